"""The five decode workloads, as shapes only (no arithmetic).

Shapes follow the model families the method page names (Llama-3-style GQA,
gpt-oss with sinks and alternating window/full layers, a Gemma-4-like pool
holding two KV geometries, Granite-style custom scale) and the MXFP8 page's
long-context decode (64 query heads, head dim 128, 128-token blocks).
``row_bytes`` is the pool stride: the natural row (payload + scale footer)
rounded up to 16 bytes, or the shared stride of the mixed-geometry pool.
"""
from dataclasses import dataclass
from typing import Optional

SEED = 20261203


@dataclass(frozen=True)
class Layer:
    name: str
    Hq: int
    Hkv: int
    D: int
    window: int = 0                 # <= 0: full attention
    sm_scale: Optional[float] = None  # None: D ** -0.5
    row_bytes: int = 0


@dataclass(frozen=True)
class Workload:
    index: int
    name: str
    B: int
    P: int
    L_lo: int
    L_hi: int
    scale_kind: str
    layers: tuple
    sinks: bool = False
    shared_pool: bool = False       # all layers index one K pool and one V pool


TINY = Workload(0, "tiny", B=1, P=16, L_lo=256, L_hi=256, scale_kind="page_head",
                layers=(Layer("full", 8, 2, 64, sm_scale=0.125, row_bytes=2064),))
LLAMA3_8B = Workload(1, "llama3-8b-decode", B=32, P=16, L_lo=1024, L_hi=8192, scale_kind="page_head",
                     layers=(Layer("full", 32, 8, 128, sm_scale=128 ** -0.5, row_bytes=16416),))
GPT_OSS = Workload(2, "gpt-oss-decode", B=64, P=16, L_lo=2048, L_hi=32768, scale_kind="page_head",
                   layers=(Layer("window128", 64, 8, 64, window=128, row_bytes=8224),
                           Layer("full", 64, 8, 64, row_bytes=8224)), sinks=True)
GEMMA4_MIXED = Workload(3, "gemma4-mixed-pool", B=16, P=32, L_lo=4096, L_hi=16384, scale_kind="page_head",
                        layers=(Layer("window1024", 16, 8, 256, window=1024, sm_scale=1.0, row_bytes=65568),
                                Layer("full", 16, 2, 512, sm_scale=1.0, row_bytes=65568)), shared_pool=True)
LONG_MXFP8 = Workload(4, "long-context-mxfp8", B=4, P=128, L_lo=131072, L_hi=131072, scale_kind="e8m0_32",
                      layers=(Layer("full", 64, 8, 128, row_bytes=135168),))

ALL = (TINY, LLAMA3_8B, GPT_OSS, GEMMA4_MIXED, LONG_MXFP8)
