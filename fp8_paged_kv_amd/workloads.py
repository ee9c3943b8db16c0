"""Device-resident synthetic decode workloads (the shapes in ``configs``),
built with the library's own append kernel from seeded bf16 inputs.

Per layer: by default K pool in the "heads_d64" layout, V pool in "heads_dmajor",
both with the workload's scale kind and row stride; pages that hold no attended position
(before a window) get no row (their table entries are -1); unused slots and
spare rows hold 0xFF (NaN codes and scales).  Raw K/V of sequence b in layer l
are N(0,1) bf16 drawn for positions [first attended page * P, L) only, with
per-(layer, sequence) seeds so any sequence can be regenerated alone.
"""
from dataclasses import dataclass, field
from typing import Optional

import numpy as np
import torch

from . import configs, inputs, ops

POISON = 0xFF


@dataclass
class DeviceLayer:
    name: str
    Hq: int
    Hkv: int
    D: int
    P: int
    window: int
    sm_scale: float
    scale_kind: str
    row_bytes: int
    pool_rows: int
    kd: ops.PoolDesc
    vd: ops.PoolDesc
    k_pool: torch.Tensor
    v_pool: torch.Tensor
    block_table: torch.Tensor
    table_np: np.ndarray
    seq_lens: torch.Tensor
    lens: np.ndarray
    first_pos: np.ndarray          # first raw position written per sequence
    q: torch.Tensor
    sinks: Optional[torch.Tensor]
    sinks_np: Optional[np.ndarray]
    max_seq_len: int
    layer_index: int = 0
    extra: dict = field(default_factory=dict)

    def attended_pages(self, b):
        return [p for p in range(self.table_np.shape[1]) if self.table_np[b, p] >= 0]


def raw_kv(seed, wl, layer_index, b, tensor, n_pos, Hkv, D):
    """bf16-exact N(0,1) float32 [n_pos, Hkv, D] of one sequence of one layer."""
    return inputs.normal_bf16(seed, wl.index, tensor, layer_index * 4096 + b, (n_pos, Hkv, D))


GROUP_DIMS = {"f32_g8": 8, "f32_g16": 16, "f32_g32": 32, "f32_g64": 64, "f32_g128": 128, "f32_g256": 256}


def scale_block_bytes(scale_kind, Hkv, P, D):
    if scale_kind in GROUP_DIMS:
        return 4 * Hkv * P * (D // GROUP_DIMS[scale_kind])
    return {"page_head": 4 * Hkv, "token_head": 4 * Hkv * P, "e8m0_32": Hkv * P * D // 32}[scale_kind]


def v_kind_of(scale_kind):
    """V scale kind paired with a K kind: per-(token, head) V for sub-row K groups."""
    return "token_head" if scale_kind in GROUP_DIMS else scale_kind


def rows_can_align(row_bytes, payload, scales):
    """Whether every payload shift rows of this width take (to the 64-byte
    grid) leaves room for the payload and the scale block."""
    for r in range(64):
        sh = (-r * row_bytes) % 64
        end = sh + payload if sh >= scales else sh + payload + scales
        if end > row_bytes:
            return False
    return True


def first_attended_page(L, window, P):
    start = max(0, L - window) if window > 0 else 0
    return start // P


def build_workload(wl: configs.Workload, seed=configs.SEED, device="cuda:0", layers=None, verbose=False,
                   k_layout="heads_d64", v_layout="heads_dmajor", scale_kind=None, row_align=16):
    """Build the device pools of the workload's layers (all, or the indices in
    ``layers``).  Layers of a shared-pool workload index disjoint rows of one
    K pool and one V pool.  ``k_layout``, ``v_layout`` and ``scale_kind``
    replace the defaults (the workload's own scale kind); a scale block that
    does not fit the layer's row width widens the rows to the natural row,
    rounded up to 16 bytes.  ``row_align`` > 16 rounds the row width up to a
    multiple of it (128: every row starts on a 128-byte line, as token-major
    pools need for whole-line loads)."""
    scale_kind = wl.scale_kind if scale_kind is None else scale_kind
    lens = inputs.seq_lens(seed, wl.index, wl.B, wl.L_lo, wl.L_hi)
    P = wl.P
    idx = list(range(len(wl.layers))) if layers is None else list(layers)
    ranges = {}
    for li, lay in enumerate(wl.layers):
        ranges[li] = [(first_attended_page(int(L), lay.window, P), -(-int(L) // P)) for L in lens]
    tables = {}
    width = -(-int(wl.L_hi) // P)        # table width covers the longest sequence the workload allows
    if wl.shared_pool:
        need = sum(e - a for li in range(len(wl.layers)) for a, e in ranges[li])
        pool_rows = need + max(1, int(np.ceil(need * 0.05)))
        taken = np.zeros(0, dtype=np.int64)
        for li in range(len(wl.layers)):
            t, rows, _ = inputs.block_table_ranges(seed, wl.index, ranges[li], P, pool_rows=pool_rows, tag=li,
                                                   exclude=taken, width=width)
            taken = np.concatenate([taken, rows])
            tables[li] = (t, pool_rows)
    else:
        for li in range(len(wl.layers)):
            t, _, pool_rows = inputs.block_table_ranges(seed, wl.index, ranges[li], P, tag=li, width=width)
            tables[li] = (t, pool_rows)
    row_width = {}
    for li, lay in enumerate(wl.layers):
        natural = P * lay.Hkv * lay.D + max(scale_block_bytes(scale_kind, lay.Hkv, P, lay.D),
                                            scale_block_bytes(v_kind_of(scale_kind), lay.Hkv, P, lay.D))
        row_width[li] = max(lay.row_bytes, -(-natural // 16) * 16)
        row_width[li] = -(-row_width[li] // row_align) * row_align
    if wl.shared_pool:   # one row width for the layers of a shared pool
        row_width = {li: max(row_width.values()) for li in row_width}
    sinks_np = inputs.sinks(seed, wl.index, wl.layers[0].Hq) if wl.sinks else None
    shared = {}
    out = []
    for li in idx:
        lay = wl.layers[li]
        table, pool_rows = tables[li]
        rb = row_width[li]
        # Rows are placed with their payloads on the 64-byte grid when the row
        # width leaves room for it (the row widths carry a 32-byte scale
        # footer, so half the rows would start 32 bytes off the grid).
        al = all(rows_can_align(rb, P * lay.Hkv * lay.D, scale_block_bytes(k, lay.Hkv, P, lay.D))
                 for k in (scale_kind, v_kind_of(scale_kind)))
        kd = ops.pool_desc(lay.Hkv, lay.D, P, k_layout, scale_kind, rb, pool_rows, align64=al)
        vd = ops.pool_desc(lay.Hkv, lay.D, P, v_layout, v_kind_of(scale_kind), rb, pool_rows, align64=al)
        if wl.shared_pool and "k" in shared:
            k_pool, v_pool = shared["k"], shared["v"]
        else:
            k_pool = torch.full((pool_rows * rb,), POISON, dtype=torch.uint8, device=device)
            v_pool = torch.full((pool_rows * rb,), POISON, dtype=torch.uint8, device=device)
            if wl.shared_pool:
                shared["k"], shared["v"] = k_pool, v_pool
        bt = torch.from_numpy(table).to(device)
        first = np.array([a * P for a, _ in ranges[li]], dtype=np.int64)
        for b, L in enumerate(lens):
            n = int(L) - int(first[b])
            if n <= 0:
                continue
            xk = torch.from_numpy(raw_kv(seed, wl, li, b, "k", n, lay.Hkv, lay.D)).to(torch.bfloat16)
            xv = torch.from_numpy(raw_kv(seed, wl, li, b, "v", n, lay.Hkv, lay.D)).to(torch.bfloat16)
            ops.append_quant(xk.to(device)[None], xv.to(device)[None], k_pool, v_pool, kd, vd, bt[b:b + 1],
                             torch.tensor([int(first[b])], dtype=torch.int32, device=device))
            if verbose and b % 16 == 0:
                print(f"  {wl.name}/{lay.name}: appended sequence {b}/{len(lens)}", flush=True)
        q = torch.from_numpy(inputs.normal_bf16(seed, wl.index, "q", li, (wl.B, lay.Hq, lay.D))).to(
            torch.bfloat16).to(device)
        out.append(DeviceLayer(
            name=f"{wl.name}/{lay.name}", Hq=lay.Hq, Hkv=lay.Hkv, D=lay.D, P=P, window=lay.window,
            sm_scale=lay.D ** -0.5 if lay.sm_scale is None else lay.sm_scale, scale_kind=scale_kind,
            row_bytes=rb, pool_rows=pool_rows, kd=kd, vd=vd, k_pool=k_pool, v_pool=v_pool, block_table=bt,
            table_np=table, seq_lens=torch.from_numpy(lens.astype(np.int32)).to(device), lens=lens,
            first_pos=first, q=q, sinks=None if sinks_np is None else torch.from_numpy(sinks_np).to(device),
            sinks_np=sinks_np, max_seq_len=int(wl.L_hi), layer_index=li))
    torch.cuda.synchronize()
    return out


def decode_layer(layer: DeviceLayer, out=None, workspace=None, workgroups=0, stream=None, variant="auto"):
    return ops.decode(layer.q, layer.k_pool, layer.v_pool, layer.kd, layer.vd, layer.block_table, layer.seq_lens,
                      layer.max_seq_len, window=layer.window, sinks=layer.sinks, sm_scale=layer.sm_scale,
                      workgroups=workgroups, variant=variant, out=out, workspace=workspace, stream=stream)


def kv_bytes(layer: DeviceLayer):
    """Algorithmic KV bytes one decode call must read: the E4M3 codes of the
    attended positions of K and V plus the scale bytes those positions touch."""
    total = 0
    for L in layer.lens:
        L = int(L)
        start = max(0, L - layer.window) if layer.window > 0 else 0
        n = L - start
        if n <= 0:
            continue
        payload = 2 * n * layer.D * layer.Hkv
        if layer.scale_kind == "page_head":
            pages = (L - 1) // layer.P - start // layer.P + 1
            sc = 2 * 4 * pages * layer.Hkv
        elif layer.scale_kind == "token_head":
            sc = 2 * 4 * n * layer.Hkv
        elif layer.scale_kind in GROUP_DIMS:   # K: one fp32 per group; V: one per (token, head)
            sc = 4 * n * (layer.D // GROUP_DIMS[layer.scale_kind]) * layer.Hkv + 4 * n * layer.Hkv
        else:
            sc = 2 * n * (layer.D // 32) * layer.Hkv
        total += payload + sc
    return total
