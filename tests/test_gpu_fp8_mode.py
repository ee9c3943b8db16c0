"""The fp8 compute mode (FP8PA_VARIANT_MFMA_FP8) on the GPU: QK^T on the fp8
MFMA with each query row rounded to E4M3 like a KV block (codes of q / s).
Against the oracle that models that one rounding (decode of ``fp8_query(q)``)
it meets the default parity bound; against the exact oracle it meets the
page's fp8 tolerance class (1.5e-1) on every served case (the mode serves
|sm_scale| <= D^-0.5 only); the counter records the mode; requests it cannot
serve are refused, never downgraded."""
import numpy as np
import pytest
import torch

from fp8_paged_kv_amd import ops
from oracle import attention as oatt
from tests.gpu_util import assert_parity, gpu_decode, say, to_np
from tests.problems import make_problem

pytestmark = pytest.mark.gpu

FP8_TOL = 1.5e-1


def oracle(p, q=None):
    return oatt.decode_ref(p.q if q is None else q, p.k_pool, p.v_pool, p.kdesc, p.vdesc, p.table, p.seq_lens,
                           window=p.window, sinks=p.sinks, sm_scale=p.sm_scale)


CASES = [
    ("d64-g4", dict(B=3, Hq=8, Hkv=2, D=64, P=16, lens=[300, 17, 129])),
    ("d128-g4", dict(B=3, Hq=16, Hkv=4, D=128, P=16, lens=[513, 64, 1])),
    ("d128-g8-sinks-token-scales", dict(B=2, Hq=16, Hkv=2, D=128, P=16, lens=[400, 77], sinks=True,
                                        scale_kind="token_head")),
    ("d64-window-sinks", dict(B=3, Hq=16, Hkv=2, D=64, P=16, lens=[500, 100, 20], window=128, sinks=True)),
    ("d128-aligned-rows", dict(B=3, Hq=16, Hkv=4, D=128, P=16, lens=[700, 65, 300], row_pad=32, align64=True)),
    ("d128-ktokens", dict(B=2, Hq=8, Hkv=2, D=128, P=16, lens=[260, 5], k_layout="tokens")),
    ("d128-kheads-p32", dict(B=2, Hq=8, Hkv=2, D=128, P=32, lens=[260, 77], k_layout="heads")),
    ("d256-window", dict(B=2, Hq=4, Hkv=2, D=256, P=32, lens=[700, 33], window=100)),
    ("d512-g8", dict(B=2, Hq=8, Hkv=1, D=512, P=32, lens=[333, 64])),
    ("d256-p16-small-scale", dict(B=2, Hq=8, Hkv=2, D=256, P=16, lens=[300, 41], sm_scale=0.03)),
    ("empty-and-short", dict(B=4, Hq=8, Hkv=2, D=64, P=16, lens=[0, 1, 15, 65])),
]


@pytest.mark.parametrize("name,kw", CASES, ids=[c[0] for c in CASES])
@pytest.mark.parametrize("workgroups", [1, 0, 3])
def test_fp8_mode_parity(name, kw, workgroups):
    say("fp8 mode parity", name, "workgroups", workgroups)
    p = make_problem(401, **kw)
    ops.reset_counters()
    got = to_np(gpu_decode(p, workgroups=workgroups, variant="mfma_fp8"))
    c = ops.counters()
    assert c["decode_mfma_fp8"] == 1 and c["decode_mfma_bf16"] == 0
    # the one rounding the mode adds, modelled exactly: the default bound
    assert_parity(got, oracle(p, oatt.fp8_query(p.q)), name)
    # the exact result: the page's fp8 tolerance class
    want = oracle(p)
    assert np.all(np.abs(got - want) <= FP8_TOL + FP8_TOL * np.abs(want)), name


def test_fp8_mode_rounds_q_and_keeps_query_range():
    """The mode differs from the bf16 one (q is rounded), and a query row of any
    magnitude is served by its own scale: rows 2**-12 and 2**12 times larger
    than N(0,1), and an all-zero row (uniform attention)."""
    p = make_problem(402, B=2, Hq=16, Hkv=4, D=128, P=16, lens=[300, 90], sm_scale=2.0 ** -10)
    q = p.q.astype(np.float64).copy()
    q[0, 1] *= 2.0 ** -12
    q[0, 2] *= 2.0 ** 12
    q[1, 3] = 0.0
    from dataclasses import replace
    p2 = replace(p, q=q.astype(np.float32))
    got = to_np(gpu_decode(p2, variant="mfma_fp8"))
    assert_parity(got, oracle(p2, oatt.fp8_query(p2.q)), "query range")
    bf = to_np(gpu_decode(p2))
    assert not np.array_equal(got, bf)


def test_fp8_mode_refusals():
    p = make_problem(403, B=2, Hq=16, Hkv=2, D=64, P=128, lens=[300, 90], scale_kind="e8m0_32")
    ops.reset_counters()
    with pytest.raises(RuntimeError):                  # E8M0 at 64 dims: the MX MFMA contracts 128
        gpu_decode(p, variant="mfma_fp8")
    p = make_problem(403, B=2, Hq=16, Hkv=2, D=128, P=16, lens=[300, 90], v_layout="tokens")
    with pytest.raises(RuntimeError):
        gpu_decode(p, variant="mfma_fp8")
    # score scales above D^-0.5 (sm_scale = 1 at D = 256 and at D = 64)
    for D, P in ((256, 32), (64, 16)):
        p = make_problem(403, B=2, Hq=8, Hkv=2, D=D, P=P, lens=[300, 90], sm_scale=1.0)
        with pytest.raises(RuntimeError):
            gpu_decode(p, variant="mfma_fp8")
    c = ops.counters()
    assert c["decode_calls"] == 0 and c["decode_mfma_fp8"] == 0 and c["errors"] == 4


def test_fp8_mode_append_decode_takes_two_launches():
    """fp8pa_append_decode in the fp8 mode: the append kernel, then the fp8
    decode; the same pools and output as fp8pa_append_quant then the decode."""
    from tests.gpu_util import DEV, desc_of
    p = make_problem(404, B=3, Hq=16, Hkv=4, D=128, P=16, lens=[300, 33, 16])
    kd, vd = desc_of(p.kdesc), desc_of(p.vdesc)
    table = torch.from_numpy(np.ascontiguousarray(p.table)).to(DEV)
    sl = torch.from_numpy(p.seq_lens.astype(np.int32)).to(DEV)
    q = torch.from_numpy(np.ascontiguousarray(p.q)).to(torch.bfloat16).to(DEV)
    g = torch.Generator().manual_seed(5)
    kn = torch.randn((3, 4, 128), generator=g).to(torch.bfloat16).to(DEV)
    vn = torch.randn((3, 4, 128), generator=g).to(torch.bfloat16).to(DEV)
    ka, va = torch.from_numpy(p.k_pool).to(DEV), torch.from_numpy(p.v_pool).to(DEV)
    kb, vb = ka.clone(), va.clone()
    pos = (sl - 1).to(torch.int32)
    ops.append_quant(kn[:, None], vn[:, None], ka, va, kd, vd, table, pos)
    want = ops.decode(q, ka, va, kd, vd, table, sl, int(p.seq_lens.max()), sm_scale=p.sm_scale, variant="mfma_fp8")
    ops.reset_counters()
    got = ops.append_decode(q, kn, vn, kb, vb, kd, vd, table, sl, int(p.seq_lens.max()), sm_scale=p.sm_scale,
                            variant="mfma_fp8")
    torch.cuda.synchronize()
    c = ops.counters()
    assert c["append_launches"] == 1 and c["fused_appends"] == 0 and c["decode_mfma_fp8"] == 1
    assert torch.equal(kb, ka) and torch.equal(vb, va)
    assert torch.equal(got.view(torch.int16), want.view(torch.int16))


MX_CASES = [
    ("d128-p128", dict(B=2, Hq=16, Hkv=2, D=128, P=128, lens=[1000, 130])),
    ("d128-p16-sinks", dict(B=3, Hq=16, Hkv=4, D=128, P=16, lens=[513, 64, 1], sinks=True)),
    ("d128-window", dict(B=2, Hq=16, Hkv=2, D=128, P=32, lens=[900, 77], window=200)),
    ("d128-kheads", dict(B=2, Hq=8, Hkv=2, D=128, P=32, lens=[260, 77], k_layout="heads")),
    ("d128-ktokens", dict(B=2, Hq=8, Hkv=2, D=128, P=16, lens=[260, 5], k_layout="tokens")),
    ("d256", dict(B=2, Hq=8, Hkv=2, D=256, P=32, lens=[300, 41])),
    ("d512-g8", dict(B=2, Hq=8, Hkv=1, D=512, P=32, lens=[333, 64])),
    ("empty-and-short", dict(B=4, Hq=8, Hkv=2, D=128, P=16, lens=[0, 1, 15, 65])),
]


@pytest.mark.parametrize("name,kw", MX_CASES, ids=[c[0] for c in MX_CASES])
@pytest.mark.parametrize("workgroups", [1, 0, 3])
def test_mx_fp8_mode_parity(name, kw, workgroups):
    """The fp8 mode over E8M0 pools: q rounded to MXFP8 (E8M0 per 32 dims),
    QK^T on the MX-scaled fp8 MFMA.  Within the default bound of the oracle
    decoding fp8_query_mx(q), and within the page's fp8 class of the exact
    oracle; the MX counter records it."""
    say("mx fp8 mode parity", name, "workgroups", workgroups)
    p = make_problem(411, scale_kind="e8m0_32", **kw)
    ops.reset_counters()
    got = to_np(gpu_decode(p, workgroups=workgroups, variant="mfma_fp8"))
    c = ops.counters()
    assert c["decode_mfma_fp8"] == 1 and c["decode_mfma_mxfp8"] == 1 and c["decode_mfma_bf16"] == 0
    assert_parity(got, oracle(p, oatt.fp8_query_mx(p.q)), name)
    want = oracle(p)
    assert np.all(np.abs(got - want) <= FP8_TOL + FP8_TOL * np.abs(want)), name


def test_mx_fp8_mode_refusals():
    p = make_problem(412, B=2, Hq=8, Hkv=2, D=64, P=16, lens=[300, 90], scale_kind="e8m0_32")
    ops.reset_counters()
    with pytest.raises(RuntimeError):                  # 64 dims: the MX MFMA contracts 128
        gpu_decode(p, variant="mfma_fp8")
    p = make_problem(412, B=2, Hq=8, Hkv=2, D=128, P=16, lens=[300, 90], scale_kind="e8m0_32", v_layout="tokens")
    with pytest.raises(RuntimeError):
        gpu_decode(p, variant="mfma_fp8")
    c = ops.counters()
    assert c["decode_calls"] == 0 and c["decode_mfma_mxfp8"] == 0 and c["errors"] == 2
