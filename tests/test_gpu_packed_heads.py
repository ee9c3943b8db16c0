"""Packed heads (FP8PA_VARIANT_PACKED_HEADS) on the GPU: one workgroup per
(sequence, group of KV heads), one head per wave, no split.  Parity against
the float64 oracle over head dims 64-512, every scale kind, windows, sinks,
aligned rows, KV-head counts that do not fill a workgroup, empty and short
sequences; the plan's fixed grid; the counter; refusals; the append + decode
call; and poison outside the attended positions."""
from dataclasses import replace

import numpy as np
import pytest
import torch

from fp8_paged_kv_amd import ops
from oracle import attention as oatt
from tests.gpu_util import DEV, assert_parity, desc_of, gpu_decode, say, to_np
from tests.problems import add_guard_rows, make_problem

pytestmark = pytest.mark.gpu


def oracle(p):
    return oatt.decode_ref(p.q, p.k_pool, p.v_pool, p.kdesc, p.vdesc, p.table, p.seq_lens, window=p.window,
                           sinks=p.sinks, sm_scale=p.sm_scale)


CASES = [
    ("tiny-hkv2", dict(B=1, Hq=8, Hkv=2, D=64, P=16, lens=[256])),
    ("d64-g8-window-sinks", dict(B=3, Hq=64, Hkv=8, D=64, P=16, lens=[500, 100, 20], window=128, sinks=True)),
    ("d128-g4", dict(B=3, Hq=16, Hkv=4, D=128, P=16, lens=[513, 64, 1])),
    ("d128-hkv8-ktokens", dict(B=2, Hq=32, Hkv=8, D=128, P=16, lens=[260, 5], k_layout="tokens")),
    ("d128-hkv6-kheads", dict(B=2, Hq=24, Hkv=6, D=128, P=32, lens=[260, 77], k_layout="heads")),
    ("d128-token-scales", dict(B=2, Hq=16, Hkv=4, D=128, P=16, lens=[700, 65], scale_kind="token_head")),
    ("d128-aligned-rows", dict(B=3, Hq=16, Hkv=4, D=128, P=16, lens=[700, 65, 300], row_pad=32, align64=True)),
    ("d128-e8m0-p128", dict(B=2, Hq=16, Hkv=2, D=128, P=128, lens=[1000, 130], scale_kind="e8m0_32")),
    ("d256-hkv8-window", dict(B=2, Hq=16, Hkv=8, D=256, P=32, lens=[1500, 33], window=1024, sm_scale=1.0)),
    ("d256-p16", dict(B=3, Hq=16, Hkv=4, D=256, P=16, lens=[300, 65, 7], sinks=True, sm_scale=1.0)),
    ("d512-g8", dict(B=2, Hq=16, Hkv=2, D=512, P=32, lens=[333, 64], sm_scale=1.0)),
    ("g16-hkv1", dict(B=1, Hq=16, Hkv=1, D=64, P=64, lens=[450])),
    ("empty-and-short", dict(B=4, Hq=8, Hkv=2, D=64, P=16, lens=[0, 1, 15, 65], sinks=True)),
    ("long-20k", dict(B=1, Hq=8, Hkv=2, D=64, P=16, lens=[20000])),
]


@pytest.mark.parametrize("name,kw", CASES, ids=[c[0] for c in CASES])
def test_packed_heads_parity(name, kw):
    say("packed heads parity", name)
    p = make_problem(501, **kw)
    plan = ops.decode_plan(p.B, p.Hq, desc_of(p.kdesc), desc_of(p.vdesc), int(p.seq_lens.max()), p.window, variant="packed_heads")
    assert plan.workgroups == p.B * -(-p.Hkv // 4) and plan.workspace_bytes == 0
    ops.reset_counters()
    got = to_np(gpu_decode(p, variant="packed_heads"))
    c = ops.counters()
    assert c["decode_packed_heads"] == 1 and c["decode_split"] == 0 and c["decode_mfma_bf16"] == 1
    assert_parity(got, oracle(p), name)


def test_packed_heads_poison_never_leaks():
    p = make_problem(502, B=3, Hq=8, Hkv=2, D=64, P=16, lens=[37, 16, 250], window=50, sinks=True)
    p, guard = add_guard_rows(p)
    t = p.table.copy()
    for b in range(3):
        used = -(-int(p.seq_lens[b]) // 16)
        t[b, used:] = -1
    t[2, : (250 - 50) // 16] = -7
    t[2, 0], t[0, -1] = guard      # never-read entries on poisoned guard rows
    got = to_np(gpu_decode(replace(p, table=t), variant="packed_heads"))
    assert np.all(np.isfinite(got))
    assert_parity(got, oracle(p), "poison")


@pytest.mark.parametrize("v_layout,D", [("tokens", 64), ("heads", 128), ("tokens", 256), ("heads", 512)])
def test_packed_heads_token_major_v(v_layout, D):
    """Packed heads with V in the page's token-major orders: the packed kernel
    with a per-wave V stage, its fixed grid and no workspace.  (These calls
    once went to the split kernel for token-major V, handed the packed grid
    and no partial buffers; at head dim 256 that kernel cut a unit and stored
    its partial through a null pointer.)"""
    say("packed heads V", v_layout, D)
    p = make_problem(505, B=3, Hq=16, Hkv=4, D=D, P=16, lens=[300, 65, 7], v_layout=v_layout, sinks=True,
                     sm_scale=1.0 if D >= 256 else None)
    plan = ops.decode_plan(p.B, p.Hq, desc_of(p.kdesc), desc_of(p.vdesc), 300, variant="packed_heads")
    assert plan.variant == ops.VARIANTS["packed_heads"] and plan.workgroups == 3 and plan.workspace_bytes == 0
    ops.reset_counters()
    got = to_np(gpu_decode(p, variant="packed_heads"))
    c = ops.counters()
    assert c["decode_packed_heads"] == 1 and c["decode_v_token_major"] == 1 and c["decode_split"] == 0
    assert_parity(got, oracle(p), f"V {v_layout}")


def test_packed_heads_refusals():
    p = make_problem(503, B=2, Hq=8, Hkv=2, D=64, P=16, lens=[100, 30], scale_kind="f32_g32")
    with pytest.raises(RuntimeError):
        gpu_decode(p, variant="packed_heads")
    p = make_problem(503, B=2, Hq=8, Hkv=2, D=64, P=16, lens=[100, 30])
    with pytest.raises(RuntimeError):
        gpu_decode(p, variant="packed_heads", workgroups=3)


def test_packed_heads_append_decode():
    """fp8pa_append_decode with packed heads: the append kernel, then the
    packed decode; the same pools and output as the two calls."""
    p = make_problem(504, B=3, Hq=32, Hkv=8, D=64, P=16, lens=[200, 33, 16], window=128)
    kd, vd = desc_of(p.kdesc), desc_of(p.vdesc)
    table = torch.from_numpy(np.ascontiguousarray(p.table)).to(DEV)
    sl = torch.from_numpy(p.seq_lens.astype(np.int32)).to(DEV)
    q = torch.from_numpy(np.ascontiguousarray(p.q)).to(torch.bfloat16).to(DEV)
    g = torch.Generator().manual_seed(6)
    kn = torch.randn((3, 8, 64), generator=g).to(torch.bfloat16).to(DEV)
    vn = torch.randn((3, 8, 64), generator=g).to(torch.bfloat16).to(DEV)
    ka, va = torch.from_numpy(p.k_pool).to(DEV), torch.from_numpy(p.v_pool).to(DEV)
    kb, vb = ka.clone(), va.clone()
    msl = int(p.seq_lens.max())
    ops.append_quant(kn[:, None], vn[:, None], ka, va, kd, vd, table, (sl - 1).to(torch.int32))
    want = ops.decode(q, ka, va, kd, vd, table, sl, msl, window=128, sm_scale=p.sm_scale, variant="packed_heads")
    ops.reset_counters()
    got = ops.append_decode(q, kn, vn, kb, vb, kd, vd, table, sl, msl, window=128, sm_scale=p.sm_scale,
                            variant="packed_heads")
    torch.cuda.synchronize()
    c = ops.counters()
    assert c["append_launches"] == 1 and c["fused_appends"] == 0 and c["decode_packed_heads"] == 1
    assert torch.equal(kb, ka) and torch.equal(vb, va)
    assert torch.equal(got.view(torch.int16), want.view(torch.int16))


def test_auto_takes_packed_heads_when_units_fill_the_device():
    """A batch whose (sequence, four KV heads) units fill every resident
    workgroup slot: an automatic call runs packed heads (and the append +
    decode call runs the append kernel, then that decode); V token-major or a
    small batch keeps the split kernel."""
    say("auto packed")
    p = make_problem(506, B=320, Hq=32, Hkv=8, D=64, P=16, lens=list(range(1, 321)), sinks=True)
    kd = desc_of(p.kdesc)
    plan = ops.decode_plan(p.B, p.Hq, kd, desc_of(p.vdesc), int(p.seq_lens.max()))
    assert plan.variant == ops.VARIANTS["packed_heads"] and plan.workspace_bytes == 0
    assert plan.workgroups == p.B * 2
    ops.reset_counters()
    got = gpu_decode(p)
    c = ops.counters()
    assert c["decode_packed_heads"] == 1 and c["decode_split"] == 0
    assert_parity(to_np(got), oracle(p), "auto packed")
    # V token-major, or a small batch: the split kernel
    pv = make_problem(506, B=320, Hq=32, Hkv=8, D=64, P=16, lens=list(range(1, 321)), v_layout="tokens")
    assert ops.decode_plan(pv.B, pv.Hq, kd, desc_of(pv.vdesc), 320).variant == ops.VARIANTS["mfma_bf16"]
    ops.reset_counters()
    assert_parity(to_np(gpu_decode(pv)), oracle(pv), "auto V tokens")
    assert ops.counters()["decode_packed_heads"] == 0
    ps = make_problem(507, B=3, Hq=32, Hkv=8, D=64, P=16, lens=[100, 30, 5])
    ops.reset_counters()
    gpu_decode(ps)
    assert ops.counters()["decode_packed_heads"] == 0
    # append + decode: two launches, the same output as append then decode
    table = torch.from_numpy(np.ascontiguousarray(p.table)).to(DEV)
    sl = torch.from_numpy(p.seq_lens.astype(np.int32)).to(DEV)
    q = torch.from_numpy(np.ascontiguousarray(p.q)).to(torch.bfloat16).to(DEV)
    sinks = torch.from_numpy(p.sinks).to(DEV)
    g = torch.Generator().manual_seed(7)
    kn = torch.randn((p.B, 8, 64), generator=g).to(torch.bfloat16).to(DEV)
    vn = torch.randn((p.B, 8, 64), generator=g).to(torch.bfloat16).to(DEV)
    ka, va = torch.from_numpy(p.k_pool).to(DEV), torch.from_numpy(p.v_pool).to(DEV)
    kb, vb = ka.clone(), va.clone()
    msl = int(p.seq_lens.max())
    vd = desc_of(p.vdesc)
    ops.append_quant(kn[:, None], vn[:, None], ka, va, kd, vd, table, (sl - 1).to(torch.int32))
    want = ops.decode(q, ka, va, kd, vd, table, sl, msl, sinks=sinks, sm_scale=p.sm_scale)
    ops.reset_counters()
    out = ops.append_decode(q, kn, vn, kb, vb, kd, vd, table, sl, msl, sinks=sinks, sm_scale=p.sm_scale)
    torch.cuda.synchronize()
    c = ops.counters()
    assert c["append_launches"] == 1 and c["fused_appends"] == 0 and c["decode_packed_heads"] == 1
    assert torch.equal(kb, ka) and torch.equal(vb, va)
    assert torch.equal(out.view(torch.int16), want.view(torch.int16))
