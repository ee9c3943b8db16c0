"""fp32 sub-row scales (FP8PA_SCALE_F32_G8..G256, the page's k_groups and
v_groups) on the GPU: decode parity against the float64 oracle over head dims
64-512, every group width a head dim takes (8-dim key groups included), K in
HEADS_D64 / HEADS / TOKENS, V d-major and token-major, V per token or in its
own sub-row groups, windows, sinks, split counts, empty and short sequences;
groups of very different ranges (the reason for the format); the append +
decode call; and the refusals of the variants that do not read them."""
from dataclasses import replace

import numpy as np
import pytest
import torch

from fp8_paged_kv_amd import ops
from oracle import attention as oatt, pool as opool
from tests.gpu_util import DEV, assert_parity, desc_of, gpu_decode, say, to_np
from tests.problems import make_problem

pytestmark = pytest.mark.gpu


def oracle(p):
    return oatt.decode_ref(p.q, p.k_pool, p.v_pool, p.kdesc, p.vdesc, p.table, p.seq_lens, window=p.window,
                           sinks=p.sinks, sm_scale=p.sm_scale)


CASES = [
    ("d64-g32", dict(B=3, Hq=8, Hkv=2, D=64, P=16, lens=[300, 17, 129], scale_kind="f32_g32")),
    ("d64-g64-sinks", dict(B=2, Hq=8, Hkv=2, D=64, P=16, lens=[200, 33], scale_kind="f32_g64", sinks=True)),
    ("d128-g32", dict(B=3, Hq=32, Hkv=8, D=128, P=16, lens=[1500, 64, 700], scale_kind="f32_g32")),
    ("d128-g64-window", dict(B=3, Hq=16, Hkv=4, D=128, P=16, lens=[900, 100, 20], scale_kind="f32_g64",
                             window=300, sinks=True)),
    ("d128-g32-kheads", dict(B=2, Hq=16, Hkv=2, D=128, P=32, lens=[400, 77], scale_kind="f32_g32",
                             k_layout="heads")),
    ("d128-g32-ktokens-p128", dict(B=2, Hq=16, Hkv=4, D=128, P=128, lens=[1000, 130], scale_kind="f32_g32",
                                   k_layout="tokens")),
    ("d128-g32-aligned", dict(B=3, Hq=16, Hkv=4, D=128, P=16, lens=[700, 65, 300], scale_kind="f32_g32",
                              row_pad=32, align64=True)),
    ("d256-g64-window", dict(B=2, Hq=16, Hkv=8, D=256, P=32, lens=[1500, 33], scale_kind="f32_g64", window=1024,
                             sm_scale=1.0)),
    ("d256-g128", dict(B=2, Hq=8, Hkv=2, D=256, P=32, lens=[600, 90], scale_kind="f32_g128")),
    ("d512-g32", dict(B=2, Hq=16, Hkv=2, D=512, P=32, lens=[333, 64], scale_kind="f32_g32", sm_scale=1.0)),
    ("d512-g256", dict(B=2, Hq=16, Hkv=2, D=512, P=32, lens=[333, 64], scale_kind="f32_g256")),
    ("g1-hkv8", dict(B=2, Hq=8, Hkv=8, D=64, P=16, lens=[90, 3], scale_kind="f32_g32")),
    ("empty-and-short", dict(B=4, Hq=8, Hkv=2, D=64, P=16, lens=[0, 1, 15, 65], scale_kind="f32_g32",
                             sinks=True)),
    # key groups narrower than 32 dims (k_groups 8 and 16 at head dim 128)
    ("d128-g16", dict(B=3, Hq=16, Hkv=4, D=128, P=16, lens=[700, 65, 9], scale_kind="f32_g16", sinks=True)),
    ("d128-g8-window", dict(B=2, Hq=16, Hkv=2, D=128, P=32, lens=[900, 77], scale_kind="f32_g8", window=200)),
    ("d64-g8-ktokens", dict(B=2, Hq=8, Hkv=2, D=64, P=16, lens=[300, 31], scale_kind="f32_g8", k_layout="tokens")),
    ("d256-g16-kheads", dict(B=2, Hq=8, Hkv=2, D=256, P=32, lens=[500, 40], scale_kind="f32_g16",
                             k_layout="heads")),
]


@pytest.mark.parametrize("name,kw", CASES, ids=[c[0] for c in CASES])
@pytest.mark.parametrize("workgroups", [1, 0, 5])
def test_kgroups_parity(name, kw, workgroups):
    say("k groups parity", name, "workgroups", workgroups)
    p = make_problem(701, **kw)
    assert p.vdesc.scale_kind == "token_head"
    ops.reset_counters()
    got = to_np(gpu_decode(p, workgroups=workgroups))
    c = ops.counters()
    assert c["decode_mfma_bf16"] == 1 and c["decode_packed_heads"] == 0
    assert_parity(got, oracle(p), name)


@pytest.mark.parametrize("v_layout", ["heads", "tokens"])
@pytest.mark.parametrize("D,kind", [(64, "f32_g32"), (128, "f32_g64"), (256, "f32_g32")])
def test_kgroups_token_major_v(v_layout, D, kind):
    say("k groups V", v_layout, D, kind)
    p = make_problem(702, B=3, Hq=16, Hkv=4, D=D, P=16, lens=[300, 65, 7], scale_kind=kind, v_layout=v_layout,
                     sinks=True, sm_scale=1.0 if D >= 256 else None)
    ops.reset_counters()
    got = to_np(gpu_decode(p))
    assert ops.counters()["decode_v_token_major"] == 1
    assert_parity(got, oracle(p), f"V {v_layout}")


def test_kgroups_of_very_different_ranges():
    """One 32-dim group of each key row 2**10 times larger than the rest: the
    small groups keep their precision, and the result matches the oracle."""
    say("k groups ranges")
    p = make_problem(703, B=2, Hq=16, Hkv=4, D=128, P=16, lens=[500, 70], scale_kind="f32_g32", k_layout="heads",
                     poison=True)
    from oracle import pool as _pool
    ks = []
    for x in p.raw_k:
        x = x.astype(np.float32).copy()
        x[:, :, 32:64] *= np.float32(1024.0)
        ks.append(x)
    k_pool = _pool.pack_sequences(np.full_like(p.k_pool, 0xFF), p.kdesc, p.table, ks)
    q = p.q.copy()
    q[:, :, 32:64] *= np.float32(2.0 ** -10)
    p2 = replace(p, k_pool=k_pool, q=q, raw_k=ks)
    assert_parity(to_np(gpu_decode(p2, workgroups=3)), oracle(p2), "ranges")


def test_kgroups_append_decode_takes_two_launches():
    """fp8pa_append_decode with sub-row K scales: the append kernel, then the
    decode; the same pools and output as fp8pa_append_quant then the decode."""
    p = make_problem(704, B=3, Hq=16, Hkv=4, D=128, P=16, lens=[300, 33, 16], scale_kind="f32_g32")
    kd, vd = desc_of(p.kdesc), desc_of(p.vdesc)
    table = torch.from_numpy(np.ascontiguousarray(p.table)).to(DEV)
    sl = torch.from_numpy(p.seq_lens.astype(np.int32)).to(DEV)
    q = torch.from_numpy(np.ascontiguousarray(p.q)).to(torch.bfloat16).to(DEV)
    g = torch.Generator().manual_seed(8)
    kn = torch.randn((3, 4, 128), generator=g).to(torch.bfloat16).to(DEV)
    vn = torch.randn((3, 4, 128), generator=g).to(torch.bfloat16).to(DEV)
    ka, va = torch.from_numpy(p.k_pool).to(DEV), torch.from_numpy(p.v_pool).to(DEV)
    kb, vb = ka.clone(), va.clone()
    pos = (sl - 1).to(torch.int32)
    ops.append_quant(kn[:, None], vn[:, None], ka, va, kd, vd, table, pos)
    msl = int(p.seq_lens.max())
    want = ops.decode(q, ka, va, kd, vd, table, sl, msl, sm_scale=p.sm_scale)
    ops.reset_counters()
    got = ops.append_decode(q, kn, vn, kb, vb, kd, vd, table, sl, msl, sm_scale=p.sm_scale)
    torch.cuda.synchronize()
    c = ops.counters()
    assert c["append_launches"] == 1 and c["fused_appends"] == 0
    assert torch.equal(kb, ka) and torch.equal(vb, va)
    assert torch.equal(got.view(torch.int16), want.view(torch.int16))
    # the appended pools are the oracle's, and the decode over them meets the bound
    wk = opool.append_ref(p.k_pool, p.kdesc, p.table, p.seq_lens - 1, kn.float().cpu().numpy()[:, None])
    wv = opool.append_ref(p.v_pool, p.vdesc, p.table, p.seq_lens - 1, vn.float().cpu().numpy()[:, None])
    assert np.array_equal(ka.cpu().numpy(), wk) and np.array_equal(va.cpu().numpy(), wv)
    assert_parity(to_np(got), oatt.decode_ref(p.q, wk, wv, p.kdesc, p.vdesc, p.table, p.seq_lens,
                                              sm_scale=p.sm_scale), "append + decode")


@pytest.mark.parametrize("variant", ["mfma_fp8", "packed_heads", "packed_split"])
def test_kgroups_refusals(variant):
    p = make_problem(705, B=2, Hq=16, Hkv=4, D=128, P=16, lens=[100, 30], scale_kind="f32_g32")
    ops.reset_counters()
    with pytest.raises(RuntimeError):
        gpu_decode(p, variant=variant)
    assert ops.counters()["decode_calls"] == 0
    # V in sub-row groups: refused with the packed variants and the fp8 mode too,
    # and for V groups narrower than a 16-dim PV chunk, or V groups with K per token
    pv = make_problem(705, B=2, Hq=16, Hkv=4, D=128, P=16, lens=[100, 30], scale_kind="f32_g32",
                      v_scale_kind="f32_g32")
    with pytest.raises(RuntimeError):
        gpu_decode(pv, variant=variant)
    for kk, vk in (("f32_g32", "f32_g8"), ("token_head", "f32_g32")):
        pb = make_problem(705, B=2, Hq=16, Hkv=4, D=128, P=16, lens=[100, 30], scale_kind=kk, v_scale_kind=vk)
        with pytest.raises(RuntimeError):
            gpu_decode(pb)
    assert ops.counters()["decode_calls"] == 0


VG_CASES = [
    # (name, kwargs): K and V both in fp32 sub-row groups (k_groups, v_groups)
    ("d64-k32-v32", dict(B=3, Hq=8, Hkv=2, D=64, P=16, lens=[300, 17, 129], scale_kind="f32_g32",
                         v_scale_kind="f32_g32")),
    ("d64-k8-v16-sinks", dict(B=2, Hq=8, Hkv=2, D=64, P=16, lens=[200, 33], scale_kind="f32_g8",
                              v_scale_kind="f32_g16", sinks=True)),
    ("d128-k32-v16", dict(B=3, Hq=32, Hkv=8, D=128, P=16, lens=[1500, 64, 700], scale_kind="f32_g32",
                          v_scale_kind="f32_g16")),
    ("d128-k16-v64-window", dict(B=3, Hq=16, Hkv=4, D=128, P=16, lens=[900, 100, 20], scale_kind="f32_g16",
                                 v_scale_kind="f32_g64", window=300)),
    ("d128-k64-v128-p128", dict(B=2, Hq=16, Hkv=4, D=128, P=128, lens=[1000, 130], scale_kind="f32_g64",
                                v_scale_kind="f32_g128", k_layout="tokens")),
    ("d256-k32-v32-window", dict(B=2, Hq=16, Hkv=8, D=256, P=32, lens=[1500, 33], scale_kind="f32_g32",
                                 v_scale_kind="f32_g32", window=1024, sm_scale=1.0)),
    ("d512-k64-v32", dict(B=2, Hq=16, Hkv=2, D=512, P=32, lens=[333, 64], scale_kind="f32_g64",
                          v_scale_kind="f32_g32", sm_scale=1.0)),
    ("empty-and-short", dict(B=4, Hq=8, Hkv=2, D=128, P=16, lens=[0, 1, 15, 65], scale_kind="f32_g32",
                             v_scale_kind="f32_g32", sinks=True)),
]


@pytest.mark.parametrize("name,kw", VG_CASES, ids=[c[0] for c in VG_CASES])
@pytest.mark.parametrize("workgroups", [1, 0, 5])
def test_vgroups_parity(name, kw, workgroups):
    say("v groups parity", name, "workgroups", workgroups)
    p = make_problem(706, **kw)
    got = to_np(gpu_decode(p, workgroups=workgroups))
    assert_parity(got, oracle(p), name)


@pytest.mark.parametrize("v_layout", ["heads", "tokens"])
def test_vgroups_token_major_v(v_layout):
    say("v groups V", v_layout)
    p = make_problem(707, B=3, Hq=16, Hkv=4, D=128, P=16, lens=[300, 65, 7], scale_kind="f32_g32",
                     v_scale_kind="f32_g32", v_layout=v_layout, sinks=True)
    ops.reset_counters()
    got = to_np(gpu_decode(p, workgroups=3))
    assert ops.counters()["decode_v_token_major"] == 1
    assert_parity(got, oracle(p), f"V groups {v_layout}")


def test_vgroups_of_very_different_ranges_and_poison():
    """One 16-dim V group 2**10 times larger than the rest, and NaN scales and
    codes in every unattended slot: the result matches the oracle."""
    say("v groups ranges")
    p = make_problem(708, B=2, Hq=16, Hkv=4, D=128, P=16, lens=[500, 70], scale_kind="f32_g32",
                     v_scale_kind="f32_g16", window=333)
    from oracle import pool as _pool
    vs = []
    for x in p.raw_v:
        x = x.astype(np.float32).copy()
        x[:, :, 48:64] *= np.float32(1024.0)
        vs.append(x)
    v_pool = _pool.pack_sequences(np.full_like(p.v_pool, 0xFF), p.vdesc, p.table, vs)
    p2 = replace(p, v_pool=v_pool, raw_v=vs)
    assert_parity(to_np(gpu_decode(p2, workgroups=3)), oracle(p2), "ranges")
