"""Decode parity on the GPU against the float64 oracle, on problems small
enough for the oracle yet spanning several tiles and splits with ragged tails,
plus the edge cases and invariants of the method."""
import os
from dataclasses import replace

import numpy as np
import pytest
import torch

from fp8_paged_kv_amd import ops
from oracle import attention as oatt
from tests.gpu_util import assert_parity, device_problem, gpu_decode, say, to_np
from tests.problems import add_guard_rows, make_problem, permute_rows

pytestmark = pytest.mark.gpu


def oracle(p, **kw):
    a = dict(window=p.window, sinks=p.sinks, sm_scale=p.sm_scale)
    a.update(kw)
    return oatt.decode_ref(p.q, p.k_pool, p.v_pool, p.kdesc, p.vdesc, p.table, p.seq_lens, **a)


CASES = [
    # (name, kwargs)
    ("d64-g4", dict(B=3, Hq=8, Hkv=2, D=64, P=16, lens=[300, 17, 129])),
    ("d128-g4", dict(B=3, Hq=16, Hkv=4, D=128, P=16, lens=[513, 64, 1])),
    ("d128-g8-sinks", dict(B=2, Hq=16, Hkv=2, D=128, P=16, lens=[400, 77], sinks=True)),
    ("d64-g8-window", dict(B=3, Hq=16, Hkv=2, D=64, P=16, lens=[500, 100, 20], window=128, sinks=True)),
    # rows 32 bytes off the 64-byte grid, payloads placed on it
    ("d128-aligned-rows", dict(B=3, Hq=16, Hkv=4, D=128, P=16, lens=[700, 65, 300], row_pad=32, align64=True)),
    ("d64-aligned-rows-window", dict(B=2, Hq=16, Hkv=2, D=64, P=16, lens=[900, 130], row_pad=80, align64=True,
                                     window=200, sinks=True)),
    ("d512-aligned-rows", dict(B=2, Hq=16, Hkv=2, D=512, P=32, lens=[300, 97], row_pad=16, align64=True,
                               sm_scale=1.0)),
    ("d256-g2-window-scale1", dict(B=2, Hq=4, Hkv=2, D=256, P=32, lens=[700, 33], window=100, sm_scale=1.0)),
    ("d512-g8-scale1", dict(B=2, Hq=8, Hkv=1, D=512, P=32, lens=[333, 64], sm_scale=1.0)),
    ("d128-e8m0-p128", dict(B=2, Hq=16, Hkv=2, D=128, P=128, lens=[1000, 130], scale_kind="e8m0_32")),
    ("d64-token-scale", dict(B=2, Hq=8, Hkv=2, D=64, P=16, lens=[250, 31], scale_kind="token_head")),
    ("d128-ktokens", dict(B=2, Hq=8, Hkv=2, D=128, P=16, lens=[260, 5], k_layout="tokens")),
    ("d128-kheads", dict(B=2, Hq=8, Hkv=2, D=128, P=32, lens=[260, 77], k_layout="heads")),
    ("d64-kheads-p128", dict(B=1, Hq=8, Hkv=2, D=64, P=128, lens=[700], k_layout="heads", sinks=True)),
    ("d256-p256-vblocks", dict(B=1, Hq=8, Hkv=2, D=256, P=256, lens=[900], window=300)),
    ("d256-p16", dict(B=3, Hq=16, Hkv=4, D=256, P=16, lens=[300, 65, 7], sinks=True, sm_scale=1.0)),
    ("g1-mqa-like", dict(B=2, Hq=2, Hkv=2, D=64, P=16, lens=[90, 3])),
    ("g16", dict(B=1, Hq=16, Hkv=1, D=64, P=64, lens=[450])),
    ("wide-rows", dict(B=2, Hq=8, Hkv=2, D=64, P=16, lens=[100, 50], row_pad=4096)),
    ("d256-e8m0", dict(B=1, Hq=8, Hkv=2, D=256, P=32, lens=[300], scale_kind="e8m0_32", sinks=True)),
    ("d512-e8m0-window", dict(B=1, Hq=8, Hkv=1, D=512, P=16, lens=[260], scale_kind="e8m0_32", window=40)),
]


@pytest.mark.parametrize("name,kw", CASES, ids=[c[0] for c in CASES])
@pytest.mark.parametrize("workgroups", [1, 0, 3])
def test_decode_parity(name, kw, workgroups):
    say("decode parity", name, "workgroups", workgroups)
    p = make_problem(101, **kw)
    got = to_np(gpu_decode(p, workgroups=workgroups))
    assert_parity(got, oracle(p), name)


@pytest.mark.parametrize("L", [0, 1, 2, 15, 16, 17, 63, 64, 65])
def test_short_and_empty_sequences(L):
    say("short", L)
    p = make_problem(102, B=3, Hq=8, Hkv=2, D=128, P=16, lens=[L, 1, 70], sinks=(L % 2 == 1))
    got = to_np(gpu_decode(p))
    want = oracle(p)
    assert_parity(got, want, f"L={L}")
    if L == 0:
        assert np.all(got[0] == 0)


@pytest.mark.parametrize("W", [1, 15, 16, 17, 63, 64, 65, 299, 300, 301])
def test_window_boundaries(W):
    say("window", W)
    p = make_problem(103, B=2, Hq=8, Hkv=2, D=64, P=16, lens=[300, 40], window=W)
    assert_parity(to_np(gpu_decode(p)), oracle(p), f"W={W}")


def test_zero_scale_is_the_window_mean():
    p = make_problem(104, B=1, Hq=8, Hkv=2, D=64, P=16, lens=[333], window=77, sm_scale=0.0)
    assert_parity(to_np(gpu_decode(p)), oracle(p), "mean")


def test_poison_outside_attended_positions_never_leaks():
    """Slots past L, pages before the window and spare rows hold NaN codes and
    NaN scales; table entries past the last page are -1 or out of range."""
    p = make_problem(105, B=3, Hq=8, Hkv=2, D=64, P=16, lens=[37, 16, 250], window=50, sinks=True)
    pg, guard = add_guard_rows(p)
    t = pg.table.copy()
    for b in range(3):
        used = -(-int(p.seq_lens[b]) // 16)
        t[b, used:] = guard[0] if b == 0 else -1          # past the last page: a poisoned guard row, or -1
    # pages entirely before the window: point them at the other guard row and -7
    t[2, : (250 - 50) // 16] = -7
    t[2, 0] = guard[1]
    p2 = replace(pg, table=t)
    got = to_np(gpu_decode(p2))
    assert np.all(np.isfinite(got))
    assert_parity(got, oracle(p), "poison")


def test_invariants_bit_identical():
    p = make_problem(106, B=3, Hq=16, Hkv=2, D=128, P=16, lens=[700, 130, 9], sinks=True)
    base = gpu_decode(p).cpu()
    # run twice: no races, no atomics in the result
    assert torch.equal(gpu_decode(p).cpu(), base)
    # physical rows permuted
    assert torch.equal(gpu_decode(permute_rows(p, 5)).cpu(), base)
    # window >= L is full attention
    assert torch.equal(gpu_decode(p, window=700).cpu(), base)
    assert torch.equal(gpu_decode(p, window=100000).cpu(), base)
    # sink = -inf is no sink
    dev = device_problem(p)
    nos = gpu_decode(p, dev=dev, sinks=None).cpu()
    neg = gpu_decode(p, dev=dev, sinks=torch.full((16,), -float("inf"), device="cuda:0")).cpu()
    assert torch.equal(nos, neg)


def test_workgroup_counts_agree():
    p = make_problem(107, B=2, Hq=8, Hkv=2, D=64, P=16, lens=[1500, 700], sinks=True)
    want = oracle(p)
    outs = []
    for s in [1, 2, 5, 8, 13, 40, 0]:
        o = to_np(gpu_decode(p, workgroups=s))
        assert_parity(o, want, f"workgroups={s}")
        outs.append(o)
    # different splits only change fp32 summation order
    for o in outs[1:]:
        assert np.max(np.abs(o - outs[0])) < 2e-2


@pytest.mark.parametrize("D,Hq,L,pieces", [(64, 4, 15000, 24), (64, 4, 30400, 48), (128, 8, 24000, 24),
                                             (128, 8, 48400, 48)])
def test_one_unit_in_many_pieces(D, Hq, L, pieces):
    """A single long (sequence, KV head) unit cut into 24 or 48 pieces: the
    merge takes its 32-partial register form, resp. its chunked form (the
    lengths make each share hold at least a round of tiles, so the kernel
    keeps every requested workgroup)."""
    say("one unit in pieces", D, L, pieces)
    p = make_problem(111, B=1, Hq=Hq, Hkv=1, D=D, P=16, lens=[L], sinks=True)
    dev = device_problem(p)
    want = oracle(p)
    for w in (pieces, 0):
        assert_parity(to_np(gpu_decode(p, dev=dev, workgroups=w)), want, f"workgroups={w}")


def test_more_workgroups_than_tiles():
    """Workgroups with an empty share exit; units are still complete."""
    p = make_problem(108, B=2, Hq=8, Hkv=2, D=64, P=16, lens=[130, 64])
    assert_parity(to_np(gpu_decode(p, workgroups=97)), oracle(p), "many workgroups")


def test_counters_record_what_ran():
    ops.reset_counters()
    p = make_problem(109, B=2, Hq=8, Hkv=2, D=64, P=16, lens=[1000, 64])
    gpu_decode(p, workgroups=4)
    c = ops.counters()
    assert c["decode_calls"] == 1 and c["decode_mfma_bf16"] == 1 and c["decode_split"] == 1
    assert c["merge_launches"] == 0          # cut units are merged inside the decode kernel
    gpu_decode(p, workgroups=1)
    c = ops.counters()
    assert c["decode_calls"] == 2 and c["decode_split"] == 1 and c["merge_launches"] == 0


def test_split_merge_many_calls_one_workspace():
    """Back-to-back split calls sharing one workspace, each with new queries:
    a partial read before it was written, or a stale arrival count, would show
    up as a mismatch against the oracle."""
    p = make_problem(110, B=4, Hq=16, Hkv=2, D=128, P=16, lens=[3000, 1500, 64, 2500], sinks=True)
    dev = device_problem(p)
    msl = int(p.seq_lens.max())
    plan = ops.decode_plan(p.B, p.Hq, dev["kd"], dev["vd"], msl, workgroups=8)
    assert plan.workgroups == 8
    ws = torch.empty(plan.workspace_bytes, dtype=torch.uint8, device="cuda:0")
    rng = np.random.default_rng(0)
    outs = []
    qs = []
    for i in range(24):
        q = inputs_round(rng.standard_normal((p.B, p.Hq, p.D)).astype(np.float32))
        qs.append(q)
        dev["q"] = torch.from_numpy(q).to(torch.bfloat16).to("cuda:0")
        outs.append(ops.decode(dev["q"], dev["k_pool"], dev["v_pool"], dev["kd"], dev["vd"], dev["block_table"],
                               dev["seq_lens"], msl, sinks=dev["sinks"], workgroups=8, workspace=ws))
    torch.cuda.synchronize()
    for i in (0, 1, 2, 11, 22, 23):
        assert_parity(to_np(outs[i]), oracle(replace(p, q=qs[i])), f"call {i}")


def inputs_round(x):
    from fp8_paged_kv_amd.inputs import round_to_bf16
    return round_to_bf16(x)


MANY = [
    # (B, D, Hq, Hkv, window, sinks): batches above 64 take the four-wave startup scan
    (65, 128, 16, 4, 0, True),
    (96, 64, 16, 2, 200, False),
    (200, 128, 16, 4, 300, True),
]


@pytest.mark.parametrize("B,D,Hq,Hkv,window,sinks", MANY, ids=[f"B{m[0]}-D{m[1]}" for m in MANY])
@pytest.mark.parametrize("workgroups", [0, 3, 131])
def test_many_sequences_default_kernel(B, D, Hq, Hkv, window, sinks, workgroups):
    """The default d-major split kernel at batches above 64 (LDS prefix scan by
    all waves, share bounds per thread, a binary search per segment), mixed
    lengths with empty and one-position sequences, against the oracle."""
    say("many sequences", B, D, "workgroups", workgroups)
    rng = np.random.default_rng(B * 7 + D)
    lens = rng.integers(1, 700, size=B)
    lens[::9] = 0
    lens[1] = 1
    lens[2] = 64
    lens[3] = 1500
    p = make_problem(120 + B, B=B, Hq=Hq, Hkv=Hkv, D=D, P=16, lens=lens.tolist(), window=window, sinks=sinks)
    dev = device_problem(p)
    plan = ops.decode_plan(p.B, p.Hq, dev["kd"], dev["vd"], int(lens.max()), window, workgroups)
    assert plan.variant == ops.VARIANTS["mfma_bf16"]
    ops.reset_counters()
    got = to_np(gpu_decode(p, dev=dev, workgroups=workgroups))
    assert ops.counters()["decode_packed_heads"] == 0
    assert_parity(got, oracle(p), f"B={B}")
    assert np.all(got[lens == 0] == 0)


def test_forced_merge_timeout_is_reported():
    """A merge whose wait for another workgroup's partial gives up (forced
    from the host: merges wait for a flag value no workgroup writes, with a
    short bound) writes NaN for its unit and counts itself in the device
    status; every kernel ends, and later calls are correct again."""
    say("forced merge timeout")
    p = make_problem(130, B=2, Hq=16, Hkv=4, D=128, P=16, lens=[3000, 2000], sinks=True)
    dev = device_problem(p)
    ops.device_status(reset=True)
    good = to_np(gpu_decode(p, dev=dev, workgroups=7))
    assert ops.device_status()["merge_timeouts"] == 0
    assert_parity(good, oracle(p), "before")
    ops.force_merge_timeout(True)
    try:
        bad = to_np(gpu_decode(p, dev=dev, workgroups=7))
    finally:
        ops.force_merge_timeout(False)
    st = ops.device_status(reset=True)
    assert st["merge_timeouts"] >= 1
    assert np.isnan(bad).any()
    again = to_np(gpu_decode(p, dev=dev, workgroups=7))
    assert ops.device_status()["merge_timeouts"] == 0
    assert np.array_equal(again, good)
