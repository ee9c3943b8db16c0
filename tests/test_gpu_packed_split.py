"""Packed heads with splits (FP8PA_VARIANT_PACKED_SPLIT) on the GPU: units of
four KV heads read together by one workgroup, long spans split over
workgroups and merged.  Parity against the float64 oracle at several
workgroup counts (whole units, cut units, units in many pieces), every scale
kind, windows, sinks, K layouts, empty and short sequences; the counter;
refusals."""
from dataclasses import replace

import numpy as np
import pytest
import torch

from fp8_paged_kv_amd import ops
from oracle import attention as oatt
from tests.gpu_util import assert_parity, gpu_decode, say, to_np
from tests.problems import add_guard_rows, make_problem

pytestmark = pytest.mark.gpu


def oracle(p):
    return oatt.decode_ref(p.q, p.k_pool, p.v_pool, p.kdesc, p.vdesc, p.table, p.seq_lens, window=p.window,
                           sinks=p.sinks, sm_scale=p.sm_scale)


CASES = [
    ("d64-hkv4-g4", dict(B=3, Hq=16, Hkv=4, D=64, P=16, lens=[300, 17, 129])),
    ("d128-hkv8-g4", dict(B=3, Hq=32, Hkv=8, D=128, P=16, lens=[1500, 64, 700])),
    ("d128-sinks-window", dict(B=3, Hq=32, Hkv=8, D=128, P=16, lens=[900, 100, 20], window=300, sinks=True)),
    ("d128-token-scales-ktokens", dict(B=2, Hq=16, Hkv=4, D=128, P=16, lens=[700, 65], scale_kind="token_head",
                                       k_layout="tokens")),
    ("d128-kheads-aligned", dict(B=3, Hq=16, Hkv=4, D=128, P=16, lens=[700, 65, 300], row_pad=32, align64=True,
                                 k_layout="heads")),
    ("d128-e8m0-p128", dict(B=2, Hq=16, Hkv=4, D=128, P=128, lens=[1000, 130], scale_kind="e8m0_32")),
    ("d256-hkv8-g2-window", dict(B=2, Hq=16, Hkv=8, D=256, P=32, lens=[1500, 33], window=1024, sm_scale=1.0)),
    ("d256-p16", dict(B=3, Hq=16, Hkv=4, D=256, P=16, lens=[300, 65, 7], sinks=True, sm_scale=1.0)),
    ("d512-hkv4-g1", dict(B=2, Hq=4, Hkv=4, D=512, P=32, lens=[333, 64], sm_scale=1.0)),
    ("g1-hkv8", dict(B=2, Hq=8, Hkv=8, D=64, P=16, lens=[90, 3])),
    ("empty-and-short", dict(B=4, Hq=16, Hkv=4, D=64, P=16, lens=[0, 1, 15, 65], sinks=True)),
]


@pytest.mark.parametrize("name,kw", CASES, ids=[c[0] for c in CASES])
@pytest.mark.parametrize("workgroups", [1, 0, 3, 7])
def test_packed_split_parity(name, kw, workgroups):
    say("packed split parity", name, "workgroups", workgroups)
    p = make_problem(601, **kw)
    ops.reset_counters()
    got = to_np(gpu_decode(p, workgroups=workgroups, variant="packed_split"))
    c = ops.counters()
    assert c["decode_packed_split"] == 1 and c["decode_mfma_bf16"] == 1
    assert_parity(got, oracle(p), name)


def test_packed_split_many_pieces_and_repeats():
    """Units cut into many pieces (more workgroups than units), run twice
    (bit-identical: no races), and rows permuted."""
    p = make_problem(602, B=2, Hq=16, Hkv=4, D=128, P=16, lens=[3000, 1200], sinks=True)
    want = oracle(p)
    for w in (5, 13, 40, 97):
        a = gpu_decode(p, workgroups=w, variant="packed_split")
        assert_parity(to_np(a), want, f"workgroups={w}")
        assert torch.equal(a, gpu_decode(p, workgroups=w, variant="packed_split"))


def test_packed_split_poison_never_leaks():
    p = make_problem(603, B=3, Hq=16, Hkv=4, D=64, P=16, lens=[37, 16, 250], window=50, sinks=True)
    p, guard = add_guard_rows(p)
    t = p.table.copy()
    for b in range(3):
        used = -(-int(p.seq_lens[b]) // 16)
        t[b, used:] = -1
    t[2, : (250 - 50) // 16] = -7
    t[2, 0], t[0, -1] = guard      # never-read entries on poisoned guard rows
    for w in (0, 5):
        got = to_np(gpu_decode(replace(p, table=t), workgroups=w, variant="packed_split"))
        assert np.all(np.isfinite(got))
        assert_parity(got, oracle(p), "poison")


def test_packed_split_refusals():
    p = make_problem(604, B=2, Hq=16, Hkv=2, D=64, P=16, lens=[100, 30])      # G = 8
    with pytest.raises(RuntimeError):
        gpu_decode(p, variant="packed_split")
    p = make_problem(604, B=2, Hq=12, Hkv=6, D=64, P=16, lens=[100, 30])      # Hkv % 4 != 0
    with pytest.raises(RuntimeError):
        gpu_decode(p, variant="packed_split")
    p = make_problem(604, B=2, Hq=16, Hkv=4, D=64, P=16, lens=[100, 30], v_layout="tokens")
    with pytest.raises(RuntimeError):
        gpu_decode(p, variant="packed_split")
