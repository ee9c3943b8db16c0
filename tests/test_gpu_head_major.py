"""Decode parity against the float64 oracle for grids where the split kernel
orders its units KV head first (head dims 64 and 256, H_kv a power of two,
an uncapped grid that is a multiple of 8 * H_kv, units split into tiles),
beside grids of the same problems that keep the sequence-first order.  Lengths
are chosen so that units are cut into pieces and merged; the cases cover both
set-up paths (up to 64 sequences, and more), empty sequences, windows and
sinks, and whole-unit mode (short windows)."""
import numpy as np
import pytest

from oracle import attention as oatt
from tests.gpu_util import assert_parity, device_problem, gpu_decode, say, to_np
from tests.problems import make_problem

pytestmark = pytest.mark.gpu


def oracle(p):
    return oatt.decode_ref(p.q, p.k_pool, p.v_pool, p.kdesc, p.vdesc, p.table, p.seq_lens,
                           window=p.window, sinks=p.sinks, sm_scale=p.sm_scale)


def shares_kept(lens, Hkv, D, window):
    """The split kernel's cap on the shares of a call (the most workgroups
    that each get at least one tile per wave): the cost of all units over the
    cost of a unit plus four tiles (whole-unit mode: one per unit)."""
    TT = 64 if D <= 128 else 32
    SC = 48 if D == 128 else 24
    nt = []
    for L in lens:
        st = L - window if (window > 0 and L > window) else 0
        tb = st & ~(TT - 1)
        nt.append((L - tb + TT - 1) // TT if L > st else 0)
    T = sum(nt) * Hkv
    U = sum(1 for x in nt if x) * Hkv
    unit_mode = T <= 4 * U
    TC, SC = (0, 1) if unit_mode else (4, SC)
    return max(1, (SC * U + TC * T) // (SC + TC * 4))


RNG = np.random.default_rng(20261204)
CASES = [
    # (name, problem kwargs, head-major grids, other grids)
    ("d64-hkv8-g8-sinks", dict(B=5, Hq=64, Hkv=8, D=64, P=16, lens=[6000, 3400, 0, 1800, 5000], sinks=True),
     [64, 128, 192], [200]),
    ("d64-hkv4-window", dict(B=8, Hq=16, Hkv=4, D=64, P=16, lens=[4100, 700, 2600, 9, 3000, 5000, 1600, 2300],
                             window=1500, sinks=True), [32, 64], [40]),
    ("d64-hkv2", dict(B=4, Hq=8, Hkv=2, D=64, P=16, lens=[15000, 333, 9000, 4000]), [16, 48, 80], [56]),
    ("d64-hkv1-g16", dict(B=2, Hq=16, Hkv=1, D=64, P=32, lens=[20000, 9000]), [16, 24, 40], [20]),
    ("d64-hkv2-b70", dict(B=70, Hq=4, Hkv=2, D=64, P=16, lens=[int(x) for x in RNG.integers(0, 900, 70)]),
     [32, 64], [40]),
    # whole-unit mode (short windows): one unit per share, the same assignment in both orders
    ("d64-hkv8-whole-units", dict(B=10, Hq=32, Hkv=8, D=64, P=16, lens=[int(x) for x in RNG.integers(130, 700, 10)],
                                  window=128, sinks=True), [64], [72]),
    ("d256-hkv8-window", dict(B=3, Hq=16, Hkv=8, D=256, P=32, lens=[3000, 2000, 1500], window=1024,
                              sm_scale=1.0), [64], [56]),
    ("d256-hkv2", dict(B=3, Hq=8, Hkv=2, D=256, P=16, lens=[6000, 2500, 3300], sinks=True), [16, 32, 64], [24]),
    # H_kv not a power of two: the sequence-first order at every grid
    ("d64-hkv6", dict(B=3, Hq=12, Hkv=6, D=64, P=16, lens=[3000, 1200, 2200]), [], [48, 96]),
]


@pytest.mark.parametrize("name,kw,hm_grids,other_grids", CASES, ids=[c[0] for c in CASES])
def test_head_major_grids_match_the_oracle(name, kw, hm_grids, other_grids):
    p = make_problem(911, **kw)
    want = oracle(p)
    dev = device_problem(p)
    cap = shares_kept(kw["lens"], kw["Hkv"], kw["D"], kw.get("window", 0))
    for W in hm_grids:
        assert W % (8 * kw["Hkv"]) == 0 and W <= cap, (W, cap)   # the grid keeps every share
    outs = {}
    for W in hm_grids + other_grids:
        say("head-major", name, "workgroups", W, "cap", cap)
        outs[W] = to_np(gpu_decode(p, dev=dev, workgroups=W))
        assert_parity(outs[W], want, f"{name} W={W}")
    # repeats of one grid are bit-identical
    for W in hm_grids[:1]:
        assert np.array_equal(to_np(gpu_decode(p, dev=dev, workgroups=W)), outs[W])
