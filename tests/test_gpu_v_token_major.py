"""Decode with the V pool in the page's own token-major payload orders
("heads": [Hkv][P][D], "tokens": [P][Hkv][D]), which the kernel stages through
LDS and reads back transposed.  Parity against the float64 oracle over head
dims 64-512, every scale kind, windows, sinks, aligned rows and several
workgroup counts; bit-identity with the same values stored d-major (the
transposed operand must be exactly the d-major one); the counter that records
the path; and the append + decode call on such pools."""
from dataclasses import replace

import numpy as np
import pytest
import torch

from fp8_paged_kv_amd import ops
from oracle import attention as oatt
from oracle import pool as opool
from tests.gpu_util import DEV, assert_parity, desc_of, gpu_decode, say, to_np
from tests.problems import add_guard_rows, POISON, make_problem

pytestmark = pytest.mark.gpu


def oracle(p):
    return oatt.decode_ref(p.q, p.k_pool, p.v_pool, p.kdesc, p.vdesc, p.table, p.seq_lens, window=p.window,
                           sinks=p.sinks, sm_scale=p.sm_scale)


CASES = [
    ("d64-vheads", dict(B=3, Hq=8, Hkv=2, D=64, P=16, lens=[300, 17, 129], v_layout="heads")),
    ("d64-vtokens-window-sinks", dict(B=3, Hq=16, Hkv=2, D=64, P=16, lens=[500, 100, 20], window=128, sinks=True,
                                      v_layout="tokens")),
    ("d128-vtokens-ktokens", dict(B=3, Hq=16, Hkv=4, D=128, P=16, lens=[513, 64, 1], k_layout="tokens",
                                  v_layout="tokens")),
    ("d128-vheads-kheads-p32", dict(B=2, Hq=16, Hkv=2, D=128, P=32, lens=[400, 77], k_layout="heads",
                                    v_layout="heads", sinks=True)),
    ("d128-vtokens-token-scales", dict(B=2, Hq=16, Hkv=4, D=128, P=16, lens=[700, 65], scale_kind="token_head",
                                       k_layout="tokens", v_layout="tokens")),
    ("d128-vheads-aligned-rows", dict(B=3, Hq=16, Hkv=4, D=128, P=16, lens=[700, 65, 300], row_pad=32,
                                      align64=True, v_layout="heads")),
    ("d128-vtokens-e8m0-p128", dict(B=2, Hq=16, Hkv=2, D=128, P=128, lens=[1000, 130], scale_kind="e8m0_32",
                                    k_layout="tokens", v_layout="tokens")),
    ("d64-vtokens-e8m0", dict(B=2, Hq=8, Hkv=2, D=64, P=16, lens=[250, 31], scale_kind="e8m0_32",
                              v_layout="tokens")),
    ("d256-vtokens-window", dict(B=2, Hq=4, Hkv=2, D=256, P=32, lens=[700, 33], window=100, sm_scale=1.0,
                                 v_layout="tokens")),
    ("d256-vheads-e8m0", dict(B=1, Hq=8, Hkv=2, D=256, P=32, lens=[300], scale_kind="e8m0_32", sinks=True,
                              v_layout="heads")),
    ("d256-p16-vtokens", dict(B=3, Hq=16, Hkv=4, D=256, P=16, lens=[300, 65, 7], sinks=True, sm_scale=1.0,
                              v_layout="tokens")),
    ("d256-p16-vheads", dict(B=3, Hq=16, Hkv=4, D=256, P=16, lens=[300, 65, 7], window=100, v_layout="heads")),
    ("d512-vtokens", dict(B=2, Hq=8, Hkv=1, D=512, P=32, lens=[333, 64], sm_scale=1.0, v_layout="tokens")),
    ("d512-vheads-token-scales", dict(B=2, Hq=16, Hkv=2, D=512, P=16, lens=[260, 97], sm_scale=1.0,
                                      scale_kind="token_head", k_layout="heads", v_layout="heads")),
    ("d512-vtokens-e8m0-window", dict(B=1, Hq=8, Hkv=1, D=512, P=16, lens=[260], scale_kind="e8m0_32", window=40,
                                      v_layout="tokens")),
    ("empty-and-short", dict(B=4, Hq=8, Hkv=2, D=64, P=16, lens=[0, 1, 15, 65], v_layout="tokens")),
]


@pytest.mark.parametrize("name,kw", CASES, ids=[c[0] for c in CASES])
@pytest.mark.parametrize("workgroups", [1, 0, 3])
def test_v_token_major_parity(name, kw, workgroups):
    say("V token-major parity", name, "workgroups", workgroups)
    p = make_problem(301, **kw)
    ops.reset_counters()
    got = to_np(gpu_decode(p, workgroups=workgroups))
    assert ops.counters()["decode_v_token_major"] == 1
    assert_parity(got, oracle(p), name)


@pytest.mark.parametrize("v_layout", ["heads", "tokens"])
@pytest.mark.parametrize("D", [64, 128, 256, 512])
def test_same_output_as_d_major(v_layout, D):
    """The same codes and scales stored d-major and token-major give the same
    output bit for bit: the staged transpose hands the MFMA the very operand
    the d-major load does."""
    say("V token-major vs d-major", v_layout, D)
    kw = dict(B=3, Hq=16 if D < 512 else 8, Hkv=2, D=D, P=16, lens=[333, 70, 16], sinks=True,
              sm_scale=1.0 if D >= 256 else None)
    p_t = make_problem(302, v_layout=v_layout, **kw)
    p_d = make_problem(302, v_layout="heads_dmajor", **kw)
    for w in (1, 0):
        a = gpu_decode(p_t, workgroups=w).view(torch.int16)
        b = gpu_decode(p_d, workgroups=w).view(torch.int16)
        assert torch.equal(a, b), f"workgroups={w}"


def test_poison_outside_attended_positions_never_leaks():
    p = make_problem(303, B=3, Hq=8, Hkv=2, D=64, P=16, lens=[37, 16, 250], window=50, sinks=True,
                     v_layout="tokens", scale_kind="token_head")
    p, guard = add_guard_rows(p)
    t = p.table.copy()
    for b in range(3):
        used = -(-int(p.seq_lens[b]) // 16)
        t[b, used:] = -1
    t[2, : (250 - 50) // 16] = -7
    t[2, 0], t[0, -1] = guard      # never-read entries on poisoned guard rows
    got = to_np(gpu_decode(replace(p, table=t)))
    assert np.all(np.isfinite(got))
    assert_parity(got, oracle(p), "poison")


def test_append_decode_on_token_major_pools():
    """fp8pa_append_decode on V token-major pools: the append kernel, then the
    decode; pools hold the oracle's append byte for byte."""
    say("append+decode V tokens")
    p = make_problem(304, B=3, Hq=16, Hkv=2, D=128, P=16, lens=[300, 33, 16], k_layout="tokens", v_layout="tokens",
                     scale_kind="token_head")
    k0 = opool.pack_sequences(np.full_like(p.k_pool, POISON), p.kdesc, p.table, [k[:-1] for k in p.raw_k])
    v0 = opool.pack_sequences(np.full_like(p.v_pool, POISON), p.vdesc, p.table, [v[:-1] for v in p.raw_v])
    xk = np.stack([k[-1] for k in p.raw_k]).astype(np.float32)
    xv = np.stack([v[-1] for v in p.raw_v]).astype(np.float32)
    kp, vp = torch.from_numpy(k0).to(DEV), torch.from_numpy(v0).to(DEV)
    ops.reset_counters()
    out = ops.append_decode(torch.from_numpy(np.ascontiguousarray(p.q)).to(torch.bfloat16).to(DEV),
                            torch.from_numpy(xk).to(torch.bfloat16).to(DEV),
                            torch.from_numpy(xv).to(torch.bfloat16).to(DEV), kp, vp, desc_of(p.kdesc),
                            desc_of(p.vdesc), torch.from_numpy(np.ascontiguousarray(p.table)).to(DEV),
                            torch.from_numpy(p.seq_lens.astype(np.int32)).to(DEV), int(p.seq_lens.max()))
    torch.cuda.synchronize()
    c = ops.counters()
    assert c["append_launches"] == 1 and c["fused_appends"] == 0 and c["decode_v_token_major"] == 1
    pos = [int(L) - 1 for L in p.seq_lens]
    wk = opool.append_ref(k0, p.kdesc, p.table, pos, xk[:, None], counts=[1] * p.B)
    wv = opool.append_ref(v0, p.vdesc, p.table, pos, xv[:, None], counts=[1] * p.B)
    assert np.array_equal(kp.cpu().numpy(), wk) and np.array_equal(vp.cpu().numpy(), wv)
    want = oatt.decode_ref(p.q, wk, wv, p.kdesc, p.vdesc, p.table, p.seq_lens, sm_scale=p.sm_scale)
    assert_parity(to_np(out), want, "append+decode V tokens")
