"""Fused append + decode (fp8pa_append_decode) on the GPU: after one call the
pools hold exactly the bytes that the oracle's append of each sequence's new
token writes, and the output is bit-identical to fp8pa_append_quant followed
by fp8pa_decode and within the parity bound of the oracle's decode of the
appended pools.  Cases cover every scale kind and layout the decode reads,
page scales that grow (earlier tokens re-encoded), a new token that opens a
page, empty sequences, windows, sinks and several workgroup counts."""
import numpy as np
import pytest
import torch

from fp8_paged_kv_amd import ops
from oracle import attention as oatt
from oracle import pool as opool
from tests.gpu_util import DEV, assert_parity, desc_of, say, to_np
from tests.problems import POISON, make_problem

pytestmark = pytest.mark.gpu

CASES = [
    ("d128-page-scales", dict(B=3, Hq=16, Hkv=4, D=128, P=16, lens=[513, 64, 17])),
    ("d64-window-sinks", dict(B=3, Hq=16, Hkv=2, D=64, P=16, lens=[500, 100, 33], window=128, sinks=True)),
    ("d128-aligned-rows", dict(B=2, Hq=16, Hkv=4, D=128, P=16, lens=[700, 65], row_pad=32, align64=True)),
    ("d256-window", dict(B=2, Hq=4, Hkv=2, D=256, P=32, lens=[700, 33], window=100, sm_scale=1.0)),
    ("d256-p16", dict(B=3, Hq=16, Hkv=4, D=256, P=16, lens=[300, 65, 7], sm_scale=1.0)),
    ("d512", dict(B=2, Hq=8, Hkv=1, D=512, P=32, lens=[333, 65], sm_scale=1.0)),
    ("d128-e8m0-p128", dict(B=2, Hq=16, Hkv=2, D=128, P=128, lens=[1000, 129], scale_kind="e8m0_32")),
    ("d64-token-scales", dict(B=2, Hq=8, Hkv=2, D=64, P=16, lens=[250, 31], scale_kind="token_head")),
    ("d128-ktokens", dict(B=2, Hq=8, Hkv=2, D=128, P=16, lens=[260, 5], k_layout="tokens")),
    ("empty-and-one", dict(B=3, Hq=8, Hkv=2, D=64, P=16, lens=[0, 1, 90])),
    # attended spans above 2048 positions: the append kernel, then the decode
    ("long-two-launches", dict(B=2, Hq=16, Hkv=4, D=128, P=16, lens=[2600, 130])),
    ("long-window-two-launches", dict(B=2, Hq=8, Hkv=2, D=64, P=16, lens=[3000, 40], window=2500, sinks=True)),
]


def before_and_new(p, gain):
    """Pools holding each sequence's first L-1 tokens, and the new tokens
    ([B, Hkv, D], position L-1; zeros where L = 0), scaled by gain[b]."""
    k0 = np.full_like(p.k_pool, POISON)
    v0 = np.full_like(p.v_pool, POISON)
    k0 = opool.pack_sequences(k0, p.kdesc, p.table, [k[:max(len(k) - 1, 0)] for k in p.raw_k])
    v0 = opool.pack_sequences(v0, p.vdesc, p.table, [v[:max(len(v) - 1, 0)] for v in p.raw_v])
    shape = (p.B, p.Hkv, p.D)
    xk = np.zeros(shape, np.float32)
    xv = np.zeros(shape, np.float32)
    for b in range(p.B):
        if len(p.raw_k[b]):
            # a power-of-two gain keeps the values bf16-exact
            xk[b] = p.raw_k[b][-1] * np.float32(gain[b])
            xv[b] = p.raw_v[b][-1] * np.float32(gain[b])
    return k0, v0, xk, xv


def oracle_append(pool, desc, table, lens, x):
    pos = [max(int(L) - 1, 0) for L in lens]
    counts = [1 if L > 0 else 0 for L in lens]
    return opool.append_ref(pool, desc, table, pos, x[:, None], counts=counts)


@pytest.mark.parametrize("name,kw", CASES, ids=[c[0] for c in CASES])
@pytest.mark.parametrize("workgroups", [1, 0, 3])
def test_append_decode_matches_append_then_decode(name, kw, workgroups):
    say("append+decode", name, "workgroups", workgroups)
    p = make_problem(202, **kw)
    gain = [8.0 if b % 2 == 0 else 1.0 for b in range(p.B)]   # even sequences grow their page scale
    k0, v0, xk, xv = before_and_new(p, gain)
    lens = p.seq_lens
    msl = int(lens.max())
    kd, vd = desc_of(p.kdesc), desc_of(p.vdesc)
    table = torch.from_numpy(np.ascontiguousarray(p.table)).to(DEV)
    sl = torch.from_numpy(lens.astype(np.int32)).to(DEV)
    q = torch.from_numpy(np.ascontiguousarray(p.q)).to(torch.bfloat16).to(DEV)
    sinks = None if p.sinks is None else torch.from_numpy(p.sinks).to(DEV)
    tk = torch.from_numpy(xk).to(torch.bfloat16).to(DEV)
    tv = torch.from_numpy(xv).to(torch.bfloat16).to(DEV)

    # two calls: append the new tokens, then decode
    ka, va = torch.from_numpy(k0).to(DEV), torch.from_numpy(v0).to(DEV)
    pos = torch.tensor([max(int(L) - 1, 0) for L in lens], dtype=torch.int32, device=DEV)
    counts = torch.tensor([1 if L > 0 else 0 for L in lens], dtype=torch.int32, device=DEV)
    ops.append_quant(tk[:, None], tv[:, None], ka, va, kd, vd, table, pos, counts)
    out_a = ops.decode(q, ka, va, kd, vd, table, sl, msl, window=p.window, sinks=sinks, sm_scale=p.sm_scale,
                       workgroups=workgroups)
    # one call
    kb, vb = torch.from_numpy(k0).to(DEV), torch.from_numpy(v0).to(DEV)
    ops.reset_counters()
    out_b = ops.append_decode(q, tk, tv, kb, vb, kd, vd, table, sl, msl, window=p.window, sinks=sinks,
                              sm_scale=p.sm_scale, workgroups=workgroups)
    torch.cuda.synchronize()
    c = ops.counters()
    span = min(p.window, msl) if p.window > 0 else msl
    if span <= 2048:
        assert c["fused_appends"] == 1 and c["append_launches"] == 0
    else:
        assert c["fused_appends"] == 0 and c["append_launches"] == 1
    assert c["decode_calls"] == 1

    # pools: the oracle's append, byte for byte
    wk = oracle_append(k0, p.kdesc, p.table, lens, xk)
    wv = oracle_append(v0, p.vdesc, p.table, lens, xv)
    assert np.array_equal(kb.cpu().numpy(), wk), "K pool differs from the oracle append"
    assert np.array_equal(vb.cpu().numpy(), wv), "V pool differs from the oracle append"
    assert np.array_equal(ka.cpu().numpy(), wk) and np.array_equal(va.cpu().numpy(), wv)
    # output: bit-identical to append-then-decode, and within the oracle bound
    assert torch.equal(out_a.view(torch.int16), out_b.view(torch.int16)), "fused output differs from two calls"
    want = oatt.decode_ref(p.q, wk, wv, p.kdesc, p.vdesc, p.table, lens, window=p.window, sinks=p.sinks,
                           sm_scale=p.sm_scale)
    assert_parity(to_np(out_b), want, name)


def test_append_decode_graph_replays_match_eager():
    """A captured fused call replays to the same pools and output as eager
    calls (the new tokens rewrite the same slots on every replay)."""
    say("append+decode graph")
    p = make_problem(203, B=3, Hq=16, Hkv=4, D=128, P=16, lens=[300, 130, 64])
    k0, v0, xk, xv = before_and_new(p, [8.0, 1.0, 4.0])
    kd, vd = desc_of(p.kdesc), desc_of(p.vdesc)
    table = torch.from_numpy(np.ascontiguousarray(p.table)).to(DEV)
    sl = torch.from_numpy(p.seq_lens.astype(np.int32)).to(DEV)
    q = torch.from_numpy(np.ascontiguousarray(p.q)).to(torch.bfloat16).to(DEV)
    tk = torch.from_numpy(xk).to(torch.bfloat16).to(DEV)
    tv = torch.from_numpy(xv).to(torch.bfloat16).to(DEV)
    msl = int(p.seq_lens.max())
    plan = ops.decode_plan(p.B, p.Hq, kd, vd, msl)
    ws = torch.empty(max(plan.workspace_bytes, 256), dtype=torch.uint8, device=DEV)
    k_e, v_e = torch.from_numpy(k0).to(DEV), torch.from_numpy(v0).to(DEV)
    out_e = ops.append_decode(q, tk, tv, k_e, v_e, kd, vd, table, sl, msl, workspace=ws)
    torch.cuda.synchronize()
    kg_, vg_ = torch.from_numpy(k0).to(DEV), torch.from_numpy(v0).to(DEV)
    out_g = torch.empty_like(q)

    def run():
        ops.append_decode(q, tk, tv, kg_, vg_, kd, vd, table, sl, msl, out=out_g, workspace=ws)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run()
    for rep in range(3):
        kg_.copy_(torch.from_numpy(k0).to(DEV))
        vg_.copy_(torch.from_numpy(v0).to(DEV))
        out_g.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(kg_, k_e) and torch.equal(vg_, v_e), f"replay {rep}: pools differ"
        assert torch.equal(out_g.view(torch.int16), out_e.view(torch.int16)), f"replay {rep}: output differs"
    del graph
