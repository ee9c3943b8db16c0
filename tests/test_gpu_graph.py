"""Decode captured in a HIP graph: the launch depends on host values only, so
a captured call replays correctly.  Replays reuse the captured call's epoch;
the split merge clears the flags it consumed, so every replay starts clean.
Each replay is checked against the eager result (bit-identical: same kernel,
same workgroup count, same summation order), with eager work on the same
buffers between replays, and against the oracle after q changes in place."""
import numpy as np
import pytest
import torch

from fp8_paged_kv_amd import ops
from oracle import attention as oatt
from tests.gpu_util import assert_parity, device_problem, say, to_np
from tests.problems import make_problem

pytestmark = pytest.mark.gpu


def run(p, dev, out, ws, workgroups):
    return ops.decode(dev["q"], dev["k_pool"], dev["v_pool"], dev["kd"], dev["vd"], dev["block_table"],
                      dev["seq_lens"], int(p.seq_lens.max()), window=p.window, sinks=dev["sinks"],
                      sm_scale=p.sm_scale, workgroups=workgroups, out=out, workspace=ws)


@pytest.mark.parametrize("workgroups", [13, 0])
def test_graph_replays_match_eager(workgroups):
    say(f"graph capture: workgroups={workgroups}")
    p = make_problem(131, B=3, Hq=16, Hkv=2, D=128, P=16, lens=[900, 333, 40], window=512, sinks=True)
    dev = device_problem(p)
    plan = ops.decode_plan(3, 16, dev["kd"], dev["vd"], int(p.seq_lens.max()), p.window, workgroups)
    ws = torch.empty(max(plan.workspace_bytes, 256), dtype=torch.uint8, device="cuda:0")
    out = torch.empty_like(dev["q"])
    eager = run(p, dev, None, ws, workgroups).clone()
    torch.cuda.synchronize()
    assert_parity(to_np(eager), oatt.decode_ref(p.q, p.k_pool, p.v_pool, p.kdesc, p.vdesc, p.table, p.seq_lens,
                                                window=p.window, sinks=p.sinks, sm_scale=p.sm_scale), "eager")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run(p, dev, out, ws, workgroups)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run(p, dev, out, ws, workgroups)
    for i in range(4):
        out.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), f"replay {i} differs from the eager call"
        # eager work on the same workspace between replays
        again = run(p, dev, None, ws, workgroups)
        torch.cuda.synchronize()
        assert torch.equal(again, eager), f"eager call after replay {i} differs"
    # new queries written in place: the replay reads them
    q2 = np.random.default_rng(7).standard_normal(p.q.shape).astype(np.float32)
    dev["q"].copy_(torch.from_numpy(q2).to(torch.bfloat16))
    q2 = dev["q"].float().cpu().numpy().astype(np.float64)
    g.replay()
    torch.cuda.synchronize()
    want = oatt.decode_ref(q2, p.k_pool, p.v_pool, p.kdesc, p.vdesc, p.table, p.seq_lens, window=p.window,
                           sinks=p.sinks, sm_scale=p.sm_scale)
    assert_parity(to_np(out), want, "replay with new q")
    del g
