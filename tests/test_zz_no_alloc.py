"""fp8pa_decode_noalloc (the allocation-free decode: split partials in the
library's per-device scratch) through the C ABI, against fp8pa_decode with a
caller workspace on the same inputs: bit-identical outputs on two calls in a
row (the second smaller, run over the first one's scratch contents), within
the oracle bound, and a refusal (nothing launched) for a plan whose workspace
exceeds the scratch."""
import numpy as np
import pytest
import torch

from fp8_paged_kv_amd import ops
from oracle import attention as oatt
from tests.gpu_util import assert_parity, device_problem, say, to_np
from tests.problems import make_problem

pytestmark = pytest.mark.gpu


def run_both(p, workgroups=0):
    dev = device_problem(p)
    msl = int(p.seq_lens.max())
    kw = dict(window=p.window, sinks=dev["sinks"], sm_scale=p.sm_scale, workgroups=workgroups)
    plan = ops.decode_plan(p.B, p.Hq, dev["kd"], dev["vd"], msl, p.window, workgroups)
    assert 0 < plan.workspace_bytes <= ops.NOALLOC_SCRATCH_BYTES
    want = ops.decode(dev["q"], dev["k_pool"], dev["v_pool"], dev["kd"], dev["vd"], dev["block_table"],
                      dev["seq_lens"], msl, **kw)
    ops.reset_counters()
    got = ops.decode_noalloc(dev["q"], dev["k_pool"], dev["v_pool"], dev["kd"], dev["vd"], dev["block_table"],
                             dev["seq_lens"], msl, **kw)
    torch.cuda.synchronize()
    c = ops.counters()
    assert c["decode_calls"] == 1 and c["decode_split"] == 1
    return got, want


def oracle(p):
    return oatt.decode_ref(p.q, p.k_pool, p.v_pool, p.kdesc, p.vdesc, p.table, p.seq_lens, window=p.window,
                           sinks=p.sinks, sm_scale=p.sm_scale)


def test_noalloc_matches_decode_two_calls():
    say("noalloc: two calls, the second smaller")
    big = make_problem(901, B=5, Hq=32, Hkv=8, D=128, P=16, lens=[3000, 1200, 700, 64, 0], sinks=True)
    small = make_problem(902, B=2, Hq=16, Hkv=2, D=64, P=16, lens=[900, 33], window=300)
    for p, wg in ((big, 0), (small, 5)):
        got, want = run_both(p, wg)
        assert torch.equal(got.view(torch.int16), want.view(torch.int16))
        assert_parity(to_np(got), oracle(p), "noalloc")


def test_noalloc_refuses_a_workspace_beyond_the_scratch():
    say("noalloc: refusal")
    p = make_problem(903, B=2, Hq=16, Hkv=2, D=512, P=32, lens=[400, 90], sm_scale=1.0)
    dev = device_problem(p)
    wg = 600                                   # 600 x 2 x 8 x 512 x 4 bytes of partials > 16 MiB
    plan = ops.decode_plan(p.B, p.Hq, dev["kd"], dev["vd"], 400, 0, wg)
    assert plan.workspace_bytes > ops.NOALLOC_SCRATCH_BYTES
    ops.reset_counters()
    with pytest.raises(ops.Fp8paError) as e:
        ops.decode_noalloc(dev["q"], dev["k_pool"], dev["v_pool"], dev["kd"], dev["vd"], dev["block_table"],
                           dev["seq_lens"], 400, sm_scale=1.0, workgroups=wg)
    assert e.value.code == ops.EWORKSPACE
    c = ops.counters()
    assert c["decode_calls"] == 0 and c["errors"] == 1
