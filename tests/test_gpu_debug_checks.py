"""In-kernel debug checks of the device-resident arguments
(fp8pa_set_debug_checks): with valid inputs nothing is flagged and outputs
are bit-identical to unchecked calls; a table entry outside the pools in an
attended page, or a length above max_seq_len, sets its error word, is read as
row 0 / length 0 (never outside the pools), and leaves the other sequences'
outputs correct; unattended -1 entries are never read, so never flagged; the
append skips a bad row.  The bad values are planted on the host."""
import numpy as np
import pytest
import torch

from fp8_paged_kv_amd import ops
from oracle import attention as oatt
from tests.gpu_util import DEV, assert_parity, desc_of, device_problem, gpu_decode, say, to_np
from tests.problems import add_guard_rows, full_page_row, make_problem, swap_rows

pytestmark = pytest.mark.gpu


@pytest.fixture
def err():
    e = torch.zeros(2, dtype=torch.int32, device=DEV)
    ops.set_debug_checks(e)
    try:
        yield e
    finally:
        ops.set_debug_checks(None)


def oracle(p, seqs=None):
    return oatt.decode_ref(p.q, p.k_pool, p.v_pool, p.kdesc, p.vdesc, p.table, p.seq_lens, window=p.window,
                           sinks=p.sinks, sm_scale=p.sm_scale, seqs=seqs)


CASES = [
    ("split", dict(B=3, Hq=16, Hkv=4, D=128, P=16, lens=[900, 100, 20], window=300, sinks=True), {}),
    ("v-tokens", dict(B=2, Hq=16, Hkv=4, D=64, P=16, lens=[300, 65], v_layout="tokens"), {}),
    ("packed", dict(B=3, Hq=16, Hkv=4, D=128, P=16, lens=[513, 64, 1]), {"variant": "packed_heads"}),
    ("packed-split", dict(B=3, Hq=16, Hkv=4, D=128, P=16, lens=[513, 64, 1]), {"variant": "packed_split"}),
    ("many-sequences", dict(B=80, Hq=8, Hkv=2, D=64, P=16, lens=list(range(3, 243, 3))), {}),
]


@pytest.mark.parametrize("name,kw,extra", CASES, ids=[c[0] for c in CASES])
def test_checks_pass_valid_inputs_unchanged(err, name, kw, extra):
    say("debug checks valid", name)
    p = make_problem(801, **kw)
    t = p.table.copy()
    for b in range(p.B):
        t[b, -(-int(p.seq_lens[b]) // p.P):] = -1        # unattended entries: never read
    from dataclasses import replace
    p = replace(p, table=t)
    dev = device_problem(p)
    got = gpu_decode(p, dev=dev, **extra)
    assert err.tolist() == [0, 0], name
    ops.set_debug_checks(None)
    want = gpu_decode(p, dev=dev, **extra)
    assert torch.equal(got.view(torch.int16), want.view(torch.int16)), name


@pytest.mark.parametrize("guard", [0, 1])
def test_bad_table_entry_is_flagged_and_contained(err, guard):
    """An attended page's entry points at a row past num_rows (a poisoned
    guard row inside the allocation): flagged, read as row 0 instead."""
    say("debug checks table", guard)
    p0 = make_problem(802, B=3, Hq=16, Hkv=4, D=128, P=16, lens=[700, 90, 33])
    p0 = swap_rows(p0, 0, full_page_row(p0))              # row 0, read in place of a bad entry, is a full page
    p, rows = add_guard_rows(p0)
    from dataclasses import replace
    t = p.table.copy()
    t[1, 2] = rows[guard]                                 # an attended page of sequence 1
    got = to_np(gpu_decode(replace(p, table=t), workgroups=5))
    assert err.tolist() == [1, 0]
    assert np.all(np.isfinite(got[[0, 2]]))
    assert np.all(np.isfinite(got[1])), "a guard row was read"
    want = oracle(p0, seqs=[0, 2])
    for b in (0, 2):
        assert_parity(got[b], want[b], f"sequence {b}")


def test_bad_length_is_flagged_and_zeroed(err):
    say("debug checks length")
    p = make_problem(803, B=3, Hq=16, Hkv=4, D=128, P=16, lens=[300, 90, 33])
    dev = device_problem(p)
    dev["seq_lens"][1] = 5000                             # above max_seq_len = 300
    got = to_np(gpu_decode(p, dev=dev, max_seq_len=300))
    assert err.tolist() == [0, 1]
    assert np.all(got[1] == 0.0)
    want = oracle(p, seqs=[0, 2])
    for b in (0, 2):
        assert_parity(got[b], want[b], f"sequence {b}")
    err.zero_()
    dev["seq_lens"][1] = -7
    got = to_np(gpu_decode(p, dev=dev, max_seq_len=300))
    assert err.tolist() == [0, 1] and np.all(got[1] == 0.0)


def test_append_skips_a_bad_row(err):
    say("debug checks append")
    p, rows = add_guard_rows(make_problem(804, B=2, Hq=8, Hkv=2, D=64, P=16, lens=[40, 20]))
    kd, vd = desc_of(p.kdesc), desc_of(p.vdesc)
    t = p.table.copy()
    t[1, 1] = rows[0]                                     # the page of position 20: a guard row
    ka, va = torch.from_numpy(p.k_pool).to(DEV), torch.from_numpy(p.v_pool).to(DEV)
    k0, v0 = ka.clone(), va.clone()
    x = torch.randn((2, 1, 2, 64), generator=torch.Generator().manual_seed(9)).to(torch.bfloat16).to(DEV)
    ops.append_quant(x, x, ka, va, kd, vd, torch.from_numpy(t).to(DEV),
                     torch.tensor([39, 20], dtype=torch.int32, device=DEV))
    torch.cuda.synchronize()
    assert err.tolist() == [1, 0]
    # sequence 0's token is written, sequence 1's is not (and nothing else changes)
    changed = (ka != k0).nonzero().flatten().cpu().numpy()
    row0 = int(p.table[0, 39 // 16])
    rb = p.kdesc.row_bytes
    assert changed.size > 0 and np.all(changed // rb == row0)


def test_append_decode_under_checks_takes_two_launches(err):
    p = make_problem(805, B=2, Hq=8, Hkv=2, D=64, P=16, lens=[40, 20])
    kd, vd = desc_of(p.kdesc), desc_of(p.vdesc)
    dev = device_problem(p)
    x = torch.randn((2, 2, 64), generator=torch.Generator().manual_seed(10)).to(torch.bfloat16).to(DEV)
    ops.reset_counters()
    ops.append_decode(dev["q"], x, x, dev["k_pool"], dev["v_pool"], kd, vd, dev["block_table"], dev["seq_lens"],
                      40, sm_scale=p.sm_scale)
    torch.cuda.synchronize()
    c = ops.counters()
    assert c["append_launches"] == 1 and c["fused_appends"] == 0
    assert err.tolist() == [0, 0]
