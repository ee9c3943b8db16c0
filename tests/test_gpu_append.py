"""The GPU append/quantize kernel writes exactly the oracle's bytes: bulk
writes, token-by-token appends with growing page scales, counts, unaligned
starting positions, all scale kinds (fp32 sub-row groups included) and
layouts."""
import numpy as np
import pytest
import torch

from fp8_paged_kv_amd import inputs, ops
from oracle import pool as opool
from tests.gpu_util import DEV, desc_of, say
from tests.problems import round16

pytestmark = pytest.mark.gpu


def make(kind, layout, H=2, D=64, P=16, lens=(40, 17), seed=3, align64=False):
    if D % opool.GROUP_KINDS.get(kind, 1):
        pytest.skip("group wider than the head dim")
    table, rows = inputs.block_table(seed, 5, lens, P)
    d = opool.natural_desc(H, D, P, layout, kind, rows)
    from dataclasses import replace
    d = replace(d, row_bytes=round16(d.row_bytes))
    if align64:
        # a row width off the 64-byte grid, with room for every payload shift
        rb = d.row_bytes + 48
        rb += (32 - rb % 64) % 64 if rb % 64 != 32 else 0
        d = replace(d, row_bytes=rb, align64=True)
        d.check()
    return table, d


def run_gpu(pool_k, pool_v, kd, vd, table, positions, xk, xv, counts=None):
    k = torch.from_numpy(pool_k).to(DEV)
    v = torch.from_numpy(pool_v).to(DEV)
    ops.append_quant(torch.from_numpy(xk).to(torch.bfloat16).to(DEV), torch.from_numpy(xv).to(torch.bfloat16).to(DEV),
                     k, v, desc_of(kd), desc_of(vd), torch.from_numpy(table).to(DEV),
                     torch.tensor(positions, dtype=torch.int32, device=DEV),
                     None if counts is None else torch.tensor(counts, dtype=torch.int32, device=DEV))
    torch.cuda.synchronize()
    return k.cpu().numpy(), v.cpu().numpy()


@pytest.mark.parametrize("kind", opool.SCALE_KINDS)
@pytest.mark.parametrize("klayout,vlayout", [("heads", "heads_dmajor"), ("tokens", "heads_dmajor"), ("heads", "tokens"),
                                             ("heads_d64", "heads_dmajor")])
@pytest.mark.parametrize("D", [64, 128, 256])
def test_bulk_append_bit_exact(kind, klayout, vlayout, D):
    say("bulk append", kind, klayout, vlayout, D)
    lens = [40, 17]
    table, kd = make(kind, klayout, D=D, lens=lens)
    _, vd = make(kind, vlayout, D=D, lens=lens)
    from dataclasses import replace
    vd = replace(vd, num_rows=kd.num_rows)
    T = max(lens)
    xk = inputs.round_to_bf16(np.stack([inputs.normal_bf16(1, 0, "k", b, (T, 2, D)) for b in range(2)]) * np.float32(3.0))
    xv = np.stack([inputs.normal_bf16(1, 0, "v", b, (T, 2, D)) for b in range(2)])
    empty_k = np.full(kd.num_rows * kd.row_bytes, 0xFF, np.uint8)
    empty_v = np.full(vd.num_rows * vd.row_bytes, 0xFF, np.uint8)
    gk, gv = run_gpu(empty_k, empty_v, kd, vd, table, [0, 0], xk, xv, counts=lens)
    wk = opool.append_ref(empty_k, kd, table, [0, 0], xk, counts=lens)
    wv = opool.append_ref(empty_v, vd, table, [0, 0], xv, counts=lens)
    assert np.array_equal(gk, wk)
    assert np.array_equal(gv, wv)


@pytest.mark.parametrize("kind", opool.SCALE_KINDS)
def test_token_by_token_append_bit_exact(kind):
    """T=1 appends one after another, with the magnitude growing so that page
    scales grow and earlier tokens are re-encoded."""
    say("t1 append", kind)
    L, H, D, P = 37, 2, 64, 16
    table, kd = make(kind, "heads", H, D, P, lens=(L, L))
    _, vd = make(kind, "heads_dmajor", H, D, P, lens=(L, L))
    gain = np.linspace(0.2, 5.0, L).astype(np.float32)[:, None, None]
    xk = np.stack([inputs.normal_bf16(2, 0, "k", b, (L, H, D)) for b in range(2)]) * gain
    xv = np.stack([inputs.normal_bf16(2, 0, "v", b, (L, H, D)) for b in range(2)]) * gain[::-1]
    xk = xk.astype(np.float32); xv = xv.astype(np.float32)
    from fp8_paged_kv_amd.inputs import round_to_bf16
    xk, xv = round_to_bf16(xk), round_to_bf16(xv)
    gk = np.full(kd.num_rows * kd.row_bytes, 0xFF, np.uint8)
    gv = np.full(vd.num_rows * vd.row_bytes, 0xFF, np.uint8)
    wk, wv = gk.copy(), gv.copy()
    dk, dv = torch.from_numpy(gk).to(DEV), torch.from_numpy(gv).to(DEV)
    tab = torch.from_numpy(table).to(DEV)
    for t in range(L):
        ops.append_quant(torch.from_numpy(np.ascontiguousarray(xk[:, t:t + 1])).to(torch.bfloat16).to(DEV),
                         torch.from_numpy(np.ascontiguousarray(xv[:, t:t + 1])).to(torch.bfloat16).to(DEV),
                         dk, dv, desc_of(kd), desc_of(vd), tab, torch.tensor([t, t], dtype=torch.int32, device=DEV))
        wk = opool.append_ref(wk, kd, table, [t, t], xk[:, t:t + 1])
        wv = opool.append_ref(wv, vd, table, [t, t], xv[:, t:t + 1])
    torch.cuda.synchronize()
    assert np.array_equal(dk.cpu().numpy(), wk)
    assert np.array_equal(dv.cpu().numpy(), wv)


def test_chunked_append_from_unaligned_positions_bit_exact():
    say("chunked append")
    L, H, D, P = 70, 2, 128, 16
    table, kd = make("page_head", "heads", H, D, P, lens=(L,))
    _, vd = make("page_head", "heads_dmajor", H, D, P, lens=(L,))
    x = inputs.normal_bf16(3, 0, "k", 0, (L, H, D)) * np.linspace(0.5, 2, L).astype(np.float32)[:, None, None]
    x = inputs.round_to_bf16(x.astype(np.float32))
    gk = np.full(kd.num_rows * kd.row_bytes, 0xFF, np.uint8)
    gv = np.full(vd.num_rows * vd.row_bytes, 0xFF, np.uint8)
    wk, wv = gk.copy(), gv.copy()
    dk, dv = torch.from_numpy(gk).to(DEV), torch.from_numpy(gv).to(DEV)
    tab = torch.from_numpy(table).to(DEV)
    cuts = [0, 5, 23, 24, 41, 70]
    for a, c in zip(cuts[:-1], cuts[1:]):
        chunk = np.ascontiguousarray(x[None, a:c])
        ops.append_quant(torch.from_numpy(chunk).to(torch.bfloat16).to(DEV), torch.from_numpy(chunk).to(torch.bfloat16).to(DEV),
                         dk, dv, desc_of(kd), desc_of(vd), tab, torch.tensor([a], dtype=torch.int32, device=DEV))
        wk = opool.append_ref(wk, kd, table, [a], chunk)
        wv = opool.append_ref(wv, vd, table, [a], chunk)
    torch.cuda.synchronize()
    assert np.array_equal(dk.cpu().numpy(), wk)
    assert np.array_equal(dv.cpu().numpy(), wv)
    assert ops.counters()["append_launches"] >= 5


@pytest.mark.parametrize("kind", opool.SCALE_KINDS)
@pytest.mark.parametrize("P", [64, 128, 256])
def test_bulk_append_large_pages_bit_exact(kind, P):
    """Pages of 64+ tokens: blocked d-major values and 64-byte-chunked keys."""
    say("large-page append", kind, P)
    lens = [300, 129]
    table, kd = make(kind, "heads_d64", D=128, P=P, lens=lens)
    _, vd = make(kind, "heads_dmajor", D=128, P=P, lens=lens)
    T = max(lens)
    xk = np.stack([inputs.normal_bf16(4, 0, "k", b, (T, 2, 128)) for b in range(2)])
    xv = np.stack([inputs.normal_bf16(4, 0, "v", b, (T, 2, 128)) for b in range(2)])
    empty_k = np.full(kd.num_rows * kd.row_bytes, 0xFF, np.uint8)
    empty_v = np.full(vd.num_rows * vd.row_bytes, 0xFF, np.uint8)
    gk, gv = run_gpu(empty_k, empty_v, kd, vd, table, [0, 0], xk, xv, counts=lens)
    assert np.array_equal(gk, opool.append_ref(empty_k, kd, table, [0, 0], xk, counts=lens))
    assert np.array_equal(gv, opool.append_ref(empty_v, vd, table, [0, 0], xv, counts=lens))


@pytest.mark.parametrize("kind", opool.SCALE_KINDS)
@pytest.mark.parametrize("klayout,vlayout", [("heads_d64", "heads_dmajor"), ("tokens", "heads_dmajor")])
def test_append_aligned_rows_bit_exact(kind, klayout, vlayout):
    """Rows 32 bytes off the 64-byte grid, payloads placed on it: bulk writes,
    then T=1 appends with growing page scales, byte-for-byte as the oracle."""
    say("aligned append", kind, klayout, vlayout)
    lens = [70, 33]
    table, kd = make(kind, klayout, D=128, lens=lens, align64=True)
    _, vd = make(kind, vlayout, D=128, lens=lens, align64=True)
    from dataclasses import replace
    vd = replace(vd, num_rows=kd.num_rows)
    T = max(lens)
    xk = np.stack([inputs.normal_bf16(2, 0, "k", b, (T, 2, 128)) for b in range(2)])
    xv = np.stack([inputs.normal_bf16(2, 0, "v", b, (T, 2, 128)) for b in range(2)])
    k0 = np.full(kd.num_rows * kd.row_bytes, 0xFF, np.uint8)
    v0 = np.full(vd.num_rows * vd.row_bytes, 0xFF, np.uint8)
    gk, gv = run_gpu(k0, v0, kd, vd, table, [0, 0], xk, xv, counts=[40, 20])
    wk = opool.append_ref(k0, kd, table, [0, 0], xk, counts=[40, 20])
    wv = opool.append_ref(v0, vd, table, [0, 0], xv, counts=[40, 20])
    assert np.array_equal(gk, wk) and np.array_equal(gv, wv)
    for step in range(3):
        pos = [40 + step, 20 + step]
        x1k = xk[:, 40 + step:41 + step] * np.float32(1.5 ** step)
        x1v = xv[:, 40 + step:41 + step] * np.float32(1.5 ** step)
        x1k, x1v = inputs.round_to_bf16(x1k), inputs.round_to_bf16(x1v)
        gk, gv = run_gpu(gk, gv, kd, vd, table, pos, x1k, x1v)
        wk = opool.append_ref(wk, kd, table, pos, x1k)
        wv = opool.append_ref(wv, vd, table, pos, x1v)
        assert np.array_equal(gk, wk) and np.array_equal(gv, wv), f"step {step}"
