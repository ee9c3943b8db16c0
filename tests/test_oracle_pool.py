"""Pins for the oracle's pool format, packing and reference append (CPU only)."""
from dataclasses import replace

import numpy as np
import pytest

from fp8_paged_kv_amd import inputs
from oracle import fp8, pool as opool
from tests.problems import make_problem, permute_rows


def kinds_for(D):
    """Scale kinds that a head dim D can take."""
    return [k for k in opool.SCALE_KINDS if D % opool.GROUP_KINDS.get(k, 1) == 0]


@pytest.mark.parametrize("layout", opool.LAYOUTS)
@pytest.mark.parametrize("kind", opool.SCALE_KINDS)
@pytest.mark.parametrize("P,D", [(16, 64), (32, 128), (128, 128)])
def test_offsets_are_a_bijection_inside_the_row(layout, kind, P, D):
    H = 3
    if kind not in kinds_for(D):
        pytest.skip("group wider than the head dim")
    d = opool.natural_desc(H, D, P, layout, kind, 1)
    h, t, dd = np.meshgrid(np.arange(H), np.arange(P), np.arange(D), indexing="ij")
    off = opool.code_offset(d, h, t, dd).ravel()
    assert np.array_equal(np.sort(off), np.arange(H * P * D))
    if kind == "page_head":
        s = [opool.scale_offset(d, hh) + i for hh in range(H) for i in range(4)]
    elif kind == "token_head":
        s = [opool.scale_offset(d, hh, tt) + i for hh in range(H) for tt in range(P) for i in range(4)]
    elif kind in opool.GROUP_KINDS:
        ng = D // opool.GROUP_KINDS[kind]
        s = [opool.scale_offset(d, hh, tt, g) + i for hh in range(H) for tt in range(P) for g in range(ng)
             for i in range(4)]
    else:
        s = [opool.scale_offset(d, hh, tt, g) for hh in range(H) for tt in range(P) for g in range(D // 32)]
    assert np.array_equal(np.sort(s), d.footer + np.arange(d.scale_bytes))
    assert d.footer == d.payload_bytes


@pytest.mark.parametrize("kind", kinds_for(64))
def test_layouts_read_back_the_same_values(kind):
    vals = []
    for layout in opool.LAYOUTS:
        p = make_problem(1, B=2, Hq=4, Hkv=2, D=64, P=16, lens=[37, 16], scale_kind=kind,
                         k_layout=layout, v_layout=layout)
        vals.append([opool.read_tokens(p.k_pool, p.kdesc, p.table[b], np.arange(p.seq_lens[b]), h)
                     for b in range(2) for h in range(2)])
    for other in vals[1:]:
        for a, b in zip(vals[0], other):
            assert np.array_equal(a, b)


@pytest.mark.parametrize("kind", kinds_for(64))
def test_pack_read_round_trip_within_quantisation_error(kind):
    p = make_problem(2, B=2, Hq=2, Hkv=2, D=64, P=16, lens=[50, 3], scale_kind=kind)
    for b in range(2):
        for h in range(2):
            x = p.raw_k[b][:, h, :].astype(np.float64)
            xh = opool.read_tokens(p.k_pool, p.kdesc, p.table[b], np.arange(p.seq_lens[b]), h)
            if kind == "page_head":
                s = np.repeat([np.abs(x[i:i + 16]).max() / 448 for i in range(0, len(x), 16)], 16)[:len(x), None]
            elif kind == "token_head":
                s = np.abs(x).max(axis=1, keepdims=True) / 448
            elif kind in opool.GROUP_KINDS:
                S = opool.GROUP_KINDS[kind]
                s = np.repeat(np.abs(x).reshape(len(x), -1, S).max(-1) / 448, S, axis=1)
            else:
                s = np.repeat(2.0 ** np.ceil(np.log2(np.abs(x).reshape(len(x), -1, 32).max(-1) / 448)), 32, axis=1)
            # half an E4M3 step (2^-4 relative, 2^-10 absolute in scale units) plus slack for fp32 rounding
            assert np.all(np.abs(xh - x) <= np.abs(x) * (2 ** -4 + 2 ** -20) + s * 2 ** -9)


def test_row_permutation_leaves_values_unchanged():
    p = make_problem(3, B=3, Hq=4, Hkv=2, D=64, P=16, lens=[40, 1, 33])
    p2 = permute_rows(p, seed=9)
    assert not np.array_equal(p.table, p2.table)
    for b in range(3):
        for h in range(2):
            J = np.arange(p.seq_lens[b])
            assert np.array_equal(opool.read_tokens(p.k_pool, p.kdesc, p.table[b], J, h),
                                  opool.read_tokens(p2.k_pool, p2.kdesc, p2.table[b], J, h))


@pytest.mark.parametrize("kind", kinds_for(64))
@pytest.mark.parametrize("layout", ["heads", "heads_d64", "heads_dmajor"])
def test_bulk_append_equals_pack(kind, layout):
    p = make_problem(4, B=2, Hq=2, Hkv=2, D=64, P=16, lens=[35, 35], scale_kind=kind,
                     k_layout=layout, v_layout=layout)
    empty = np.full_like(p.k_pool, 0xFF)
    x = np.stack(p.raw_k)                                            # [2, 35, H, D]
    got = opool.append_ref(empty, p.kdesc, p.table, [0, 0], x)
    assert np.array_equal(got, p.k_pool)


def test_t1_appends_with_leading_page_maximum_equal_bulk():
    """When each page's first token holds the page maximum, no re-encode happens
    and token-by-token appends equal the bulk write."""
    B, L, H, D, P = 1, 40, 2, 64, 16
    x = inputs.normal_bf16(5, 0, "k", 0, (L, H, D)).astype(np.float64)
    for p0 in range(0, L, P):
        x[p0] *= 8.0                                                 # page max sits in token p0
    table, rows = inputs.block_table(5, 0, [L], P)
    d = opool.natural_desc(H, D, P, "heads", "page_head", rows)
    empty = np.full(rows * d.row_bytes, 0xFF, dtype=np.uint8)
    bulk = opool.pack_sequences(empty, d, table, [x])
    step = empty
    for t in range(L):
        step = opool.append_ref(step, d, table, [t], x[None, t:t + 1])
    assert np.array_equal(step, bulk)


def _t1_replay(x, P, seed):
    L, H, D = x.shape
    table, rows = inputs.block_table(seed, 0, [L], P)
    d = opool.natural_desc(H, D, P, "heads", "page_head", rows)
    pool_ = np.full(rows * d.row_bytes, 0xFF, dtype=np.uint8)
    for t in range(L):
        pool_ = opool.append_ref(pool_, d, table, [t], x[None, t:t + 1])
    return pool_, d, table


def test_t1_appends_end_with_page_amax_scale():
    L, H, D, P = 48, 2, 64, 16
    x = inputs.normal_bf16(6, 0, "k", 0, (L, H, D)).astype(np.float64)
    x *= np.linspace(0.1, 4.0, L)[:, None, None]                     # growing amax: many re-encodes
    pool_, d, table = _t1_replay(x, P, 6)
    for pg in range(L // P):
        for h in range(H):
            at = table[0, pg] * d.row_bytes + opool.scale_offset(d, h)
            s = float(pool_[at:at + 4].copy().view(np.float32)[0])
            assert s == float(np.float32(np.abs(x[pg * P:(pg + 1) * P, h]).max() / 448))   # rounding is monotone


def test_t1_single_growth_reencodes_once_with_bounded_error():
    """Slot 8 of each page raises the page maximum once: slots 0..7 are rounded
    twice (at most one full E4M3 step), slots 8.. once (half a step)."""
    L, H, D, P = 32, 2, 64, 16
    x = inputs.normal_bf16(7, 0, "k", 0, (L, H, D)).astype(np.float64)
    x[0::P] *= 8.0
    x[8::P] *= 64.0
    pool_, d, table = _t1_replay(x, P, 7)
    for pg in range(L // P):
        xs = x[pg * P:(pg + 1) * P]
        xh = np.stack([opool.read_tokens(pool_, d, table[0], np.arange(pg * P, (pg + 1) * P), h) for h in range(H)], 1)
        s = np.abs(xs).max(axis=(0, 2)) / 448
        err = np.abs(xh - xs)
        slack = 1 + 2 ** -16
        assert np.all(err[:8] <= (np.abs(xs[:8]) * 2 ** -3 + s[None, :, None] * 2 ** -9) * slack)
        assert np.all(err[8:] <= (np.abs(xs[8:]) * 2 ** -4 + s[None, :, None] * 2 ** -10) * slack)
        assert np.any(err[:8] > (np.abs(xs[:8]) * 2 ** -4 + s[None, :, None] * 2 ** -10) * slack), \
            "expected at least one doubly rounded code"


def test_token_scale_equals_page_scale_when_pages_hold_one_token():
    L, H, D = 9, 2, 64
    x = inputs.normal_bf16(7, 0, "k", 0, (L, H, D))
    table, rows = inputs.block_table(7, 0, [L], 1)
    a = opool.natural_desc(H, D, 1, "heads", "page_head", rows)
    b = opool.natural_desc(H, D, 1, "heads", "token_head", rows)
    pa = opool.append_ref(np.zeros(rows * a.row_bytes, np.uint8), a, table, [0], x[None])
    pb = opool.append_ref(np.zeros(rows * b.row_bytes, np.uint8), b, table, [0], x[None])
    assert np.array_equal(pa, pb)


def test_append_respects_counts_and_leaves_other_rows():
    p = make_problem(8, B=2, Hq=2, Hkv=2, D=64, P=16, lens=[20, 20])
    x = np.stack(p.raw_k)
    got = opool.append_ref(np.full_like(p.k_pool, 0xFF), p.kdesc, p.table, [0, 0], x, counts=[20, 0])
    rows_b1 = set(p.table[1][p.table[1] >= 0].tolist())
    g2 = got.reshape(p.kdesc.num_rows, -1)
    for r in rows_b1:
        assert np.all(g2[r] == 0xFF)


def _payload_as_hpd(payload, layout, H, P, D):
    """The payload stated as a C-order array whose axes the layout names,
    brought to [H, P, D] by reshapes and transposes only."""
    if layout == "heads":
        return payload.reshape(H, P, D)
    if layout == "tokens":
        return payload.reshape(P, H, D).transpose(1, 0, 2)
    if layout == "heads_d64":
        return payload.reshape(H, D // 64, P, 64).transpose(0, 2, 1, 3).reshape(H, P, D)
    W = min(P, 64)
    return payload.reshape(H, P // W, D, W).transpose(0, 1, 3, 2).reshape(H, P, D)


@pytest.mark.parametrize("layout", opool.LAYOUTS)
@pytest.mark.parametrize("kind", opool.SCALE_KINDS)
@pytest.mark.parametrize("P,D", [(16, 64), (16, 128), (128, 128), (256, 64)])
def test_row_layout_matches_reshape_views(layout, kind, P, D):
    """The row format stated a second way: the payload is a C-order array whose
    axes are named by the layout, the footer a C-order array of scales."""
    H = 2
    if kind not in kinds_for(D):
        pytest.skip("group wider than the head dim")
    p = make_problem(9, B=1, Hq=2, Hkv=H, D=D, P=P, lens=[P], scale_kind=kind, k_layout=layout, v_layout=layout)
    d = p.kdesc
    row = int(p.table[0, 0])
    r = p.k_pool[row * d.row_bytes:(row + 1) * d.row_bytes]
    codes = _payload_as_hpd(r[:d.payload_bytes], layout, H, P, D)
    foot = r[d.footer:d.footer + d.scale_bytes]
    if kind == "page_head":
        sc = foot.copy().view(np.float32).astype(np.float64)[:, None, None]
    elif kind == "token_head":
        f = foot.copy().view(np.float32).astype(np.float64)
        sc = (f.reshape(P, H).T if layout == "tokens" else f.reshape(H, P))[:, :, None]
    elif kind in opool.GROUP_KINDS:
        S = opool.GROUP_KINDS[kind]
        f = foot.copy().view(np.float32).astype(np.float64)
        f = f.reshape(P, H, D // S).transpose(1, 0, 2) if layout == "tokens" else f.reshape(H, P, D // S)
        sc = np.repeat(f, S, axis=-1)
    else:
        u = foot.reshape(P, H, D // 32).transpose(1, 0, 2) if layout == "tokens" else foot.reshape(H, P, D // 32)
        sc = np.repeat(fp8.E8M0_TABLE[u], 32, axis=-1)
    want = fp8.E4M3_TABLE[codes] * sc                                           # [H, P, D]
    for h in range(H):
        got = opool.read_tokens(p.k_pool, d, p.table[0], np.arange(P), h)
        assert np.array_equal(got, want[h])
    assert np.array_equal(np.sort(r[:d.payload_bytes]), np.sort(codes.ravel()))


@pytest.mark.parametrize("layout,H,P,D,kind,rb", [
    ("heads_d64", 8, 16, 128, "page_head", 16384 + 32),      # rows 32 bytes past a 64-byte multiple
    ("heads_dmajor", 8, 16, 64, "page_head", 8192 + 32),
    ("heads_dmajor", 2, 32, 512, "page_head", 65536 + 32),   # scales (8 B) fit in a 32-byte gap
    ("heads", 2, 16, 64, "token_head", 2048 + 128 + 48),      # shifts 0, 16, 32, 48
    ("tokens", 2, 16, 64, "e8m0_32", 2048 + 64 + 48),
])
def test_align64_rows(layout, H, P, D, kind, rb):
    """Aligned rows: every payload starts on a 64-byte boundary of the pool,
    payload and scales stay inside their row without overlapping, and the
    pool decodes to exactly what the unaligned placement of the same data
    decodes to."""
    rows = 9
    plain = opool.PoolDesc(H, D, P, layout, kind, rb, rows)
    al = replace(plain, align64=True)
    plain.check()
    al.check()
    r = np.arange(rows)
    cb = opool.row_code_base(al, r)
    sb = opool.row_scale_base(al, r)
    assert np.all(cb % 64 == 0)
    assert np.all(cb >= r * rb) and np.all(cb + al.payload_bytes <= (r + 1) * rb)
    assert np.all(sb >= r * rb) and np.all(sb + al.scale_bytes <= (r + 1) * rb)
    assert np.all((sb + al.scale_bytes <= cb) | (sb >= cb + al.payload_bytes))
    rng = np.random.default_rng(5)
    L = rows * P - 3
    table = [rng.permutation(rows)]
    x = rng.standard_normal((L, H, D))
    pp = opool.pack_sequences(np.zeros(rows * rb, np.uint8), plain, table, [x])
    pa = opool.pack_sequences(np.zeros(rows * rb, np.uint8), al, table, [x])
    pos = np.arange(L)
    for h in range(H):
        np.testing.assert_array_equal(opool.read_tokens(pa, al, table[0], pos, h),
                                      opool.read_tokens(pp, plain, table[0], pos, h))
    # the same holds for the token-by-token append (page scales that grow)
    pos0 = np.zeros(1, np.int64)
    xa = rng.standard_normal((1, 2 * P + 1, H, D))
    qa = opool.append_ref(np.zeros(rows * rb, np.uint8), al, table, pos0, xa)
    qp = opool.append_ref(np.zeros(rows * rb, np.uint8), plain, table, pos0, xa)
    for h in range(H):
        np.testing.assert_array_equal(opool.read_tokens(qa, al, table[0], np.arange(2 * P + 1), h),
                                      opool.read_tokens(qp, plain, table[0], np.arange(2 * P + 1), h))


def test_align64_needs_room():
    """A row too narrow for some payload shift is refused."""
    d = opool.PoolDesc(2, 64, 16, "heads", "token_head", 2048 + 128 + 48, 4, align64=True)
    d.check()
    with pytest.raises(AssertionError):
        replace(d, row_bytes=2048 + 128 + 48 - 64).check()
