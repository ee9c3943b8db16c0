"""Pins for the oracle's sub-row fp32 key scales ("f32_g<S>": one fp32 scale
per (token, head, S dims), the page's ``k_groups`` = D/S option; page "fp8
paged attention for MoE serving", section "Supported scope").  CPU only.

Each pin ties the grouped kind to something defined apart from its own code:
a group as wide as the head is the per-(token, head) kind byte for byte; each
group of a pool reads back exactly what a per-(token, head) pool of that group's
dims alone reads back (so a wrong group index, stride or order fails); the
per-group scale is the group's own amax/448; and decode over such a pool is
plain softmax attention over the dequantized values."""
import numpy as np
import pytest

from fp8_paged_kv_amd import inputs
from oracle import attention as oatt, fp8, pool as opool
from tests.problems import make_problem


@pytest.mark.parametrize("layout", opool.LAYOUTS)
@pytest.mark.parametrize("D,kind", [(64, "f32_g64"), (128, "f32_g128"), (256, "f32_g256")])
def test_group_as_wide_as_the_head_is_the_token_kind(layout, D, kind):
    """k_groups = 1: the same footer size, offsets, codes and scales as "token_head"."""
    a = make_problem(31, B=2, Hq=4, Hkv=2, D=D, P=16, lens=[40, 7], scale_kind=kind, k_layout=layout,
                     v_layout=layout)
    b = make_problem(31, B=2, Hq=4, Hkv=2, D=D, P=16, lens=[40, 7], scale_kind="token_head", k_layout=layout,
                     v_layout=layout)
    assert a.kdesc.scale_bytes == b.kdesc.scale_bytes and a.kdesc.row_bytes == b.kdesc.row_bytes
    assert np.array_equal(a.k_pool, b.k_pool)


@pytest.mark.parametrize("kind", ["f32_g8", "f32_g16", "f32_g32", "f32_g64"])
@pytest.mark.parametrize("layout", ["heads", "tokens", "heads_d64", "heads_dmajor"])
def test_each_group_reads_back_as_its_own_token_scaled_row(kind, layout):
    """Group g of head h holds exactly what a "token_head" pool built from the
    dims [g*S, (g+1)*S) alone holds."""
    S = opool.GROUP_KINDS[kind]
    D, P, H = 128, 16, 2
    p = make_problem(32, B=2, Hq=4, Hkv=H, D=D, P=P, lens=[45, 16], scale_kind=kind, k_layout=layout,
                     v_layout=layout)
    table, rows = p.table, p.kdesc.num_rows
    for g in range(D // S):
        d1 = opool.natural_desc(H, S, P, "heads", "token_head", rows)
        one = opool.pack_sequences(np.zeros(rows * d1.row_bytes, np.uint8), d1, table,
                                   [x[:, :, g * S:(g + 1) * S] for x in p.raw_k])
        for b in range(2):
            J = np.arange(p.seq_lens[b])
            for h in range(H):
                got = opool.read_tokens(p.k_pool, p.kdesc, table[b], J, h)[:, g * S:(g + 1) * S]
                want = opool.read_tokens(one, d1, table[b], J, h)
                assert np.array_equal(got, want), (g, b, h)


def test_group_scale_is_the_groups_amax_over_448():
    D, S, P = 128, 32, 16
    p = make_problem(33, B=1, Hq=2, Hkv=1, D=D, P=P, lens=[20], scale_kind="f32_g32", k_layout="heads")
    x = p.raw_k[0][:, 0, :].astype(np.float64)
    x[3, 40:64] = 0.0                                                # part of group 1 of token 3
    x[5, 64:96] = 0.0                                                # all of group 2 of token 5: scale 1
    d = p.kdesc
    pool = opool.pack_sequences(np.zeros_like(p.k_pool), d, p.table, [x[:, None, :]])
    for t in range(20):
        row = int(p.table[0, t // P])
        for g in range(D // S):
            at = int(opool.row_scale_base(d, row)) + opool.scale_rel(d, 0, t % P, g)
            s = float(pool[at:at + 4].copy().view(np.float32)[0])
            amax = np.abs(x[t, g * S:(g + 1) * S]).max()
            want = 1.0 if amax == 0 else float(np.float32(amax / 448.0))
            assert s == want, (t, g)


@pytest.mark.parametrize("kind", ["f32_g32", "f32_g64"])
def test_appends_equal_the_bulk_pack(kind):
    """Token-by-token reference appends (stateless per group) equal the bulk pack."""
    D, P, H, L = 128, 16, 2, 37
    x = inputs.normal_bf16(34, 0, "k", 0, (L, H, D)).astype(np.float64)
    x[:, :, :32] *= 64.0                                             # groups of very different ranges
    table, rows = inputs.block_table(34, 0, [L], P)
    d = opool.natural_desc(H, D, P, "tokens", kind, rows)
    empty = np.full(rows * d.row_bytes, 0xFF, dtype=np.uint8)
    bulk = opool.pack_sequences(empty, d, table, [x])
    step = empty
    for t in range(L):
        step = opool.append_ref(step, d, table, [t], x[None, t:t + 1])
    assert np.array_equal(step, bulk)


def test_groups_keep_small_dims_that_one_row_scale_flushes():
    """The reason for sub-row scales: with one large group in the row, the
    small dims survive per group but underflow to zero under one row scale."""
    D, P = 128, 16
    x = np.full((P, 1, D), 1e-4)
    x[:, :, :32] = 300.0
    vals = {}
    for kind in ("token_head", "f32_g32"):
        table, rows = inputs.block_table(35, 0, [P], P)
        d = opool.natural_desc(1, D, P, "heads", kind, rows)
        pool = opool.pack_sequences(np.zeros(rows * d.row_bytes, np.uint8), d, table, [x])
        vals[kind] = opool.read_tokens(pool, d, table[0], np.arange(P), 0)
    assert np.all(vals["token_head"][:, 32:] == 0.0)
    assert np.all(np.abs(vals["f32_g32"][:, 32:] - 1e-4) <= 1e-4 * 2 ** -4)


@pytest.mark.parametrize("kind", ["f32_g32", "f32_g64"])
def test_decode_over_groups_is_dense_attention_of_the_dequantized_values(kind):
    p = make_problem(36, B=2, Hq=8, Hkv=2, D=128, P=16, lens=[70, 5], scale_kind=kind, k_layout="heads",
                     window=50, sinks=True)
    got = oatt.decode_ref(p.q, p.k_pool, p.v_pool, p.kdesc, p.vdesc, p.table, p.seq_lens, window=p.window,
                          sinks=p.sinks, sm_scale=p.sm_scale)
    for b in range(2):
        L = int(p.seq_lens[b])
        J = np.arange(max(0, L - p.window), L)
        for h in range(8):
            k = opool.read_tokens(p.k_pool, p.kdesc, p.table[b], J, h // 4)
            v = opool.read_tokens(p.v_pool, p.vdesc, p.table[b], J, h // 4)
            s = (k @ p.q[b, h].astype(np.float64)) * p.scale
            m = max(s.max(), p.sinks[h])
            e = np.exp(s - m)
            want = (e @ v) / (e.sum() + np.exp(p.sinks[h] - m))
            assert np.allclose(got[b, h], want, rtol=1e-12, atol=1e-12)
    assert p.vdesc.scale_kind == "token_head"
