"""Test problems: seeded inputs (fp8_paged_kv_amd.inputs) packed into pools by
the oracle's quantizer.  Used by the oracle pins and the GPU parity tests."""
from dataclasses import dataclass, field
from typing import Optional

import numpy as np

from fp8_paged_kv_amd import inputs
from oracle import pool as opool

POISON = 0xFF      # NaN E4M3 code, NaN fp32 scale bytes, NaN E8M0 scale


def round16(n):
    return (n + 15) // 16 * 16


@dataclass
class Problem:
    B: int
    Hq: int
    Hkv: int
    D: int
    P: int
    kdesc: opool.PoolDesc
    vdesc: opool.PoolDesc
    k_pool: np.ndarray
    v_pool: np.ndarray
    table: np.ndarray
    seq_lens: np.ndarray
    q: np.ndarray                  # [B, Hq, D] float32, bf16-exact
    sinks: Optional[np.ndarray]
    window: int
    sm_scale: Optional[float]
    raw_k: list = field(default_factory=list)
    raw_v: list = field(default_factory=list)

    @property
    def scale(self):
        return self.D ** -0.5 if self.sm_scale is None else self.sm_scale


def make_problem(seed, B, Hq, Hkv, D, P, lens, scale_kind="page_head", k_layout="heads_d64",
                 v_layout="heads_dmajor", window=0, sinks=False, sm_scale=None, row_pad=0,
                 poison=True, cfg=99, spare_frac=0.1, k_gain=1.0, align64=False, v_scale_kind=None):
    """A seeded decode problem.  V takes the K scale kind, except that sub-row
    fp32 key groups ("f32_g<S>") pair with per-(token, head) V scales unless
    ``v_scale_kind`` says otherwise."""
    lens = np.asarray(lens, dtype=np.int32)
    assert len(lens) == B
    if v_scale_kind is None:
        v_scale_kind = "token_head" if scale_kind in opool.GROUP_KINDS else scale_kind
    table, rows = inputs.block_table(seed, cfg, lens, P, spare_frac=spare_frac)
    kd = opool.natural_desc(Hkv, D, P, k_layout, scale_kind, rows)
    vd = opool.natural_desc(Hkv, D, P, v_layout, v_scale_kind, rows)
    from dataclasses import replace
    kd = replace(kd, row_bytes=round16(kd.row_bytes) + row_pad, align64=align64)
    vd = replace(vd, row_bytes=round16(vd.row_bytes) + row_pad, align64=align64)
    fill = POISON if poison else 0
    k_pool = np.full(rows * kd.row_bytes, fill, dtype=np.uint8)
    v_pool = np.full(rows * vd.row_bytes, fill, dtype=np.uint8)
    ks = [inputs.normal_bf16(seed, cfg, "k", b, (int(lens[b]), Hkv, D)) * np.float32(k_gain) for b in range(B)]
    vs = [inputs.normal_bf16(seed, cfg, "v", b, (int(lens[b]), Hkv, D)) for b in range(B)]
    k_pool = opool.pack_sequences(k_pool, kd, table, ks)
    v_pool = opool.pack_sequences(v_pool, vd, table, vs)
    q = inputs.normal_bf16(seed, cfg, "q", 0, (B, Hq, D))
    s = inputs.sinks(seed, cfg, Hq) if sinks else None
    return Problem(B, Hq, Hkv, D, P, kd, vd, k_pool, v_pool, table, lens, q, s, window, sm_scale, ks, vs)


def permute_rows(prob: Problem, seed=1):
    """Same logical data with the physical rows shuffled (table updated to match)."""
    n = prob.kdesc.num_rows
    perm = np.random.default_rng(seed).permutation(n)          # old row r -> new row perm[r]
    def move(pool, desc):
        old = pool.reshape(n, desc.row_bytes)
        new = np.empty_like(old)
        new[perm] = old
        return new.reshape(-1)
    table = np.where(prob.table >= 0, perm[np.maximum(prob.table, 0)], -1).astype(np.int32)
    from dataclasses import replace
    return replace(prob, k_pool=move(prob.k_pool, prob.kdesc), v_pool=move(prob.v_pool, prob.vdesc), table=table)


def add_guard_rows(prob: Problem, n=2):
    """The same problem with n poisoned rows appended to both pools, outside
    the descriptors' num_rows: table entries planted there are invalid rows
    that still lie inside the allocation, so a read or write through one
    shows up in the results instead of faulting.  Returns (problem, rows)."""
    from dataclasses import replace
    k = np.concatenate([prob.k_pool, np.full(n * prob.kdesc.row_bytes, POISON, np.uint8)])
    v = np.concatenate([prob.v_pool, np.full(n * prob.vdesc.row_bytes, POISON, np.uint8)])
    first = prob.kdesc.num_rows
    return replace(prob, k_pool=k, v_pool=v), list(range(first, first + n))


def swap_rows(prob: Problem, r1, r2):
    """The same logical data with physical rows r1 and r2 exchanged in both
    pools (and the table updated to match)."""
    from dataclasses import replace
    def move(pool, desc):
        rows = pool[:desc.num_rows * desc.row_bytes].reshape(desc.num_rows, desc.row_bytes).copy()
        rows[[r1, r2]] = rows[[r2, r1]]
        out = pool.copy()
        out[:desc.num_rows * desc.row_bytes] = rows.reshape(-1)
        return out
    t = prob.table.copy()
    m1, m2 = t == r1, t == r2
    t[m1], t[m2] = r2, r1
    return replace(prob, k_pool=move(prob.k_pool, prob.kdesc), v_pool=move(prob.v_pool, prob.vdesc), table=t)


def full_page_row(prob: Problem):
    """A physical row holding a page whose every slot is attended data."""
    for b in range(prob.B):
        for pg in range(int(prob.seq_lens[b]) // prob.P):
            if prob.table[b, pg] >= 0:
                return int(prob.table[b, pg])
    raise ValueError("no full page")
