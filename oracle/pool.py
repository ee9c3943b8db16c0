"""Paged KV pool format for the oracle: packed rows, addressing, packing and the
reference KV append.

Test infrastructure only (see the package docstring).

Format (page "fp8 paged attention for MoE serving", sections "Supported scope"
and "Smallest correct example"): a pool is a flat byte array of rows; one row
holds one page of ``page_size`` tokens for all KV heads of a layer: the E4M3
payload first, then a scale footer at ``scale_offset`` (default: right after
the payload).  Rows are ``row_bytes`` apart, which may be wider than the natural
row so that layers of different geometry can share a pool.  A per-sequence
block table maps logical page p to a physical row.

Payload layouts (byte offset of the code for head h, in-page token t, dim d).
The page names "tokens" and "heads"; the other two are this library's own
orders, chosen so that a wave-wide 16-byte load covers whole 128-byte lines:
  "heads"        [H][P][D]:        (h*P + t)*D + d
  "tokens"       [P][H][D]:        (t*H + h)*D + d
  "heads_d64"    [H][D/64][P][64]: ((h*(D/64) + d//64)*P + t)*64 + d%64
                 (keys: 64-byte pieces of consecutive tokens side by side)
  "heads_dmajor" [H][P/W][D][W], W = min(P, 64):
                 h*P*D + (t//W)*D*W + d*W + t%W
                 (values: token-contiguous per dim, in blocks of W tokens;
                 for P <= 64 this is [H][D][P])
Row placement.  By default a row's payload starts at the row start and its
scales at ``scale_offset``.  With ``align64`` (this library's option, for rows
whose width is not a multiple of 64 bytes) the payload of row r starts at the
first 64-byte boundary of the row, r*row_bytes + ((-r*row_bytes) mod 64) from
the pool start, and the scale block sits in the gap before the payload when it
fits there, else right after the payload.

Scale footer (byte offset from the scale block's start):
  "page_head"  fp32 per (page, head):  4*h
  "token_head" fp32 per (token, head): 4*(h*P + t), or 4*(t*H + h) for "tokens"
  "e8m0_32"    one E8M0 byte per (token, head, 32 dims along D):
               (h*P + t)*(D/32) + d//32, or (t*H + h)*(D/32) + d//32 for "tokens"
  "f32_g<S>"   fp32 per (token, head, S dims along D), S in 8, 16, 32, 64, 128,
               256 (the page's sub-row groups, k_groups or v_groups = D/S):
               4*((h*P + t)*(D/S) + d//S), or 4*((t*H + h)*(D/S) + d//S) for "tokens"
"""
from dataclasses import dataclass, replace
from typing import Optional

import numpy as np

from . import fp8

LAYOUTS = ("heads", "tokens", "heads_d64", "heads_dmajor")
GROUP_KINDS = {"f32_g8": 8, "f32_g16": 16, "f32_g32": 32, "f32_g64": 64, "f32_g128": 128, "f32_g256": 256}
SCALE_KINDS = ("page_head", "token_head", "e8m0_32") + tuple(GROUP_KINDS)


@dataclass(frozen=True)
class PoolDesc:
    num_kv_heads: int
    head_dim: int
    page_size: int
    layout: str
    scale_kind: str
    row_bytes: int
    num_rows: int
    scale_offset: Optional[int] = None
    align64: bool = False

    @property
    def payload_bytes(self) -> int:
        return self.page_size * self.num_kv_heads * self.head_dim

    @property
    def scale_bytes(self) -> int:
        H, P, D = self.num_kv_heads, self.page_size, self.head_dim
        if self.scale_kind in GROUP_KINDS:
            return 4 * H * P * (D // GROUP_KINDS[self.scale_kind])
        return {"page_head": 4 * H, "token_head": 4 * H * P, "e8m0_32": H * P * D // 32}[self.scale_kind]

    @property
    def footer(self) -> int:
        return self.payload_bytes if self.scale_offset is None else self.scale_offset

    def natural_row_bytes(self) -> int:
        return self.payload_bytes + self.scale_bytes

    def shifts(self):
        """Payload shifts (bytes) that rows of this pool take."""
        if not self.align64:
            return [0]
        return sorted({(-r * self.row_bytes) % 64 for r in range(64)})

    def check(self):
        assert self.layout in LAYOUTS and self.scale_kind in SCALE_KINDS
        assert self.footer + self.scale_bytes <= self.row_bytes
        assert self.footer >= self.payload_bytes
        if self.align64:
            assert self.scale_offset is None
            for sh in self.shifts():
                end = sh + self.payload_bytes if sh >= self.scale_bytes else sh + self.payload_bytes + self.scale_bytes
                assert end <= self.row_bytes
        if self.scale_kind == "e8m0_32":
            assert self.head_dim % 32 == 0
        if self.scale_kind in GROUP_KINDS:
            assert self.head_dim % GROUP_KINDS[self.scale_kind] == 0
        if self.layout == "heads_d64":
            assert self.head_dim % 64 == 0
        if self.layout == "heads_dmajor":
            assert self.page_size <= 64 or self.page_size % 64 == 0


def natural_desc(num_kv_heads, head_dim, page_size, layout, scale_kind, num_rows, row_bytes=None):
    d = PoolDesc(num_kv_heads, head_dim, page_size, layout, scale_kind, 0, num_rows)
    nat = d.natural_row_bytes()
    return replace(d, row_bytes=nat if row_bytes is None else row_bytes)


# ---------------------------------------------------------------- addressing
def row_code_base(desc: PoolDesc, rows):
    """Byte offset of the payload of physical row(s) from the pool start."""
    base = np.asarray(rows, dtype=np.int64) * desc.row_bytes
    if not desc.align64:
        return base
    return base + (-base) % 64


def row_scale_base(desc: PoolDesc, rows):
    """Byte offset of the scale block of physical row(s) from the pool start."""
    base = np.asarray(rows, dtype=np.int64) * desc.row_bytes
    if not desc.align64:
        return base + desc.footer
    sh = (-base) % 64
    return np.where(sh >= desc.scale_bytes, base, base + sh + desc.payload_bytes)


def code_offset(desc: PoolDesc, h, t, d):
    H, P, D = desc.num_kv_heads, desc.page_size, desc.head_dim
    if desc.layout == "heads":
        return (h * P + t) * D + d
    if desc.layout == "tokens":
        return (t * H + h) * D + d
    if desc.layout == "heads_d64":
        return ((h * (D // 64) + d // 64) * P + t) * 64 + d % 64
    W = min(P, 64)
    return h * P * D + (t // W) * D * W + d * W + t % W


def scale_rel(desc: PoolDesc, h, t=0, g=0):
    """Offset of a scale inside the scale block."""
    H, P, D = desc.num_kv_heads, desc.page_size, desc.head_dim
    slot = (t * H + h) if desc.layout == "tokens" else (h * P + t)
    if desc.scale_kind == "page_head":
        return 4 * h
    if desc.scale_kind == "token_head":
        return 4 * slot
    if desc.scale_kind in GROUP_KINDS:
        return 4 * (slot * (D // GROUP_KINDS[desc.scale_kind]) + g)
    return slot * (D // 32) + g


def scale_offset(desc: PoolDesc, h, t=0, g=0):
    """Offset of a scale from the row start (pools without ``align64``)."""
    assert not desc.align64
    return desc.footer + scale_rel(desc, h, t, g)


def _page_codes(pool, desc, rows, h):
    """Codes of head h for the given physical rows: uint8 [n, P, D]."""
    H, P, D = desc.num_kv_heads, desc.page_size, desc.head_dim
    t = np.arange(P)[:, None]
    d = np.arange(D)[None, :]
    off = code_offset(desc, h, t, d)                                   # [P, D]
    base = row_code_base(desc, rows)[:, None, None]
    return pool[base + off[None]]


def _page_scales(pool, desc, rows, h):
    """Scales of head h for the rows, broadcastable against [n, P, D] (float64)."""
    P, D = desc.page_size, desc.head_dim
    base = row_scale_base(desc, rows)
    if desc.scale_kind == "page_head":
        idx = base[:, None] + scale_rel(desc, h) + np.arange(4)[None, :]
        return pool[idx].copy().view(np.float32).astype(np.float64)[:, :, None]        # [n,1,1]
    if desc.scale_kind == "token_head":
        offs = np.array([scale_rel(desc, h, t) for t in range(P)])
        idx = base[:, None, None] + offs[None, :, None] + np.arange(4)[None, None, :]
        return pool[idx].copy().view(np.float32)[..., 0].astype(np.float64)[:, :, None]  # [n,P,1]
    if desc.scale_kind in GROUP_KINDS:
        S = GROUP_KINDS[desc.scale_kind]
        offs = np.array([[scale_rel(desc, h, t, g) for g in range(D // S)] for t in range(P)])
        idx = base[:, None, None, None] + offs[None, :, :, None] + np.arange(4)[None, None, None, :]
        s = pool[idx].copy().view(np.float32)[..., 0].astype(np.float64)               # [n,P,D/S]
        return np.repeat(s, S, axis=-1)                                                # [n,P,D]
    offs = np.array([[scale_rel(desc, h, t, g) for g in range(D // 32)] for t in range(P)])
    u = pool[base[:, None, None] + offs[None]]                                         # [n,P,D/32]
    return np.repeat(fp8.E8M0_TABLE[u], 32, axis=-1)                                   # [n,P,D]


def read_tokens(pool, desc, table_row, positions, h):
    """Exact float64 dequantized values [len(positions), D] of KV head h at the
    logical positions of one sequence (page "fp8 paged attention for MoE serving",
    "Smallest correct example": the block table maps page j // P to a row)."""
    positions = np.asarray(positions, dtype=np.int64)
    if positions.size == 0:
        return np.zeros((0, desc.head_dim))
    P = desc.page_size
    pages = np.unique(positions // P)
    rows = np.asarray(table_row, dtype=np.int64)[pages]
    if (rows < 0).any() or (rows >= desc.num_rows).any():
        raise IndexError("block table entry out of range for an attended page")
    vals = fp8.E4M3_TABLE[_page_codes(pool, desc, rows, h)] * _page_scales(pool, desc, rows, h)
    where = {p: i for i, p in enumerate(pages)}
    pi = np.array([where[p] for p in positions // P])
    return vals[pi, positions % P]


# ---------------------------------------------------------------- writing
def _write_codes(pool, desc, row, h, t0, codes):
    """codes [n, D] for in-page tokens t0..t0+n-1 of head h."""
    n, D = codes.shape
    t = (t0 + np.arange(n))[:, None]
    d = np.arange(D)[None, :]
    pool[row_code_base(desc, row) + code_offset(desc, h, t, d)] = codes


def _write_f32(pool, at, value):
    pool[at:at + 4] = np.array([value], dtype=np.float32).view(np.uint8)


def _read_f32(pool, at):
    return float(pool[at:at + 4].copy().view(np.float32)[0])


def append_ref(pool, desc: PoolDesc, block_table, positions, x_new, counts=None):
    """Reference KV append: write tokens x_new[b, 0:n_b] (float values, [B, T, H, D])
    at logical positions positions[b] + t of sequence b; n_b = counts[b] (default T).
    Returns a new pool.

    The page asks for a per-token-per-head E4M3 quantizer with an fp32 scale or
    sub-row groups, and a one-launch T=1 append ("Supported scope").  Readings:
    * "token_head": stateless, one fp32 scale per (token, head).
    * "e8m0_32": stateless, one E8M0 scale per (token, head, 32 dims).
    * "f32_g<S>": stateless, one fp32 scale per (token, head, S dims), each
      group quantized like a "token_head" row of S dims.
    * "page_head": the page's scale only grows.  If this call writes the page's
      first slot, the old scale counts as 0 and there are no old tokens; else the
      old tokens are slots [0, first written slot).  s_new = max(s_old,
      fp32(amax_new / 448)), 1 if that is 0.  When s_new > s_old > 0 the old
      tokens are re-encoded as e4m3(fp32(fp32(code * s_old) / s_new)); new tokens
      are encoded with s_new.
    """
    pool = np.array(pool, dtype=np.uint8, copy=True)
    x_new = np.asarray(x_new, dtype=np.float64)
    B, T, H, D = x_new.shape
    assert H == desc.num_kv_heads and D == desc.head_dim
    P = desc.page_size
    for b in range(B):
        n_b = T if counts is None else int(counts[b])
        pos0 = int(positions[b])
        t = 0
        while t < n_b:
            pos = pos0 + t
            page, slot0 = pos // P, pos % P
            n = min(P - slot0, n_b - t)
            row = int(block_table[b][page])
            if not (0 <= row < desc.num_rows):
                raise IndexError("block table entry out of range for an appended page")
            for h in range(H):
                x = x_new[b, t:t + n, h, :]                                  # [n, D]
                if desc.scale_kind == "token_head":
                    for i in range(n):
                        c, s = fp8.quantize_fp32_block(x[i])
                        _write_codes(pool, desc, row, h, slot0 + i, c[None])
                        _write_f32(pool, row_scale_base(desc, row) + scale_rel(desc, h, slot0 + i), s)
                elif desc.scale_kind in GROUP_KINDS:
                    S = GROUP_KINDS[desc.scale_kind]
                    for i in range(n):
                        for g in range(D // S):
                            c, s = fp8.quantize_fp32_block(x[i, g * S:(g + 1) * S])
                            tt, dd = np.array([[slot0 + i]]), (g * S + np.arange(S))[None, :]
                            pool[row_code_base(desc, row) + code_offset(desc, h, tt, dd)] = c[None]
                            _write_f32(pool, row_scale_base(desc, row) + scale_rel(desc, h, slot0 + i, g), s)
                elif desc.scale_kind == "e8m0_32":
                    c, u = fp8.quantize_e8m0_g32(x)
                    _write_codes(pool, desc, row, h, slot0, c)
                    for i in range(n):
                        for g in range(D // 32):
                            pool[row_scale_base(desc, row) + scale_rel(desc, h, slot0 + i, g)] = u[i, g]
                else:
                    at = int(row_scale_base(desc, row)) + scale_rel(desc, h)
                    s_old = 0.0 if slot0 == 0 else _read_f32(pool, at)
                    amax = float(np.abs(x).max()) if x.size else 0.0
                    cand = float(fp8.to_fp32(amax / fp8.E4M3_MAX)) if amax > 0 else 0.0
                    s_new = max(s_old, cand)
                    if s_new == 0.0:
                        s_new = 1.0
                    if slot0 > 0 and s_old > 0.0 and s_new > s_old:
                        tt = np.arange(slot0)[:, None]
                        dd = np.arange(D)[None, :]
                        idx = row_code_base(desc, row) + code_offset(desc, h, tt, dd)
                        old = fp8.dequant_fp32(pool[idx], s_old)
                        pool[idx] = fp8.encode_e4m3(fp8.to_fp32(old / s_new))
                    _write_codes(pool, desc, row, h, slot0, fp8.encode_e4m3(fp8.to_fp32(x / s_new)))
                    _write_f32(pool, at, s_new)
            t += n
    return pool


def pack_sequences(pool, desc: PoolDesc, block_table, xs, heads=None):
    """Write whole sequences xs[b] ([L_b, H, D] floats) from position 0: one
    append per sequence, so every page scale is the plain amax of its tokens.
    Vectorised over pages; equal to ``append_ref`` with positions 0 (pinned).
    ``heads`` restricts the work to some KV heads (the others are not written)."""
    pool = np.array(pool, dtype=np.uint8, copy=True)
    H, P, D = desc.num_kv_heads, desc.page_size, desc.head_dim
    heads = range(H) if heads is None else heads
    tt = np.arange(P)[:, None]
    dd = np.arange(D)[None, :]
    for b, x in enumerate(xs):
        if x is None:
            continue
        x = np.asarray(x)
        L = x.shape[0]
        if L == 0:
            continue
        n_pages = -(-L // P)
        rows = np.asarray(block_table[b][:n_pages], dtype=np.int64)
        if (rows < 0).any() or (rows >= desc.num_rows).any():
            raise IndexError("block table entry out of range for a written page")
        valid = (np.arange(n_pages * P) < L).reshape(n_pages, P)
        for h in heads:
            xp = np.zeros((n_pages * P, D))
            xp[:L] = x[:, h, :]
            xp = xp.reshape(n_pages, P, D)
            if desc.scale_kind == "page_head":
                s = fp8.fp32_scale_from_amax(np.abs(xp).max(axis=(1, 2)))             # [n]
                codes = fp8.encode_e4m3(fp8.to_fp32(xp / s[:, None, None]))
                at = row_scale_base(desc, rows) + scale_rel(desc, h)
                pool[at[:, None] + np.arange(4)[None, :]] = s.astype(np.float32).view(np.uint8).reshape(-1, 4)
            elif desc.scale_kind == "token_head":
                s = fp8.fp32_scale_from_amax(np.abs(xp).max(axis=2))                  # [n, P]
                codes = fp8.encode_e4m3(fp8.to_fp32(xp / s[..., None]))
                offs = np.array([scale_rel(desc, h, t) for t in range(P)])
                idx = row_scale_base(desc, rows)[:, None, None] + offs[None, :, None] + np.arange(4)[None, None, :]
                vals = s.astype(np.float32).view(np.uint8).reshape(n_pages, P, 4)
                pool[idx[valid]] = vals[valid]
            elif desc.scale_kind in GROUP_KINDS:
                S = GROUP_KINDS[desc.scale_kind]
                xg = xp.reshape(n_pages, P, D // S, S)
                s = fp8.fp32_scale_from_amax(np.abs(xg).max(axis=3))                  # [n, P, D/S]
                codes = fp8.encode_e4m3(fp8.to_fp32(xg / s[..., None])).reshape(n_pages, P, D)
                offs = np.array([[scale_rel(desc, h, t, g) for g in range(D // S)] for t in range(P)])
                idx = (row_scale_base(desc, rows)[:, None, None, None] + offs[None, :, :, None] +
                       np.arange(4)[None, None, None, :])
                vals = s.astype(np.float32).view(np.uint8).reshape(n_pages, P, D // S, 4)
                pool[idx[valid]] = vals[valid]
            else:
                codes, u = fp8.quantize_e8m0_g32(xp)                                  # u [n, P, D/32]
                offs = np.array([[scale_rel(desc, h, t, g) for g in range(D // 32)] for t in range(P)])
                idx = row_scale_base(desc, rows)[:, None, None] + offs[None]
                pool[idx[valid]] = u[valid]
            idx = row_code_base(desc, rows)[:, None, None] + code_offset(desc, h, tt, dd)[None]   # [n, P, D]
            pool[idx[valid]] = codes[valid]
    return pool
