"""Seeded synthetic inputs for tests and benchmarks.

This module draws random numbers and lays out page tables; it holds none of the
attention or quantisation arithmetic, so the oracle and the HIP library can both
consume what it produces.  Draws use numpy's PCG64 with per-(config, tensor,
sequence) seed sequences, so one sequence can be regenerated on its own.

Value recipe (a stand-in for real models; no weights or datasets): K, V and q are
N(0, 1) float32 rounded to bf16 (round to nearest even), sinks N(0, 1) float32,
sequence lengths uniform integers over an inclusive range, physical rows a random
permutation of a pool with spare rows.
"""
import numpy as np

TENSOR_IDS = {"seq_lens": 1, "rows": 2, "k": 3, "v": 4, "q": 5, "sinks": 6, "extra": 7}


def generator(seed: int, cfg: int, tensor: str, index: int = 0) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, cfg, TENSOR_IDS[tensor], index])))


def round_to_bf16(x) -> np.ndarray:
    """float32 values rounded to the nearest bf16 (ties to even), as float32."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    bits = x.view(np.uint32).astype(np.uint64)
    bias = 0x7FFF + ((bits >> 16) & 1)
    r = ((bits + bias) & 0xFFFF0000).astype(np.uint32)
    return r.view(np.float32)


def bf16_bits(x) -> np.ndarray:
    """Upper 16 bits of bf16-exact float32 values (the bf16 encoding)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    return (x.view(np.uint32) >> 16).astype(np.uint16)


def seq_lens(seed, cfg, B, lo, hi) -> np.ndarray:
    return generator(seed, cfg, "seq_lens").integers(lo, hi + 1, size=B).astype(np.int32)


def normal_bf16(seed, cfg, tensor, index, shape) -> np.ndarray:
    return round_to_bf16(generator(seed, cfg, tensor, index).standard_normal(shape, dtype=np.float32))


def sinks(seed, cfg, Hq) -> np.ndarray:
    return generator(seed, cfg, "sinks").standard_normal(Hq, dtype=np.float32)


def block_table(seed, cfg, lens, page_size, spare_frac=0.05, min_rows=0, exclude=None, pool_rows=None):
    """Random page table.  Returns (table [B, max_pages] int32 with -1 in unused
    entries, total rows the pool needs).  Rows are a random permutation of a pool
    with ~spare_frac unused rows; ``exclude`` (a set of row ids) is skipped, and
    ``pool_rows`` fixes the pool size (for pools shared between two tables)."""
    lens = np.asarray(lens, dtype=np.int64)
    pages = -(-lens // page_size)
    need = int(pages.sum())
    max_pages = max(1, int(pages.max()) if len(pages) else 1)
    if pool_rows is None:
        pool_rows = max(min_rows, need + max(1, int(np.ceil(need * spare_frac))))
    g = generator(seed, cfg, "rows")
    avail = np.arange(pool_rows, dtype=np.int64)
    if exclude is not None and len(exclude):
        avail = avail[~np.isin(avail, np.fromiter(exclude, dtype=np.int64))]
    if len(avail) < need:
        raise ValueError("pool too small for the table")
    rows = g.permutation(avail)[:need]
    table = np.full((len(lens), max_pages), -1, dtype=np.int32)
    at = 0
    for b, n in enumerate(pages):
        table[b, :n] = rows[at:at + n]
        at += n
    return table, pool_rows


def block_table_ranges(seed, cfg, ranges, page_size, spare_frac=0.05, pool_rows=None, tag=0, exclude=None,
                       width=None):
    """Random page table giving rows only to pages [first, end) of each sequence
    (ranges[b] = (first, end)); other entries are -1.  Returns (table, rows used,
    pool rows).  Rows come from a random permutation of the pool, skipping
    ``exclude`` (rows another table of a shared pool already holds)."""
    ranges = [(int(a), int(e)) for a, e in ranges]
    need = sum(e - a for a, e in ranges)
    width = max([e for _, e in ranges] + [1] + ([width] if width else []))
    if pool_rows is None:
        pool_rows = need + max(1, int(np.ceil(need * spare_frac)))
    g = generator(seed, cfg, "rows", tag)
    avail = np.arange(pool_rows, dtype=np.int64)
    if exclude is not None and len(exclude):
        avail = np.setdiff1d(avail, np.asarray(exclude, dtype=np.int64), assume_unique=True)
    if len(avail) < need:
        raise ValueError("pool too small for the table")
    rows = g.permutation(avail)[:need]
    table = np.full((len(ranges), width), -1, dtype=np.int32)
    at = 0
    for b, (a, e) in enumerate(ranges):
        table[b, a:e] = rows[at:at + e - a]
        at += e - a
    return table, rows, pool_rows
