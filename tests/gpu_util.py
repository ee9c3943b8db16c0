"""Helpers for the GPU parity tests: move a test problem to the device, run the
HIP decode through the C-ABI binding, and compare with the oracle."""
import sys

import numpy as np
import torch

from fp8_paged_kv_amd import ops

# |gpu - oracle| <= ATOL + RTOL * |oracle|, elementwise.
ATOL = 4e-3
RTOL = 1e-2

DEV = "cuda:0"


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def desc_of(d):
    """ops.PoolDesc from an oracle PoolDesc."""
    return ops.pool_desc(d.num_kv_heads, d.head_dim, d.page_size, d.layout, d.scale_kind, d.row_bytes, d.num_rows,
                         -1 if d.scale_offset is None else d.scale_offset, align64=d.align64)


def device_problem(p):
    return dict(
        q=torch.from_numpy(np.ascontiguousarray(p.q)).to(torch.bfloat16).to(DEV),
        k_pool=torch.from_numpy(p.k_pool).to(DEV), v_pool=torch.from_numpy(p.v_pool).to(DEV),
        kd=desc_of(p.kdesc), vd=desc_of(p.vdesc),
        block_table=torch.from_numpy(np.ascontiguousarray(p.table)).to(DEV),
        seq_lens=torch.from_numpy(p.seq_lens.astype(np.int32)).to(DEV),
        sinks=None if p.sinks is None else torch.from_numpy(p.sinks).to(DEV),
    )


def gpu_decode(p, dev=None, workgroups=0, max_seq_len=None, window=None, sinks="same", **kw):
    dev = device_problem(p) if dev is None else dev
    msl = int(p.seq_lens.max()) if max_seq_len is None else max_seq_len
    s = dev["sinks"] if isinstance(sinks, str) else sinks
    out = ops.decode(dev["q"], dev["k_pool"], dev["v_pool"], dev["kd"], dev["vd"], dev["block_table"],
                     dev["seq_lens"], msl, window=p.window if window is None else window, sinks=s,
                     sm_scale=p.sm_scale, workgroups=workgroups, **kw)
    torch.cuda.synchronize()
    return out


def to_np(t):
    return t.float().cpu().numpy().astype(np.float64)


def assert_parity(got, want, what=""):
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    assert got.shape == want.shape
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    err = np.abs(got - want)
    bound = ATOL + RTOL * np.abs(want)
    bad = err > bound
    if bad.any():
        i = np.unravel_index(np.argmax(err - bound), err.shape)
        raise AssertionError(f"{what}: {bad.sum()} of {bad.size} outside tolerance; worst at {i}: "
                             f"gpu={got[i]!r} oracle={want[i]!r}")
    return float(err.max()), float((err / bound).max())
