"""fp8pa_merge_splits against the oracle's log-sum-exp merge."""
import numpy as np
import pytest
import torch

from fp8_paged_kv_amd import ops
from oracle import attention as oatt
from tests.gpu_util import DEV, assert_parity, say, to_np

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("D", [64, 128, 256, 512])
@pytest.mark.parametrize("sinks", [False, True])
def test_merge_matches_oracle(D, sinks):
    say("merge", D, sinks)
    rng = np.random.default_rng(D + sinks)
    B, H, S = 3, 8, 7
    o = rng.standard_normal((B, H, S, D)).astype(np.float32)
    lse = (rng.standard_normal((B, H, S)) * 3).astype(np.float32)
    lse[0, 0, :] = -np.inf                 # nothing attended
    lse[1, 2, ::2] = -np.inf               # some empty splits
    o[1, 2, ::2] = np.nan                  # whose outputs must be ignored
    s = rng.standard_normal(H).astype(np.float32) if sinks else None
    got = ops.merge_splits(torch.from_numpy(o).to(DEV), torch.from_numpy(lse).to(DEV),
                           None if s is None else torch.from_numpy(s).to(DEV))
    torch.cuda.synchronize()
    want = oatt.merge_ref(o, lse, s)
    assert_parity(to_np(got), want, "merge")
    assert np.all(to_np(got)[0, 0] == 0)
