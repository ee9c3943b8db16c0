"""Dequantization on the GPU is bit-exact against the oracle: every E4M3 code
times a set of fp32 scales (tiny, huge, subnormal products) and E8M0 scales,
through the conversion the decode kernel uses."""
import numpy as np
import pytest
import torch

from fp8_paged_kv_amd import ops
from oracle import fp8
from tests.gpu_util import DEV, say

pytestmark = pytest.mark.gpu

CODES = np.array([c for c in range(256) if c not in fp8.E4M3_NAN_CODES], dtype=np.uint8)


def test_dequant_fp32_scales_bit_exact():
    say("dequant fp32 scales")
    scales = np.array([1.0, 2.0 ** -7, 0.0123, 3.7, 1e-3, 250.0, 1e-38, 3e-39, 2.0 ** -140, 1e30, 7.1e-6],
                      dtype=np.float32)
    codes = np.tile(CODES, len(scales))
    sc = np.repeat(scales, len(CODES))
    got = ops.debug_dequant(torch.from_numpy(codes).to(DEV), torch.from_numpy(sc).to(DEV), "page_head")
    want = fp8.dequant_fp32(codes, sc.astype(np.float64)).astype(np.float32)
    g = got.cpu().numpy()
    assert np.array_equal(g.view(np.uint32), want.view(np.uint32))


def test_dequant_e8m0_bit_exact():
    say("dequant e8m0")
    us = np.arange(10, 246, dtype=np.uint8)
    codes = np.tile(CODES, len(us))
    u = np.repeat(us, len(CODES))
    got = ops.debug_dequant(torch.from_numpy(codes).to(DEV), torch.from_numpy(u).to(DEV), "e8m0_32")
    want = fp8.dequant_fp32(codes, fp8.E8M0_TABLE[u]).astype(np.float32)
    assert np.array_equal(got.cpu().numpy().view(np.uint32), want.view(np.uint32))
    assert ops.counters()["debug_launches"] >= 1


def test_dequant_sub_row_key_conversion_bit_exact():
    """The sub-row key path's fp32(code x scale), formed before its hi/lo bf16
    split: every finite code times fp32 scales including subnormal products."""
    say("dequant sub-row key conversion")
    scales = np.array([1.0, 2.0 ** -7, 0.0123, 3.7, 1e-3, 250.0, 1e-38, 3e-39, 2.0 ** -140, 1e30, 7.1e-6,
                       0.1, 1.0 / 448.0], dtype=np.float32)
    codes = np.tile(CODES, len(scales))
    sc = np.repeat(scales, len(CODES))
    for kind in ("f32_g32", "f32_g64", "f32_g128", "f32_g256"):
        got = ops.debug_dequant(torch.from_numpy(codes).to(DEV), torch.from_numpy(sc).to(DEV), kind)
        want = fp8.dequant_fp32(codes, sc.astype(np.float64)).astype(np.float32)
        assert np.array_equal(got.cpu().numpy().view(np.uint32), want.view(np.uint32)), kind
