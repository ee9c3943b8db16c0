"""The five workloads at full size, in the launch configuration the benchmark
times.  Pools are built on the GPU by the append kernel; for sampled
(sequence, KV head) panels the oracle re-quantizes the same seeded inputs, the
GPU bytes must equal the oracle's, and the GPU decode output of those panels
must match the oracle's decode within tolerance.  The tiny workload is checked
on every panel."""
import numpy as np
import pytest
import torch

from fp8_paged_kv_amd import configs, workloads
from oracle import attention as oatt, pool as opool
from tests.gpu_util import assert_parity, say, to_np

pytestmark = pytest.mark.gpu


def oracle_panel(wl, layer, b, g, seed=configs.SEED):
    """Host pools holding sequence b, KV head g of the layer, quantized by the oracle."""
    al = bool(layer.kd.flags & 1)
    kd = opool.PoolDesc(layer.Hkv, layer.D, layer.P, "heads_d64", layer.scale_kind, layer.row_bytes, layer.pool_rows,
                        align64=al)
    vd = opool.PoolDesc(layer.Hkv, layer.D, layer.P, "heads_dmajor", workloads.v_kind_of(layer.scale_kind),
                        layer.row_bytes, layer.pool_rows, align64=al)
    L, first = int(layer.lens[b]), int(layer.first_pos[b])
    n = L - first
    xk = workloads.raw_kv(seed, wl, layer.layer_index, b, "k", n, layer.Hkv, layer.D)
    xv = workloads.raw_kv(seed, wl, layer.layer_index, b, "v", n, layer.Hkv, layer.D)
    hk = np.zeros(layer.pool_rows * layer.row_bytes, np.uint8)
    hv = np.zeros(layer.pool_rows * layer.row_bytes, np.uint8)
    tb = layer.table_np
    if first == 0:
        xs_k = [None] * len(layer.lens); xs_k[b] = xk
        xs_v = [None] * len(layer.lens); xs_v[b] = xv
        hk = opool.pack_sequences(hk, kd, tb, xs_k, heads=[g])
        hv = opool.pack_sequences(hv, vd, tb, xs_v, heads=[g])
    else:
        hk = opool.append_ref(hk, kd, tb[b:b + 1], [first], xk[None])
        hv = opool.append_ref(hv, vd, tb[b:b + 1], [first], xv[None])
    return kd, vd, hk, hv


def panel_byte_index(desc, rows, g):
    P, D = desc.page_size, desc.head_dim
    t = np.arange(P)[:, None]
    d = np.arange(D)[None, :]
    code = opool.code_offset(desc, g, t, d).ravel()
    if desc.scale_kind == "page_head":
        sc = opool.scale_rel(desc, g) + np.arange(4)
    elif desc.scale_kind == "token_head":
        sc = np.array([opool.scale_rel(desc, g, tt) + i for tt in range(P) for i in range(4)])
    elif desc.scale_kind in opool.GROUP_KINDS:
        ng = D // opool.GROUP_KINDS[desc.scale_kind]
        sc = np.array([opool.scale_rel(desc, g, tt, gg) + i for tt in range(P) for gg in range(ng) for i in range(4)])
    else:
        sc = np.array([opool.scale_rel(desc, g, tt, gg) for tt in range(P) for gg in range(D // 32)])
    rows = np.asarray(rows, np.int64)
    cb = opool.row_code_base(desc, rows)[:, None] + code[None, :]
    sb = opool.row_scale_base(desc, rows)[:, None] + sc[None, :]
    return np.concatenate([cb, sb], axis=1).ravel()


def check_panel(wl, layer, out_np, b, g):
    kd, vd, hk, hv = oracle_panel(wl, layer, b, g)
    L = int(layer.lens[b])
    start = max(0, L - layer.window) if layer.window > 0 else 0
    pages = np.arange(start // layer.P, (L - 1) // layer.P + 1)
    rows = layer.table_np[b, pages]
    # bytes of every attended page: codes of the written slots and the scales
    P = layer.P
    written = np.zeros((len(pages), P), bool)
    for i, p in enumerate(pages):
        lo = max(int(layer.first_pos[b]), p * P)
        written[i, lo - p * P:min(L, (p + 1) * P) - p * P] = True
    for desc, host, dev in ((kd, hk, layer.k_pool), (vd, hv, layer.v_pool)):
        idx = panel_byte_index(desc, rows, g)
        got = dev[torch.from_numpy(idx).to(dev.device)].cpu().numpy()
        want = host[idx]
        # compare written slots only: the GPU pool keeps poison in the unwritten tail of the last page
        n_code = P * desc.head_dim
        per_row = len(idx) // len(rows)
        gr = got.reshape(len(rows), per_row)
        wr = want.reshape(len(rows), per_row)
        # panel_byte_index lists codes in (slot, dim) order for every layout
        code_slot = np.broadcast_to(np.arange(P)[:, None], (P, desc.head_dim)).ravel()
        keep_code = written[:, code_slot]
        assert np.array_equal(gr[:, :n_code][keep_code], wr[:, :n_code][keep_code]), f"{layer.name} b={b} g={g} codes"
        if desc.scale_kind == "page_head":
            assert np.array_equal(gr[:, n_code:], wr[:, n_code:]), f"{layer.name} b={b} g={g} scales"
        else:
            per_tok = (per_row - n_code) // P
            ks = np.repeat(written, per_tok, axis=1)
            assert np.array_equal(gr[:, n_code:][ks], wr[:, n_code:][ks]), f"{layer.name} b={b} g={g} scales"
    q = workloads.inputs.normal_bf16(configs.SEED, wl.index, "q", layer.layer_index, (len(layer.lens), layer.Hq, layer.D))
    want = oatt.decode_ref(q, hk, hv, kd, vd, layer.table_np, layer.lens, window=layer.window,
                           sinks=layer.sinks_np, sm_scale=layer.sm_scale, seqs=[b], heads=[g])
    G = layer.Hq // layer.Hkv
    return assert_parity(out_np[b, g * G:(g + 1) * G], want[b, g * G:(g + 1) * G], f"{layer.name} b={b} g={g}")


@pytest.mark.parametrize("wl", configs.ALL, ids=[w.name for w in configs.ALL])
def test_workload_full_size(wl):
    say("workload", wl.name)
    layers = workloads.build_workload(wl)
    rng = np.random.default_rng(wl.index)
    for layer in layers:
        out = workloads.decode_layer(layer)
        torch.cuda.synchronize()
        out_np = to_np(out)
        assert np.all(np.isfinite(out_np)), layer.name
        if wl is configs.TINY:
            pairs = [(b, g) for b in range(len(layer.lens)) for g in range(layer.Hkv)]
        else:
            pairs = [(int(np.argmax(layer.lens)), int(rng.integers(layer.Hkv))),
                     (int(rng.integers(len(layer.lens))), int(rng.integers(layer.Hkv)))]
        for b, g in pairs:
            err, frac = check_panel(wl, layer, out_np, b, g)
            say(f"  {layer.name} b={b} L={int(layer.lens[b])} g={g}: max err {err:.2e} ({frac:.2f} of bound)")


@pytest.fixture(scope="module")
def llama_layer():
    return workloads.build_workload(configs.LLAMA3_8B)[0]


@pytest.mark.parametrize("variant", ["packed_split", "packed_heads"])
def test_llama_full_size_other_variants(llama_layer, variant):
    """The Llama-3-8B-shaped call at full size through the packed variants:
    sampled panels (the longest sequence among them) within the oracle bound,
    and the same output as the default variant up to summation order."""
    say("workload variant", variant)
    layer = llama_layer
    out = workloads.decode_layer(layer, variant=variant)
    ref = workloads.decode_layer(layer)
    torch.cuda.synchronize()
    out_np = to_np(out)
    assert np.all(np.isfinite(out_np))
    rng = np.random.default_rng(17)
    for b, g in [(int(np.argmax(layer.lens)), int(rng.integers(layer.Hkv))),
                 (int(rng.integers(len(layer.lens))), int(rng.integers(layer.Hkv)))]:
        err, frac = check_panel(configs.LLAMA3_8B, layer, out_np, b, g)
        say(f"  {variant} b={b} g={g}: max err {err:.2e} ({frac:.2f} of bound)")
    assert float((out.float() - ref.float()).abs().max()) < 2e-2


def test_llama_full_size_sub_row_key_scales():
    """The Llama-3-8B-shaped call at full size with fp32 K scales per 32 dims
    (V per token): sampled panels within the oracle bound."""
    say("workload k groups")
    layer = workloads.build_workload(configs.LLAMA3_8B, scale_kind="f32_g32")[0]
    out = workloads.decode_layer(layer)
    torch.cuda.synchronize()
    out_np = to_np(out)
    assert np.all(np.isfinite(out_np))
    rng = np.random.default_rng(23)
    for b, g in [(int(np.argmax(layer.lens)), int(rng.integers(layer.Hkv))),
                 (int(rng.integers(len(layer.lens))), int(rng.integers(layer.Hkv)))]:
        err, frac = check_panel(configs.LLAMA3_8B, layer, out_np, b, g)
        say(f"  f32_g32 b={b} g={g}: max err {err:.2e} ({frac:.2f} of bound)")
