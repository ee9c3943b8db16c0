"""The five workloads at full size, in the launch configuration the benchmark
times.  Pools are built on the GPU by the append kernel; for every (sequence,
KV head) panel the oracle re-quantizes the same seeded inputs (in worker
processes that never touch the GPU), the GPU bytes must equal the oracle's,
and the GPU decode output must match the oracle's decode within tolerance.
The packed and sub-row-scale variants are checked on sampled panels."""
import hashlib
import multiprocessing as mp
import os

import numpy as np
import pytest
import torch

from fp8_paged_kv_amd import configs, inputs, ops, workloads
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


def written_slots(L, first, pages, P):
    """[len(pages), P] bool: the slots the workload's build wrote (positions in [first, L))."""
    w = np.zeros((len(pages), P), bool)
    for i, p in enumerate(pages):
        lo = max(first, p * P)
        w[i, lo - p * P:min(L, (p + 1) * P) - p * P] = True
    return w


def panel_bytes(gathered, desc, written):
    """The written bytes of one KV head's panel: `gathered` holds the panel's
    bytes in panel_byte_index order (per row: codes in (slot, dim) order, then
    the scales); kept are the codes of written slots and their scales (all of
    a page scale), in logical order whatever the layout and placement."""
    P, D = desc.page_size, desc.head_dim
    g = np.asarray(gathered, np.uint8).reshape(written.shape[0], -1)
    n_code = P * D
    codes = g[:, :n_code][written[:, np.repeat(np.arange(P), D)]]
    sc = g[:, n_code:]
    if desc.scale_kind != "page_head":
        sc = sc[np.repeat(written, sc.shape[1] // P, axis=1)]
    return np.concatenate([codes.ravel(), sc.ravel()])


def digest(a):
    return hashlib.sha256(np.ascontiguousarray(a, np.uint8).tobytes()).hexdigest()


def layer_geometry(layer):
    """What an oracle worker needs to rebuild one layer's data (host values only)."""
    return dict(Hkv=layer.Hkv, Hq=layer.Hq, D=layer.D, P=layer.P, window=layer.window, sm_scale=layer.sm_scale,
                scale_kind=layer.scale_kind, row_bytes=layer.row_bytes, align64=bool(layer.kd.flags & 1),
                layer_index=layer.layer_index, sinks=layer.sinks_np, lens=np.asarray(layer.lens),
                first_pos=np.asarray(layer.first_pos))


def oracle_sequence(job):
    """Worker (no GPU): sequence b of one layer re-quantized from the seeded
    inputs into a compact host pool by the oracle (its attended pages as rows
    0..n-1), then per KV head: the digest of its written bytes and the oracle
    decode of its G query heads."""
    wl_index, geo, b, heads = job
    wl = configs.ALL[wl_index]
    P, D, Hkv = geo["P"], geo["D"], geo["Hkv"]
    L, first = int(geo["lens"][b]), int(geo["first_pos"][b])
    start = max(0, L - geo["window"]) if geo["window"] > 0 else 0
    pages = np.arange(start // P, (L - 1) // P + 1) if L > 0 else np.arange(0)
    n_rows = max(1, (L - 1) // P + 1 - first // P) if L > 0 else 1
    B = len(geo["lens"])
    table = np.full((B, max(1, -(-int(wl.L_hi) // P))), -1, np.int32)
    if L > 0:
        table[b, first // P:(L - 1) // P + 1] = np.arange(n_rows, dtype=np.int32)
    kd = opool.PoolDesc(Hkv, D, P, "heads_d64", geo["scale_kind"], geo["row_bytes"], n_rows, align64=geo["align64"])
    vd = opool.PoolDesc(Hkv, D, P, "heads_dmajor", workloads.v_kind_of(geo["scale_kind"]), geo["row_bytes"], n_rows,
                        align64=geo["align64"])
    hk = np.zeros(n_rows * geo["row_bytes"], np.uint8)
    hv = np.zeros(n_rows * geo["row_bytes"], np.uint8)
    n = L - first
    if n > 0:
        xk = workloads.raw_kv(configs.SEED, wl, geo["layer_index"], b, "k", n, Hkv, D)
        xv = workloads.raw_kv(configs.SEED, wl, geo["layer_index"], b, "v", n, Hkv, D)
        if first == 0:
            xs = [None] * B
            xs[b] = xk
            hk = opool.pack_sequences(hk, kd, table, xs, heads=heads)
            xs[b] = xv
            hv = opool.pack_sequences(hv, vd, table, xs, heads=heads)
        else:
            hk = opool.append_ref(hk, kd, table[b:b + 1], [first], xk[None])
            hv = opool.append_ref(hv, vd, table[b:b + 1], [first], xv[None])
        del xk, xv
    q = inputs.normal_bf16(configs.SEED, wl.index, "q", geo["layer_index"], (B, geo["Hq"], D))
    want = oatt.decode_ref(q, hk, hv, kd, vd, table, geo["lens"], window=geo["window"], sinks=geo["sinks"],
                           sm_scale=geo["sm_scale"], seqs=[b], heads=heads)
    G = geo["Hq"] // Hkv
    res = {}
    if L > 0:
        local = table[b, pages]
        wr = written_slots(L, first, pages, P)
    for g in heads:
        dk = digest(panel_bytes(hk[panel_byte_index(kd, local, g)], kd, wr)) if L > 0 else None
        dv = digest(panel_bytes(hv[panel_byte_index(vd, local, g)], vd, wr)) if L > 0 else None
        res[g] = (dk, dv, want[b, g * G:(g + 1) * G].copy())
    return b, res


def workers():
    return max(1, min(16, len(os.sched_getaffinity(0))))


def unit_pieces(layer, W_plan):
    """How many workgroup shares each (sequence, KV head) unit of the layer is
    cut into by the decode kernel's cost-balanced split (the kernel's integer
    share rule, restated on the host to pick test panels; W_plan = the plan's
    workgroups).  Returns {(b, g): pieces}."""
    D = layer.D
    TT, NW, SCd = (64, 4, 36) if D == 128 else ((64, 4, 24) if D == 64 else (32, 4, 24))
    lens = [int(x) for x in layer.lens]

    def tiles_of(L):
        st = max(0, L - layer.window) if layer.window > 0 else 0
        tb = st & ~(TT - 1)
        return (L - tb + TT - 1) // TT if L > st else 0
    nt = [tiles_of(L) for L in lens]
    T, U = sum(nt) * layer.Hkv, sum(1 for x in nt if x > 0) * layer.Hkv
    unit_mode = T <= NW * U
    TC, SC = (0, 1) if unit_mode else (4, SCd)
    Ct = SC * U + TC * T
    W = min(W_plan, max(1, Ct // (SC + TC * NW))) if T else 0
    out, c = {}, 0
    for b, n in enumerate(nt):
        for g in range(layer.Hkv):
            if n == 0:
                continue
            first, last = c + SC, c + SC + TC * (n - 1)
            wg = lambda x: ((x + 1) * W + Ct - 1) // Ct - 1
            out[(b, g)] = wg(last) - wg(first) + 1
            c += SC + TC * n
    return out


@pytest.fixture(scope="module")
def oracle_pool():
    ctx = mp.get_context("spawn")
    with ctx.Pool(workers()) as pool:
        yield pool


def jobs_of(wl, layer, geo):
    """Oracle jobs for every panel: a job per sequence, its heads split so that
    a batch with few sequences still keeps every worker busy."""
    B, H = len(layer.lens), layer.Hkv
    chunks = max(1, min(H, -(-workers() // B)))
    parts = [list(range(H))[i::chunks] for i in range(chunks)]
    return [(wl.index, geo, b, hs) for b in range(B) for hs in parts]


@pytest.mark.parametrize("wl", configs.ALL, ids=[w.name for w in configs.ALL])
def test_workload_full_size(wl, oracle_pool):
    """Every (sequence, KV head) panel of every layer at full size, in the
    launch configuration the benchmark times: the pool bytes the GPU append
    wrote equal the oracle quantizer's (by digest, written slots only), and
    the GPU decode of each panel is within the oracle bound."""
    say("workload", wl.name, "oracle workers", workers())
    layers = workloads.build_workload(wl)
    pool = oracle_pool
    for layer in layers:
        out = workloads.decode_layer(layer)
        torch.cuda.synchronize()
        out_np = to_np(out)
        assert np.all(np.isfinite(out_np)), layer.name
        plan = ops.decode_plan(len(layer.lens), layer.Hq, layer.kd, layer.vd, layer.max_seq_len, layer.window)
        pieces = unit_pieces(layer, plan.workgroups)
        say(f"  {layer.name}: {plan.workgroups} workgroups, {len(pieces)} units, "
            f"{sum(1 for v in pieces.values() if v >= 3)} cut into 3+ pieces, max {max(pieces.values(), default=0)}")
        geo = layer_geometry(layer)
        al = bool(layer.kd.flags & 1)
        kdg = opool.PoolDesc(layer.Hkv, layer.D, layer.P, "heads_d64", layer.scale_kind, layer.row_bytes,
                             layer.pool_rows, align64=al)
        vdg = opool.PoolDesc(layer.Hkv, layer.D, layer.P, "heads_dmajor", workloads.v_kind_of(layer.scale_kind),
                             layer.row_bytes, layer.pool_rows, align64=al)
        G = layer.Hq // layer.Hkv
        jobs = jobs_of(wl, layer, geo)
        worst, npanels = 0.0, 0
        for b, res in pool.imap_unordered(oracle_sequence, jobs):
            L, first = int(layer.lens[b]), int(layer.first_pos[b])
            start = max(0, L - layer.window) if layer.window > 0 else 0
            pages = np.arange(start // layer.P, (L - 1) // layer.P + 1)
            rows = layer.table_np[b, pages]
            wr = written_slots(L, first, pages, layer.P)
            for g, (dk, dv, want) in res.items():
                if L > 0:
                    for desc, dev, d_or in ((kdg, layer.k_pool, dk), (vdg, layer.v_pool, dv)):
                        idx = torch.from_numpy(panel_byte_index(desc, rows, g)).to(dev.device)
                        assert digest(panel_bytes(dev[idx].cpu().numpy(), desc, wr)) == d_or, \
                            f"{layer.name} b={b} g={g}: pool bytes differ from the oracle quantizer"
                err, frac = assert_parity(out_np[b, g * G:(g + 1) * G], want, f"{layer.name} b={b} g={g}")
                worst = max(worst, frac)
                npanels += 1
            say(f"  {layer.name} b={b} L={L} heads {sorted(res)}: ok (worst so far {worst:.2f} of the bound)")
        assert npanels == len(layer.lens) * layer.Hkv
        say(f"  {layer.name}: all {npanels} panels within the bound, worst {worst:.2f} of it")


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


def test_long_context_full_size_mx_fp8_mode():
    """The long-context MXFP8 call at full size in the fp8 mode (the MX-scaled
    fp8 MFMA): sampled panels within the default bound of the oracle decoding
    the MXFP8-rounded query, and within the page's fp8 class of the exact
    oracle."""
    say("workload mx fp8")
    wl = configs.LONG_MXFP8
    layer = workloads.build_workload(wl)[0]
    ops.reset_counters()
    out = workloads.decode_layer(layer, variant="mfma_fp8")
    torch.cuda.synchronize()
    assert ops.counters()["decode_mfma_mxfp8"] == 1
    out_np = to_np(out)
    assert np.all(np.isfinite(out_np))
    q = inputs.normal_bf16(configs.SEED, wl.index, "q", 0, (len(layer.lens), layer.Hq, layer.D))
    qmx = oatt.fp8_query_mx(q)
    G = layer.Hq // layer.Hkv
    for b, g in [(0, 3), (2, 7)]:
        kd, vd, hk, hv = oracle_panel(wl, layer, b, g)
        want = oatt.decode_ref(qmx, hk, hv, kd, vd, layer.table_np, layer.lens, sm_scale=layer.sm_scale,
                               seqs=[b], heads=[g])
        err, frac = assert_parity(out_np[b, g * G:(g + 1) * G], want[b, g * G:(g + 1) * G], f"mx b={b} g={g}")
        exact = oatt.decode_ref(q, hk, hv, kd, vd, layer.table_np, layer.lens, sm_scale=layer.sm_scale,
                                seqs=[b], heads=[g])[b, g * G:(g + 1) * G]
        assert np.all(np.abs(out_np[b, g * G:(g + 1) * G] - exact) <= 0.15 + 0.15 * np.abs(exact))
        say(f"  mx b={b} g={g}: max err {err:.2e} ({frac:.2f} of bound)")
