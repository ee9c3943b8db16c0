#!/usr/bin/env python3
"""Decode benchmark: KV-read HBM GB/s (and % of the MI355X 8 TB/s peak) plus µs
per decode call, on seeded synthetic workloads resident in HBM.

By default all five workloads are measured in one run; the headline is the
largest single-GPU one, the gpt-oss-shaped decode (B=64, Hq=64, Hkv=8, D=64,
page 16, seq_lens U[2048, 32768], a window-128 layer and a full layer, sinks,
E4M3 K/V with fp32 per-(page, head) scales).  One step = one decode call per
layer of the workload (plan, decode kernel; split merges run inside it).
Pools are built once by the library's append kernel; several copies are
rotated so that consecutive steps never read a pool that could still sit in
the 256 MB last-level cache.  Every other workload is reported under
"configs" with its own µs per step, GB/s and fraction of peak.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
       [--sweep] [--formats] [--graph] [--no-cpu-baseline] [--copy-probe]
Prints one JSON line (rank 0, N=1).
"""
import argparse
import ctypes
import hashlib
import json
import os
import re
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "KV-read HBM GB/s (% of MI355X peak) + µs per decode call, batch×context sweep"
PEAK_GBPS = 8000.0
PROFILE_PMC = os.path.join(ROOT, "profiles", "decode_{}_pmc.json")
KERNEL_SOURCES = ["fp8_paged_kv_amd/csrc/decode.hip", "fp8_paged_kv_amd/csrc/decode_kernel.h",
                  "fp8_paged_kv_amd/csrc/append_common.h", "fp8_paged_kv_amd/csrc/device_common.h",
                  "fp8_paged_kv_amd/csrc/fp8pa_internal.h"]


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="", help="one workload only (default: all five, headline gpt-oss-decode)")
    ap.add_argument("--workgroups", type=int, default=0, help="0: one resident generation (auto)")
    ap.add_argument("--copies", type=int, default=0, help="pool copies to rotate (0: enough for 2 GiB)")
    ap.add_argument("--sweep", action="store_true", help="batch x context sweep (CSV on stderr, JSON per point)")
    ap.add_argument("--sweep-points", default="", help="--sweep: only these BxL points, e.g. 256x1024,1024x256")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--variant", default="auto", choices=["auto", "mfma_bf16", "mfma_fp8", "packed_heads", "packed_split"],
                    help="decode variant (mfma_fp8: the fp8 compute mode, q rounded to E4M3; packed_heads: one "
                         "workgroup per sequence and group of KV heads, no split)")
    ap.add_argument("--cpu-budget", type=float, default=20.0, help="CPU seconds of oracle work in the CPU baseline")
    ap.add_argument("--copy-probe", action="store_true", help="also run a plain 1 GiB copy (PMC scale reference)")
    ap.add_argument("--formats", action="store_true",
                    help="time the workload's decode in each pool format (K layout x scale kind; JSON per format)")
    ap.add_argument("--graph", action="store_true",
                    help="time one step of all layers as eager launches and as a replayed HIP graph")
    ap.add_argument("--graph-depth", type=int, default=1,
                    help="--graph: decodes of the layer list per step (a model's depth), pool copies in turn")
    return ap.parse_args()


class Hip:
    """hipEvent API of the HIP runtime torch already loaded (one runtime per process)."""

    def __init__(self):
        path = None
        for m in re.findall(r"/\S*libamdhip64\.so\S*", open("/proc/self/maps").read()):
            path = m
            break
        self.lib = ctypes.CDLL(path or "libamdhip64.so")
        self.lib.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.lib.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.lib.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        self.lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.lib.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def events(self, n):
        out = []
        for _ in range(n):
            e = ctypes.c_void_p()
            if self.lib.hipEventCreate(ctypes.byref(e)) != 0:
                raise RuntimeError("hipEventCreate failed")
            out.append(e.value)
        return out

    def record(self, ev, stream):
        if self.lib.hipEventRecord(ctypes.c_void_p(ev), ctypes.c_void_p(stream)) != 0:
            raise RuntimeError("hipEventRecord failed")

    def elapsed_ms(self, a, b):
        self.lib.hipEventSynchronize(ctypes.c_void_p(b))
        ms = ctypes.c_float()
        if self.lib.hipEventElapsedTime(ctypes.byref(ms), ctypes.c_void_p(a), ctypes.c_void_p(b)) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return ms.value

    def destroy(self, evs):
        for e in evs:
            self.lib.hipEventDestroy(ctypes.c_void_p(e))


def source_digest():
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        h.update(open(os.path.join(ROOT, p), "rb").read())
    return h.hexdigest()[:16]


def stored_traffic(workload):
    """HBM bytes per decode launch from the committed rocprofv3 PMC summary, if
    it was taken on the current kernel sources; else None."""
    try:
        rec = json.load(open(PROFILE_PMC.format(workload)))
    except (OSError, ValueError):
        return None
    if rec.get("source_digest") != source_digest() or rec.get("workload") != workload:
        return None
    return rec.get("traffic_bytes_per_launch")


def time_layers(layers_copies, steps, warmup, hip, ops, workloads, torch, workgroups, variant="auto"):
    """`warmup` untimed steps, then the timed region: exactly `steps` steps (a
    step decodes every layer once, pool copy k % R), bracketed by
    synchronizations, timed by the wall clock and by one pair of HIP events
    on the launch stream around the same launches.  Then, per layer, a region
    of `steps` back-to-back launches of that layer alone, timed the same two
    ways (its mean is the layer's kernel time; it includes the short gaps
    between consecutive launches).  Last, a pass with an event between steps
    gives the step-time distribution."""
    R = len(layers_copies)
    nl = len(layers_copies[0])
    outs = [torch.empty_like(l.q) for l in layers_copies[0]]
    ws = []
    for l in layers_copies[0]:
        p = ops.decode_plan(len(l.lens), l.Hq, l.kd, l.vd, l.max_seq_len, l.window, workgroups, variant)
        ws.append(torch.empty(max(p.workspace_bytes, 256), dtype=torch.uint8, device="cuda:0"))
    stream = torch.cuda.current_stream().cuda_stream

    def step(k):
        for j, l in enumerate(layers_copies[k % R]):
            workloads.decode_layer(l, out=outs[j], workspace=ws[j], workgroups=workgroups, variant=variant)

    def region(fn, n):
        ev = hip.events(2)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        hip.record(ev[0], stream)
        for k in range(n):
            fn(k)
        hip.record(ev[1], stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        ms = hip.elapsed_ms(ev[0], ev[1])
        hip.destroy(ev)
        return wall, ms / 1e3

    # Settle: untimed steps for SETTLE_S seconds of wall time, so that the
    # device's clocks have ramped up (measured: the first ~20 ms of sustained
    # decode run up to 12% slower, then the step time is flat), then the
    # `warmup` steps, then the timed region.
    torch.cuda.synchronize()
    t_settle, k = time.perf_counter(), 0
    while time.perf_counter() - t_settle < SETTLE_S:
        step(k)
        k += 1
        if k % 8 == 0:
            torch.cuda.synchronize()
    for k in range(warmup):
        step(k)
    wall, ev_s = region(step, steps)
    kern = []
    for j in range(nl):
        def one(k, j=j):
            l = layers_copies[k % R][j]
            workloads.decode_layer(l, out=outs[j], workspace=ws[j], workgroups=workgroups, variant=variant)
        t_settle, k = time.perf_counter(), 0
        while time.perf_counter() - t_settle < SETTLE_S / 2:
            one(k)
            k += 1
            if k % 8 == 0:
                torch.cuda.synchronize()
        kw, ke = region(one, steps)
        kern.append({"wall_s": kw, "event_s": ke})
    step_ev = hip.events(steps + 1)
    torch.cuda.synchronize()
    for k in range(steps):
        hip.record(step_ev[k], stream)
        step(k)
    hip.record(step_ev[steps], stream)
    torch.cuda.synchronize()
    step_ms = [hip.elapsed_ms(step_ev[k], step_ev[k + 1]) for k in range(steps)]
    hip.destroy(step_ev)
    return {"wall_s": wall, "event_s": ev_s, "kern": kern, "step_ms": step_ms}, outs


def time_fused(copies, j, steps, hip, ops, workloads, torch):
    """One decode step of layer j with its KV append: fp8pa_append_quant of
    each sequence's new token (position seq_lens - 1) then fp8pa_decode, against
    fp8pa_append_decode (one launch).  Batch events around `steps` steps each,
    pool copies rotated.  The appends rewrite each sequence's last token."""
    R = len(copies)
    l0 = copies[0][j]
    B, Hkv, D = len(l0.lens), l0.Hkv, l0.D
    g = torch.Generator(device="cuda:0")
    g.manual_seed(20261203)
    k_new = torch.randn((B, Hkv, D), generator=g, device="cuda:0").to(torch.bfloat16)
    v_new = torch.randn((B, Hkv, D), generator=g, device="cuda:0").to(torch.bfloat16)
    pos = (l0.seq_lens - 1).clamp(min=0).to(torch.int32)
    counts = (l0.seq_lens > 0).to(torch.int32)
    out = torch.empty_like(l0.q)
    p = ops.decode_plan(B, l0.Hq, l0.kd, l0.vd, l0.max_seq_len, l0.window)
    ws = torch.empty(max(p.workspace_bytes, 256), dtype=torch.uint8, device="cuda:0")
    stream = torch.cuda.current_stream().cuda_stream

    def two(l):
        ops.append_quant(k_new[:, None], v_new[:, None], l.k_pool, l.v_pool, l.kd, l.vd, l.block_table, pos, counts)
        workloads.decode_layer(l, out=out, workspace=ws)

    def one(l):
        ops.append_decode(l.q, k_new, v_new, l.k_pool, l.v_pool, l.kd, l.vd, l.block_table, l.seq_lens,
                          l.max_seq_len, window=l.window, sinks=l.sinks, sm_scale=l.sm_scale, out=out, workspace=ws)

    res = {}
    for name, fn in (("append_then_decode", two), ("fused", one)):
        for k in range(5):
            fn(copies[k % R][j])
        ev = hip.events(2)
        torch.cuda.synchronize()
        hip.record(ev[0], stream)
        for k in range(steps):
            fn(copies[k % R][j])
        hip.record(ev[1], stream)
        torch.cuda.synchronize()
        res[name] = hip.elapsed_ms(ev[0], ev[1]) / steps * 1e3
        hip.destroy(ev)
    return res


def clone_layer(l, torch):
    import dataclasses
    return dataclasses.replace(l, k_pool=l.k_pool.clone(), v_pool=l.v_pool.clone())


def _seq_kv_bytes(L, window, P, D, Hkv, scale_kind):
    """Algorithmic KV bytes of one sequence of one layer (all its KV heads):
    the codes of the attended positions of K and V and the scales they touch."""
    start = max(0, L - window) if window > 0 else 0
    n = L - start
    if n <= 0:
        return 0
    if scale_kind == "page_head":
        sc = 2 * 4 * ((L - 1) // P - start // P + 1)
    elif scale_kind == "token_head":
        sc = 2 * 4 * n
    else:
        sc = 2 * n * (D // 32)
    return (2 * n * D + sc) * Hkv


def _oracle_inputs(wl_index, li, b):
    """The oracle's own pools for sequence b of layer li of a workload: the
    same seeded inputs as the GPU build, quantized by the oracle into a host
    pool holding just this sequence's attended pages (rows 0..n-1)."""
    import numpy as np

    from fp8_paged_kv_amd import configs, inputs, workloads
    from oracle import pool as opool
    wl = configs.ALL[wl_index]
    lay = wl.layers[li]
    P, D, Hkv = wl.P, lay.D, lay.Hkv
    lens = inputs.seq_lens(configs.SEED, wl.index, wl.B, wl.L_lo, wl.L_hi)
    L = int(lens[b])
    first = workloads.first_attended_page(L, lay.window, P) * P
    n_rows = max(1, -(-L // P) - first // P)
    table = np.full((wl.B, -(-int(wl.L_hi) // P)), -1, np.int32)
    table[b, first // P:first // P + n_rows] = np.arange(n_rows, dtype=np.int32)
    sk = wl.scale_kind
    kd = opool.PoolDesc(Hkv, D, P, "heads_d64", sk, P * Hkv * D + workloads.scale_block_bytes(sk, Hkv, P, D), n_rows)
    vd = opool.PoolDesc(Hkv, D, P, "heads_dmajor", sk, kd.row_bytes, n_rows)
    hk = np.zeros(n_rows * kd.row_bytes, np.uint8)
    hv = np.zeros(n_rows * vd.row_bytes, np.uint8)
    n = L - first
    if n > 0:
        xs = [None] * wl.B
        xs[b] = workloads.raw_kv(configs.SEED, wl, li, b, "k", n, Hkv, D)
        if first == 0:
            hk = opool.pack_sequences(hk, kd, table, xs)
        else:
            hk = opool.append_ref(hk, kd, table[b:b + 1], [first], xs[b][None])
        xs[b] = workloads.raw_kv(configs.SEED, wl, li, b, "v", n, Hkv, D)
        if first == 0:
            hv = opool.pack_sequences(hv, vd, table, xs)
        else:
            hv = opool.append_ref(hv, vd, table[b:b + 1], [first], xs[b][None])
    q = inputs.normal_bf16(configs.SEED, wl.index, "q", li, (wl.B, lay.Hq, D))
    sinks = inputs.sinks(configs.SEED, wl.index, lay.Hq) if wl.sinks else None
    sm = lay.D ** -0.5 if lay.sm_scale is None else lay.sm_scale
    return dict(q=q, hk=hk, hv=hv, kd=kd, vd=vd, table=table, lens=lens, window=lay.window, sinks=sinks, sm=sm, b=b,
                nbytes=_seq_kv_bytes(L, lay.window, P, D, Hkv, sk))


def _oracle_worker(wl_index, tasks, repeats, barrier, queue):
    """One host core: builds its share of the oracle's inputs (untimed), waits
    for every worker, then decodes its share `repeats` times, timed."""
    from threadpoolctl import threadpool_limits

    from oracle import attention as oatt
    with threadpool_limits(1):
        built = [_oracle_inputs(wl_index, li, b) for li, b in tasks]
        barrier.wait()
        t0 = time.perf_counter()
        nbytes = 0
        for _ in range(repeats):
            for x in built:
                oatt.decode_ref(x["q"], x["hk"], x["hv"], x["kd"], x["vd"], x["table"], x["lens"], window=x["window"],
                                sinks=x["sinks"], sm_scale=x["sm"], seqs=[x["b"]])
                nbytes += x["nbytes"]
        t1 = time.perf_counter()
    queue.put((nbytes, t0, t1))


def cpu_baseline(wl, budget_s):
    """The oracle (float64 numpy, one BLAS thread per process) on every host
    core the process may use, over the whole decode step of the workload (all
    layers, all sequences; inputs re-quantized by the oracle first, untimed):
    one process per core, each a balanced share of the (layer, sequence)
    panels, all started together; the step is repeated until about `budget_s`
    seconds of CPU work.  GB/s = algorithmic KV bytes / wall time of the
    decode phase."""
    import multiprocessing as mp

    from fp8_paged_kv_amd import configs, inputs
    cores = len(os.sched_getaffinity(0))
    lens = inputs.seq_lens(configs.SEED, wl.index, wl.B, wl.L_lo, wl.L_hi)
    tasks = [(li, b, _seq_kv_bytes(int(lens[b]), lay.window, wl.P, lay.D, lay.Hkv, wl.scale_kind))
             for li, lay in enumerate(wl.layers) for b in range(wl.B)]
    tasks.sort(key=lambda t: -t[2])
    share = [[] for _ in range(min(cores, len(tasks)))]
    load = [0] * len(share)
    for li, b, nb in tasks:                       # largest first, to the least loaded core
        i = load.index(min(load))
        share[i].append((li, b))
        load[i] += nb
    total = sum(t[2] for t in tasks)
    est_cpu_s = total / 0.1e9                    # about 0.1 GB/s per core for this oracle
    repeats = int(max(1, min(20, round(budget_s / max(est_cpu_s, 1e-9)))))
    ctx = mp.get_context("spawn")
    barrier = ctx.Barrier(len(share))
    queue = ctx.Queue()
    procs = [ctx.Process(target=_oracle_worker, args=(wl.index, sh, repeats, barrier, queue)) for sh in share]
    for pr in procs:
        pr.start()
    res = [queue.get() for _ in procs]
    for pr in procs:
        pr.join()
    nbytes = sum(r[0] for r in res)
    wall = max(r[2] for r in res) - min(r[1] for r in res)
    busy = sum(r[2] - r[1] for r in res)
    return {"value": round(nbytes / wall / 1e9, 4), "unit": "GB/s", "cores": len(share), "kind": "oracle",
            "sample": f"the whole decode step of {wl.name} ({len(wl.layers)} layer(s) x {wl.B} sequences, "
                      f"{total} KV bytes), decoded {repeats}x by {len(share)} processes of float64 numpy with one "
                      f"BLAS thread each; {wall:.2f} s wall, {busy:.1f} s of CPU; quantization excluded",
            "host_cpus": cores, "os_cpu_count": os.cpu_count()}


def run_sweep(args, torch, ops, workloads, hip):
    """C2 geometry at fixed L for B x L points; pools built on the GPU from a
    seeded torch generator (timing only: content does not change the work)."""
    import numpy as np
    D, Hq, Hkv, P = 128, 32, 8, 16
    rb = 16416
    gen = torch.Generator(device="cuda:0")
    only = {tuple(int(x) for x in pt.split("x")) for pt in args.sweep_points.split(",") if pt}
    print("B,L,us_per_call_median,kv_gbps,pct_peak", file=sys.stderr)
    for L in (128, 1024, 4096, 16384, 32000, 131072):
        for B in (1, 8, 32, 128, 256, 1024):
            if B > 128 and L > 4096:
                continue
            if only and (B, L) not in only:
                continue
            pages = -(-L // P)
            rows = B * pages
            if rows * rb * 2 > 60e9:
                continue
            gen.manual_seed(L * 1000 + B)
            k_pool = torch.full((rows * rb,), 0xFF, dtype=torch.uint8, device="cuda:0")
            v_pool = torch.full((rows * rb,), 0xFF, dtype=torch.uint8, device="cuda:0")
            kd = ops.pool_desc(Hkv, D, P, "heads", "page_head", rb, rows)
            vd = ops.pool_desc(Hkv, D, P, "heads_dmajor", "page_head", rb, rows)
            perm = torch.randperm(rows, generator=gen, device="cuda:0").to(torch.int32)
            table = perm.view(B, pages).contiguous()
            for b in range(B):
                x = torch.randn((1, L, Hkv, D), generator=gen, device="cuda:0").to(torch.bfloat16)
                y = torch.randn((1, L, Hkv, D), generator=gen, device="cuda:0").to(torch.bfloat16)
                ops.append_quant(x, y, k_pool, v_pool, kd, vd, table[b:b + 1],
                                 torch.zeros(1, dtype=torch.int32, device="cuda:0"))
            q = torch.randn((B, Hq, D), generator=gen, device="cuda:0").to(torch.bfloat16)
            lens = torch.full((B,), L, dtype=torch.int32, device="cuda:0")
            layer = workloads.DeviceLayer(
                name=f"sweep-B{B}-L{L}", Hq=Hq, Hkv=Hkv, D=D, P=P, window=0, sm_scale=D ** -0.5,
                scale_kind="page_head", row_bytes=rb, pool_rows=rows, kd=kd, vd=vd, k_pool=k_pool, v_pool=v_pool,
                block_table=table, table_np=None, seq_lens=lens, lens=np.full(B, L), first_pos=np.zeros(B),
                q=q, sinks=None, sinks_np=None, max_seq_len=L)
            nbytes = workloads.kv_bytes(layer)
            R = max(1, min(8, int(np.ceil(2 * 2 ** 30 / (2 * rows * rb)))))
            copies = [[layer]] + [[clone_layer(layer, torch)] for _ in range(R - 1)]
            steps = max(20, min(args.steps, 200))
            t, _ = time_layers(copies, steps, 5, hip, ops, workloads, torch, args.workgroups, args.variant)
            med = statistics.median(t["step_ms"]) * 1e3
            gbps = nbytes / (t["kern"][0]["event_s"] / steps) / 1e9
            print(f"{B},{L},{med:.2f},{gbps:.1f},{100 * gbps / PEAK_GBPS:.1f}", file=sys.stderr, flush=True)
            print(json.dumps({"sweep_point": {"B": B, "L": L, "variant": args.variant,
                                              "us_per_call_median": round(med, 2),
                                              "kernel_gbps": round(gbps, 1),
                                              "pct_peak": round(100 * gbps / PEAK_GBPS, 1)}}), flush=True)
            del copies, layer, k_pool, v_pool
            torch.cuda.empty_cache()


# (K layout, V layout, scale kind; None: the workload's own).  Rows 7-10 are
# the page's own payload orders for both pools; the last three take fp32
# sub-row K scales (V per (token, head)).
FORMATS = (("heads_d64", "heads_dmajor", None), ("heads", "heads_dmajor", None), ("tokens", "heads_dmajor", None),
           ("heads_d64", "heads_dmajor", "token_head"), ("heads", "heads_dmajor", "token_head"),
           ("tokens", "heads_dmajor", "token_head"), ("heads", "heads", None), ("tokens", "tokens", None),
           ("heads", "heads", "token_head"), ("tokens", "tokens", "token_head"),
           ("heads_d64", "heads_dmajor", "f32_g32"), ("heads_d64", "heads_dmajor", "f32_g64"),
           ("tokens", "tokens", "f32_g32"))
# The same formats with rows on 128-byte lines (row width a multiple of 128):
# token-major pools then load whole lines.
FORMATS_ROW128 = (("heads_d64", "heads_dmajor", None), ("heads", "heads_dmajor", None),
                  ("tokens", "heads_dmajor", None), ("heads", "heads", None), ("tokens", "tokens", None),
                  ("tokens", "tokens", "token_head"))


def copies_of(layers, wl, R, torch):
    copies = [layers]
    for _ in range(R - 1):
        if wl.shared_pool:
            import dataclasses
            k2, v2 = layers[0].k_pool.clone(), layers[0].v_pool.clone()
            copies.append([dataclasses.replace(l, k_pool=k2, v_pool=v2) for l in layers])
        else:
            copies.append([clone_layer(l, torch) for l in layers])
    torch.cuda.synchronize()
    return copies


def rotation(layers, wl, np):
    per_copy = sum(2 * l.k_pool.numel() for l in layers) if not wl.shared_pool else 2 * layers[0].k_pool.numel()
    return max(2, min(16, int(np.ceil(2 * 2 ** 30 / per_copy))))


def run_formats(args, wl, torch, np, ops, workloads, hip):
    """The workload in each pool format: same seeded values, written by the
    library's append in that format.  Formats that share a scale kind hold the
    same codes and scales, so their outputs must agree bit for bit."""
    first = {}
    for kl, vl, sk, ra in [f + (16,) for f in FORMATS] + [f + (128,) for f in FORMATS_ROW128]:
        if args.variant in ("mfma_fp8", "packed_heads", "packed_split") and (vl != "heads_dmajor" or
                                                                              (sk or "").startswith("f32_g")):
            continue   # these variants read V d-major only, and no sub-row K scales
        sk = wl.scale_kind if sk is None else sk
        layers = workloads.build_workload(wl, k_layout=kl, v_layout=vl, scale_kind=sk, row_align=ra)
        R = args.copies or rotation(layers, wl, np)
        copies = copies_of(layers, wl, R, torch)
        outs = [workloads.decode_layer(l, variant=args.variant).clone() for l in layers]
        if sk in first:
            for j, o in enumerate(outs):
                assert torch.equal(o.view(torch.int16), first[sk][j].view(torch.int16)), \
                    f"{kl}/{sk}: output differs from {sk} in another layout"
        else:
            first[sk] = outs
        t, _ = time_layers(copies, args.steps, args.warmup, hip, ops, workloads, torch, args.workgroups,
                           args.variant)
        rows = []
        for l, k in zip(layers, t["kern"]):
            km = k["event_s"] / args.steps * 1e3
            b = workloads.kv_bytes(l)
            rows.append({"name": l.name, "kernel_us_mean": round(km * 1e3, 2), "kv_bytes": b,
                         "kernel_gbps": round(b / (km * 1e-3) / 1e9, 1),
                         "pct_peak": round(100 * b / (km * 1e-3) / 1e9 / PEAK_GBPS, 1)})
        print(json.dumps({"format": {"k_layout": kl, "v_layout": vl, "scale_kind": sk,
                                     "row_bytes": layers[0].row_bytes, "row_align": ra}, "variant": args.variant,
                          "workload": wl.name, "layers": rows,
                          "timing": f"hipEvents around {args.steps} back-to-back launches per layer, "
                                    f"{R} pool copies rotated"}), flush=True)
        del copies, layers
        torch.cuda.empty_cache()


def run_graph(args, wl, torch, np, ops, workloads, hip):
    """One decode step, `--graph-depth` passes over all layers of the workload
    (pass r reads pool copy r mod R, so a deep step still streams from HBM):
    eager launches against a replayed HIP graph (one graph per starting copy,
    grids fixed at capture)."""
    layers = workloads.build_workload(wl)
    R = args.copies or rotation(layers, wl, np)
    copies = copies_of(layers, wl, R, torch)
    depth = max(1, args.graph_depth)
    outs = [torch.empty_like(l.q) for l in layers]
    ws = []
    for l in layers:
        p = ops.decode_plan(len(l.lens), l.Hq, l.kd, l.vd, l.max_seq_len, l.window)
        ws.append(torch.empty(max(p.workspace_bytes, 256), dtype=torch.uint8, device="cuda:0"))

    def step(c0):
        for r in range(depth):
            for j, l in enumerate(copies[(c0 + r) % R]):
                workloads.decode_layer(l, out=outs[j], workspace=ws[j])

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step(0)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    eager = [o.clone() for o in outs]
    graphs = []
    for c0 in range(R):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            step(c0)
        graphs.append(g)
    torch.cuda.synchronize()
    for o in outs:
        o.zero_()
    graphs[0].replay()
    torch.cuda.synchronize()
    for o, e in zip(outs, eager):
        assert torch.equal(o.view(torch.int16), e.view(torch.int16)), "graph replay differs from eager"
    stream = torch.cuda.current_stream().cuda_stream
    res = {}
    for name, fn in (("eager", lambda k: step(k % R)), ("graph", lambda k: graphs[k % R].replay())):
        for k in range(args.warmup):
            fn(k)
        ev = hip.events(2)
        torch.cuda.synchronize()
        hip.record(ev[0], stream)
        for k in range(args.steps):
            fn(k)
        hip.record(ev[1], stream)
        torch.cuda.synchronize()
        res[name] = hip.elapsed_ms(ev[0], ev[1]) / args.steps * 1e3
        hip.destroy(ev)
    print(json.dumps({"graph_step": {"workload": wl.name, "layers": [l.name for l in layers], "depth": depth,
                                     "us_per_step_eager": round(res["eager"], 2),
                                     "us_per_step_graph": round(res["graph"], 2),
                                     "timing": f"hipEvents around {args.steps} steps, {R} pool copies rotated"}}),
          flush=True)
    del graphs


HEADLINE = "gpt-oss-decode"   # the largest single-GPU config (most KV bytes per step)
SETTLE_S = 0.2                 # untimed decode before each timed region (clock ramp-up)
GATED = {"llama3-8b-decode", "gpt-oss-decode", "gemma4-mixed-pool", "long-context-mxfp8"}


def measure(wl, args, hip, torch, np, ops, workloads):
    """Build the workload, check that the rotated pool copies decode alike, and
    time it (time_layers).  Returns (record, layers, copies)."""
    t_build = time.perf_counter()
    layers = workloads.build_workload(wl)
    build_s = time.perf_counter() - t_build
    R = args.copies or rotation(layers, wl, np)
    copies = copies_of(layers, wl, R, torch)
    # Copies hold identical bytes: every copy must give the same output bit for bit.
    ref = [workloads.decode_layer(l, variant=args.variant).clone() for l in copies[0]]
    for c in copies[1:]:
        for j, l in enumerate(c):
            assert torch.equal(workloads.decode_layer(l, variant=args.variant), ref[j]), "pool copies disagree"
    torch.cuda.synchronize()
    t, _ = time_layers(copies, args.steps, args.warmup, hip, ops, workloads, torch, args.workgroups, args.variant)
    layer_bytes = [workloads.kv_bytes(l) for l in layers]
    total = sum(layer_bytes)
    step_s = t["wall_s"] / args.steps
    step_ev_s = t["event_s"] / args.steps
    plans = [ops.decode_plan(len(l.lens), l.Hq, l.kd, l.vd, l.max_seq_len, l.window, args.workgroups, args.variant)
             for l in layers]
    us = sorted(x * 1e3 for x in t["step_ms"])
    pct = lambda q: us[min(len(us) - 1, int(q * len(us)))]
    lay_rec = []
    for l, b, p, k in zip(layers, layer_bytes, plans, t["kern"]):
        ku = k["event_s"] / args.steps * 1e6
        lay_rec.append({"name": l.name, "Hq": l.Hq, "Hkv": l.Hkv, "D": l.D, "window": l.window,
                        "sm_scale": round(l.sm_scale, 6), "kv_bytes": b, "workgroups": p.workgroups,
                        "variant": {v: k_ for k_, v in ops.VARIANTS.items()}[p.variant],
                        "kernel_us": round(ku, 2), "kernel_us_wall": round(k["wall_s"] / args.steps * 1e6, 2),
                        "kernel_gbps": round(b / (ku * 1e-6) / 1e9, 1),
                        "frac": round(b / (ku * 1e-6) / 1e9 / PEAK_GBPS, 4)})
    gbps = total / step_s / 1e9
    rec = {"B": wl.B, "page": wl.P, "seq_lens": f"U[{wl.L_lo},{wl.L_hi}]", "scales": wl.scale_kind,
           "kv_bytes_per_step": total, "us_per_step": round(step_s * 1e6, 2),
           "us_per_step_events": round(step_ev_s * 1e6, 2), "gbps": round(gbps, 1),
           "frac": round(gbps / PEAK_GBPS, 4),
           "gate": "long-context: >= 0.70 of 8 TB/s" if wl.name in GATED else "launch-bound: reported in us, not gated",
           "step_us_median": round(pct(0.5), 2), "step_us_p10": round(pct(0.1), 2), "step_us_p90": round(pct(0.9), 2),
           "layers": lay_rec, "pool_copies_rotated": R, "build_s": round(build_s, 1)}
    return rec, layers, copies


def copy_probe(torch, hip):
    """A plain 1 GiB device copy: its counters scale the PMC byte counts of
    a profiled run."""
    n = 1 << 30
    stream = torch.cuda.current_stream().cuda_stream
    a = torch.empty(n, dtype=torch.uint8, device="cuda:0")
    b = torch.empty_like(a)
    ev = hip.events(2)
    for _ in range(3):
        b.copy_(a)
    hip.record(ev[0], stream)
    for _ in range(5):
        b.copy_(a)
    hip.record(ev[1], stream)
    ms = hip.elapsed_ms(ev[0], ev[1]) / 5
    hip.destroy(ev)
    del a, b
    return {"bytes_read": n, "bytes_written": n, "us": round(ms * 1e3, 2),
            "read_plus_write_gbps": round(2 * n / (ms * 1e-3) / 1e9, 1)}


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py: this library runs on one GPU only; the decode path shards by sequence or KV head with no "
              "exchange, which needs no multi-GPU run to measure (run with --gpus 1)", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    from fp8_paged_kv_amd import configs, ops, workloads

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    ops.lib()
    hip = Hip()
    if args.sweep:
        run_sweep(args, torch, ops, workloads, hip)
        return
    by_name = {w.name: w for w in configs.ALL}
    if args.formats:
        run_formats(args, by_name[args.workload or "llama3-8b-decode"], torch, np, ops, workloads, hip)
        if args.copy_probe:
            print(json.dumps({"copy_probe": copy_probe(torch, hip)}), flush=True)
        return
    if args.graph:
        run_graph(args, by_name[args.workload or "llama3-8b-decode"], torch, np, ops, workloads, hip)
        return
    # The headline workload first (on a fresh device), then the other configs.
    head = by_name[args.workload or HEADLINE]
    order = [head] + ([w for w in configs.ALL if w is not head] if not args.workload else [])
    recs = {}
    for wl in order:
        print(f"bench: measuring {wl.name}", file=sys.stderr, flush=True)
        rec, layers, copies = measure(wl, args, hip, torch, np, ops, workloads)
        recs[wl.name] = rec
        if wl is head:
            hrec, hlayers = rec, layers
            dom = int(np.argmax([l["kv_bytes"] for l in rec["layers"]]))
            fu = time_fused(copies, dom, args.steps, hip, ops, workloads, torch)
            ld = layers[dom]
            span = min(ld.window, ld.max_seq_len) if ld.window > 0 else ld.max_seq_len
            fused = {"layer": ld.name, "us_append_quant_then_decode": round(fu["append_then_decode"], 2),
                     "us_append_decode": round(fu["fused"], 2),
                     "append_decode_path": "one launch" if span <= 2048 else "append kernel, then decode",
                     "timing": f"hipEvents around {args.steps} steps (new token per sequence appended, then "
                               f"decoded); mean per step"}
        del copies, layers
        torch.cuda.empty_cache()
    dl = hrec["layers"][dom]
    traffic = stored_traffic(head.name)
    out = {
        "metric": METRIC,
        "value": hrec["gbps"],
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(hrec["us_per_step"] / 1e3, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if args.variant != "mfma_fp8" else "fp8 QK (q rounded to e4m3), bf16 PV",
        "data": "synthetic",
        "config": {"workload": head.name, "B": head.B, "page": head.P, "seq_lens": hrec["seq_lens"], "kv": "e4m3",
                   "scales": head.scale_kind, "layers": [l["name"] for l in hrec["layers"]],
                   "kv_bytes_per_step": hrec["kv_bytes_per_step"], "parallelism": "single GPU",
                   "step": "one decode call per layer of the workload (window-128 layer and full layer), split "
                           "merges inside the decode launch",
                   "settle": f"{SETTLE_S} s of untimed decode steps, then the warm-up steps, before each timed "
                             f"region"},
        "pct_of_peak": round(100 * hrec["gbps"] / PEAK_GBPS, 2),
        "us_per_step_events": hrec["us_per_step_events"],
        "roofline": {"bound": "hbm", "achieved": dl["kernel_gbps"], "peak": PEAK_GBPS, "unit": "GB/s",
                     "frac": dl["frac"], "traffic": traffic,
                     "kernel": f"decode_kernel D={dl['D']} ({dl['name']})", "kernel_us_mean": dl["kernel_us"],
                     "kernel_us_mean_wall": dl["kernel_us_wall"], "bytes_per_launch": dl["kv_bytes"],
                     "timing": f"one hipEvent pair on the launch stream around {args.steps} back-to-back launches "
                               f"of this layer (pool copies rotated); mean per launch"},
        "configs": recs,
    }
    # Streaming-read ceiling measured on this machine: the library's plain read
    # probe over 4 GiB (reads only, the same HBM direction as decode).
    x = torch.empty((4 << 30,), dtype=torch.uint8, device="cuda:0")
    sink = torch.zeros(4, dtype=torch.int32, device="cuda:0")
    ev = hip.events(2)
    stream = torch.cuda.current_stream().cuda_stream
    for _ in range(2):
        ops.stream_read(x, sink)
    hip.record(ev[0], stream)
    for _ in range(5):
        ops.stream_read(x, sink)
    hip.record(ev[1], stream)
    ms = hip.elapsed_ms(ev[0], ev[1]) / 5
    hip.destroy(ev)
    out["read_probe"] = {"bytes": 4 << 30, "us": round(ms * 1e3, 2), "gbps": round((4 << 30) / (ms * 1e-3) / 1e9, 1),
                         "kernel": "fp8pa_stream_read over 4 GiB"}
    out["roofline"]["frac_of_measured_read"] = round(dl["kernel_gbps"] / out["read_probe"]["gbps"], 4)
    del x
    if args.copy_probe:
        out["copy_probe"] = copy_probe(torch, hip)
    out["fused_append_decode"] = fused
    out["cpu_baseline"] = None if args.no_cpu_baseline else cpu_baseline(head, args.cpu_budget)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
