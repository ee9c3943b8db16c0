#!/usr/bin/env python3
"""Decode benchmark: KV-read HBM GB/s (and % of the MI355X 8 TB/s peak) plus µs
per decode call, on seeded synthetic workloads resident in HBM.

Default workload: the Llama-3-8B-shaped decode (B=32, Hq=32, Hkv=8, D=128,
page 16, seq_lens U[1024, 8192], E4M3 K/V with fp32 per-(page, head) scales,
full attention).  One step = one decode call over the batch (plan, decode
kernel, split merge).  Pools are built once by the library's append kernel;
several copies are rotated so that consecutive steps never read a pool that
could still sit in the 256 MB last-level cache.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
       [--sweep] [--no-cpu-baseline] [--copy-probe]
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
PROFILE_PMC = os.path.join(ROOT, "profiles", "decode_llama3-8b-decode_pmc.json")
KERNEL_SOURCES = ["fp8_paged_kv_amd/csrc/decode.hip", "fp8_paged_kv_amd/csrc/decode_kernel.h",
                  "fp8_paged_kv_amd/csrc/append_common.h", "fp8_paged_kv_amd/csrc/device_common.h",
                  "fp8_paged_kv_amd/csrc/fp8pa_internal.h"]


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="llama3-8b-decode")
    ap.add_argument("--workgroups", type=int, default=0, help="0: one resident generation (auto)")
    ap.add_argument("--copies", type=int, default=0, help="pool copies to rotate (0: enough for 2 GiB)")
    ap.add_argument("--sweep", action="store_true", help="batch x context sweep (CSV on stderr, JSON per point)")
    ap.add_argument("--sweep-points", default="", help="--sweep: only these BxL points, e.g. 256x1024,1024x256")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--variant", default="auto", choices=["auto", "mfma_bf16", "mfma_fp8", "packed_heads", "packed_split"],
                    help="decode variant (mfma_fp8: the fp8 compute mode, q rounded to E4M3; packed_heads: one "
                         "workgroup per sequence and group of KV heads, no split)")
    ap.add_argument("--cpu-budget", type=float, default=15.0, help="seconds of oracle work in the CPU baseline")
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
        rec = json.load(open(PROFILE_PMC))
    except (OSError, ValueError):
        return None
    if rec.get("source_digest") != source_digest() or rec.get("workload") != workload:
        return None
    return rec.get("traffic_bytes_per_launch")


def time_layers(layers_copies, steps, warmup, hip, ops, workloads, torch, workgroups, variant="auto"):
    """Runs `steps` timed steps; a step decodes every layer once (copy k % R).
    Returns wall seconds, per-step GPU ms, and per-layer mean decode ms."""
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

    for k in range(warmup):
        step(k)
    # Throughput: K steps with nothing else in the stream.
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(steps):
        step(k)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    # Step durations: the same K steps again, with an event between steps.
    step_ev = hip.events(steps + 1)
    torch.cuda.synchronize()
    for k in range(steps):
        hip.record(step_ev[k], stream)
        step(k)
    hip.record(step_ev[steps], stream)
    torch.cuda.synchronize()
    step_ms = [hip.elapsed_ms(step_ev[k], step_ev[k + 1]) for k in range(steps)]
    hip.destroy(step_ev)
    # Kernel durations: per layer, K back-to-back launches of that layer alone
    # (pool copies rotated) between two events on the launch stream; the mean
    # includes the short gap between consecutive launches.
    kern_ms = []
    for j in range(nl):
        ev = hip.events(2)
        torch.cuda.synchronize()
        hip.record(ev[0], stream)
        for k in range(steps):
            l = layers_copies[k % R][j]
            workloads.decode_layer(l, out=outs[j], workspace=ws[j], workgroups=workgroups, variant=variant)
        hip.record(ev[1], stream)
        torch.cuda.synchronize()
        kern_ms.append(hip.elapsed_ms(ev[0], ev[1]) / steps)
        hip.destroy(ev)
    return wall, step_ms, kern_ms, outs


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


def cpu_baseline(wl, layers, budget_s):
    """The oracle (float64 numpy, one BLAS thread) timed on a bounded sample of
    the same workload: whole sequences of the first layer, oracle-quantized
    from the same seeded inputs, until about `budget_s` seconds of decode_ref."""
    import numpy as np
    from threadpoolctl import threadpool_limits

    from fp8_paged_kv_amd import configs, inputs, workloads
    from oracle import attention as oatt, pool as opool

    lay = layers[0]
    kd = opool.PoolDesc(lay.Hkv, lay.D, lay.P, "heads_d64", lay.scale_kind, lay.row_bytes, lay.pool_rows)
    vd = opool.PoolDesc(lay.Hkv, lay.D, lay.P, "heads_dmajor", lay.scale_kind, lay.row_bytes, lay.pool_rows)
    q = inputs.normal_bf16(configs.SEED, wl.index, "q", lay.layer_index, (len(lay.lens), lay.Hq, lay.D))
    spent, nbytes, seqs = 0.0, 0, 0
    with threadpool_limits(1):
        for b in range(len(lay.lens)):
            if spent >= budget_s:
                break
            L, first = int(lay.lens[b]), int(lay.first_pos[b])
            xk = workloads.raw_kv(configs.SEED, wl, lay.layer_index, b, "k", L - first, lay.Hkv, lay.D)
            xv = workloads.raw_kv(configs.SEED, wl, lay.layer_index, b, "v", L - first, lay.Hkv, lay.D)
            hk = np.zeros(lay.pool_rows * lay.row_bytes, np.uint8)
            hv = np.zeros(lay.pool_rows * lay.row_bytes, np.uint8)
            if first == 0:
                xs = [None] * len(lay.lens)
                xs[b] = xk
                hk = opool.pack_sequences(hk, kd, lay.table_np, xs)
                xs[b] = xv
                hv = opool.pack_sequences(hv, vd, lay.table_np, xs)
            else:
                hk = opool.append_ref(hk, kd, lay.table_np[b:b + 1], [first], xk[None])
                hv = opool.append_ref(hv, vd, lay.table_np[b:b + 1], [first], xv[None])
            t0 = time.perf_counter()
            oatt.decode_ref(q, hk, hv, kd, vd, lay.table_np, lay.lens, window=lay.window, sinks=lay.sinks_np,
                            sm_scale=lay.sm_scale, seqs=[b])
            spent += time.perf_counter() - t0
            start = max(0, L - lay.window) if lay.window > 0 else 0
            n = L - start
            sc = (2 * 4 * ((L - 1) // lay.P - start // lay.P + 1) * lay.Hkv if lay.scale_kind == "page_head"
                  else 2 * n * (lay.D // 32) * lay.Hkv)
            nbytes += 2 * n * lay.D * lay.Hkv + sc
            seqs += 1
    return {"value": round(nbytes / spent / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"{seqs} of {len(lay.lens)} sequences of {lay.name} (all KV heads), float64 numpy, "
                      f"{spent:.1f} s of decode_ref, quantisation excluded",
            "host_cpus": len(os.sched_getaffinity(0))}


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
            wall, step_ms, kern_ms, _ = time_layers(copies, steps, 5, hip, ops, workloads, torch, args.workgroups,
                                                    args.variant)
            med = statistics.median(step_ms) * 1e3
            gbps = nbytes / (kern_ms[0] * 1e-3) / 1e9
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
    for kl, vl, sk in FORMATS:
        if args.variant in ("mfma_fp8", "packed_heads", "packed_split") and (vl != "heads_dmajor" or
                                                                              (sk or "").startswith("f32_g")):
            continue   # these variants read V d-major only, and no sub-row K scales
        sk = wl.scale_kind if sk is None else sk
        layers = workloads.build_workload(wl, k_layout=kl, v_layout=vl, scale_kind=sk)
        R = args.copies or rotation(layers, wl, np)
        copies = copies_of(layers, wl, R, torch)
        outs = [workloads.decode_layer(l, variant=args.variant).clone() for l in layers]
        if sk in first:
            for j, o in enumerate(outs):
                assert torch.equal(o.view(torch.int16), first[sk][j].view(torch.int16)), \
                    f"{kl}/{sk}: output differs from {sk} in another layout"
        else:
            first[sk] = outs
        _, step_ms, kern_ms, _ = time_layers(copies, args.steps, args.warmup, hip, ops, workloads, torch,
                                             args.workgroups, args.variant)
        rows = []
        for l, km in zip(layers, kern_ms):
            b = workloads.kv_bytes(l)
            rows.append({"name": l.name, "kernel_us_mean": round(km * 1e3, 2), "kv_bytes": b,
                         "kernel_gbps": round(b / (km * 1e-3) / 1e9, 1),
                         "pct_peak": round(100 * b / (km * 1e-3) / 1e9 / PEAK_GBPS, 1)})
        print(json.dumps({"format": {"k_layout": kl, "v_layout": vl, "scale_kind": sk,
                                     "row_bytes": layers[0].row_bytes}, "variant": args.variant,
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
    wl = {w.name: w for w in configs.ALL}[args.workload]
    if args.formats:
        run_formats(args, wl, torch, np, ops, workloads, hip)
        return
    if args.graph:
        run_graph(args, wl, torch, np, ops, workloads, hip)
        return
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

    wall, step_ms, kern_ms, _ = time_layers(copies, args.steps, args.warmup, hip, ops, workloads, torch,
                                            args.workgroups, args.variant)
    layer_bytes = [workloads.kv_bytes(l) for l in layers]
    total_bytes = sum(layer_bytes)
    ms_per_step = wall * 1e3 / args.steps
    value = total_bytes / (wall / args.steps) / 1e9
    dom = int(np.argmax(layer_bytes))
    kern_avg_ms = kern_ms[dom]
    achieved = layer_bytes[dom] / (kern_avg_ms * 1e-3) / 1e9
    traffic = stored_traffic(wl.name)
    us = sorted(x * 1e3 for x in step_ms)
    pct = lambda p: us[min(len(us) - 1, int(p * len(us)))]
    plans = [ops.decode_plan(len(l.lens), l.Hq, l.kd, l.vd, l.max_seq_len, l.window, args.workgroups, args.variant)
             for l in layers]
    rec = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if args.variant != "mfma_fp8" else "fp8 QK (q rounded to e4m3), bf16 PV",
        "data": "synthetic",
        "config": {
            "workload": wl.name, "B": wl.B, "page": wl.P, "seq_lens": f"U[{wl.L_lo},{wl.L_hi}]",
            "kv": "e4m3", "scales": wl.scale_kind,
            "layers": [{"name": l.name, "Hq": l.Hq, "Hkv": l.Hkv, "D": l.D, "window": l.window,
                        "sm_scale": round(l.sm_scale, 6), "kv_bytes": b, "workgroups": p.workgroups,
                        "tile_tokens": p.tile_tokens, "kernel_us_mean": round(km * 1e3, 2),
                        "kernel_gbps": round(b / (km * 1e-3) / 1e9, 1)}
                       for l, b, p, km in zip(layers, layer_bytes, plans, kern_ms)],
            "kv_bytes_per_step": total_bytes, "pool_copies_rotated": R, "parallelism": "single GPU",
        },
        "us_per_call": {"median": round(pct(0.5), 2), "p10": round(pct(0.1), 2), "p90": round(pct(0.9), 2),
                        "note": "GPU time per step between hipEvents (one decode launch per layer; split merges run inside it)"},
        "pct_of_peak": round(100 * value / PEAK_GBPS, 2),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_GBPS, "unit": "GB/s",
                     "frac": round(achieved / PEAK_GBPS, 4), "traffic": traffic,
                     "kernel": f"decode_kernel D={layers[dom].D} ({layers[dom].name})",
                     "kernel_us_mean": round(kern_avg_ms * 1e3, 2), "bytes_per_launch": layer_bytes[dom],
                     "timing": f"hipEvents around {args.steps} back-to-back launches of this layer; mean per launch"},
        "build_s": round(build_s, 1),
    }
    if args.copy_probe:
        # A plain device copy of known size: its counters scale the PMC byte
        # counts, and its rate is a measured streaming ceiling on this machine.
        n = 1 << 30
        a = torch.empty(n, dtype=torch.uint8, device="cuda:0")
        b = torch.empty_like(a)
        ev = hip.events(2)
        stream = torch.cuda.current_stream().cuda_stream
        for _ in range(3):
            b.copy_(a)
        hip.record(ev[0], stream)
        for _ in range(5):
            b.copy_(a)
        hip.record(ev[1], stream)
        ms = hip.elapsed_ms(ev[0], ev[1]) / 5
        hip.destroy(ev)
        rec["copy_probe"] = {"bytes_read": n, "bytes_written": n, "us": round(ms * 1e3, 2),
                             "read_plus_write_gbps": round(2 * n / (ms * 1e-3) / 1e9, 1)}
        del a, b
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
    rec["read_probe"] = {"bytes": 4 << 30, "us": round(ms * 1e3, 2), "gbps": round((4 << 30) / (ms * 1e-3) / 1e9, 1),
                         "kernel": "fp8pa_stream_read over 4 GiB"}
    rec["roofline"]["frac_of_measured_read"] = round(achieved / rec["read_probe"]["gbps"], 4)
    del x
    rec["cpu_baseline"] = None if args.no_cpu_baseline else cpu_baseline(wl, layers, args.cpu_budget)
    # Last, as it rewrites each sequence's last token in the pools.
    fu = time_fused(copies, dom, args.steps, hip, ops, workloads, torch)
    ld = layers[dom]
    span = min(ld.window, ld.max_seq_len) if ld.window > 0 else ld.max_seq_len
    rec["fused_append_decode"] = {
        "layer": ld.name, "us_append_quant_then_decode": round(fu["append_then_decode"], 2),
        "us_append_decode": round(fu["fused"], 2),
        "append_decode_path": "one launch" if span <= 2048 else "append kernel, then decode",
        "timing": f"hipEvents around {args.steps} steps (new token per sequence appended, then decoded); mean per step"}
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
