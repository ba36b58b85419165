#!/usr/bin/env python3
"""Benchmark of the SWA hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]

Prints ONE JSON line.  The headline step is the full-sequence SWA forward on
the prefill workload (B=1, H=Hkv=32, N=8192, W=512, d=128, bf16, tiles
128x64), whose block metadata is built once on the host beforehand (a fixed
pattern reuses its metadata); `value` is useful TFLOP/s = 4*d*(visible pairs)
per step over the wall time of K steps, replayed from a HIP graph that holds
them (the eager per-step wall time is reported beside it).  The same run also
measures, each on its own synthetic workload, the GQA prefill with
per-sequence lengths, the chunked prefill against a ring cache and the ring
decode (KV GB/s), and times the fp64 oracle on a bounded sample on the host
cores.
Inputs are seeded synthetic tensors already resident in HBM.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0      # MI355X HBM3E


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only", default="",
                    help="comma list: prefill,gqa,chunk,decode,bwd,sink,variants")
    ap.add_argument("--calibrate-copy-mib", type=int, default=0,
                    help="only run a plain device-to-device copy of this many MiB, 5 times "
                         "(scale for rocprofv3 FETCH_SIZE / WRITE_SIZE counters)")
    ap.add_argument("--probe-coexec", action="store_true",
                    help="only time the matrix/vector co-execution probe "
                         "(libswa_measure.so) and print its JSON line")
    return ap.parse_args()


def probe_coexec(torch, dev):
    """Times one workgroup of eight waves per CU: matrix-only, vector-only and
    both (two waves per SIMD, one of each kind), for accumulators in AGPRs or
    arch VGPRs and exp2 or FMA vector work; overlap = (t_m + t_v - t_both) /
    min(t_m, t_v), 1 when the shorter work hides entirely under the longer."""
    import ctypes
    lib = ctypes.CDLL(os.path.join(ROOT, "causal_sliding_window_swa_amd", "libswa_measure.so"))
    lib.swa_measure_coexec.argtypes = [ctypes.c_void_p] + [ctypes.c_int] * 6 + [ctypes.c_void_p]
    blocks = torch.cuda.get_device_properties(dev).multi_processor_count
    out = torch.zeros(blocks * 512, device=dev)
    st = torch.cuda.current_stream(dev)

    def run(im, iv, mode, agpr, trans, reps=5):
        call = lambda: lib.swa_measure_coexec(out.data_ptr(), blocks, im, iv, mode, agpr, trans,
                                              ctypes.c_void_p(st.cuda_stream))
        for _ in range(2):
            if call() != 0:
                raise RuntimeError("coexec probe launch failed")
        torch.cuda.synchronize()
        ts = []
        for _ in range(reps):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(st)
            call()
            b.record(st)
            torch.cuda.synchronize()
            ts.append(a.elapsed_time(b))
        return min(ts)

    res = {"workload": "co-execution probe, %d workgroups of 512 threads" % blocks}
    for agpr in (0, 1):
        for trans, iv in ((1, 3200), (0, 8000)):
            t = {m: run(4000, iv, m, agpr, trans) for m in (1, 2, 3)}
            res["acc_%s_%s" % ("agpr" if agpr else "vgpr", "exp2" if trans else "fma")] = {
                "matrix_ms": round(t[1], 4), "vector_ms": round(t[2], 4), "both_ms": round(t[3], 4),
                "overlap": round((t[1] + t[2] - t[3]) / min(t[1], t[2]), 3)}
    print(json.dumps(res), flush=True)


def src_digest(*names):
    """sha256 prefix of the kernel sources with comments and whitespace
    removed: the code the counters in profiles/hbm_traffic.json were taken
    on (a comment edit keeps the record valid, a code edit voids it)."""
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "causal_sliding_window_swa_amd", "csrc", n)) as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def counters_for(kernel_key, digest):
    """HBM traffic per launch measured by rocprofv3 counters, if the record in
    profiles/ was taken on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", "hbm_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f).get(kernel_key)
    if not rec or rec.get("source_digest") != digest:
        return None
    return rec.get("bytes_per_launch")


def counter_summary(name, digest):
    """The rocprofv3 record of this kernel in profiles/counters_<name>.json
    (kernel trace and counter passes of one run), if it was taken on the
    current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", "counters_%s.json" % name)
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("source_digest") != digest:
        return None
    d = rec["derived"]
    return {"record": "profiles/counters_%s.json" % name,
            "trace_mean_ms": rec["trace"]["mean_ms"],
            "frac_from_trace": rec["frac_of_bf16_peak_from_trace"],
            "mfma_busy": d["mfma_busy_frac_of_simd_cycles"],
            "valu_coexec_of_mfma_busy": d["valu_coexec_frac_of_mfma_busy"],
            "l2_hit": d["l2_hit_frac"]}


def main():
    args = parse()
    if args.gpus != 1:
        sys.stderr.write("bench.py measures one GPU only; --gpus %d is not supported "
                         "(each request and KV head is an independent unit, so a sharded run "
                         "would need no communication; no multi-GPU path is built)\n"
                         % args.gpus)
        sys.exit(2)
    import numpy as np
    import torch

    sys.path.insert(0, ROOT)
    import causal_sliding_window_swa_amd as swa
    from causal_sliding_window_swa_amd import synth

    only = set(args.only.split(",")) if args.only else {"prefill", "gqa", "chunk", "decode",
                                                         "bwd", "sink", "variants"}
    dev = torch.device("cuda:0")
    if args.probe_coexec:
        probe_coexec(torch, dev)
        return
    if args.calibrate_copy_mib:
        n = args.calibrate_copy_mib << 20
        src = torch.ones(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_per_launch": n}), flush=True)
        return
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)
    K, WU = args.steps, args.warmup
    log = lambda *a: print(*a, file=sys.stderr, flush=True)

    SETTLE_S = 1.0
    WARM_S = 2.0  # load before the first timed region of the run
    last_events = []  # per-launch event times (ms) of the latest timed() call

    def timed(fn, steps, warmup, reset=None, graph=True):
        """(ms per step, event-timed ms per step, eager wall ms per step).

        The first figure is the host wall time of one replay of a HIP graph
        holding the `steps` steps, bracketed by device synchronisations, so
        that the host's per-launch cost between steps is not counted; the
        second is the same replay timed by HIP events recorded on the launch
        stream around it (the GPU time of the timed region over `steps`,
        which is what a kernel trace's mean duration of a one-kernel step
        reproduces).  The GPU lowers its clocks within milliseconds of going
        idle and needs tens of milliseconds of load to raise them again
        (graph capture and instantiation leave it idle), so after the
        `warmup` eager steps and the capture the graph is replayed, untimed,
        for SETTLE_S seconds before the timed replay; a pass with one event
        pair per step (last_events: their spread) and an eager pass follow
        while the GPU is still busy.  graph=False (steps with host work): the
        eager wall time only."""
        def step():
            if reset:
                reset()
            fn()
        for _ in range(warmup):
            step()
        torch.cuda.synchronize()
        if not graph:
            t0 = time.perf_counter()
            for _ in range(steps):
                step()
            torch.cuda.synchronize()
            wall = (time.perf_counter() - t0) * 1e3 / steps
            return wall, wall, wall
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(steps):
                step()
        g.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < SETTLE_S:
            g.replay()
            torch.cuda.synchronize()
        r0, r1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        r0.record(stream)
        g.replay()
        r1.record(stream)
        torch.cuda.synchronize()
        gms = (time.perf_counter() - t0) * 1e3 / steps
        region = r0.elapsed_time(r1) / steps
        del g
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(steps)]
        for s, e in evs:
            if reset:
                reset()
            s.record(stream)
            fn()
            e.record(stream)
        torch.cuda.synchronize()
        last_events[:] = sorted(s.elapsed_time(e) for s, e in evs)
        t0 = time.perf_counter()
        for _ in range(steps):
            step()
        torch.cuda.synchronize()
        wall = (time.perf_counter() - t0) * 1e3 / steps
        return gms, region, wall

    out = {}

    # ---------------- prefill workload (headline) ----------------
    inp = synth.make("prefill")
    B, H, N, d = inp["q"].shape
    # tiles: 128x128 for the headline (no sinks: the 128-key tile kernel then
    # spreads its loads like the 64-key one and has half the metadata entries);
    # 128x64 for the other workloads, the backward and the sink variant
    W, tq, tk, tk_pf = 512, 128, 64, 128
    t0 = time.perf_counter()
    meta = swa.swa_blockmask_build(B, N, N, W, tq, tk_pf)
    t_meta = (time.perf_counter() - t0) * 1e3
    swa.meta_to_device(meta, dev)  # first transfer pays one-time runtime set-up
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    md = swa.meta_to_device(meta, dev)
    torch.cuda.synchronize()
    t_h2d = (time.perf_counter() - t0) * 1e3
    q, k, v = (inp[x].to(dev) for x in ("q", "k", "v"))
    o = torch.empty_like(q)
    flops = 4.0 * d * meta["valid_pairs"] * H
    fwd = lambda: swa.swa_fwd(q, k, v, o, W, md)
    # two seconds of the headline step before the first timed region of the
    # run, so that it starts from steady clocks like the regions after it
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < WARM_S:
        for _ in range(20):
            fwd()
        torch.cuda.synchronize()
    wall_ms, ev_ms, eager_ms = timed(fwd, K, WU)
    ev_median, ev_min = last_events[K // 2], last_events[0]
    log("prefill: graph %.4f ms/step, eager %.4f ms/step, event-timed region %.4f ms/step, "
        "per-launch events median %.4f ms" % (wall_ms, eager_ms, ev_ms, ev_median))
    # end to end with the metadata rebuilt and copied each step
    def fwd_with_meta():
        m = swa.swa_blockmask_build(B, N, N, W, tq, tk_pf)
        mdd = swa.meta_to_device(m, dev)
        swa.swa_fwd(q, k, v, o, W, mdd)
    e2e_ms, _, _ = timed(fwd_with_meta, max(5, K // 5), 2, graph=False)
    prefill = dict(wall_ms=wall_ms, kernel_ms=ev_ms, kernel_ms_median=ev_median,
                   kernel_ms_min=ev_min, eager_ms=eager_ms, flops=flops,
                   meta_ms=t_meta, meta_h2d_ms=t_h2d, e2e_ms=e2e_ms, stats=meta)
    out["prefill"] = prefill

    # ---------------- prefill variants: 64-row tiles, cold caches, W = N -------------
    if "variants" in only:
        m64 = swa.swa_blockmask_build(B, N, N, W, 64, 64)
        md64 = swa.meta_to_device(m64, dev)
        w64, e64, _ = timed(lambda: swa.swa_fwd(q, k, v, o, W, md64), K, WU)
        prefill["tile64"] = dict(wall_ms=w64, kernel_ms=e64, n_live=m64["n_live"],
                                 covered=m64["covered_coords"])
        log("prefill tile 64: graph %.4f ms/step, event %.4f ms" % (w64, e64))
        # 64-key metadata tiles (the headline streams its 128-key tiles as
        # 64-key halves; here every 64-key tile has its own metadata entry)
        m128 = swa.swa_blockmask_build(B, N, N, W, 128, 64)
        md128 = swa.meta_to_device(m128, dev)
        w128, e128, _ = timed(lambda: swa.swa_fwd(q, k, v, o, W, md128), K, WU)
        prefill["tile128x64"] = dict(wall_ms=w128, kernel_ms=e128, n_live=m128["n_live"],
                                     covered=m128["covered_coords"])
        log("prefill tiles 128x64: graph %.4f ms/step, event %.4f ms" % (w128, e128))
        # cold caches: 1 GiB written between launches evicts L2 and the
        # 256 MB Infinity Cache; only the kernel is inside the events
        flush = torch.empty(1 << 28, dtype=torch.float32, device=dev)
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(K)]
        for i, (s_, e_) in enumerate(evs):
            flush.fill_(float(i))
            s_.record(stream)
            fwd()
            e_.record(stream)
        torch.cuda.synchronize()
        cold = sorted(s_.elapsed_time(e_) for s_, e_ in evs)
        prefill["cold"] = dict(median_ms=cold[K // 2], min_ms=cold[0])
        del flush
        log("prefill cold: median %.4f ms, min %.4f ms" % (cold[K // 2], cold[0]))
        # skipping check: W = N is dense causal, with 8.26x the visible pairs
        mden = swa.swa_blockmask_build(B, N, N, N, tq, tk_pf)
        mdd = swa.meta_to_device(mden, dev)
        _, eden, _ = timed(lambda: swa.swa_fwd(q, k, v, o, N, mdd), max(3, K // 10), 2)
        prefill["dense"] = dict(kernel_ms=eden, valid_pairs=mden["valid_pairs"])
        log("prefill at W=N: event %.4f ms" % eden)
        del mdd, md64, md128

    # ---------------- backward on the prefill workload -------------
    if "bwd" in only:
        gen = torch.Generator(device="cpu").manual_seed(1 + 7919)
        dout = (torch.randn(q.shape, generator=gen) * 0.5).to(torch.bfloat16).to(dev)
        lse = torch.empty((B, H, N), dtype=torch.float32, device=dev)
        mdb = swa.meta_to_device(swa.swa_blockmask_build(B, N, N, W, tq, tk), dev)  # 64-key tiles
        swa.swa_fwd(q, k, v, o, W, mdb, lse=lse)
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        wsb = torch.empty(swa.swa_bwd_workspace_size(B, H, N) // 4, dtype=torch.float32,
                          device=dev)
        fb = lambda: swa.swa_bwd(q, k, v, o, dout, lse, dq, dk, dv, wsb, W, mdb)
        wb, eb, _ = timed(fb, max(3, K // 10), 1)
        out["bwd"] = dict(wall_ms=wb, kernel_ms=eb, flops=2.5 * flops)
        log("bwd: wall %.3f ms, event %.3f ms" % (wb, eb))
        del dout, lse, dq, dk, dv, wsb, mdb

    # ---------------- prefill with 4 attention sinks -------------
    if "sink" in only:
        ms = swa.swa_blockmask_build(B, N, N, W, tq, tk, n_sink=4)
        mds = swa.meta_to_device(ms, dev)
        fs = lambda: swa.swa_fwd(q, k, v, o, W, mds)
        ws_, es_, _ = timed(fs, K, WU)
        out["prefill_sink"] = dict(wall_ms=ws_, kernel_ms=es_,
                                   flops=4.0 * d * ms["valid_pairs"] * H)
        log("prefill sink: wall %.4f ms, event %.4f ms" % (ws_, es_))
    del inp

    # ---------------- GQA prefill with per-sequence lengths -------------
    if "gqa" in only:
        inp = synth.make("prefill_gqa")
        B3, H3, N3, d3 = inp["q"].shape
        L = inp["q_len"].numpy()
        m3 = swa.swa_blockmask_build(B3, N3, N3, 4096, tq, tk, q_len=L, k_len=L)
        md3 = swa.meta_to_device(m3, dev)
        q3, k3, v3 = (inp[x].to(dev) for x in ("q", "k", "v"))
        ql3 = inp["q_len"].to(dev)
        o3 = torch.empty_like(q3)
        del inp
        f3 = lambda: swa.swa_fwd(q3, k3, v3, o3, 4096, md3, q_len=ql3)
        w3, e3, _ = timed(f3, max(3, K // 10), 2)
        out["gqa"] = dict(wall_ms=w3, kernel_ms=e3, flops=4.0 * d3 * m3["valid_pairs"] * H3)
        log("gqa: wall %.3f ms, event %.3f ms" % (w3, e3))
        # 256-row query tiles: the eight-wave kernel whose wave groups
        # alternate matrix and vector work (swa_pp_bf16.hip)
        m3b = swa.swa_blockmask_build(B3, N3, N3, 4096, 256, 64, q_len=L, k_len=L)
        md3b = swa.meta_to_device(m3b, dev)
        f3b = lambda: swa.swa_fwd(q3, k3, v3, o3, 4096, md3b, q_len=ql3)
        w3b, e3b, _ = timed(f3b, max(3, K // 10), 2)
        out["gqa_tile256"] = dict(wall_ms=w3b, kernel_ms=e3b, flops=out["gqa"]["flops"],
                                  live=len(m3b["col"]))
        log("gqa tiles 256x64: wall %.3f ms, event %.3f ms" % (w3b, e3b))
        del md3b
        # the same sequences packed token-major without padding (swa_fwd_varlen)
        lens = [int(x) for x in L]
        pk = [torch.cat([t[b, :, :n].transpose(0, 1) for b, n in enumerate(lens)]).contiguous()
              for t in (q3, k3, v3)]
        del q3, k3, v3, o3
        cu = torch.tensor([0] + list(np.cumsum(lens)), dtype=torch.int32, device=dev)
        op = torch.empty_like(pk[0])
        f3p = lambda: swa.swa_fwd_varlen(pk[0], pk[1], pk[2], op, 4096, md3, cu)
        w3p, e3p, _ = timed(f3p, max(3, K // 10), 2)
        out["gqa_packed"] = dict(wall_ms=w3p, kernel_ms=e3p, flops=out["gqa"]["flops"],
                                 tokens=int(sum(lens)))
        log("gqa packed: wall %.3f ms, event %.3f ms" % (w3p, e3p))
        if "bwd" in only:
            # its backward (swa_bwd_varlen), for a seeded output gradient
            gen = torch.Generator(device="cpu").manual_seed(3 + 7919)
            dop = (torch.randn(op.shape, generator=gen) * 0.5).to(torch.bfloat16).to(dev)
            lsp = torch.empty(op.shape[:2], dtype=torch.float32, device=dev)
            swa.swa_fwd_varlen(pk[0], pk[1], pk[2], op, 4096, md3, cu, lse=lsp)
            gq, gk, gv = (torch.empty_like(t) for t in pk)
            wsp = torch.empty(swa.swa_bwd_workspace_size(1, H3, op.shape[0]) // 4,
                              dtype=torch.float32, device=dev)
            fbp = lambda: swa.swa_bwd_varlen(pk[0], pk[1], pk[2], op, dop, lsp, gq, gk, gv, wsp,
                                             4096, md3, cu)
            wbp, ebp, _ = timed(fbp, 3, 1)
            out["gqa_bwd_packed"] = dict(wall_ms=wbp, kernel_ms=ebp,
                                         flops=2.5 * out["gqa"]["flops"], tokens=int(sum(lens)))
            log("gqa packed bwd: wall %.3f ms, event %.3f ms" % (wbp, ebp))
            del dop, lsp, gq, gk, gv, wsp
        del pk, op

    # ---------------- chunked prefill against the ring -------------
    if "chunk" in only:
        inp = synth.make("chunk")
        B4, H4, Tq, d4 = inp["q"].shape
        W4 = 4096
        p = inp["next_pos"].numpy()
        inp_rs, inp_cl = inp["ring_start"].numpy(), inp["cache_len"].numpy()
        m4 = swa.swa_blockmask_build(B4, Tq, Tq, W4, tq, tk, q_start=p, k_start=p, W_ring=W4,
                                     ring_start=inp_rs, cache_len=inp_cl, next_pos=p)
        md4 = swa.meta_to_device(m4, dev)
        dv = {x: inp[x].to(dev) for x in inp}
        # the ring state as three rows of one tensor, so that a step's reset is
        # one small copy
        st3 = torch.stack([dv[x] for x in ("ring_start", "cache_len", "next_pos")]).contiguous()
        for i, x in enumerate(("ring_start", "cache_len", "next_pos")):
            dv[x] = st3[i]
        state0 = {x: dv[x].clone() for x in ("ring_start", "cache_len", "next_pos")}
        st3_0 = st3.clone()
        o4 = torch.empty_like(dv["q"])
        del inp

        def reset4():  # same ring state each step, so the metadata stays valid
            st3.copy_(st3_0)

        f4 = lambda: swa.swa_prefill_chunk(dv["q"], dv["k_new"], dv["v_new"], dv["k_cache"],
                                           dv["v_cache"], dv["ring_start"], dv["cache_len"],
                                           dv["next_pos"], o4, W4, md4)
        w4, e4, _ = timed(f4, max(5, K // 5), 2, reset=reset4)
        out["chunk"] = dict(wall_ms=w4, kernel_ms=e4, flops=4.0 * d4 * m4["valid_pairs"] * H4,
                            keys_touched_per_request=m4["keys_touched"] // B4)
        log("chunk: wall %.3f ms, event %.3f ms" % (w4, e4))
        # 256-row query tiles (swa_pp_bf16.hip)
        m4b = swa.swa_blockmask_build(B4, Tq, Tq, W4, 256, 64, q_start=p, k_start=p, W_ring=W4,
                                      ring_start=inp_rs, cache_len=inp_cl, next_pos=p)
        md4b = swa.meta_to_device(m4b, dev)
        f4b = lambda: swa.swa_prefill_chunk(dv["q"], dv["k_new"], dv["v_new"], dv["k_cache"],
                                            dv["v_cache"], dv["ring_start"], dv["cache_len"],
                                            dv["next_pos"], o4, W4, md4b)
        w4b, e4b, _ = timed(f4b, max(5, K // 5), 2, reset=reset4)
        out["chunk_tile256"] = dict(wall_ms=w4b, kernel_ms=e4b, flops=out["chunk"]["flops"],
                                    live=len(m4b["col"]))
        log("chunk tiles 256x64: wall %.3f ms, event %.3f ms" % (w4b, e4b))
        # a real stream of chunk steps: the ring moves every step, so the
        # block metadata is rebuilt before each one (the figure above resets
        # the ring state to reuse one build).  (a) on the device, in stream
        # order, from the device ring state; (b) on the host, from a copy of
        # the ring state, then copied to the device
        for x in state0:
            dv[x].copy_(state0[x])
        mdev = swa.chunk_meta_buffers(B4, Tq, W4, tq, tk, dev, stats=False)

        def f4d():
            swa.swa_chunk_blockmask_dev(mdev, dv["ring_start"], dv["cache_len"], dv["next_pos"])
            swa.swa_prefill_chunk(dv["q"], dv["k_new"], dv["v_new"], dv["k_cache"],
                                  dv["v_cache"], dv["ring_start"], dv["cache_len"],
                                  dv["next_pos"], o4, W4, mdev)
        w4d, e4d, _ = timed(f4d, max(5, K // 5), 2)
        out["chunk_stream_dev"] = dict(wall_ms=w4d, kernel_ms=e4d)
        log("chunk stream, device metadata: wall %.3f ms, event %.3f ms" % (w4d, e4d))

        def f4h():
            rs_h, cl_h, np_h = (dv[x].cpu().numpy() for x in ("ring_start", "cache_len",
                                                             "next_pos"))
            mh = swa.swa_blockmask_build(B4, Tq, Tq, W4, tq, tk, q_start=np_h, k_start=np_h,
                                         W_ring=W4, ring_start=rs_h, cache_len=cl_h,
                                         next_pos=np_h)
            swa.swa_prefill_chunk(dv["q"], dv["k_new"], dv["v_new"], dv["k_cache"],
                                  dv["v_cache"], dv["ring_start"], dv["cache_len"],
                                  dv["next_pos"], o4, W4, swa.meta_to_device(mh, dev))
        w4h, _, _ = timed(f4h, max(5, K // 5), 2, graph=False)
        out["chunk_stream_host"] = dict(wall_ms=w4h)
        log("chunk stream, host metadata: wall %.3f ms" % w4h)
        for x in state0:
            dv[x].copy_(state0[x])
        if "sink" in only:  # 4 sinks from a sink cache, far behind every window
            m4s = swa.swa_blockmask_build(B4, Tq, Tq, W4, tq, tk, q_start=p, k_start=p,
                                          W_ring=W4, ring_start=state0["ring_start"].cpu().numpy(),
                                          cache_len=state0["cache_len"].cpu().numpy(), next_pos=p,
                                          n_sink=4)
            md4s = swa.meta_to_device(m4s, dev)
            sk4 = torch.zeros(B4, dv["k_new"].shape[1], 4, d4, dtype=dv["q"].dtype, device=dev)
            sv4 = torch.zeros_like(sk4)
            f4s = lambda: swa.swa_prefill_chunk(dv["q"], dv["k_new"], dv["v_new"],
                                                dv["k_cache"], dv["v_cache"], dv["ring_start"],
                                                dv["cache_len"], dv["next_pos"], o4, W4, md4s,
                                                sink_k=sk4, sink_v=sv4)
            w4s, e4s, _ = timed(f4s, max(5, K // 5), 2, reset=reset4)
            out["chunk_sink"] = dict(wall_ms=w4s, kernel_ms=e4s,
                                     flops=4.0 * d4 * m4s["valid_pairs"] * H4)
            log("chunk sink: wall %.3f ms, event %.3f ms" % (w4s, e4s))
        del dv, o4

    # ---------------- ring decode -------------
    if "decode" in only:
        inp = synth.make("decode")
        B5, H5, d5 = inp["q"].shape
        Hkv5 = inp["k_new"].shape[1]
        W5 = 4096
        dv = {x: inp[x].to(dev) for x in inp}
        o5 = torch.empty_like(dv["q"])
        ws = torch.empty(swa.swa_decode_workspace_size(B5, H5, d5, W5) // 4 + 4,
                         dtype=torch.float32, device=dev)
        del inp
        f5 = lambda: swa.swa_decode(dv["q"], dv["k_new"], dv["v_new"], dv["k_cache"],
                                    dv["v_cache"], dv["ring_start"], dv["cache_len"],
                                    dv["next_pos"], o5, ws, W5)
        w5, e5, we5 = timed(f5, max(10, K), 5)
        kv_bytes = 2.0 * B5 * Hkv5 * W5 * d5 * 2
        out["decode"] = dict(wall_ms=w5, kernel_ms=e5, eager_ms=we5, kv_bytes=kv_bytes)
        log("decode: wall %.4f ms, event %.4f ms" % (w5, e5))
        if "sink" in only:  # 4 sinks, all outside the window at these positions
            sk = torch.zeros(B5, Hkv5, 4, d5, dtype=dv["k_cache"].dtype, device=dev)
            sv = torch.zeros_like(sk)
            f6 = lambda: swa.swa_decode(dv["q"], dv["k_new"], dv["v_new"], dv["k_cache"],
                                        dv["v_cache"], dv["ring_start"], dv["cache_len"],
                                        dv["next_pos"], o5, ws, W5, n_sink=4, sink_k=sk,
                                        sink_v=sv)
            w6, e6, _ = timed(f6, max(10, K), 5)
            out["decode_sink"] = dict(wall_ms=w6, kernel_ms=e6,
                                      kv_bytes=kv_bytes + 2.0 * B5 * Hkv5 * 4 * d5 * 2)
            log("decode sink: wall %.4f ms, event %.4f ms" % (w6, e6))
        del dv

    # ---------------- HBM read ceiling of this GPU -------------
    # a plain streaming read (libswa_measure.so, measurement support only) of
    # as many bytes as the decode step reads, at a few grid sizes; the best
    # is the practical ceiling beside the 8 TB/s specification
    if "decode" in only:
        import ctypes
        mlib = ctypes.CDLL(os.path.join(ROOT, "causal_sliding_window_swa_amd",
                                        "libswa_measure.so"))
        mlib.swa_measure_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t,
                                                 ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p]
        nbytes = 1 << 30
        buf = torch.ones(nbytes // 2, dtype=torch.bfloat16, device=dev)
        sink = torch.empty(1 << 16, dtype=torch.int32, device=dev)
        best = None
        for blocks in (2048, 8192, 16384, 32768, 65536):
            fr = lambda: mlib.swa_measure_stream_read(
                ctypes.c_void_p(buf.data_ptr()), ctypes.c_size_t(nbytes),
                ctypes.c_void_p(sink.data_ptr()), blocks,
                ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream))
            _, ms_r, _ = timed(fr, 20, 3)
            gbs_r = nbytes / (ms_r * 1e-3) / 1e9
            if best is None or gbs_r > best[1]:
                best = (blocks, gbs_r, ms_r)
        out["hbm_stream"] = dict(bytes=nbytes, blocks=best[0], GB_per_s=best[1], ms=best[2])
        log("hbm stream read: %.1f GB/s (%d blocks)" % (best[1], best[0]))
        del buf, sink

    # ---------------- oracle on the host cores -------------
    # the whole prefill workload in fp64, repeated until about 10 s of work
    cpu = None
    if not args.no_cpu_baseline:
        sys.path.insert(0, ROOT)
        import oracle
        inp = synth.make("prefill")
        qs = inp["q"].float().numpy().astype(np.float64)
        ks = inp["k"].float().numpy().astype(np.float64)
        vs = inp["v"].float().numpy().astype(np.float64)
        del inp
        reps, sec = 0, 0.0
        while sec < 10.0 and reps < 50:
            t0 = time.perf_counter()
            oracle.fwd(qs, ks, vs, 512, 1 / math.sqrt(128))
            sec += time.perf_counter() - t0
            reps += 1
        sample_flops = 4.0 * 128 * meta["valid_pairs"] * 32 * reps
        cpu = {"value": round(sample_flops / sec / 1e12, 5), "unit": "TFLOP/s",
               "cores": oracle.num_threads(), "kind": "oracle",
               "sample": "the whole prefill workload (B=1, H=32, N=8192, W=512, d=128) "
                         "in fp64, %d passes, %.1f s" % (reps, sec)}
        log("oracle: %d passes in %.2f s" % (reps, sec))
        # the same at one thread, on 2 of the 32 heads
        nthr = oracle.num_threads()
        oracle.set_num_threads(1)
        q2, k2, v2 = (x[:, :2].copy() for x in (qs, ks, vs))
        reps1, sec1 = 0, 0.0
        while sec1 < 5.0 and reps1 < 20:
            t0 = time.perf_counter()
            oracle.fwd(q2, k2, v2, 512, 1 / math.sqrt(128))
            sec1 += time.perf_counter() - t0
            reps1 += 1
        oracle.set_num_threads(nthr)
        cpu["single_thread"] = {
            "value": round(4.0 * 128 * meta["valid_pairs"] * 2 * reps1 / sec1 / 1e12, 6),
            "unit": "TFLOP/s", "cores": 1,
            "sample": "2 of the 32 heads of the prefill workload in fp64, %d passes, %.1f s"
                      % (reps1, sec1)}
        log("oracle, one thread: %d passes in %.2f s" % (reps1, sec1))

    pf = out["prefill"]
    value = pf["flops"] / (pf["wall_ms"] * 1e-3) / 1e12
    achieved = pf["flops"] / (pf["kernel_ms"] * 1e-3) / 1e12
    tile_digest = src_digest("swa_tile_bf16.hip")
    line = {
        "metric": "SWA prefill useful TFLOP/s + decode KV GB/s, each as % of MI355X peak",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": WU,
        "ms_per_step": round(pf["wall_ms"], 5),
        "settle_s_before_timing": SETTLE_S,
        "warm_s_before_first_timing": WARM_S,
        "eager_ms_per_step": round(pf["eager_ms"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "prefill B=1 H=32 Hkv=32 N=8192 W=512 d=128 bf16, "
                               "tiles 128x128, metadata prebuilt",
                   "global_batch": 1, "seq_len": 8192, "window": 512,
                   "parallelism": "single GPU"},
        "pct_of_peak": round(100.0 * value / PEAK_BF16_TFLOPS, 2),
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2),
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": counters_for("swa_fwd_prefill", tile_digest),
                     "kernel": "swa::tile_kernel<0,128,4,false,2,false> (swa_fwd)",
                     "kernel_ms": round(pf["kernel_ms"], 5),
                     "kernel_ms_timing": "HIP events on the launch stream around the timed "
                                         "graph replay of the K steps, divided by K",
                     "per_launch_event_ms_median": round(pf["kernel_ms_median"], 5),
                     "per_launch_event_ms_min": round(pf["kernel_ms_min"], 5),
                     "counters": counter_summary("prefill", tile_digest)},
        "metadata": {"build_ms": round(pf["meta_ms"], 4), "h2d_ms": round(pf["meta_h2d_ms"], 4),
                     "e2e_ms_per_step_with_build": round(pf["e2e_ms"], 4),
                     "e2e_TFLOPs_with_build": round(pf["flops"] / (pf["e2e_ms"] * 1e-3) / 1e12,
                                                    2),
                     "valid_pairs": pf["stats"]["valid_pairs"],
                     "live_blocks": pf["stats"]["n_live"],
                     "covered_coords": pf["stats"]["covered_coords"]},
        "cpu_baseline": cpu,
    }
    # the fraction of the computed tile area that holds visible pairs
    line["roofline"]["useful_fraction_of_covered"] = round(
        pf["stats"]["valid_pairs"] / pf["stats"]["covered_coords"], 4)
    # the same launch against the HBM roofline: Q, K, V, O once
    alg_bytes = 4.0 * B * H * N * d * 2
    line["prefill_hbm"] = {"algorithmic_bytes": int(alg_bytes),
                           "GB_per_s": round(alg_bytes / (pf["kernel_ms"] * 1e-3) / 1e9, 1),
                           "pct_of_peak": round(100 * alg_bytes / (pf["kernel_ms"] * 1e-3) /
                                                1e9 / PEAK_HBM_GBS, 2)}
    if "tile64" in pf:
        t64 = pf["tile64"]
        line["prefill_tile64"] = {
            "workload": "prefill workload with 64x64 tiles (%d live tiles)" % t64["n_live"],
            "TFLOP_per_s": round(pf["flops"] / (t64["wall_ms"] * 1e-3) / 1e12, 2),
            "kernel_TFLOP_per_s": round(pf["flops"] / (t64["kernel_ms"] * 1e-3) / 1e12, 2),
            "ms_per_step": round(t64["wall_ms"], 5),
            "useful_fraction_of_covered": round(pf["stats"]["valid_pairs"] / t64["covered"], 4)}
    if "tile128x64" in pf:
        t128 = pf["tile128x64"]
        line["prefill_tile128x64"] = {
            "workload": "prefill workload with 128x64 tiles (%d live tiles)" % t128["n_live"],
            "TFLOP_per_s": round(pf["flops"] / (t128["wall_ms"] * 1e-3) / 1e12, 2),
            "kernel_TFLOP_per_s": round(pf["flops"] / (t128["kernel_ms"] * 1e-3) / 1e12, 2),
            "ms_per_step": round(t128["wall_ms"], 5),
            "useful_fraction_of_covered": round(pf["stats"]["valid_pairs"] / t128["covered"],
                                                4)}
    if "cold" in pf:
        line["prefill_cold_caches"] = {
            "workload": "prefill workload, 1 GiB written between launches (L2 and Infinity "
                        "Cache evicted)",
            "median_ms": round(pf["cold"]["median_ms"], 5),
            "min_ms": round(pf["cold"]["min_ms"], 5),
            "TFLOP_per_s": round(pf["flops"] / (pf["cold"]["median_ms"] * 1e-3) / 1e12, 2)}
    if "dense" in pf:
        dn = pf["dense"]
        line["skip_check"] = {
            "workload": "prefill workload at W = N (dense causal)",
            "kernel_ms": round(dn["kernel_ms"], 4),
            "time_ratio": round(dn["kernel_ms"] / pf["kernel_ms"], 2),
            "pair_ratio": round(dn["valid_pairs"] / pf["stats"]["valid_pairs"], 2)}
    if "decode" in out:
        dd = out["decode"]
        gbs = dd["kv_bytes"] / (dd["wall_ms"] * 1e-3) / 1e9
        gbs_k = dd["kv_bytes"] / (dd["kernel_ms"] * 1e-3) / 1e9
        line["decode"] = {"workload": "decode B=64 H=32 Hkv=8 W=4096 d=128 bf16, full rings",
                          "GB_per_s": round(gbs, 1),
                          "pct_of_peak": round(100 * gbs / PEAK_HBM_GBS, 2),
                          "ms_per_step": round(dd["wall_ms"], 5),
                          "eager_ms_per_step": round(dd["eager_ms"], 5),
                          "roofline": {"bound": "hbm", "achieved": round(gbs_k, 1),
                                       "peak": PEAK_HBM_GBS, "unit": "GB/s",
                                       "frac": round(gbs_k / PEAK_HBM_GBS, 4),
                                       "traffic": counters_for(
                                           "swa_decode", src_digest("swa_decode_bf16.hip")),
                                       "kernel_ms": round(dd["kernel_ms"], 5),
                                       "kernels": "split + combine"}}
    if "hbm_stream" in out:
        hs = out["hbm_stream"]
        line["hbm_stream"] = {"workload": "plain streaming read of 1 GiB (one pass, 16-byte "
                                          "loads, %d workgroups of 256)" % hs["blocks"],
                              "GB_per_s": round(hs["GB_per_s"], 1),
                              "pct_of_peak": round(100 * hs["GB_per_s"] / PEAK_HBM_GBS, 2)}
        if "decode" in line:
            line["decode"]["pct_of_stream_read"] = round(
                100 * line["decode"]["roofline"]["achieved"] / hs["GB_per_s"], 2)
    if "prefill_sink" in out:
        ps = out["prefill_sink"]
        t = ps["flops"] / (ps["wall_ms"] * 1e-3) / 1e12
        line["prefill_sink"] = {"workload": "prefill workload with 4 attention sinks",
                                "TFLOP_per_s": round(t, 2),
                                "pct_of_peak": round(100 * t / PEAK_BF16_TFLOPS, 2),
                                "ms_per_step": round(ps["wall_ms"], 5)}
    if "decode_sink" in out:
        ds = out["decode_sink"]
        gbs = ds["kv_bytes"] / (ds["wall_ms"] * 1e-3) / 1e9
        line["decode_sink"] = {"workload": "decode workload with 4 attention sinks",
                               "GB_per_s": round(gbs, 1),
                               "pct_of_peak": round(100 * gbs / PEAK_HBM_GBS, 2),
                               "ms_per_step": round(ds["wall_ms"], 5)}
    if "bwd" in out:
        bb = out["bwd"]
        t = bb["flops"] / (bb["wall_ms"] * 1e-3) / 1e12
        line["backward"] = {"workload": "backward of the prefill workload (dq, dk, dv), "
                                        "useful FLOPs = 2.5 x forward = 10 d (visible pairs)",
                            "TFLOP_per_s": round(t, 2),
                            "pct_of_peak": round(100 * t / PEAK_BF16_TFLOPS, 2),
                            "ms_per_step": round(bb["wall_ms"], 4)}
    if "gqa" in out:
        g3 = out["gqa"]
        t = g3["flops"] / (g3["wall_ms"] * 1e-3) / 1e12
        line["prefill_gqa"] = {"workload": "prefill B=4 H=32 Hkv=8 N=32768 W=4096 d=128 bf16, "
                                           "lengths U[8192,32768]",
                               "TFLOP_per_s": round(t, 2),
                               "pct_of_peak": round(100 * t / PEAK_BF16_TFLOPS, 2),
                               "ms_per_step": round(g3["wall_ms"], 4),
                               "kernel_ms": round(g3["kernel_ms"], 4),
                               "useful_GFLOP": round(g3["flops"] / 1e9, 3)}
    if "gqa_tile256" in out:
        g4 = out["gqa_tile256"]
        t = g4["flops"] / (g4["wall_ms"] * 1e-3) / 1e12
        line["prefill_gqa_tile256"] = {"workload": "the GQA workload with 256x64 tiles (%d live "
                                                   "tiles; one eight-wave workgroup per query "
                                                   "tile, two wave groups alternating matrix "
                                                   "and vector work)" % g4["live"],
                                       "TFLOP_per_s": round(t, 2),
                                       "pct_of_peak": round(100 * t / PEAK_BF16_TFLOPS, 2),
                                       "ms_per_step": round(g4["wall_ms"], 4),
                                       "kernel_ms": round(g4["kernel_ms"], 4),
                                       "counters": counter_summary(
                                           "gqa_tile256", src_digest("swa_pp_bf16.hip"))}
    if "gqa_packed" in out:
        gp = out["gqa_packed"]
        t = gp["flops"] / (gp["wall_ms"] * 1e-3) / 1e12
        line["prefill_gqa_packed"] = {"workload": "the GQA workload's sequences packed "
                                                  "token-major (cu_seqlens, %d tokens, no "
                                                  "padding)" % gp["tokens"],
                                      "TFLOP_per_s": round(t, 2),
                                      "pct_of_peak": round(100 * t / PEAK_BF16_TFLOPS, 2),
                                      "ms_per_step": round(gp["wall_ms"], 4),
                                      "kernel_ms": round(gp["kernel_ms"], 4),
                                      "useful_GFLOP": round(gp["flops"] / 1e9, 3)}
    if "gqa_bwd_packed" in out:
        gb = out["gqa_bwd_packed"]
        t = gb["flops"] / (gb["wall_ms"] * 1e-3) / 1e12
        line["backward_gqa_packed"] = {"workload": "backward of the packed GQA workload "
                                                   "(swa_bwd_varlen, %d tokens), useful FLOPs "
                                                   "= 2.5 x forward" % gb["tokens"],
                                       "TFLOP_per_s": round(t, 2),
                                       "pct_of_peak": round(100 * t / PEAK_BF16_TFLOPS, 2),
                                       "ms_per_step": round(gb["wall_ms"], 4)}
    if "chunk_tile256" in out:
        c5 = out["chunk_tile256"]
        t = c5["flops"] / (c5["wall_ms"] * 1e-3) / 1e12
        line["chunk_tile256"] = {"workload": "the chunk workload with 256x64 tiles (%d live tiles; "
                                             "one eight-wave workgroup per query tile)" % c5["live"],
                                 "TFLOP_per_s": round(t, 2),
                                 "pct_of_peak": round(100 * t / PEAK_BF16_TFLOPS, 2),
                                 "ms_per_step": round(c5["wall_ms"], 4),
                                 "kernel_ms": round(c5["kernel_ms"], 4),
                                 "counters": counter_summary(
                                     "chunk_tile256", src_digest("swa_pp_bf16.hip"))}
    if "chunk_sink" in out:
        cs = out["chunk_sink"]
        t = cs["flops"] / (cs["wall_ms"] * 1e-3) / 1e12
        line["chunk_sink"] = {"workload": "chunk workload with 4 attention sinks",
                              "TFLOP_per_s": round(t, 2),
                              "pct_of_peak": round(100 * t / PEAK_BF16_TFLOPS, 2),
                              "ms_per_step": round(cs["wall_ms"], 4)}
    if "chunk" in out:
        c4 = out["chunk"]
        t = c4["flops"] / (c4["wall_ms"] * 1e-3) / 1e12
        line["chunk"] = {"workload": "chunked prefill B=8 H=32 Hkv=8 Tq=512 W=4096 d=128 bf16",
                         "TFLOP_per_s": round(t, 2),
                         "pct_of_peak": round(100 * t / PEAK_BF16_TFLOPS, 2),
                         "ms_per_step": round(c4["wall_ms"], 4),
                         "kernel_ms": round(c4["kernel_ms"], 4),
                         "useful_GFLOP": round(c4["flops"] / 1e9, 3),
                         "keys_touched_per_request": c4["keys_touched_per_request"]}
    if "chunk_stream_dev" in out:
        c4 = out["chunk"]
        fl = c4["flops"]
        line["chunk_stream"] = {
            "workload": "the chunk workload as a stream of steps (the ring advances 512 "
                        "positions per step), block metadata rebuilt before every step",
            "device_metadata": {"ms_per_step": round(out["chunk_stream_dev"]["wall_ms"], 4),
                                "TFLOP_per_s": round(fl / (out["chunk_stream_dev"]["wall_ms"]
                                                           * 1e-3) / 1e12, 2)},
            "host_metadata": {"ms_per_step": round(out["chunk_stream_host"]["wall_ms"], 4),
                              "TFLOP_per_s": round(fl / (out["chunk_stream_host"]["wall_ms"]
                                                         * 1e-3) / 1e12, 2)}}
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
