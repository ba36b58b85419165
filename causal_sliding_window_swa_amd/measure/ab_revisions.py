"""A/B timing of two or more builds of the library (measurement support, not
part of the library).

Build, on a machine with hipcc and the git history (no GPU needed):

    python -m causal_sliding_window_swa_amd.measure.ab_revisions build REV [REV ...] --out DIR

  exports each revision's package and include/ with `git archive`, builds it
  with that revision's own build script for gfx950 and leaves
  DIR/libswa_<REV>.so.

Time, on the GPU:

    python -m causal_sliding_window_swa_amd.measure.ab_revisions time LIB [LIB ...] \\
        --workload prefill|gqa|chunk|decode [--tile-k 64|128] [--rounds N]

  loads the libraries side by side through ctypes (the C ABI of include/swa.h),
  runs each once on the same inputs and compares every output bit for bit with
  the first library's, warms the GPU up for a second, then times the libraries
  in interleaved rounds (so that clock drift and the box affect them alike) and
  prints one JSON line per library with the median and minimum time per call.
  Inputs and block metadata come from this tree (synth, swa_blockmask_build).
"""
import argparse
import ctypes
import json
import math
import os
import shutil
import subprocess
import sys
import tempfile
import time

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))


def build(revs, out):
    os.makedirs(out, exist_ok=True)
    for rev in revs:
        tmp = tempfile.mkdtemp(prefix="swa_ab_")
        try:
            arch = subprocess.run(["git", "-C", ROOT, "archive", rev,
                                   "causal_sliding_window_swa_amd", "include"],
                                  check=True, stdout=subprocess.PIPE).stdout
            subprocess.run(["tar", "-x", "-C", tmp], input=arch, check=True)
            subprocess.run([sys.executable, "-m", "causal_sliding_window_swa_amd.build"],
                           cwd=tmp, check=True, stdout=subprocess.DEVNULL)
            dst = os.path.join(out, "libswa_%s.so" % rev.replace("/", "_"))
            shutil.copy(os.path.join(tmp, "causal_sliding_window_swa_amd", "libswa.so"), dst)
            print(dst, flush=True)
        finally:
            shutil.rmtree(tmp, ignore_errors=True)


def _load(path):
    P, I, F, Z = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    L = ctypes.CDLL(os.path.abspath(path))
    L.swa_fwd.argtypes = [I] * 10 + [P] * 9 + [F, P]
    L.swa_prefill_chunk.argtypes = [I] * 8 + [P, P, I, I] + [P] * 12 + [F, P]
    L.swa_decode.argtypes = [I] * 7 + [P] * 12 + [Z, F, P]
    L.swa_decode_workspace_size.argtypes = [I] * 4
    L.swa_decode_workspace_size.restype = Z
    return L


def time_libs(libs, workload, tile_k, rounds):
    import numpy as np
    import torch
    sys.path.insert(0, ROOT)
    import causal_sliding_window_swa_amd as swa
    from causal_sliding_window_swa_amd import synth

    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream().cuda_stream
    L = [_load(p) for p in libs]
    bf16 = swa.SWA_BF16

    def check(*ts):  # the bf16 entry points take 2-byte elements only
        for t in ts:
            if t.dtype != torch.bfloat16 or t.element_size() != 2:
                raise SystemExit("inputs must be bf16")

    if workload in ("prefill", "gqa"):
        inp = synth.make("prefill" if workload == "prefill" else "prefill_gqa")
        B, H, N, d = inp["q"].shape
        Hkv = inp["k"].shape[1]
        W = 512 if workload == "prefill" else 4096
        qlen = inp.get("q_len")
        lens = None if qlen is None else qlen.numpy()
        meta = swa.swa_blockmask_build(B, N, N, W, 128, tile_k, q_len=lens, k_len=lens)
        md = swa.meta_to_device(meta, dev)
        q, k, v = (inp[x].to(dev) for x in ("q", "k", "v"))
        ql = None if qlen is None else qlen.to(dev)
        del inp
        flop = 4.0 * d * meta["valid_pairs"] * H
        rep = 20 if workload == "prefill" else 2

        def out_like():
            return torch.zeros_like(q)

        def call(lib, o):
            check(q, k, v, o)
            rc = lib.swa_fwd(bf16, B, H, Hkv, N, d, W, 0, 128, tile_k, q.data_ptr(), k.data_ptr(),
                             v.data_ptr(), o.data_ptr(), None if ql is None else ql.data_ptr(),
                             md["row_ptr"].data_ptr(), md["col"].data_ptr(),
                             md["col_cls"].data_ptr(), None, 1 / math.sqrt(d), stream)
            if rc:
                raise SystemExit("swa_fwd failed: %d" % rc)
        rate = lambda ms: {"TFLOP_per_s": round(flop / ms / 1e9, 1)}
    elif workload == "chunk":
        inp = synth.make("chunk")
        B, H, Tq, d = inp["q"].shape
        Hkv, W = inp["k_new"].shape[1], 4096
        p = inp["next_pos"].numpy()
        meta = swa.swa_blockmask_build(B, Tq, Tq, W, 128, tile_k, q_start=p, k_start=p,
                                       W_ring=W, ring_start=inp["ring_start"].numpy(),
                                       cache_len=inp["cache_len"].numpy(), next_pos=p)
        md = swa.meta_to_device(meta, dev)
        dv = {x: inp[x].to(dev) for x in inp}
        del inp
        st = torch.stack([dv[x] for x in ("ring_start", "cache_len", "next_pos")]).contiguous()
        st0, kc0, vc0 = st.clone(), dv["k_cache"].clone(), dv["v_cache"].clone()
        flop = 4.0 * d * meta["valid_pairs"] * H
        rep = 10

        def out_like():  # a fresh ring as well, so that every library sees the same inputs
            dv["k_cache"].copy_(kc0)
            dv["v_cache"].copy_(vc0)
            return torch.zeros_like(dv["q"])

        def call(lib, o):  # the state is reset each call so the metadata stays valid
            check(dv["q"], dv["k_new"], dv["v_new"], dv["k_cache"], dv["v_cache"], o)
            st.copy_(st0)
            rc = lib.swa_prefill_chunk(
                bf16, B, H, Hkv, Tq, d, W, 0, None, None, 128, tile_k, dv["q"].data_ptr(),
                dv["k_new"].data_ptr(), dv["v_new"].data_ptr(), dv["k_cache"].data_ptr(),
                dv["v_cache"].data_ptr(), st[0].data_ptr(), st[1].data_ptr(), st[2].data_ptr(),
                md["row_ptr"].data_ptr(), md["col"].data_ptr(), md["col_cls"].data_ptr(),
                o.data_ptr(), 1 / math.sqrt(d), stream)
            if rc:
                raise SystemExit("swa_prefill_chunk failed: %d" % rc)
        rate = lambda ms: {"TFLOP_per_s": round(flop / ms / 1e9, 1)}
    elif workload == "decode":
        inp = synth.make("decode")
        B, H, d = inp["q"].shape
        Hkv, W = inp["k_new"].shape[1], 4096
        dv = {x: inp[x].to(dev) for x in inp}
        del inp
        st0 = {x: dv[x].clone() for x in ("ring_start", "cache_len", "next_pos")}
        kc0, vc0 = dv["k_cache"].clone(), dv["v_cache"].clone()
        wsz = max(int(lib.swa_decode_workspace_size(B, H, d, W)) for lib in L)
        ws = torch.empty(wsz // 4 + 4, dtype=torch.float32, device=dev)
        kv = 2.0 * B * Hkv * W * d * 2
        rep = 20

        def out_like():
            for x in st0:
                dv[x].copy_(st0[x])
            dv["k_cache"].copy_(kc0)
            dv["v_cache"].copy_(vc0)
            return torch.zeros_like(dv["q"])

        def call(lib, o):
            check(dv["q"], dv["k_new"], dv["v_new"], dv["k_cache"], dv["v_cache"], o)
            rc = lib.swa_decode(bf16, B, H, Hkv, d, W, 0, None, None, dv["q"].data_ptr(),
                                dv["k_new"].data_ptr(), dv["v_new"].data_ptr(),
                                dv["k_cache"].data_ptr(), dv["v_cache"].data_ptr(),
                                dv["ring_start"].data_ptr(), dv["cache_len"].data_ptr(),
                                dv["next_pos"].data_ptr(), o.data_ptr(), ws.data_ptr(),
                                ws.numel() * 4, 1 / math.sqrt(d), stream)
            if rc:
                raise SystemExit("swa_decode failed: %d" % rc)
        rate = lambda ms: {"GB_per_s": round(kv / ms / 1e6, 1)}
    else:
        raise SystemExit("unknown workload " + workload)

    ref = None
    for lib, path in zip(L, libs):
        o = out_like()
        call(lib, o)
        torch.cuda.synchronize()
        if ref is None:
            ref = o
        else:
            print(json.dumps({"lib": path, "bit_identical_to": libs[0],
                              "value": bool(torch.equal(o, ref))}), flush=True)
    o = torch.empty_like(ref)
    t0 = time.time()
    while time.time() - t0 < 1.0:
        for lib in L:
            for _ in range(5):
                call(lib, o)
        torch.cuda.synchronize()
    res = [[] for _ in L]
    for _ in range(rounds):
        for i, lib in enumerate(L):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(rep):
                call(lib, o)
            e1.record()
            torch.cuda.synchronize()
            res[i].append(e0.elapsed_time(e1) / rep)
    for path, r in zip(libs, res):
        med = float(np.median(r))
        line = {"lib": path, "workload": workload, "tile_k": tile_k, "rounds": rounds,
                "calls_per_round": rep, "median_ms": round(med, 5), "min_ms": round(min(r), 5)}
        line.update(rate(med))
        print(json.dumps(line), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__,
                                 formatter_class=argparse.RawDescriptionHelpFormatter)
    sub = ap.add_subparsers(dest="cmd", required=True)
    b = sub.add_parser("build")
    b.add_argument("revs", nargs="+")
    b.add_argument("--out", required=True)
    t = sub.add_parser("time")
    t.add_argument("libs", nargs="+")
    t.add_argument("--workload", default="prefill")
    t.add_argument("--tile-k", type=int, default=64)
    t.add_argument("--rounds", type=int, default=16)
    a = ap.parse_args()
    if a.cmd == "build":
        build(a.revs, a.out)
    else:
        time_libs(a.libs, a.workload, a.tile_k, a.rounds)


if __name__ == "__main__":
    main()
