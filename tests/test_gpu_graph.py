"""The entry points captured in a HIP graph (through torch.cuda.CUDAGraph) and
replayed several times, with other eager GPU work and synchronisations between
the replays: every replay must reproduce the eager call bit for bit.  The
library enqueues kernels only (no allocation, no memset), so its calls can be
captured; bench.py times its steps this way.
"""
import math

import numpy as np
import pytest
import torch

import causal_sliding_window_swa_amd as swa
import oracle
from causal_sliding_window_swa_amd import synth

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
REPLAYS = 3


def f64(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def other_work():
    """Unrelated eager work between replays."""
    x = torch.randn(512, 512, device=DEV)
    (x @ x).sum().item()
    torch.cuda.synchronize()


def capture(fn):
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def test_graph_fwd_replays():
    inp = synth.gen_fwd(2, 8, 2, 700, 128, seed=31, len_lo=300, len_hi=700)
    B, H, N, d = inp["q"].shape
    L = inp["q_len"].numpy()
    md = swa.meta_to_device(swa.swa_blockmask_build(B, N, N, 96, 128, 64, q_len=L, k_len=L),
                            DEV)
    q, k, v, ql = (inp[x].to(DEV) for x in ("q", "k", "v", "q_len"))
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=DEV)
    run = lambda: swa.swa_fwd(q, k, v, o, 96, md, q_len=ql, lse=lse)
    run()
    torch.cuda.synchronize()
    o_ref, lse_ref = o.clone(), lse.clone()
    ref = oracle.fwd(f64(inp["q"]), f64(inp["k"]), f64(inp["v"]), 96, 1 / math.sqrt(d), q_len=L)
    assert np.abs(f64(o_ref) - ref).max() <= 2e-2
    g = capture(run)
    for r in range(REPLAYS):
        o.fill_(float("nan"))
        lse.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(o, o_ref), "replay %d" % r
        assert torch.equal(lse, lse_ref), "replay %d" % r
        other_work()


def test_graph_decode_replays():
    W = 512
    inp = synth.gen_decode(4, 16, 4, W, 128, seed=32, pos_lo=W, pos_hi=3 * W)
    inp["cache_len"][1] = 100
    inp["next_pos"][1] = 100
    dev0 = {k: v.to(DEV).contiguous() for k, v in inp.items()}
    dev = {k: v.clone() for k, v in dev0.items()}
    B, H, d = dev["q"].shape
    ws = torch.empty(swa.swa_decode_workspace_size(B, H, d, W) // 4 + 4, dtype=torch.float32,
                     device=DEV)
    o = torch.empty_like(dev["q"])
    run = lambda: swa.swa_decode(dev["q"], dev["k_new"], dev["v_new"], dev["k_cache"],
                                 dev["v_cache"], dev["ring_start"], dev["cache_len"],
                                 dev["next_pos"], o, ws, W)

    def reset():
        for k in dev:
            dev[k].copy_(dev0[k])
        torch.cuda.synchronize()

    run()
    torch.cuda.synchronize()
    ref = {k: v.clone() for k, v in dev.items()}
    o_ref = o.clone()
    reset()
    g = capture(run)
    for r in range(REPLAYS):
        reset()
        o.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(o, o_ref), "replay %d" % r
        for k in ("k_cache", "v_cache", "ring_start", "cache_len", "next_pos"):
            assert torch.equal(dev[k], ref[k]), (k, r)
        other_work()


def test_graph_chunk_replays():
    W, Tq = 256, 100
    inp = synth.gen_chunk(2, 8, 2, Tq, W, 128, seed=33, p=[300, 700])
    p = inp["next_pos"].numpy()
    meta = swa.swa_blockmask_build(2, Tq, Tq, W, 128, 64, q_start=p, k_start=p, W_ring=W,
                                   ring_start=inp["ring_start"].numpy(),
                                   cache_len=inp["cache_len"].numpy(), next_pos=p)
    md = swa.meta_to_device(meta, DEV)
    dev0 = {k: v.to(DEV).contiguous() for k, v in inp.items()}
    dev = {k: v.clone() for k, v in dev0.items()}
    o = torch.empty_like(dev["q"])
    run = lambda: swa.swa_prefill_chunk(dev["q"], dev["k_new"], dev["v_new"], dev["k_cache"],
                                        dev["v_cache"], dev["ring_start"], dev["cache_len"],
                                        dev["next_pos"], o, W, md)

    def reset():
        for k in dev:
            dev[k].copy_(dev0[k])
        torch.cuda.synchronize()

    run()
    torch.cuda.synchronize()
    ref = {k: v.clone() for k, v in dev.items()}
    o_ref = o.clone()
    reset()
    g = capture(run)
    for r in range(REPLAYS):
        reset()
        o.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(o, o_ref), "replay %d" % r
        for k in ("k_cache", "v_cache", "ring_start", "cache_len", "next_pos"):
            assert torch.equal(dev[k], ref[k]), (k, r)
        other_work()


def test_graph_bwd_replays():
    inp = synth.gen_bwd(1, 4, 2, 500, 128, seed=34)
    B, H, N, d = inp["q"].shape
    md = swa.meta_to_device(swa.swa_blockmask_build(B, N, N, 64, 128, 64), DEV)
    q, k, v, dout = (inp[x].to(DEV) for x in ("q", "k", "v", "dout"))
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=DEV)
    swa.swa_fwd(q, k, v, o, 64, md, lse=lse)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws = torch.empty(swa.swa_bwd_workspace_size(B, H, N) // 4, dtype=torch.float32, device=DEV)
    run = lambda: swa.swa_bwd(q, k, v, o, dout, lse, dq, dk, dv, ws, 64, md)
    run()
    torch.cuda.synchronize()
    refs = (dq.clone(), dk.clone(), dv.clone())
    g = capture(run)
    for r in range(REPLAYS):
        for t in (dq, dk, dv):
            t.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for got, want in zip((dq, dk, dv), refs):
            assert torch.equal(got, want), "replay %d" % r
        other_work()
