"""GPU parity of the 256-row query tiling of the bf16 forward (swa_pp_bf16.hip).

"Weight sparsity vs attention sparsity" (AI-infra KB) §04 leaves the block
shape open; with tile_q = 256 the metadata lists the key tiles of 256 query
rows and one workgroup of eight waves runs them, two groups of four waves
taking turns between matrix and vector work.  Each wave visits the key tiles
its 32 rows see, in increasing order, with the arithmetic of the 128-row
kernel, and a tile none of its rows sees changes nothing, so the outputs (and
the row log-sum-exp) must equal the (128, 64) tiling's bit for bit; they are
also checked against the fp64 oracle at the bars of the other tilings (bf16
max-abs 2e-2, mean-abs 2e-3; ring state and caches bit-exact).  The three
long-window workloads are compared whole, every output element.
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
BF16_MAX, BF16_MEAN = 2e-2, 2e-3


def f64(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def check(got, ref, where):
    got = f64(got) if torch.is_tensor(got) else got
    assert np.all(np.isfinite(got)), "non-finite output " + where
    err = np.abs(got - ref)
    assert err.max() <= BF16_MAX, (where, float(err.max()))
    assert err.mean() <= BF16_MEAN, (where, float(err.mean()))


def fwd(dev, W, tq, tk, L=None, S=0, lse=False):
    q = dev["q"]
    B, H, N, d = q.shape
    meta = swa.swa_blockmask_build(B, N, N, W, tq, tk, q_len=L, k_len=L, n_sink=S)
    o = torch.full_like(q, float("nan"))
    ls = torch.full((B, H, N), float("nan"), device=DEV) if lse else None
    swa.swa_fwd(q, dev["k"], dev["v"], o, W, swa.meta_to_device(meta, DEV),
                q_len=None if L is None else torch.tensor(L, dtype=torch.int32, device=DEV),
                lse=ls)
    torch.cuda.synchronize()
    return o, ls, meta


@pytest.mark.parametrize("W,S", [(1, 0), (17, 0), (100, 0), (255, 0), (256, 0), (333, 0),
                                 (1000, 0), (17, 4), (100, 1), (40, 130), (600, 70)])
@pytest.mark.parametrize("N", [333, 700])
def test_fwd_tq256_small(W, S, N):
    """Padded lengths (some sequences shorter than a tile, whole query tiles of
    padding), windows from 1 to beyond the sequence, attention sinks: outputs
    and lse against the oracle and bit for bit the (128, 64) tiling."""
    inp = synth.gen_fwd(3, 4, 2, N, 128, seed=1300 + W + S + N, std=0.5, len_lo=1, len_hi=N)
    inp["q_len"][0] = N
    L = inp["q_len"].numpy()
    dev = {x: inp[x].to(DEV) for x in ("q", "k", "v")}
    o, ls, meta = fwd(dev, W, 256, 64, L, S, lse=True)
    o128, ls128, _ = fwd(dev, W, 128, 64, L, S, lse=True)
    ref = oracle.fwd(f64(inp["q"]), f64(inp["k"]), f64(inp["v"]), W, 1 / math.sqrt(128), q_len=L,
                     n_sink=S)
    check(o, ref, "tq256 W=%d S=%d N=%d" % (W, S, N))
    assert meta["tile_q"] == 256
    assert torch.equal(o, o128), "256-row tiling differs from the 128-row tiling"
    for b, n in enumerate(L):
        assert torch.all(o[b, :, int(n):] == 0)
        assert torch.equal(ls[b, :, :int(n)], ls128[b, :, :int(n)])


@pytest.mark.parametrize("N", [1, 5, 64, 256, 257, 511])
def test_fwd_tq256_short(N):
    """Sequences of one tile or less (group 1 of the workgroup, or most of
    its waves, have no rows), against the oracle and the 128-row tiling."""
    inp = synth.gen_fwd(2, 4, 4, N, 128, seed=50 + N, std=0.5)
    dev = {x: inp[x].to(DEV) for x in ("q", "k", "v")}
    o, _, _ = fwd(dev, 200, 256, 64)
    o128, _, _ = fwd(dev, 200, 128, 64)
    ref = oracle.fwd(f64(inp["q"]), f64(inp["k"]), f64(inp["v"]), 200, 1 / math.sqrt(128))
    check(o, ref, "tq256 N=%d" % N)
    assert torch.equal(o, o128)


def _large(B, H, Hkv, N, d, seed, qk_std, bias):
    g = torch.Generator().manual_seed(seed)
    u = torch.randn(d, generator=g)
    u = u / u.norm()
    q = torch.randn(B, H, N, d, generator=g) * 0.3 + qk_std * math.sqrt(d) * u
    k = torch.randn(B, Hkv, N, d, generator=g) * 0.3 + bias * qk_std * math.sqrt(d) * u
    k = k + torch.randn(B, Hkv, N, 1, generator=g) * qk_std * math.sqrt(d) * 0.2 * u
    v = torch.randn(B, Hkv, N, d, generator=g) * 0.5
    return q.to(torch.bfloat16), k.to(torch.bfloat16), v.to(torch.bfloat16)


@pytest.mark.parametrize("qk_std,bias", [(1.5, 1.0), (3.0, 1.0), (1.5, -1.0), (3.0, -1.0)])
@pytest.mark.parametrize("W", [64, 600])
def test_fwd_tq256_large_scores(qk_std, bias, W):
    """Scores far from the fixed softmax reference: the rescale path (a
    recompute of the tile's scores in the vector slot) must give the oracle's
    result and the 128-row tiling's bits."""
    q, k, v = _large(2, 4, 2, 700, 128, int(qk_std * 10) + W, qk_std, bias)
    dev = {"q": q.to(DEV), "k": k.to(DEV), "v": v.to(DEV)}
    o, ls, _ = fwd(dev, W, 256, 64, lse=True)
    o128, ls128, _ = fwd(dev, W, 128, 64, lse=True)
    ref = oracle.fwd(f64(q), f64(k), f64(v), W, 1 / math.sqrt(128))
    check(o, ref, "tq256 large scores std=%g bias=%g W=%d" % (qk_std, bias, W))
    assert torch.equal(o, o128) and torch.equal(ls, ls128)


@pytest.mark.parametrize("H,Hkv", [(3, 3), (8, 1), (16, 2), (6, 3)])
def test_fwd_tq256_group_sizes(H, Hkv):
    """Query heads per KV head G = 1 (odd head count), 2 and 8."""
    inp = synth.gen_fwd(2, H, Hkv, 600, 128, seed=60 + H, std=0.5, len_lo=100, len_hi=600)
    L = inp["q_len"].numpy()
    dev = {x: inp[x].to(DEV) for x in ("q", "k", "v")}
    o, _, _ = fwd(dev, 300, 256, 64, L)
    o128, _, _ = fwd(dev, 300, 128, 64, L)
    ref = oracle.fwd(f64(inp["q"]), f64(inp["k"]), f64(inp["v"]), 300, 1 / math.sqrt(128),
                     q_len=L)
    check(o, ref, "tq256 H=%d Hkv=%d" % (H, Hkv))
    assert torch.equal(o, o128)


def test_varlen_tq256_packed():
    """Sequences packed token-major (swa_fwd_varlen), empty ones included:
    every row against the oracle and bit for bit the padded call's rows."""
    inp = synth.gen_fwd(4, 8, 2, 900, 128, seed=78, std=0.5, len_lo=0, len_hi=900)
    inp["q_len"][0] = 900
    inp["q_len"][2] = 0
    L = inp["q_len"].numpy()
    dev = {x: inp[x].to(DEV) for x in ("q", "k", "v")}
    W = 500
    o, _, meta = fwd(dev, W, 256, 64, L)
    lens = [int(x) for x in L]
    pk = [torch.cat([dev[x][b, :, :n].transpose(0, 1) for b, n in enumerate(lens)]).contiguous()
          for x in ("q", "k", "v")]
    cu = torch.tensor([0] + list(np.cumsum(lens)), dtype=torch.int32, device=DEV)
    op = torch.full_like(pk[0], float("nan"))
    swa.swa_fwd_varlen(pk[0], pk[1], pk[2], op, W, swa.meta_to_device(meta, DEV), cu)
    torch.cuda.synchronize()
    ref = oracle.fwd(f64(inp["q"]), f64(inp["k"]), f64(inp["v"]), W, 1 / math.sqrt(128), q_len=L)
    for b, n in enumerate(lens):
        seg = op[int(cu[b]):int(cu[b + 1])].transpose(0, 1)
        if n:
            check(seg, ref[b, :, :n], "packed tq256 sequence %d" % b)
        assert torch.equal(seg, o[b, :, :n]), "packed rows differ from padded, sequence %d" % b


def _chunk_inputs(B, H, Hkv, Tq, W, d, S, seed):
    inp = synth.gen_chunk(B, H, Hkv, Tq, W, d, seed=seed, std=0.5, p=[0] * B)
    rng = np.random.default_rng(seed)
    for b in range(B):
        cl = W if b % 2 == 0 else int(rng.integers(0, W))
        inp["cache_len"][b] = cl
        inp["next_pos"][b] = cl + int(rng.integers(0, 3 * W))
        inp["ring_start"][b] = int(rng.integers(0, W))
    gen = torch.Generator().manual_seed(seed + 1)
    sk = (torch.randn(B, Hkv, max(S, 1), d, generator=gen) * 0.5).to(torch.bfloat16)
    sv = (torch.randn(B, Hkv, max(S, 1), d, generator=gen) * 0.5).to(torch.bfloat16)
    # a sink position the ring still holds carries the ring's row, as in a
    # stream (both copies come from the same new row)
    for b in range(B):
        oldest = int(inp["next_pos"][b]) - int(inp["cache_len"][b])
        for p in range(max(oldest, 0), min(S, int(inp["next_pos"][b]))):
            slot = (int(inp["ring_start"][b]) + p - oldest) % W
            sk[b, :, p] = inp["k_cache"][b, :, slot]
            sv[b, :, p] = inp["v_cache"][b, :, slot]
    return inp, sk[:, :, :S].contiguous(), sv[:, :, :S].contiguous()


def run_chunk(inp, sk, sv, W, tq, tk, S):
    B, H, Tq, d = inp["q"].shape
    p = inp["next_pos"].numpy()
    meta = swa.swa_blockmask_build(B, Tq, Tq, W, tq, tk, q_start=p, k_start=p, W_ring=W,
                                   ring_start=inp["ring_start"].numpy(),
                                   cache_len=inp["cache_len"].numpy(), next_pos=p, n_sink=S)
    dev = {k: v.to(DEV).contiguous() for k, v in inp.items()}
    skd, svd = sk.to(DEV), sv.to(DEV)
    o = torch.full_like(dev["q"], float("nan"))
    swa.swa_prefill_chunk(dev["q"], dev["k_new"], dev["v_new"], dev["k_cache"], dev["v_cache"],
                          dev["ring_start"], dev["cache_len"], dev["next_pos"], o, W,
                          swa.meta_to_device(meta, DEV),
                          sink_k=skd if S else None, sink_v=svd if S else None)
    torch.cuda.synchronize()
    return o, dev, skd, svd


@pytest.mark.parametrize("Tq", [1, 37, 256, 300, 512])
@pytest.mark.parametrize("S", [0, 3, 70])
def test_chunk_tq256_small(Tq, S):
    """Chunked prefill over rings that are full or filling (wrap points inside
    tiles), with and without sink caches: output, rings, sink caches and state
    against the oracle; output bit for bit the (128, 64) tiling's."""
    W, d = 512, 128
    inp, sk, sv = _chunk_inputs(4, 8, 2, Tq, W, d, S, seed=700 + Tq + S)
    o, dev, skd, svd = run_chunk(inp, sk, sv, W, 256, 64, S)
    o128, _, _, _ = run_chunk(inp, sk, sv, W, 128, 64, S)
    kw = dict(n_sink=S, sink_k=f64(sk), sink_v=f64(sv)) if S else {}
    ro, kc, vc, rs, cl, npos = oracle.chunk(
        f64(inp["q"]), f64(inp["k_new"]), f64(inp["v_new"]), f64(inp["k_cache"]),
        f64(inp["v_cache"]), inp["ring_start"].numpy(), inp["cache_len"].numpy(),
        inp["next_pos"].numpy(), W, 1 / math.sqrt(d), **kw)[:6]
    check(o, ro, "chunk tq256 Tq=%d S=%d" % (Tq, S))
    assert torch.equal(o, o128), "256-row tiling differs from the 128-row tiling"
    assert np.array_equal(f64(dev["k_cache"]), kc) and np.array_equal(f64(dev["v_cache"]), vc)
    assert np.array_equal(dev["ring_start"].cpu().numpy(), rs)
    assert np.array_equal(dev["cache_len"].cpu().numpy(), cl)
    assert np.array_equal(dev["next_pos"].cpu().numpy(), npos)


def test_prefill_workload_tq256_full():
    """B=1, H=32, N=8192, W=512 at tiles (256, 64): every output element bit
    for bit the (128, 64) tiling's, which the parity tests hold to the oracle
    over the whole workload; and a slice against the oracle directly."""
    inp = synth.make("prefill")
    dev = {x: inp[x].to(DEV) for x in ("q", "k", "v")}
    o, _, _ = fwd(dev, 512, 256, 64)
    o128, _, _ = fwd(dev, 512, 128, 64)
    assert torch.equal(o, o128)
    ref = oracle.fwd(f64(inp["q"][:, :2]), f64(inp["k"][:, :2]), f64(inp["v"][:, :2]), 512,
                     1 / math.sqrt(128))
    check(o[:, :2], ref, "prefill workload tq256, heads 0-1")


def test_gqa_workload_tq256_full():
    """B=4, H=32, Hkv=8, N=32768 padded, W=4096: every element of the padded
    and of the packed call bit for bit the (128, 64) tiling's padded output
    (itself held to the oracle on every valid row by the parity tests); the
    first 512 rows of each sequence against the oracle directly."""
    inp = synth.make("prefill_gqa")
    L = inp["q_len"].numpy()
    dev = {x: inp[x].to(DEV) for x in ("q", "k", "v")}
    o, _, meta = fwd(dev, 4096, 256, 64, L)
    o128, _, _ = fwd(dev, 4096, 128, 64, L)
    assert torch.equal(o, o128)
    del o128
    lens = [int(x) for x in L]
    pk = [torch.cat([dev[x][b, :, :n].transpose(0, 1) for b, n in enumerate(lens)]).contiguous()
          for x in ("q", "k", "v")]
    cu = torch.tensor([0] + list(np.cumsum(lens)), dtype=torch.int32, device=DEV)
    op = torch.full_like(pk[0], float("nan"))
    swa.swa_fwd_varlen(pk[0], pk[1], pk[2], op, 4096, swa.meta_to_device(meta, DEV), cu)
    torch.cuda.synchronize()
    for b, n in enumerate(lens):
        assert torch.equal(op[int(cu[b]):int(cu[b + 1])].transpose(0, 1), o[b, :, :n])
    del pk, op
    sc = 1 / math.sqrt(128)
    for b in range(4):
        ref = oracle.fwd(f64(inp["q"][b:b + 1, :, :512]), f64(inp["k"][b:b + 1, :, :512]),
                         f64(inp["v"][b:b + 1, :, :512]), 4096, sc)
        check(o[b:b + 1, :, :512], ref, "gqa workload tq256 sequence %d" % b)


def test_chunk_workload_tq256_full():
    """B=8, H=32, Hkv=8, Tq=512, W=4096 at tiles (256, 64): every output bit for
    bit the (128, 64) tiling's and against the oracle's chunk."""
    inp = synth.make("chunk")
    none = torch.zeros(0, dtype=torch.bfloat16)
    o, dev, _, _ = run_chunk(inp, none, none, 4096, 256, 64, 0)
    o128, _, _, _ = run_chunk(inp, none, none, 4096, 128, 64, 0)
    assert torch.equal(o, o128), "256-row tiling differs from the 128-row tiling"
    ro = oracle.chunk(f64(inp["q"]), f64(inp["k_new"]), f64(inp["v_new"]), f64(inp["k_cache"]),
                      f64(inp["v_cache"]), inp["ring_start"].numpy(), inp["cache_len"].numpy(),
                      inp["next_pos"].numpy(), 4096, 1 / math.sqrt(128))[0]
    check(o, ro, "chunk workload tq256")
