"""GPU parity of the 128-key tiling of the bf16 forward kernels.

"Weight sparsity vs attention sparsity" (AI-infra KB) §04 trades block size
against masked work: with tile_k = 128 the metadata lists 128-key tiles and
the kernel streams each as two 64-key halves through its LDS stages.  The
outputs are checked against the fp64 oracle at the bars of the 64-key tiling
(bf16 max-abs 2e-2, mean-abs 2e-3 over the compared outputs; ring state and
caches bit-exact), and bit for bit against the 64-key tiling on the same
inputs: both run the same 64-key steps in the same order, a half that no row
of the query tile sees changes no state, and a full half inside a partial
128-key tile is masked with a mask that keeps every key.
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


def fwd(dev, W, tq, tk, L=None, S=0):
    q = dev["q"]
    B, H, N, d = q.shape
    meta = swa.swa_blockmask_build(B, N, N, W, tq, tk, q_len=L, k_len=L, n_sink=S)
    o = torch.full_like(q, float("nan"))
    swa.swa_fwd(q, dev["k"], dev["v"], o, W, swa.meta_to_device(meta, DEV),
                q_len=None if L is None else torch.tensor(L, dtype=torch.int32, device=DEV))
    torch.cuda.synchronize()
    return o, meta


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("tq", [128, 64])
@pytest.mark.parametrize("W,S", [(1, 0), (17, 0), (100, 0), (128, 0), (333, 0), (1000, 0),
                                 (17, 4), (100, 1), (40, 130)])
def test_fwd_tk128_small(d, tq, W, S):
    inp = synth.gen_fwd(2, 4, 2, 333, d, seed=900 + W + S, std=0.5, len_lo=100, len_hi=333)
    L = inp["q_len"].numpy()
    dev = {x: inp[x].to(DEV) for x in ("q", "k", "v")}
    o128, m128 = fwd(dev, W, tq, 128, L, S)
    o64, _ = fwd(dev, W, tq, 64, L, S)
    ref = oracle.fwd(f64(inp["q"]), f64(inp["k"]), f64(inp["v"]), W, 1 / math.sqrt(d), q_len=L,
                     n_sink=S)
    check(o128, ref, "tk128 d=%d tq=%d W=%d S=%d" % (d, tq, W, S))
    assert torch.equal(o128, o64), "128-key tiling differs from the 64-key tiling"
    for b, n in enumerate(L):
        assert torch.all(o128[b, :, int(n):] == 0)
    assert m128["tile_k"] == 128


def test_varlen_tk128_packed():
    """GQA sequences packed token-major (swa_fwd_varlen) with 128-key tiles:
    every row against the oracle, and bit for bit the padded call's rows."""
    inp = synth.gen_fwd(3, 8, 2, 700, 128, seed=77, std=0.5, len_lo=1, len_hi=700)
    inp["q_len"][0] = 700
    L = inp["q_len"].numpy()
    dev = {x: inp[x].to(DEV) for x in ("q", "k", "v")}
    W = 300
    o, meta = fwd(dev, W, 128, 128, L)
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
        check(seg, ref[b, :, :n], "packed tk128 sequence %d" % b)
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


@pytest.mark.parametrize("Tq", [1, 37, 128, 200, 256])
@pytest.mark.parametrize("S", [0, 3])
def test_chunk_tk128_small(Tq, S):
    """Chunked prefill over rings that are full or filling, with and without
    a sink cache (sink slots rounded up to 128): output, rings, sink caches
    and state against the oracle; output bit for bit the 64-key tiling's."""
    W, d = 256, 128
    inp, sk, sv = _chunk_inputs(4, 8, 2, Tq, W, d, S, seed=300 + Tq + S)
    o, dev, skd, svd = run_chunk(inp, sk, sv, W, 128, 128, S)
    o64, _, _, _ = run_chunk(inp, sk, sv, W, 128, 64, S)
    kw = dict(n_sink=S, sink_k=f64(sk), sink_v=f64(sv)) if S else {}
    ro, kc, vc, rs, cl, npos = oracle.chunk(
        f64(inp["q"]), f64(inp["k_new"]), f64(inp["v_new"]), f64(inp["k_cache"]),
        f64(inp["v_cache"]), inp["ring_start"].numpy(), inp["cache_len"].numpy(),
        inp["next_pos"].numpy(), W, 1 / math.sqrt(d), **kw)[:6]
    check(o, ro, "chunk tk128 Tq=%d S=%d" % (Tq, S))
    assert torch.equal(o, o64), "128-key tiling differs from the 64-key tiling"
    assert np.array_equal(f64(dev["k_cache"]), kc) and np.array_equal(f64(dev["v_cache"]), vc)
    assert np.array_equal(dev["ring_start"].cpu().numpy(), rs)
    assert np.array_equal(dev["cache_len"].cpu().numpy(), cl)
    assert np.array_equal(dev["next_pos"].cpu().numpy(), npos)


def test_prefill_workload_tk128_full():
    """B=1, H=32, N=8192, W=512, d=128 at tiles (128, 128): every output
    element against the oracle, and bit for bit the (128, 64) tiling."""
    inp = synth.make("prefill")
    dev = {x: inp[x].to(DEV) for x in ("q", "k", "v")}
    o, meta = fwd(dev, 512, 128, 128)
    assert meta["valid_pairs"] == 4063488
    o64, _ = fwd(dev, 512, 128, 64)
    assert torch.equal(o, o64), "128-key tiling differs from the 64-key tiling"
    ref = oracle.fwd(f64(inp["q"]), f64(inp["k"]), f64(inp["v"]), 512, 1 / math.sqrt(128))
    check(o, ref, "prefill workload tk128")


def test_chunk_workload_tk128_full():
    """B=8, H=32, Hkv=8, Tq=512, W=4096 at tiles (128, 128): every output
    against the oracle's chunk, and bit for bit the (128, 64) tiling."""
    inp = synth.make("chunk")
    none = torch.zeros(0, dtype=torch.bfloat16)
    o, dev, _, _ = run_chunk(inp, none, none, 4096, 128, 128, 0)
    o64, _, _, _ = run_chunk(inp, none, none, 4096, 128, 64, 0)
    assert torch.equal(o, o64), "128-key tiling differs from the 64-key tiling"
    ro = oracle.chunk(f64(inp["q"]), f64(inp["k_new"]), f64(inp["v_new"]), f64(inp["k_cache"]),
                      f64(inp["v_cache"]), inp["ring_start"].numpy(), inp["cache_len"].numpy(),
                      inp["next_pos"].numpy(), 4096, 1 / math.sqrt(128))[0]
    check(o, ro, "chunk workload tk128")


@pytest.mark.parametrize("H,Hkv", [(3, 3), (8, 1), (16, 2), (6, 3)])
@pytest.mark.parametrize("tk", [64, 128])
def test_fwd_group_sizes(H, Hkv, tk):
    """Query heads per KV head G = 1 (odd head count), 2 and 8, at both key
    tilings, with padded lengths: every output against the oracle."""
    inp = synth.gen_fwd(2, H, Hkv, 333, 128, seed=40 + H + tk, std=0.5, len_lo=100, len_hi=333)
    L = inp["q_len"].numpy()
    dev = {x: inp[x].to(DEV) for x in ("q", "k", "v")}
    o, _ = fwd(dev, 100, 128, tk, L)
    ref = oracle.fwd(f64(inp["q"]), f64(inp["k"]), f64(inp["v"]), 100, 1 / math.sqrt(128),
                     q_len=L)
    check(o, ref, "H=%d Hkv=%d tk=%d" % (H, Hkv, tk))


@pytest.mark.parametrize("tk", [64, 128])
def test_chunk_group_size_8(tk):
    """A chunk with 8 query heads per KV head (H = 16, Hkv = 2) at both key
    tilings: output, rings and state against the oracle."""
    W, d, Tq = 256, 128, 100
    inp, sk, sv = _chunk_inputs(3, 16, 2, Tq, W, d, 0, seed=77 + tk)
    o, dev, _, _ = run_chunk(inp, sk, sv, W, 128, tk, 0)
    ro, kc, vc, rs, cl, npos = oracle.chunk(
        f64(inp["q"]), f64(inp["k_new"]), f64(inp["v_new"]), f64(inp["k_cache"]),
        f64(inp["v_cache"]), inp["ring_start"].numpy(), inp["cache_len"].numpy(),
        inp["next_pos"].numpy(), W, 1 / math.sqrt(d))[:6]
    check(o, ro, "chunk G=8 tk=%d" % tk)
    assert np.array_equal(f64(dev["k_cache"]), kc) and np.array_equal(f64(dev["v_cache"]), vc)
    assert np.array_equal(dev["next_pos"].cpu().numpy(), npos)
