"""GPU parity: the HIP path through the C ABI against the fp64 oracle.

Bars: bf16 inputs (fp32 accumulation) max-abs <= 2e-2 and mean-abs <= 2e-3 over
the compared outputs; fp32 path <= 1e-4; ring contents after a commit are
copies, so they must be bit-identical; padded rows exactly 0.  The oracle gets
the very values the GPU gets (bf16 rounded on the host, widened to fp64).
"""
import math

import numpy as np
import pytest
import torch

import causal_sliding_window_swa_amd as swa
import oracle
from causal_sliding_window_swa_amd import synth

pytestmark = pytest.mark.gpu

BF16_MAX, BF16_MEAN, F32_MAX = 2e-2, 2e-3, 1e-4
DEV = "cuda:0"


def f64(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def check(got, ref, dtype, where=""):
    got = f64(got) if torch.is_tensor(got) else got
    err = np.abs(got - ref)
    assert np.all(np.isfinite(got)), "non-finite output " + where
    if dtype == torch.bfloat16:
        assert err.max() <= BF16_MAX, (where, float(err.max()))
        assert err.mean() <= BF16_MEAN, (where, float(err.mean()))
    else:
        assert err.max() <= F32_MAX, (where, float(err.max()))


def run_fwd(inp, W, tq, tk, scale=None):
    q, k, v, ql = inp["q"], inp["k"], inp["v"], inp["q_len"]
    B, H, N, d = q.shape
    L = None if ql is None else ql.numpy()
    meta = swa.swa_blockmask_build(B, N, N, W, tq, tk, q_len=L, k_len=L)
    md = swa.meta_to_device(meta, DEV)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    od = torch.full_like(qd, float("nan"))
    qld = None if ql is None else ql.to(DEV)
    swa.swa_fwd(qd, kd, vd, od, W, md, q_len=qld, scale=scale)
    torch.cuda.synchronize()
    return od, meta


# ---------------------------------------------------------------------------
# full-sequence forward

def test_tiny_workload_fp32():
    inp = synth.make("tiny")
    for tile in (2, 4):
        o, meta = run_fwd(inp, 3, tile, tile, scale=0.5)
        ref = oracle.fwd(f64(inp["q"]), f64(inp["k"]), f64(inp["v"]), 3, 0.5)
        check(o, ref, torch.float32, "tiny tile %d" % tile)
        assert meta["valid_pairs"] == 21
    # zero scores with values 1..8: 4.5 causal, 7 at W=3 on the last row
    q = torch.zeros(1, 1, 8, 4)
    k = inp["k"].clone()
    v = torch.arange(1, 9, dtype=torch.float32)[:, None].repeat(1, 4)[None, None].contiguous()
    z = dict(q=q, k=k, v=v, q_len=None)
    o3, _ = run_fwd(z, 3, 2, 2, scale=0.5)
    o8, _ = run_fwd(z, 8, 4, 4, scale=0.5)
    assert abs(float(o3[0, 0, 7, 0]) - 7.0) <= 1e-6
    assert abs(float(o8[0, 0, 7, 0]) - 4.5) <= 1e-6


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("tq", [128, 64])
@pytest.mark.parametrize("W", [1, 17, 64, 100, 333, 1000])
def test_fwd_bf16_small(d, tq, W):
    inp = synth.gen_fwd(2, 4, 2, 333, d, seed=100 + W, std=0.5)
    o, _ = run_fwd(inp, W, tq, 64)
    ref = oracle.fwd(f64(inp["q"]), f64(inp["k"]), f64(inp["v"]), W, 1 / math.sqrt(d))
    check(o, ref, torch.bfloat16, "fwd d=%d tq=%d W=%d" % (d, tq, W))


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_fwd_padded_lengths(dtype):
    inp = synth.gen_fwd(3, 8, 2, 300, 128 if dtype == "bf16" else 36, seed=7, std=0.5,
                        dtype=dtype, len_lo=1, len_hi=300)
    inp["q_len"][0] = 300
    inp["q_len"][1] = 1
    o, _ = run_fwd(inp, 50, 128 if dtype == "bf16" else 16, 64 if dtype == "bf16" else 8)
    L = inp["q_len"].numpy()
    ref = oracle.fwd(f64(inp["q"]), f64(inp["k"]), f64(inp["v"]), 50,
                     1 / math.sqrt(inp["q"].shape[-1]), q_len=L)
    check(o, ref, inp["q"].dtype, "padded " + dtype)
    for b, l in enumerate(L):
        assert torch.all(o[b, :, int(l):] == 0)


@pytest.mark.parametrize("d", [4, 8, 36, 64, 128])
def test_fwd_fp32_small(d):
    inp = synth.gen_fwd(2, 4, 4, 77, d, seed=d, std=1.0, dtype="f32")
    for W, tq, tk in ((5, 8, 8), (13, 3, 7), (77, 16, 32), (200, 64, 64)):
        o, _ = run_fwd(inp, W, tq, tk)
        ref = oracle.fwd(f64(inp["q"]), f64(inp["k"]), f64(inp["v"]), W, 1 / math.sqrt(d))
        check(o, ref, torch.float32, "fp32 d=%d W=%d" % (d, W))


def test_fwd_window_locality_bitwise():
    """Changing K/V outside row i's window leaves row i bit-identical."""
    inp = synth.gen_fwd(1, 2, 1, 256, 128, seed=3, std=0.5)
    W, i = 40, 150
    o1, _ = run_fwd(inp, W, 128, 64)
    inp2 = {k: (v.clone() if torch.is_tensor(v) else v) for k, v in inp.items()}
    inp2["k"][0, 0, :i - W + 1] = 1.0
    inp2["v"][0, 0, :i - W + 1] = -1.0
    inp2["k"][0, 0, i + 1:] = 2.0
    inp2["v"][0, 0, i + 1:] = 3.0
    o2, _ = run_fwd(inp2, W, 128, 64)
    assert torch.equal(o1[:, :, i], o2[:, :, i])


def test_prefill_workload_full():
    """B=1, H=32, N=8192, W=512, bf16, tiles (128, 64): every output element
    against the oracle's forward of the whole workload (mean-abs over all of it)."""
    inp = synth.make("prefill")
    o, meta = run_fwd(inp, 512, 128, 64)
    assert meta["valid_pairs"] == 32 * 0 + 4063488  # per head; B=1
    ref = oracle.fwd(f64(inp["q"]), f64(inp["k"]), f64(inp["v"]), 512, 1 / math.sqrt(128))
    check(o, ref, torch.bfloat16, "prefill workload")


def test_prefill_gqa_workload_full():
    """B=4, H=32, Hkv=8, N=32768 padded, W=4096, lengths U[8192, 32768]: every
    valid row of every sequence against the oracle (each sequence's forward
    over its valid length: keys past it are never visible, so the rows are
    the padded batch's), padded rows exactly 0; and the same sequences packed
    token-major (swa_fwd_varlen) give the padded call's rows bit for bit."""
    inp = synth.make("prefill_gqa")
    o, meta = run_fwd(inp, 4096, 128, 64)
    L = inp["q_len"].numpy()
    sc = 1 / math.sqrt(128)
    errs, n = [], 0
    for b in range(4):
        n_b = int(L[b])
        ref = oracle.fwd(f64(inp["q"][b:b + 1, :, :n_b]), f64(inp["k"][b:b + 1, :, :n_b]),
                         f64(inp["v"][b:b + 1, :, :n_b]), 4096, sc)
        got = f64(o[b:b + 1, :, :n_b])
        assert np.all(np.isfinite(got)), "non-finite output, sequence %d" % b
        err = np.abs(got - ref)
        errs.append((float(err.max()), float(err.sum())))
        n += err.size
        assert torch.all(o[b, :, n_b:] == 0)
        del ref, got, err
    assert max(e[0] for e in errs) <= BF16_MAX, errs
    assert sum(e[1] for e in errs) / n <= BF16_MEAN, errs
    # packed layout: same kernel, other addressing, same arithmetic
    lens = [int(x) for x in L]
    pk = [torch.cat([inp[x][b, :, :n_b].transpose(0, 1) for b, n_b in enumerate(lens)])
          .contiguous().to(DEV) for x in ("q", "k", "v")]
    cu = torch.tensor([0] + list(np.cumsum(lens)), dtype=torch.int32, device=DEV)
    op = torch.full_like(pk[0], float("nan"))
    swa.swa_fwd_varlen(pk[0], pk[1], pk[2], op, 4096, swa.meta_to_device(meta, DEV), cu)
    torch.cuda.synchronize()
    for b, n_b in enumerate(lens):
        seg = op[int(cu[b]):int(cu[b + 1])].transpose(0, 1)
        assert torch.equal(seg, o[b, :, :n_b]), "packed rows differ from padded, sequence %d" % b


# ---------------------------------------------------------------------------
# chunked prefill against the ring

def run_chunk(inp, W, tq, tk, scale=None):
    q = inp["q"]
    B, H, Tq, d = q.shape
    p = inp["next_pos"].numpy()
    meta = swa.swa_blockmask_build(B, Tq, Tq, W, tq, tk, q_start=p, k_start=p, W_ring=W,
                                   ring_start=inp["ring_start"].numpy(),
                                   cache_len=inp["cache_len"].numpy(), next_pos=p)
    md = swa.meta_to_device(meta, DEV)
    dev = {k: v.to(DEV).contiguous() for k, v in inp.items()}
    o = torch.full_like(dev["q"], float("nan"))
    swa.swa_prefill_chunk(dev["q"], dev["k_new"], dev["v_new"], dev["k_cache"],
                          dev["v_cache"], dev["ring_start"], dev["cache_len"],
                          dev["next_pos"], o, W, md, scale=scale)
    torch.cuda.synchronize()
    return o, dev, meta


def oracle_chunk(inp, W, scale, bsel=None):
    sel = slice(None) if bsel is None else bsel
    g = {k: (v[sel] if torch.is_tensor(v) else v) for k, v in inp.items()}
    return oracle.chunk(f64(g["q"]), f64(g["k_new"]), f64(g["v_new"]), f64(g["k_cache"]),
                        f64(g["v_cache"]), g["ring_start"].numpy(), g["cache_len"].numpy(),
                        g["next_pos"].numpy(), W, scale)


def _ring_inputs(B, H, Hkv, Tq, W, d, seed, dtype, fill):
    inp = synth.gen_chunk(B, H, Hkv, Tq, W, d, seed=seed, std=0.5, dtype=dtype,
                          p=[0] * B)
    rng = np.random.default_rng(seed)
    for b in range(B):
        cl = W if fill[b] else int(rng.integers(0, W))
        p = cl + int(rng.integers(0, 3 * W))
        inp["cache_len"][b] = cl
        inp["next_pos"][b] = p
        inp["ring_start"][b] = int(rng.integers(0, W))
    return inp


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("Tq", [1, 37, 64, 128, 256])
def test_chunk_small(dtype, Tq):
    W = 256
    d = 128 if dtype == "bf16" else 20
    inp = _ring_inputs(4, 8, 2, Tq, W, d, seed=Tq, dtype=dtype, fill=[1, 0, 1, 0])
    tq, tk = (128, 64) if dtype == "bf16" else (32, 16)
    o, dev, meta = run_chunk(inp, W, tq, tk)
    ref_o, kc, vc, rs, cl, npos = oracle_chunk(inp, W, 1 / math.sqrt(d))
    check(o, ref_o, inp["q"].dtype, "chunk %s Tq=%d" % (dtype, Tq))
    assert np.array_equal(dev["ring_start"].cpu().numpy(), rs)
    assert np.array_equal(dev["cache_len"].cpu().numpy(), cl)
    assert np.array_equal(dev["next_pos"].cpu().numpy(), npos)
    assert np.array_equal(f64(dev["k_cache"]), kc) and np.array_equal(f64(dev["v_cache"]), vc)


def test_chunk_workload_full():
    """B=8, H=32, Hkv=8, Tq=512, W=4096, p U[4096, 65536], start = p mod W:
    every output of every request, every ring and the state against the
    oracle's chunk of the whole batch."""
    inp = synth.make("chunk")
    o, dev, meta = run_chunk(inp, 4096, 128, 64)
    assert meta["keys_touched"] == 8 * 4607
    ref_o, kc, vc, rs, cl, npos = oracle_chunk(inp, 4096, 1 / math.sqrt(128))
    check(o, ref_o, torch.bfloat16, "chunk workload")
    assert np.array_equal(f64(dev["k_cache"]), kc)
    assert np.array_equal(f64(dev["v_cache"]), vc)
    assert np.array_equal(dev["ring_start"].cpu().numpy(), rs)
    assert np.array_equal(dev["cache_len"].cpu().numpy(), cl)
    assert np.array_equal(dev["next_pos"].cpu().numpy(), npos)
    p = inp["next_pos"].numpy()
    assert np.array_equal(npos, p + 512) and np.array_equal(rs, (p + 512) % 4096)


# ---------------------------------------------------------------------------
# decode

def run_decode(inp, W):
    dev = {k: v.to(DEV).contiguous() for k, v in inp.items()}
    B, H, d = dev["q"].shape
    ws = torch.empty(max(1, swa.swa_decode_workspace_size(B, H, d, W)) // 4 + 4,
                     dtype=torch.float32, device=DEV)
    o = torch.full_like(dev["q"], float("nan"))
    swa.swa_decode(dev["q"], dev["k_new"], dev["v_new"], dev["k_cache"], dev["v_cache"],
                   dev["ring_start"], dev["cache_len"], dev["next_pos"], o, ws, W)
    torch.cuda.synchronize()
    return o, dev


def oracle_decode(inp, W, scale):
    return oracle.decode(f64(inp["q"]), f64(inp["k_new"]), f64(inp["v_new"]),
                         f64(inp["k_cache"]), f64(inp["v_cache"]), inp["ring_start"].numpy(),
                         inp["cache_len"].numpy(), inp["next_pos"].numpy(), W, scale)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("G", [1, 2, 4, 8])
@pytest.mark.parametrize("W", [64, 300, 1024])
def test_decode_small(dtype, G, W):
    d = 128 if dtype == "bf16" else 12
    B, Hkv = 5, 2
    inp = synth.gen_decode(B, G * Hkv, Hkv, W, d, seed=G * 1000 + W, std=0.5, dtype=dtype,
                           pos_lo=W, pos_hi=4 * W)
    inp["cache_len"][1] = 0
    inp["cache_len"][2] = W // 3
    inp["next_pos"][2] = W // 3 + 7
    inp["cache_len"][3] = W - 1
    o, dev = run_decode(inp, W)
    ref_o, kc, vc, rs, cl, npos = oracle_decode(inp, W, 1 / math.sqrt(d))
    check(o, ref_o, inp["q"].dtype, "decode %s G=%d W=%d" % (dtype, G, W))
    assert np.array_equal(f64(dev["k_cache"]), kc) and np.array_equal(f64(dev["v_cache"]), vc)
    assert np.array_equal(dev["ring_start"].cpu().numpy(), rs)
    assert np.array_equal(dev["cache_len"].cpu().numpy(), cl)
    assert np.array_equal(dev["next_pos"].cpu().numpy(), npos)


def test_decode_d64():
    inp = synth.gen_decode(3, 8, 2, 512, 64, seed=64, std=0.5, pos_lo=512, pos_hi=2000)
    o, dev = run_decode(inp, 512)
    ref_o = oracle_decode(inp, 512, 1 / 8.0)[0]
    check(o, ref_o, torch.bfloat16, "decode d=64")


def test_decode_workload_full():
    """B=64, H=32, Hkv=8, d=128, W=4096: every output against the oracle."""
    inp = synth.make("decode")
    o, dev = run_decode(inp, 4096)
    ref_o, kc, vc, rs, cl, npos = oracle_decode(inp, 4096, 1 / math.sqrt(128))
    check(o, ref_o, torch.bfloat16, "decode workload")
    assert np.array_equal(dev["ring_start"].cpu().numpy(), rs)
    assert np.array_equal(f64(dev["k_cache"]), kc)


def test_decode_steps_chain():
    """Ten decode steps in a row from a partly filled ring match the oracle."""
    W, B, H, Hkv, d = 128, 2, 8, 2, 128
    inp = synth.gen_decode(B, H, Hkv, W, d, seed=11, std=0.5, pos_lo=120, pos_hi=130)
    inp["cache_len"][0] = 120
    inp["next_pos"][0] = 120
    inp["ring_start"][0] = 0
    dev = {k: v.to(DEV).contiguous() for k, v in inp.items()}
    ws = torch.empty(swa.swa_decode_workspace_size(B, H, d, W) // 4 + 4, dtype=torch.float32,
                     device=DEV)
    state = {k: (f64(v) if v.dtype != torch.int32 else v.numpy().copy()) for k, v in inp.items()}
    gen = torch.Generator().manual_seed(5)
    for step in range(10):
        q = (torch.randn(B, H, d, generator=gen) * 0.5).to(torch.bfloat16)
        kn = (torch.randn(B, Hkv, d, generator=gen) * 0.5).to(torch.bfloat16)
        vn = (torch.randn(B, Hkv, d, generator=gen) * 0.5).to(torch.bfloat16)
        o = torch.empty(B, H, d, dtype=torch.bfloat16, device=DEV)
        swa.swa_decode(q.to(DEV), kn.to(DEV), vn.to(DEV), dev["k_cache"], dev["v_cache"],
                       dev["ring_start"], dev["cache_len"], dev["next_pos"], o, ws, W)
        ro, state["k_cache"], state["v_cache"], state["ring_start"], state["cache_len"], \
            state["next_pos"] = oracle.decode(f64(q), f64(kn), f64(vn), state["k_cache"],
                                              state["v_cache"], state["ring_start"],
                                              state["cache_len"], state["next_pos"], W,
                                              1 / math.sqrt(d))
        torch.cuda.synchronize()
        check(o, ro, torch.bfloat16, "decode step %d" % step)
    assert np.array_equal(dev["cache_len"].cpu().numpy(), state["cache_len"])
    assert np.array_equal(f64(dev["k_cache"]), state["k_cache"])
