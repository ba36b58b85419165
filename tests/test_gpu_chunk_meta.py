"""The device-built block metadata of a chunk step (swa_chunk_blockmask_dev)
against the oracle's brute force, bit for bit, and a stream of chunk steps
that rebuilds it on the device before every step, against the oracle step by
step ("Weight sparsity vs attention sparsity" §07: a pattern that moves with
the input is rebuilt each time; "LLMs from scratch" ch.10 §10.2: the chunk)."""
import math

import numpy as np
import pytest
import torch

import causal_sliding_window_swa_amd as swa
import oracle
from causal_sliding_window_swa_amd import synth

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
STATS = oracle.STAT_NAMES


def f64(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def device_meta(B, Tq, W, tq, tk, rs, cl, p, S=0):
    meta = swa.chunk_meta_buffers(B, Tq, W, tq, tk, DEV, n_sink=S)
    state = [torch.tensor(np.asarray(x, dtype=np.int32), device=DEV) for x in (rs, cl, p)]
    swa.swa_chunk_blockmask_dev(meta, *state)
    torch.cuda.synchronize()
    return meta


def assert_same(meta, ref, where):
    nnz = int(ref["row_ptr"][-1])
    B, nqt, nkt = ref["cls"].shape
    assert np.array_equal(meta["cls"].cpu().numpy()[:B * nqt * nkt].reshape(B, nqt, nkt),
                          ref["cls"]), where
    assert np.array_equal(meta["row_ptr"].cpu().numpy(), ref["row_ptr"]), where
    assert np.array_equal(meta["col"].cpu().numpy()[:nnz], ref["col"]), where
    assert np.array_equal(meta["col_cls"].cpu().numpy()[:nnz], ref["col_cls"]), where
    st = meta["stats"].cpu().numpy()
    for i, n in enumerate(STATS):
        assert int(st[i]) == ref[n], (where, n, int(st[i]), ref[n])


def test_random_ring_states():
    """Rings filling and full, random starts and positions, odd tiles, with
    and without sinks."""
    rng = np.random.default_rng(11)
    for case in range(300):
        B = int(rng.integers(1, 4))
        tq = int(rng.integers(1, 9))
        tk = int(rng.integers(1, 9))
        Wr = tk * int(rng.integers(1, 6))
        Tq = int(rng.integers(1, 30))
        S = int(rng.integers(0, 20)) if case % 2 else 0
        cl = rng.integers(0, Wr + 1, size=B)
        p = cl + rng.integers(0, 50, size=B)
        rs = rng.integers(0, Wr, size=B)
        # the chunk's window is the ring's size
        meta = device_meta(B, Tq, Wr, tq, tk, rs, cl, p, S)
        ref = oracle.blockmask(B, Tq, Tq, Wr, tq, tk, q_start=p, k_start=p, W_ring=Wr,
                               ring_start=rs, cache_len=cl, next_pos=p, n_sink=S)
        assert_same(meta, ref, "case %d" % case)


@pytest.mark.parametrize("S", [0, 4])
@pytest.mark.parametrize("tq,tk", [(128, 64), (64, 64), (128, 128)])
def test_chunk_workload(S, tq, tk):
    inp = synth.make("chunk", H=1, Hkv=1, d=1)
    p = inp["next_pos"].numpy()
    rs, cl = inp["ring_start"].numpy(), inp["cache_len"].numpy()
    meta = device_meta(8, 512, 4096, tq, tk, rs, cl, p, S)
    ref = oracle.blockmask(8, 512, 512, 4096, tq, tk, q_start=p, k_start=p, W_ring=4096,
                           ring_start=rs, cache_len=cl, next_pos=p, n_sink=S)
    assert_same(meta, ref, "chunk workload")
    assert ref["keys_touched"] == 8 * 4607 or S > 0


@pytest.mark.parametrize("dtype,tiles", [("bf16", (128, 64)), ("bf16", (128, 128)),
                                         ("bf16", (64, 128)), ("f32", (16, 16))])
def test_chunk_stream_with_device_metadata(dtype, tiles):
    """Six chunk steps of sizes 37, 64, 128, 5, 64, 100 from rings partly
    filled, each preceded by the device metadata build on the same stream and
    no host copy of the ring state: every step's output, and the rings and
    state at the end, against the oracle run step by step (bf16 at 64- and
    128-key tiles)."""
    W = 256
    d = 128 if dtype == "bf16" else 20
    tq, tk = tiles
    B, H, Hkv = 3, 8, 2
    init = synth.gen_chunk(B, H, Hkv, 1, W, d, seed=21, std=0.5, dtype=dtype, p=[0] * B)
    init["cache_len"][:] = torch.tensor([0, 100, W], dtype=torch.int32)
    init["next_pos"][:] = torch.tensor([0, 140, 900], dtype=torch.int32)
    init["ring_start"][:] = torch.tensor([0, 7, 33], dtype=torch.int32)
    kc, vc = init["k_cache"].to(DEV), init["v_cache"].to(DEV)
    state = [init[x].clone().to(DEV) for x in ("ring_start", "cache_len", "next_pos")]
    ref = [f64(init["k_cache"]), f64(init["v_cache"])] + [init[x].numpy().copy() for x in
                                                          ("ring_start", "cache_len", "next_pos")]
    sc = 1 / math.sqrt(d)
    for step, Tq in enumerate((37, 64, 128, 5, 64, 100)):
        ci = synth.gen_chunk(B, H, Hkv, Tq, W, d, seed=100 + step, std=0.5, dtype=dtype,
                             p=[0] * B)
        q, kn, vn = (ci[x].to(DEV) for x in ("q", "k_new", "v_new"))
        meta = swa.chunk_meta_buffers(B, Tq, W, tq, tk, DEV)
        swa.swa_chunk_blockmask_dev(meta, *state)
        o = torch.full_like(q, float("nan"))
        swa.swa_prefill_chunk(q, kn, vn, kc, vc, *state, o, W, meta)
        ro, ref[0], ref[1], ref[2], ref[3], ref[4] = oracle.chunk(
            f64(ci["q"]), f64(ci["k_new"]), f64(ci["v_new"]), ref[0], ref[1], ref[2], ref[3],
            ref[4], W, sc)
        torch.cuda.synchronize()
        err = np.abs(f64(o) - ro)
        assert np.all(np.isfinite(f64(o))), step
        if dtype == "bf16":
            assert err.max() <= 2e-2 and err.mean() <= 2e-3, (step, float(err.max()))
        else:
            assert err.max() <= 1e-4, (step, float(err.max()))
    assert np.array_equal(f64(kc), ref[0]) and np.array_equal(f64(vc), ref[1])
    for i in range(3):
        assert np.array_equal(state[i].cpu().numpy(), ref[2 + i])
