"""Library metadata builder against the oracle's brute force: bit-exact class
grids, CSR arrays and statistics (CPU only, host code of libswa.so)."""
import numpy as np
import pytest

import causal_sliding_window_swa_amd as swa
import oracle
from causal_sliding_window_swa_amd import synth

STATS = oracle.STAT_NAMES


def _same(a, b):
    assert np.array_equal(a["cls"], b["cls"])
    assert np.array_equal(a["row_ptr"], b["row_ptr"])
    assert np.array_equal(a["col"], b["col"])
    assert np.array_equal(a["col_cls"], b["col_cls"])
    for s in STATS:
        assert a[s] == b[s], (s, a[s], b[s])


def both(*args, **kw):
    lib = swa.swa_blockmask_build(*args, **kw)
    ref = oracle.blockmask(*args, **kw)
    _same(lib, ref)
    return lib


@pytest.mark.parametrize("tile", [1, 2, 3, 4, 8])
def test_tiny_workload(tile):
    m = both(1, 8, 8, 3, tile, tile)
    assert m["valid_pairs"] == 21


@pytest.mark.parametrize("tq,tk", [(128, 64), (64, 64), (128, 128), (64, 32)])
def test_prefill_workload(tq, tk):
    m = both(1, 8192, 8192, 512, tq, tk)
    assert m["valid_pairs"] == 4063488


def test_prefill_gqa_workload():
    inp = synth.make("prefill_gqa", H=1, Hkv=1, d=1)  # same lengths, tiny tensors
    L = inp["q_len"].numpy()
    m = both(4, 32768, 32768, 4096, 128, 64, q_len=L, k_len=L)
    want = sum(int(l) * 4096 - 4096 * 4095 // 2 for l in L)
    assert m["valid_pairs"] == want


@pytest.mark.parametrize("tq,tk", [(128, 64), (64, 64)])
def test_chunk_workload(tq, tk):
    inp = synth.make("chunk", H=1, Hkv=1, d=1)
    p = inp["next_pos"].numpy()
    m = both(8, 512, 512, 4096, tq, tk, q_start=p, k_start=p, W_ring=4096,
             ring_start=inp["ring_start"].numpy(), cache_len=inp["cache_len"].numpy(),
             next_pos=p)
    assert m["keys_touched"] == 8 * 4607
    assert m["valid_pairs"] == 8 * 512 * 4096


def test_random_small_cases():
    rng = np.random.default_rng(0)
    for _ in range(300):
        B = int(rng.integers(1, 4))
        W = int(rng.integers(1, 40))
        tq = int(rng.integers(1, 9))
        tk = int(rng.integers(1, 9))
        if rng.random() < 0.5:
            N = int(rng.integers(1, 70))
            L = rng.integers(0, N + 1, size=B)
            both(B, N, N, W, tq, tk, q_len=L, k_len=L)
        else:
            Wr = tk * int(rng.integers(1, 6))
            Tq = int(rng.integers(1, 30))
            cl = rng.integers(0, Wr + 1, size=B)
            p = cl + rng.integers(0, 50, size=B)
            rs = rng.integers(0, Wr, size=B)
            both(B, Tq, Tq, W, tq, tk, q_start=p, k_start=p, W_ring=Wr, ring_start=rs,
                 cache_len=cl, next_pos=p)


def test_random_small_cases_with_sinks():
    """Attention sinks ("Sparse attention taxonomy" §3.2): bit-exact metadata
    against the brute force, with lengths, ragged tiles and sink counts below,
    at and beyond the window and the length."""
    rng = np.random.default_rng(1)
    for _ in range(200):
        B = int(rng.integers(1, 4))
        W = int(rng.integers(1, 30))
        S = int(rng.integers(1, 40))
        tq = int(rng.integers(1, 9))
        tk = int(rng.integers(1, 9))
        N = int(rng.integers(1, 70))
        L = rng.integers(0, N + 1, size=B)
        both(B, N, N, W, tq, tk, q_len=L, k_len=L, n_sink=S)


def test_prefill_workload_with_sinks():
    both(1, 8192, 8192, 512, 128, 64, n_sink=4)


def test_random_ring_cases_with_sinks():
    """The chunk's key axis with sinks: a sink segment of S slots (rounded up
    to the key tile) before the ring; rings still filling, full, holding
    positions below S or not."""
    rng = np.random.default_rng(2)
    for _ in range(300):
        B = int(rng.integers(1, 4))
        W = int(rng.integers(1, 40))
        S = int(rng.integers(1, 20))
        tq = int(rng.integers(1, 9))
        tk = int(rng.integers(1, 9))
        Wr = tk * int(rng.integers(1, 6))
        Tq = int(rng.integers(1, 30))
        cl = rng.integers(0, Wr + 1, size=B)
        p = cl + rng.integers(0, 50, size=B)
        rs = rng.integers(0, Wr, size=B)
        both(B, Tq, Tq, W, tq, tk, q_start=p, k_start=p, W_ring=Wr, ring_start=rs,
             cache_len=cl, next_pos=p, n_sink=S)


@pytest.mark.parametrize("tq,tk", [(128, 64), (64, 64)])
def test_chunk_workload_with_sinks(tq, tk):
    inp = synth.make("chunk", H=1, Hkv=1, d=1)
    p = inp["next_pos"].numpy()
    m = both(8, 512, 512, 4096, tq, tk, q_start=p, k_start=p, W_ring=4096,
             ring_start=inp["ring_start"].numpy(), cache_len=inp["cache_len"].numpy(),
             next_pos=p, n_sink=4)
    # every query sees its W window plus 4 sinks far behind it
    assert m["valid_pairs"] == 8 * 512 * (4096 + 4)
