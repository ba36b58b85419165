"""KV-cache estimator of the C library against the oracle, bit-exact (CPU only).

swa_layer_plan resolves a local:global ratio into per-layer windows and
swa_cache_bytes sums the persistent K/V bytes of such a stack
("LLMs from scratch, chapter 10: SWA and DSA", §10.2; per-layer windows as
in "Dense attention vs sliding-window sparse attention", §3.1).  Both are
host integer code, so every case runs without a GPU.
"""
import numpy as np
import pytest

import causal_sliding_window_swa_amd as swa
import oracle


@pytest.mark.parametrize("L,ratio", [(26, "5:1"), (32, (3, 1)), (7, "2:3"), (5, "0:1"),
                                     (5, "1:0"), (0, "1:1"), (1, "5:1"), (48, "1:7")])
def test_layer_plan_matches_oracle(L, ratio):
    a, b = (int(x) for x in (ratio.split(":") if isinstance(ratio, str) else ratio))
    W_layer, ns, nf = swa.swa_layer_plan(L, ratio, 512)
    flags, ons, onf = oracle.layer_plan(L, a, b)
    assert (ns, nf) == (ons, onf)
    assert np.array_equal(W_layer, np.where(flags == 1, 512, -1).astype(np.int32))


def test_cache_bytes_matches_oracle_sweep():
    rng = np.random.default_rng(2024)
    for _ in range(400):
        B = int(rng.integers(1, 129))
        G = int(rng.choice([1, 2, 4, 8, 32]))
        d = int(rng.choice([64, 128, 256]))
        s = int(rng.choice([1, 2, 4]))
        L = int(rng.integers(0, 81))
        T = int(rng.choice([0, 1, int(rng.integers(1, 1 << 20))]))
        W_layer = rng.choice([-1, 1, 128, 512, 1024, 4096, 131072], size=L).astype(np.int32)
        assert swa.swa_cache_bytes(B, G, d, s, T, W_layer) == \
            oracle.cache_bytes_layers(B, G, d, s, T, W_layer)


@pytest.mark.parametrize("L,ratio,W,T", [(26, "5:1", 1024, 32768), (26, "5:1", 1024, 100),
                                         (80, "3:1", 4096, 131072), (12, "1:0", 512, 8192)])
def test_plan_and_bytes_equal_the_pages_formula(L, ratio, W, T):
    """The plan fed to the byte count equals 2BGds[L_s min(T,W) + L_f T]."""
    W_layer, ns, nf = swa.swa_layer_plan(L, ratio, W)
    for B, G, d, s in [(1, 8, 128, 2), (64, 8, 128, 2), (3, 1, 64, 4)]:
        assert swa.swa_cache_bytes(B, G, d, s, T, W_layer) == \
            oracle.cache_bytes(B, G, d, s, T, W, ns, nf)


def test_decode_ring_bytes():
    """One windowed layer after at least W tokens holds exactly the ring
    caches that swa_decode streams: [B][Hkv][W][d] for K and for V."""
    B, G, W, d = 64, 8, 4096, 128
    ring = 2 * B * G * W * d * 2
    assert swa.swa_cache_bytes(B, G, d, 2, 131072, [W]) == ring == 1073741824


def test_estimator_validation():
    with pytest.raises(swa.SwaError):
        swa.swa_layer_plan(4, "0:0", 16)
    with pytest.raises(swa.SwaError):
        swa.swa_layer_plan(4, "-1:2", 16)
    with pytest.raises(swa.SwaError):
        swa.swa_layer_plan(4, "1:1", 0)
    with pytest.raises(swa.SwaError):
        swa.swa_layer_plan(-1, "1:1", 16)
    with pytest.raises(ValueError):
        swa.swa_layer_plan(4, "1:1:1", 16)
    with pytest.raises(swa.SwaError):
        swa.swa_cache_bytes(1, 1, 1, 2, 10, [0])
    with pytest.raises(swa.SwaError):
        swa.swa_cache_bytes(1, 1, 1, 2, 10, [-2])
    with pytest.raises(swa.SwaError):
        swa.swa_cache_bytes(1, 1, 1, 2, -1, [4])
    with pytest.raises(swa.SwaError):
        swa.swa_cache_bytes(0, 1, 1, 2, 10, [4])
    with pytest.raises(swa.SwaError, match="overflows"):
        swa.swa_cache_bytes(65535, 65535, 65535, 8, 1 << 40, [-1])
    assert swa.swa_cache_bytes(1, 1, 1, 2, 10, []) == 0
