"""Pins of the fp64 oracle: what the pages and plain mathematics fix.

Each ``pin_*`` function takes an ``oracle.Oracle`` and raises AssertionError when
the oracle disagrees with a value printed on a page (fixtures under
``tests/golden/``, each with its citation), a closed form, a textbook or library
routine (torch's scaled_dot_product_attention, numpy's tril), an invariant, or a
brute force built another way.  ``test_oracle_pins.py`` runs them against the
oracle; ``test_oracle_mutants.py`` runs them against copies of the oracle with a
planted mistake and requires that some pin fails for each.

Sources, by page title and section:
  [M003] "Weight sparsity vs attention sparsity" (AI-infra KB)
  [Ch10] "LLMs from scratch, chapter 10: SWA and DSA"
  [Blog] "Dense attention vs sliding-window sparse attention" (maplevalley)
"""
from __future__ import annotations

import json
import math
import os

import numpy as np
import torch

GOLD = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def gold(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


def _rng(seed):
    return np.random.default_rng(seed)


def _band_mask(nq_pos, nk_pos, W):
    """Visible pairs built from library triangles: causal triangle minus the
    causal triangle shifted W to the left (positions are 0..N-1 here)."""
    n = max(nq_pos, nk_pos)
    causal = np.tril(np.ones((n, n), dtype=bool), 0)
    too_old = np.tril(np.ones((n, n), dtype=bool), -W)
    return (causal & ~too_old)[:nq_pos, :nk_pos]


def _sdpa(q, k, v, mask=None, causal=False):
    """torch's scaled_dot_product_attention in fp64 on the CPU, GQA by
    repeating each KV head over its contiguous group of query heads."""
    q = torch.from_numpy(np.asarray(q, dtype=np.float64))
    k = torch.from_numpy(np.asarray(k, dtype=np.float64))
    v = torch.from_numpy(np.asarray(v, dtype=np.float64))
    G = q.shape[1] // k.shape[1]
    k = k.repeat_interleave(G, dim=1)
    v = v.repeat_interleave(G, dim=1)
    m = None if mask is None else torch.from_numpy(mask)
    out = torch.nn.functional.scaled_dot_product_attention(q, k, v, attn_mask=m,
                                                           is_causal=causal)
    return out.numpy()


def _page_ring_fill(positions_k, positions_v, W, d, Hkv=1):
    """Fill an empty W-slot ring with the rows of the given positions in order,
    by the update rule of [Blog §3.2]: below W rows, write the next free slot;
    when full, overwrite the start slot and advance the start by one mod W.
    positions_k/v: [Hkv, n, d].  Returns (k_ring, v_ring, start, len)."""
    kr = np.zeros((Hkv, W, d))
    vr = np.zeros((Hkv, W, d))
    start, length = 0, 0
    for t in range(positions_k.shape[1]):
        if length < W:
            slot = length
            length += 1
        else:
            slot = start
            start = (start + 1) % W
        kr[:, slot] = positions_k[:, t]
        vr[:, slot] = positions_v[:, t]
    return kr, vr, start, length


def _slot_position(s, ring_start, cache_len, next_pos, W):
    """Logical position held by ring slot s, or None for an unfilled slot:
    the row r-th oldest (r = (s - start) mod W) sits at next_pos - len + r."""
    r = (s - ring_start) % W
    if r >= cache_len:
        return None
    return next_pos - cache_len + r


# ---------------------------------------------------------------------------
# visibility rule and pair counts

def pin_window_visible_sets(O):
    """[M003 §03] rows 0,1,2,7 at N=8, W=3; [Ch10 §10.1] W=3,t=4 -> {2,3,4};
    [Ch10 §10.6 ex. 1] W=4,t=9 -> {6,7,8,9}.  Read off the tile-1 class grid,
    which is the visibility matrix itself."""
    g = gold("m003_window_counts.json")
    m = O.blockmask(1, g["N"], g["N"], g["W"], 1, 1)
    for row, vis in g["visible"].items():
        got = [j for j in range(g["N"]) if m["cls"][0, int(row), j] == 1]
        assert got == vis, (row, got, vis)
    for case in gold("ch10_windows.json")["visible_sets"]:
        n = case["t"] + 1
        m = O.blockmask(1, n, n, case["W"], 1, 1)
        got = [j for j in range(n) if m["cls"][0, case["t"], j] == 1]
        assert got == case["visible"], (case, got)


def pin_pair_counts(O):
    """[M003 §03]: 21 window pairs vs 36 causal at N=8, W=3, and the closed
    form N*W - W(W-1)/2 (N >= W-1; N(N+1)/2 below) for every N<=64, W<=70."""
    g = gold("m003_window_counts.json")
    assert O.blockmask(1, 8, 8, 3, 1, 1)["valid_pairs"] == g["valid_pairs_window"]
    assert O.blockmask(1, 8, 8, 8, 1, 1)["valid_pairs"] == g["valid_pairs_causal"]
    for N in range(1, 65):
        for W in (1, 2, 3, 5, 8, 13, 31, 32, 33, 63, 64, 65, 70):
            want = N * W - W * (W - 1) // 2 if N >= W - 1 else N * (N + 1) // 2
            got = O.blockmask(1, N, N, W, 7, 5)["valid_pairs"]
            assert got == want, (N, W, got, want)
    # the prefill workload's count (N=8192, W=512) against 33 558 528 causal
    assert O.blockmask(1, 8192, 8192, 512, 128, 128)["valid_pairs"] == 4063488
    assert 8192 * 8193 // 2 == 33558528


def pin_block_coverage(O):
    """[M003 §04]: N=8, W=3 gives 7 live blocks / 28 coordinates at tile 2 and
    3 blocks / 48 at tile 4.  Plus the prefill workload's counts from the
    interval argument: q-tile qt of size T sees key tiles max(0,qt-W/T)..qt,
    the diagonal one and (when it exists) the farthest one partial."""
    g = gold("m003_block_coverage.json")
    for t in g["tiles"]:
        m = O.blockmask(1, g["N"], g["N"], g["W"], t["tile"], t["tile"])
        assert m["valid_pairs"] == g["valid_pairs"]
        assert m["n_live"] == t["live_blocks"], (t, m["n_live"])
        assert m["covered_coords"] == t["covered_coords"], (t, m["covered_coords"])
    N, W = 8192, 512
    for T in (64, 128):
        nqt, r = N // T, W // T
        live = sum(min(qt, r) + 1 for qt in range(nqt))
        partial = sum(1 + (qt >= r) for qt in range(nqt))
        m = O.blockmask(1, N, N, W, T, T)
        assert (m["n_live"], m["n_full"], m["n_partial"]) == (live, live - partial, partial)
    assert (live, live - partial, partial) == (310, 186, 124)  # T=128
    m = O.blockmask(1, N, N, W, 64, 64)
    assert (m["n_live"], m["n_full"], m["n_partial"]) == (1116, 868, 248)


def pin_blockmask_by_aggregation(O):
    """Class grid, CSR and statistics against a numpy aggregation of the
    element visibility matrix (built from library triangles and the slot
    position formula), for ragged tiles, lengths and rings."""
    rng = _rng(7)
    cases = [
        dict(B=2, nq=37, nk_lin=37, W=9, tq=8, tk=5, q_len=[37, 21]),
        dict(B=1, nq=64, nk_lin=64, W=70, tq=16, tk=16, q_len=None),
        dict(B=3, nq=11, nk_lin=11, W=1, tq=3, tk=4, q_len=[11, 1, 6]),
    ]
    for c in cases:
        B, nq, W = c["B"], c["nq"], c["W"]
        m = O.blockmask(B, nq, c["nk_lin"], W, c["tq"], c["tk"], q_len=c["q_len"],
                        k_len=c["q_len"])
        band = _band_mask(nq, nq, W)
        _check_aggregation(m, [band & _valid2(nq, nq, None if c["q_len"] is None
                                               else c["q_len"][b]) for b in range(B)],
                           c["tq"], c["tk"])
    # ring + linear keys (chunked prefill geometry)
    for W, Tq, tq, tk in ((8, 5, 4, 4), (16, 16, 8, 4), (12, 3, 2, 3)):
        B = 3
        p = rng.integers(0, 3 * W, size=B)
        rs = rng.integers(0, W, size=B)
        cl = np.minimum(p, W)
        m = O.blockmask(B, Tq, Tq, W, tq, tk, q_start=p, k_start=p, W_ring=W,
                        ring_start=rs, cache_len=cl, next_pos=p)
        masks = []
        for b in range(B):
            kpos = [_slot_position(s, rs[b], cl[b], p[b], W) for s in range(W)]
            kpos += [p[b] + t for t in range(Tq)]
            M = np.zeros((Tq, W + Tq), dtype=bool)
            for i in range(Tq):
                for j, kp in enumerate(kpos):
                    if kp is not None:
                        M[i, j] = kp <= p[b] + i and kp >= p[b] + i - W + 1
            masks.append(M)
        _check_aggregation(m, masks, tq, tk)


def _valid2(nq, nk, L):
    if L is None:
        return np.ones((nq, nk), dtype=bool)
    v = np.zeros((nq, nk), dtype=bool)
    v[:L, :L] = True
    return v


def _check_aggregation(m, masks, tq, tk):
    B = len(masks)
    nq, nk = masks[0].shape
    nqt, nkt = -(-nq // tq), -(-nk // tk)
    row_ptr, col, ccls = [0], [], []
    pairs = covered = touched = full = part = 0
    for b, M in enumerate(masks):
        Mp = np.zeros((nqt * tq, nkt * tk), dtype=np.int64)
        Mp[:nq, :nk] = M
        area_q = np.minimum(tq, nq - np.arange(nqt) * tq)
        area_k = np.minimum(tk, nk - np.arange(nkt) * tk)
        cnt = Mp.reshape(nqt, tq, nkt, tk).sum(axis=(1, 3))
        area = area_q[:, None] * area_k[None, :]
        cls = np.where(cnt == 0, 0, np.where(cnt == area, 1, 2)).astype(np.uint8)
        assert np.array_equal(cls, m["cls"][b]), b
        for qt in range(nqt):
            live = np.nonzero(cls[qt])[0]
            col += list(live)
            ccls += list(cls[qt, live])
            row_ptr.append(len(col))
        pairs += int(M.sum())
        covered += int((area * (cls > 0)).sum())
        touched += int(M.any(axis=0).sum())
        full += int((cls == 1).sum())
        part += int((cls == 2).sum())
    assert np.array_equal(m["row_ptr"], np.array(row_ptr, dtype=np.int32))
    assert np.array_equal(m["col"], np.array(col, dtype=np.int32))
    assert np.array_equal(m["col_cls"], np.array(ccls, dtype=np.uint8))
    assert m["valid_pairs"] == pairs
    assert m["covered_coords"] == covered
    assert m["keys_touched"] == touched
    assert (m["n_full"], m["n_partial"], m["n_live"]) == (full, part, full + part)


# ---------------------------------------------------------------------------
# softmax semantics

def pin_zero_scores(O):
    """[M003 §05]: all scores 0, values 1..8: the causal output of the last
    row is 4.5 and the W=3 output is 7 (exact).  Every row is then the plain
    mean of the values it can see."""
    g = gold("m003_zero_scores.json")
    N = g["N"]
    rng = _rng(1)
    q = np.zeros((1, 1, N, 4))
    k = rng.standard_normal((1, 1, N, 4))
    v = np.repeat(np.array(g["values"], dtype=np.float64)[:, None], 4, axis=1)[None, None]
    o_causal = O.fwd(q, k, v, W=N, scale=0.5)
    o_win = O.fwd(q, k, v, W=3, scale=0.5)
    assert o_causal[0, 0, N - 1, 0] == g["last_row_output_causal"]
    assert o_win[0, 0, N - 1, 0] == g["last_row_output_window3"]
    for i in range(N):
        vis = g["values"][max(0, i - 2): i + 1]
        assert abs(o_win[0, 0, i, 0] - sum(vis) / len(vis)) <= 1e-15
        assert np.all(o_win[0, 0, i] == o_win[0, 0, i, 0])


def pin_dense_causal_reduction(O):
    """W >= N is plain causal attention: torch SDPA(is_causal=True), fp64,
    default scale 1/sqrt(d), with grouped KV heads repeated over their group."""
    rng = _rng(2)
    B, H, Hkv, N, d = 2, 4, 2, 37, 16
    q = rng.standard_normal((B, H, N, d))
    k = rng.standard_normal((B, Hkv, N, d))
    v = rng.standard_normal((B, Hkv, N, d))
    ref = _sdpa(q, k, v, causal=True)
    for W in (N, N + 1, 1000):
        got = O.fwd(q, k, v, W=W, scale=1.0 / math.sqrt(d))
        assert np.max(np.abs(got - ref)) <= 1e-12, W


def pin_window_mask_sdpa(O):
    """Windowed attention equals SDPA with the boolean mask of library
    triangles (causal minus causal shifted by W), for several W and GQA."""
    rng = _rng(3)
    B, H, Hkv, N, d = 1, 8, 2, 45, 8
    q = rng.standard_normal((B, H, N, d))
    k = rng.standard_normal((B, Hkv, N, d))
    v = rng.standard_normal((B, Hkv, N, d))
    for W in (1, 2, 3, 7, 16, 44):
        ref = _sdpa(q, k, v, mask=_band_mask(N, N, W))
        got = O.fwd(q, k, v, W=W, scale=1.0 / math.sqrt(d))
        assert np.max(np.abs(got - ref)) <= 1e-12, W


def pin_dense_table_with_mask(O):
    """[M003 §07]'s correctness baseline: the full score table, entries outside
    the window set to -inf, softmax, then V.  Also W=1 returns V itself."""
    rng = _rng(4)
    N, d, W, scale = 29, 6, 5, 0.3
    q = rng.standard_normal((1, 1, N, d))
    k = rng.standard_normal((1, 1, N, d))
    v = rng.standard_normal((1, 1, N, d))
    S = scale * q[0, 0] @ k[0, 0].T
    S[~_band_mask(N, N, W)] = -np.inf
    P = np.exp(S - S.max(axis=1, keepdims=True))
    ref = (P / P.sum(axis=1, keepdims=True)) @ v[0, 0]
    got = O.fwd(q, k, v, W=W, scale=scale)[0, 0]
    assert np.max(np.abs(got - ref)) <= 1e-12
    assert np.array_equal(O.fwd(q, k, v, W=1, scale=scale), v)


def pin_padding_rows(O):
    """Per-sequence valid lengths: padded rows are 0, valid rows equal the
    attention of the truncated sequence (SDPA with the window mask)."""
    rng = _rng(5)
    B, H, Hkv, N, d, W = 3, 2, 1, 33, 8, 6
    lens = [33, 17, 1]
    q = rng.standard_normal((B, H, N, d))
    k = rng.standard_normal((B, Hkv, N, d))
    v = rng.standard_normal((B, Hkv, N, d))
    got = O.fwd(q, k, v, W=W, scale=0.25, q_len=lens)
    for b, L in enumerate(lens):
        assert np.all(got[b, :, L:] == 0)
        mask = _band_mask(L, L, W)
        qb, kb, vb = q[b:b + 1, :, :L] * 0.25 * math.sqrt(d), k[b:b + 1, :, :L], v[b:b + 1, :, :L]
        ref = _sdpa(qb, kb, vb, mask=mask)
        assert np.max(np.abs(got[b:b + 1, :, :L] - ref)) <= 1e-12, b


def pin_causality_and_window_locality(O):
    """[Ch10 §10.5]: editing future values leaves past outputs unchanged, and
    so does editing keys that fell out of the window (bit-exact); editing a
    key inside the window changes the row."""
    rng = _rng(6)
    N, d, W, i = 24, 5, 5, 13
    q = rng.standard_normal((1, 1, N, d))
    k = rng.standard_normal((1, 1, N, d))
    v = rng.standard_normal((1, 1, N, d))
    base = O.fwd(q, k, v, W=W, scale=0.4)
    for j in list(range(0, i - W + 1)) + list(range(i + 1, N)):
        k2, v2 = k.copy(), v.copy()
        k2[0, 0, j] += 3.0
        v2[0, 0, j] -= 2.0
        o2 = O.fwd(q, k2, v2, W=W, scale=0.4)
        assert np.array_equal(o2[0, 0, i], base[0, 0, i]), j
        assert np.array_equal(o2[0, 0, :min(i, j)], base[0, 0, :min(i, j)])
    for j in range(i - W + 1, i + 1):
        v2 = v.copy()
        v2[0, 0, j] += 1.0
        assert not np.array_equal(O.fwd(q, k, v2, W=W, scale=0.4)[0, 0, i], base[0, 0, i])


def pin_normalisation(O):
    """Weights sum to one: constant V rows give that constant back."""
    rng = _rng(8)
    B, H, Hkv, N, d = 1, 2, 2, 40, 4
    q = rng.standard_normal((B, H, N, d)) * 3
    k = rng.standard_normal((B, Hkv, N, d)) * 3
    v = np.full((B, Hkv, N, d), 2.5)
    got = O.fwd(q, k, v, W=9, scale=0.5)
    assert np.max(np.abs(got - 2.5)) <= 1e-14


def pin_large_scores_stable(O):
    """[Ch10 §10.3] warns of NaN in softmax; large scores must stay finite and
    agree with SDPA (which subtracts the row maximum too)."""
    rng = _rng(9)
    B, H, N, d, W = 1, 1, 20, 16, 6
    q = rng.standard_normal((B, H, N, d)) * 40
    k = rng.standard_normal((B, H, N, d)) * 40
    v = rng.standard_normal((B, H, N, d))
    got = O.fwd(q, k, v, W=W, scale=1.0 / math.sqrt(d))
    assert np.all(np.isfinite(got))
    ref = _sdpa(q, k, v, mask=_band_mask(N, N, W))
    assert np.max(np.abs(got - ref)) <= 1e-9


# ---------------------------------------------------------------------------
# ring cache: chunked prefill and decode

def pin_chunked_equals_full(O):
    """[Ch10 §10.5]: 7 tokens, W=3, chunks [0:2],[2:5],[5:7] through the ring
    give exactly the full-sequence outputs (error 0)."""
    g = gold("ch10_windows.json")["chunked_vs_full"]
    N, W = g["N"], g["W"]
    rng = _rng(10)
    H, Hkv, d = 2, 1, 8
    q = rng.standard_normal((1, H, N, d))
    k = rng.standard_normal((1, Hkv, N, d))
    v = rng.standard_normal((1, Hkv, N, d))
    full = O.fwd(q, k, v, W=W, scale=0.35)
    kc = np.zeros((1, Hkv, W, d))
    vc = np.zeros((1, Hkv, W, d))
    rs, cl, npos = [0], [0], [0]
    outs = []
    for a, b in g["chunks"]:
        o, kc, vc, rs, cl, npos = O.chunk(q[:, :, a:b], k[:, :, a:b], v[:, :, a:b], kc, vc,
                                          rs, cl, npos, W=W, scale=0.35)
        outs.append(o)
    got = np.concatenate(outs, axis=2)
    assert np.max(np.abs(got - full)) == g["max_abs_error"]
    assert int(npos[0]) == N and int(cl[0]) == W and 0 <= int(rs[0]) < W


def pin_chunk_against_full_sequence(O):
    """A chunk at a random position p whose ring was filled by the page's
    update rule equals the full-sequence rows p..p+Tq-1 bit-exactly; after it
    the ring holds the last W positions (slot -> position by the start/len
    formula), including chunks longer than W and rings not yet full."""
    rng = _rng(11)
    H, Hkv, d, W = 4, 2, 6, 16
    for p, Tq in ((40, 8), (17, 16), (5, 3), (0, 7), (70, 2 * 16 + 3), (16, 1)):
        n = p + Tq
        q = rng.standard_normal((1, H, n, d))
        k = rng.standard_normal((1, Hkv, n, d))
        v = rng.standard_normal((1, Hkv, n, d))
        full = O.fwd(q, k, v, W=W, scale=0.3)
        kr, vr, start, length = _page_ring_fill(k[0, :, :p], v[0, :, :p], W, d, Hkv)
        o, kc, vc, rs, cl, npos = O.chunk(q[:, :, p:], k[:, :, p:], v[:, :, p:], kr[None],
                                          vr[None], [start], [length], [p], W=W, scale=0.3)
        assert np.array_equal(o, full[:, :, p:]), (p, Tq)
        assert int(npos[0]) == n and int(cl[0]) == min(W, n) and 0 <= int(rs[0]) < W
        for s in range(W):
            pos = _slot_position(s, int(rs[0]), int(cl[0]), int(npos[0]), W)
            if pos is None:
                continue
            assert n - W <= pos < n
            assert np.array_equal(kc[0, :, s], k[0, :, pos]) and np.array_equal(
                vc[0, :, s], v[0, :, pos]), (p, Tq, s)


def pin_chunk_union(O):
    """[Ch10 §10.2]: W=3, positions up to 4 cached, chunk 5,6,7 touches keys
    3..7 (5 = W+Tq-1); [Ch10 §10.6 ex. 2]: W=4, Tq=5 touches 8; the chunked
    prefill workload (W=4096, Tq=512) touches 4607 per request."""
    g = gold("ch10_windows.json")["chunk_unions"]
    c = g[0]
    W, p, Tq = c["W"], c["cached_upto"] + 1, len(c["chunk"])
    rs, cl = p % W, W   # a ring filled from empty by the page's rule
    m = O.blockmask(1, Tq, Tq, W, 1, 1, q_start=[p], k_start=[p], W_ring=W,
                    ring_start=[rs], cache_len=[cl], next_pos=[p])
    assert m["keys_touched"] == c["count"]
    touched = []
    for s in range(W):
        if m["cls"][0, :, s].any():
            touched.append(_slot_position(s, rs, cl, p, W))
    touched += [p + t for t in range(Tq) if m["cls"][0, :, W + t].any()]
    assert sorted(touched) == c["union"]
    c = g[1]
    m = O.blockmask(1, c["Tq"], c["Tq"], c["W"], 2, 2, q_start=[10], k_start=[10],
                    W_ring=c["W"], ring_start=[10 % c["W"]], cache_len=[c["W"]],
                    next_pos=[10])
    assert m["keys_touched"] == c["count"]
    for p in (4096, 5000, 65536):
        m = O.blockmask(1, 512, 512, 4096, 64, 64, q_start=[p], k_start=[p], W_ring=4096,
                        ring_start=[p % 4096], cache_len=[4096], next_pos=[p])
        assert m["keys_touched"] == 4096 + 512 - 1
        assert m["valid_pairs"] == 512 * 4096


def pin_decode_against_full_sequence(O):
    """A decode step (append, then attend) on a ring filled by the page's rule
    equals the full-sequence row of the new token bit-exactly, for full rings,
    rings still filling, and rings whose start is not 0."""
    rng = _rng(12)
    H, Hkv, d, W = 4, 2, 6, 8
    for qpos in (0, 3, 7, 8, 9, 30):
        n = qpos + 1
        q = rng.standard_normal((1, H, n, d))
        k = rng.standard_normal((1, Hkv, n, d))
        v = rng.standard_normal((1, Hkv, n, d))
        full = O.fwd(q, k, v, W=W, scale=0.3)
        kr, vr, start, length = _page_ring_fill(k[0, :, :qpos], v[0, :, :qpos], W, d, Hkv)
        o, kc, vc, rs, cl, npos = O.decode(q[:, :, qpos], k[:, :, qpos], v[:, :, qpos],
                                           kr[None], vr[None], [start], [length], [qpos],
                                           W=W, scale=0.3)
        assert np.array_equal(o[0], full[0, :, qpos]), qpos
        assert int(npos[0]) == n and int(cl[0]) == min(W, n) and 0 <= int(rs[0]) < W
        for s in range(W):
            pos = _slot_position(s, int(rs[0]), int(cl[0]), n, W)
            if pos is not None:
                assert np.array_equal(kc[0, :, s], k[0, :, pos])
    # a partly filled ring whose start index is not 0: logical row r sits in
    # slot (start + r) mod W; the appended row goes to the next one
    qpos, length, start = 5, 5, 6
    n = qpos + 1
    q = rng.standard_normal((1, H, n, d))
    k = rng.standard_normal((1, Hkv, n, d))
    v = rng.standard_normal((1, Hkv, n, d))
    full = O.fwd(q, k, v, W=W, scale=0.3)
    kr = np.full((1, Hkv, W, d), 7.0)
    vr = np.full((1, Hkv, W, d), -7.0)
    for r in range(length):
        kr[0, :, (start + r) % W] = k[0, :, r]
        vr[0, :, (start + r) % W] = v[0, :, r]
    o, kc, vc, rs, cl, npos = O.decode(q[:, :, qpos], k[:, :, qpos], v[:, :, qpos], kr, vr,
                                       [start], [length], [qpos], W=W, scale=0.3)
    assert np.array_equal(o[0], full[0, :, qpos])
    assert np.array_equal(kc[0, :, (start + length) % W], k[0, :, qpos])
    assert int(rs[0]) == start and int(cl[0]) == length + 1


def pin_decode_rotation_invariance(O):
    """Rotating the physical ring together with its start index changes
    nothing: slots carry logical positions, not their own index [M003 §06]."""
    rng = _rng(13)
    B, H, Hkv, d, W = 2, 4, 1, 8, 12
    q = rng.standard_normal((B, H, d))
    kn = rng.standard_normal((B, Hkv, d))
    vn = rng.standard_normal((B, Hkv, d))
    kc = rng.standard_normal((B, Hkv, W, d))
    vc = rng.standard_normal((B, Hkv, W, d))
    rs = np.array([3, 0])
    base = O.decode(q, kn, vn, kc, vc, rs, [W, W], [100, 12], W=W, scale=0.5)
    for shift in (1, 5, 11):
        kc2 = np.roll(kc, shift, axis=2)
        vc2 = np.roll(vc, shift, axis=2)
        got = O.decode(q, kn, vn, kc2, vc2, (rs + shift) % W, [W, W], [100, 12], W=W,
                       scale=0.5)
        assert np.array_equal(got[0], base[0]), shift
        assert np.array_equal(np.roll(got[1], -shift, axis=2), base[1])


# ---------------------------------------------------------------------------
# Gradients ([M003] §07: Q/K/V gradients of the masked attention are checked by
# finite differences; §08: outputs and gradients, boundaries, valid lengths).

def _bwd_case(seed, B=2, H=4, Hkv=2, N=13, d=5):
    rng = _rng(seed)
    return (rng.standard_normal((B, H, N, d)), rng.standard_normal((B, Hkv, N, d)),
            rng.standard_normal((B, Hkv, N, d)), rng.standard_normal((B, H, N, d)), rng)


def pin_bwd_finite_differences(O):
    """Directional derivatives of L = <o(q, k, v), dout> by central differences
    of the forward equal <grad, direction> for q, k and v, with grouped heads,
    padded sequences and windows shorter than, inside and beyond the length."""
    for seed, W, ql in ((40, 3, [13, 8]), (41, 1, [13, 13]), (42, 20, [9, 13]),
                        (43, 6, [1, 12])):
        q, k, v, do, rng = _bwd_case(seed)
        sc = 0.6
        dq, dk, dv, _ = O.bwd(q, k, v, do, W=W, scale=sc, q_len=ql)
        eps = 1e-5

        def loss(q_, k_, v_):
            return float((O.fwd(q_, k_, v_, W=W, scale=sc, q_len=ql) * do).sum())

        for name, g in (("q", dq), ("k", dk), ("v", dv)):
            x = {"q": q, "k": k, "v": v}
            e = rng.standard_normal(x[name].shape)
            xp, xm = dict(x), dict(x)
            xp[name] = x[name] + eps * e
            xm[name] = x[name] - eps * e
            fd = (loss(xp["q"], xp["k"], xp["v"]) - loss(xm["q"], xm["k"], xm["v"])) / (2 * eps)
            an = float((g * e).sum())
            assert abs(fd - an) <= 1e-6 * max(1.0, abs(fd)), (seed, name, fd, an)


def pin_bwd_window_mask_autograd(O):
    """Gradients and row log-sum-exp equal torch autograd through SDPA with the
    band mask of library triangles (fp64, grouped heads by repeat)."""
    rng = _rng(44)
    B, H, Hkv, N, d = 1, 6, 2, 33, 8
    q = rng.standard_normal((B, H, N, d))
    k = rng.standard_normal((B, Hkv, N, d))
    v = rng.standard_normal((B, Hkv, N, d))
    do = rng.standard_normal((B, H, N, d))
    sc = 1.0 / math.sqrt(d)
    for W in (1, 4, 17, 40):
        qt, kt, vt = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
        G = H // Hkv
        mask = torch.from_numpy(_band_mask(N, N, W))
        out = torch.nn.functional.scaled_dot_product_attention(
            qt, kt.repeat_interleave(G, dim=1), vt.repeat_interleave(G, dim=1), attn_mask=mask,
            scale=sc)
        out.backward(torch.from_numpy(do))
        dq, dk, dv, lse = O.bwd(q, k, v, do, W=W, scale=sc)
        for got, ref in ((dq, qt.grad), (dk, kt.grad), (dv, vt.grad)):
            assert np.max(np.abs(got - ref.numpy())) <= 1e-12, W
        scores = (torch.from_numpy(q) @ torch.from_numpy(k).repeat_interleave(G, dim=1)
                  .transpose(-1, -2)) * sc
        ref_lse = torch.logsumexp(scores.masked_fill(~mask, -math.inf), dim=-1)
        assert np.max(np.abs(lse - ref_lse.numpy())) <= 1e-12, W


def pin_bwd_closed_forms(O):
    """Sum over keys of dk is 0 (each row's dS sums to 0); sum over keys of dv
    equals the sum of dout over the group's valid rows (each row's P sums to
    1); equal keys give dq = 0; padded rows and keys get zero gradients and
    padded rows a log-sum-exp of -inf."""
    q, k, v, do, rng = _bwd_case(45, N=15)
    ql = [15, 6]
    W = 4
    dq, dk, dv, lse = O.bwd(q, k, v, do, W=W, scale=0.8, q_len=ql)
    G = q.shape[1] // k.shape[1]
    for b in range(2):
        L = ql[b]
        for g in range(k.shape[1]):
            assert np.max(np.abs(dk[b, g].sum(axis=0))) <= 1e-12
            want = do[b, g * G:(g + 1) * G, :L].sum(axis=(0, 1))
            assert np.max(np.abs(dv[b, g].sum(axis=0) - want)) <= 1e-12
        assert np.all(dq[b, :, L:] == 0) and np.all(dk[b, :, L:] == 0)
        assert np.all(dv[b, :, L:] == 0) and np.all(np.isneginf(lse[b, :, L:]))
        assert np.all(np.isfinite(lse[b, :, :L]))
    kc = np.broadcast_to(k[:, :, :1], k.shape).copy()
    dq2, _, _, _ = O.bwd(q, kc, v, do, W=W, scale=0.8, q_len=ql)
    assert np.max(np.abs(dq2)) <= 1e-12


def pin_bwd_selection_matches(O):
    """The selected-entry gradients equal the corresponding full gradients."""
    q, k, v, do, rng = _bwd_case(46, N=17)
    ql = [17, 11]
    W = 5
    dq, dk, dv, _ = O.bwd(q, k, v, do, W=W, scale=0.5, q_len=ql)
    qrows = [[0, 0, 0], [1, 3, 10], [1, 2, 16], [0, 1, 9]]
    keys = [[0, 1, 0], [1, 0, 10], [1, 1, 16], [0, 0, 12]]
    sq, sk, sv = O.bwd_sel(q, k, v, do, W=W, scale=0.5, qrows=qrows, keys=keys, q_len=ql)
    for r, (b, h, i) in enumerate(qrows):
        assert np.array_equal(sq[r], dq[b, h, i])
    for r, (b, g, j) in enumerate(keys):
        assert np.array_equal(sk[r], dk[b, g, j]) and np.array_equal(sv[r], dv[b, g, j])



def pin_fwd_rows_matches(O):
    """The selected-row forward equals the corresponding rows of the full
    forward, bit for bit: every (b, h, i) of a batch with grouped heads
    (H = 6 over Hkv = 2), padded lengths (rows past a length included) and
    attention sinks, requested in a shuffled order so that a row written to
    the wrong slot, a wrong batch length or a wrong KV group shows."""
    rng = _rng(47)
    B, H, Hkv, N, d = 3, 6, 2, 21, 5
    q = rng.standard_normal((B, H, N, d))
    k = rng.standard_normal((B, Hkv, N, d))
    v = rng.standard_normal((B, Hkv, N, d))
    ql = [21, 9, 1]
    rows = np.array([[b, h, i] for b in range(B) for h in range(H) for i in range(N)],
                    dtype=np.int32)
    rows = rows[rng.permutation(len(rows))]
    for W, S in ((4, 0), (7, 3), (30, 0), (1, 2)):
        full = O.fwd(q, k, v, W=W, scale=0.6, q_len=ql, n_sink=S)
        got = O.fwd_rows(q, k, v, W=W, scale=0.6, rows=rows, q_len=ql, n_sink=S)
        for r, (b, h, i) in enumerate(rows):
            assert np.array_equal(got[r], full[b, h, i]), (W, S, b, h, i)

# ---------------------------------------------------------------------------
# Attention sinks ("Sparse attention taxonomy" §3.2: StreamingLLM keeps the
# first 4 tokens besides the most recent W, a rule on positions only).

def _sink_mask(n, W, S):
    """Causal band of library triangles plus the causal part of the first S
    columns."""
    causal = np.tril(np.ones((n, n), dtype=bool), 0)
    cols = np.zeros((n, n), dtype=bool)
    cols[:, :S] = True
    return _band_mask(n, n, W) | (cols & causal)


def pin_sink_visible_sets(O):
    """The first 4 tokens plus the last W=3, written out from the page's rule:
    row 10 sees {0,1,2,3,8,9,10}; row 5 sees {0..5} (window 3..5 meets the
    sinks); row 2 sees {0,1,2}; row 0 sees {0}."""
    m = O.blockmask(1, 16, 16, 3, 1, 1, n_sink=4)
    vis = m["cls"][0] > 0
    want = {10: {0, 1, 2, 3, 8, 9, 10}, 5: {0, 1, 2, 3, 4, 5}, 2: {0, 1, 2}, 0: {0},
            15: {0, 1, 2, 3, 13, 14, 15}}
    for r, keys in want.items():
        assert set(np.nonzero(vis[r])[0].tolist()) == keys, r


def pin_sink_pair_counts_and_blocks(O):
    """Visible pairs = sum over rows of min(t+1, W) + max(0, min(S, t-W+1)); the
    block metadata with sinks equals a numpy aggregation of the element mask,
    with lengths and ragged tiles."""
    for N, W, S in ((40, 5, 4), (33, 1, 2), (64, 70, 4), (50, 8, 12)):
        m = O.blockmask(1, N, N, W, 16, 8, n_sink=S)
        want = sum(min(t + 1, W) + max(0, min(S, t - W + 1)) for t in range(N))
        assert m["valid_pairs"] == want, (N, W, S)
    N, W, S = 45, 6, 4
    L = [45, 30]
    m = O.blockmask(2, N, N, W, 16, 8, q_len=L, k_len=L, n_sink=S)
    masks = [_sink_mask(N, W, S) & _valid2(N, N, l) for l in L]
    _check_aggregation(m, masks, 16, 8)


def pin_sink_ring_metadata(O):
    """Chunk metadata with sinks (sink segment before the ring): every query at
    position t sees each position p <= t with p >= t-W+1 or p < S exactly once,
    among the positions the sink segment, the ring and the chunk hold, so the
    visible pairs are sum_t min(S, t+1) + max(0, t + 1 - max(S, t-W+1, oldest))
    (oldest = first position the ring holds).  The sink slots come first and
    are NS = S rounded up to tile_k."""
    for W, S, Tq, tk, states in ((16, 4, 7, 8, [(3, 16, 40), (0, 5, 5), (9, 16, 18), (0, 0, 0)]),
                                 (8, 3, 8, 4, [(2, 8, 30), (1, 4, 4), (5, 8, 9)])):
        for rs, cl, p0 in states:
            m = O.blockmask(1, Tq, Tq, W, 4, tk, q_start=[p0], k_start=[p0], W_ring=W,
                            ring_start=[rs], cache_len=[cl], next_pos=[p0], n_sink=S)
            oldest = p0 - cl
            want = sum(min(S, t + 1) + max(0, t + 1 - max(S, t - W + 1, oldest))
                       for t in range(p0, p0 + Tq))
            assert m["valid_pairs"] == want, (W, S, rs, cl, p0, m["valid_pairs"], want)
            ns = -(-S // tk) * tk
            assert m["cls"].shape[2] == (ns + W + Tq + tk - 1) // tk


def pin_sink_mask_sdpa(O):
    """Forward with sinks equals SDPA with the library-built mask; n_sink = 0
    gives the plain window exactly."""
    rng = _rng(60)
    B, H, Hkv, N, d = 1, 4, 2, 40, 8
    q = rng.standard_normal((B, H, N, d))
    k = rng.standard_normal((B, Hkv, N, d))
    v = rng.standard_normal((B, Hkv, N, d))
    for W, S in ((1, 4), (5, 4), (5, 1), (12, 20), (39, 4)):
        ref = _sdpa(q, k, v, mask=_sink_mask(N, W, S))
        got = O.fwd(q, k, v, W=W, scale=1.0 / math.sqrt(d), n_sink=S)
        assert np.max(np.abs(got - ref)) <= 1e-12, (W, S)
    a = O.fwd(q, k, v, W=5, scale=0.3, n_sink=0)
    b = O.fwd(q, k, v, W=5, scale=0.3)
    assert np.array_equal(a, b)


def pin_sink_decode_streams_like_full(O):
    """Streaming every token through decode with sinks (empty ring at the start)
    gives, at every step, the full-sequence sink forward's row for that
    position, including steps where the sinks are still inside the window."""
    rng = _rng(61)
    B, H, Hkv, T, d, W, S = 2, 4, 2, 23, 6, 5, 3
    q = rng.standard_normal((B, H, T, d))
    k = rng.standard_normal((B, Hkv, T, d))
    v = rng.standard_normal((B, Hkv, T, d))
    full = O.fwd(q, k, v, W=W, scale=0.5, n_sink=S)
    kc = np.zeros((B, Hkv, W, d))
    vc = np.zeros((B, Hkv, W, d))
    sk = np.zeros((B, Hkv, S, d))
    sv = np.zeros((B, Hkv, S, d))
    rs, cl, npos = np.array([0, 2]), np.array([0, 0]), np.array([0, 0])
    for t in range(T):
        out = O.decode(q[:, :, t], k[:, :, t], v[:, :, t], kc, vc, rs, cl, npos, W=W,
                       scale=0.5, n_sink=S, sink_k=sk, sink_v=sv)
        o, kc, vc, rs, cl, npos, sk, sv = out
        assert np.max(np.abs(o - full[:, :, t])) <= 1e-12, t
    assert np.array_equal(sk, k[:, :, :S].transpose(0, 1, 2, 3))


def pin_sink_chunk_streams_like_full(O):
    """Chunked prefill with sinks, chunks of several sizes mixed with decode
    steps from an empty ring, reproduces the full-sequence sink forward row by
    row; the sink cache ends up holding exactly the first S positions."""
    rng = _rng(62)
    B, H, Hkv, T, d, W, S = 2, 4, 2, 29, 6, 5, 3
    q = rng.standard_normal((B, H, T, d))
    k = rng.standard_normal((B, Hkv, T, d))
    v = rng.standard_normal((B, Hkv, T, d))
    full = O.fwd(q, k, v, W=W, scale=0.5, n_sink=S)
    kc = np.zeros((B, Hkv, W, d))
    vc = np.zeros((B, Hkv, W, d))
    sk = np.zeros((B, Hkv, S, d))
    sv = np.zeros((B, Hkv, S, d))
    rs, cl, npos = np.array([0, 4]), np.array([0, 0]), np.array([0, 0])
    t = 0
    for n in [2, 1, 4, 1, 5, 3, 1, 1, 5, 2, 4]:  # 1 = a decode step
        if n == 1:
            out = O.decode(q[:, :, t], k[:, :, t], v[:, :, t], kc, vc, rs, cl, npos, W=W,
                           scale=0.5, n_sink=S, sink_k=sk, sink_v=sv)
        else:
            out = O.chunk(q[:, :, t:t + n], k[:, :, t:t + n], v[:, :, t:t + n], kc, vc, rs, cl,
                          npos, W=W, scale=0.5, n_sink=S, sink_k=sk, sink_v=sv)
        o, kc, vc, rs, cl, npos, sk, sv = out
        ref = full[:, :, t] if n == 1 else full[:, :, t:t + n]
        assert np.max(np.abs(o - ref)) <= 1e-12, (t, n)
        t += n
    assert t == T
    assert np.array_equal(sk, k[:, :, :S]) and np.array_equal(sv, v[:, :, :S])


def pin_sink_bwd(O):
    """Gradients with sinks: central differences of the sink forward, and torch
    autograd through SDPA with the library-built mask."""
    rng = _rng(62)
    B, H, Hkv, N, d = 1, 4, 2, 21, 5
    q = rng.standard_normal((B, H, N, d))
    k = rng.standard_normal((B, Hkv, N, d))
    v = rng.standard_normal((B, Hkv, N, d))
    do = rng.standard_normal((B, H, N, d))
    W, S, sc = 4, 3, 0.7
    dq, dk, dv, lse = O.bwd(q, k, v, do, W=W, scale=sc, n_sink=S)
    qt, kt, vt = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    G = H // Hkv
    out = torch.nn.functional.scaled_dot_product_attention(
        qt, kt.repeat_interleave(G, dim=1), vt.repeat_interleave(G, dim=1),
        attn_mask=torch.from_numpy(_sink_mask(N, W, S)), scale=sc)
    out.backward(torch.from_numpy(do))
    for got, ref in ((dq, qt.grad), (dk, kt.grad), (dv, vt.grad)):
        assert np.max(np.abs(got - ref.numpy())) <= 1e-12
    eps = 1e-5
    e = rng.standard_normal(k.shape)
    lp = float((O.fwd(q, k + eps * e, v, W=W, scale=sc, n_sink=S) * do).sum())
    lm = float((O.fwd(q, k - eps * e, v, W=W, scale=sc, n_sink=S) * do).sum())
    assert abs((lp - lm) / (2 * eps) - float((dk * e).sum())) <= 1e-6
    rows = [[0, 1, 20], [0, 3, 2]]
    keys = [[0, 0, 1], [0, 1, 15], [0, 1, 2]]
    sq, sk_, sv_ = O.bwd_sel(q, k, v, do, W=W, scale=sc, qrows=rows, keys=keys, n_sink=S)
    for r, (b, h, i) in enumerate(rows):
        assert np.array_equal(sq[r], dq[b, h, i])
    for r, (b, g, j) in enumerate(keys):
        assert np.array_equal(sk_[r], dk[b, g, j]) and np.array_equal(sv_[r], dv[b, g, j])


# ---------------------------------------------------------------------------
# Packed variable-length batches ("Dense vs sliding-window sparse attention"
# §3.3 passes cu_seqlens; §5.2: windows are per sequence).

def pin_varlen_equals_per_sequence(O):
    """A packed batch equals the padded forward of each sequence on its own
    (exactly), and changing one sequence's K/V leaves every other sequence's
    output bit-identical (no window crosses a sequence boundary)."""
    rng = _rng(70)
    lens = [13, 1, 30, 7, 22]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    total, H, Hkv, d = int(cu[-1]), 4, 2, 6
    q = rng.standard_normal((total, H, d))
    k = rng.standard_normal((total, Hkv, d))
    v = rng.standard_normal((total, Hkv, d))
    for W, S in ((4, 0), (1, 0), (9, 3), (40, 0)):
        got = O.fwd_varlen(q, k, v, cu, W=W, scale=0.4, n_sink=S)
        for b, L in enumerate(lens):
            sl = slice(int(cu[b]), int(cu[b + 1]))
            ref = O.fwd(q[sl].transpose(1, 0, 2)[None], k[sl].transpose(1, 0, 2)[None],
                        v[sl].transpose(1, 0, 2)[None], W=W, scale=0.4, n_sink=S)
            assert np.array_equal(got[sl], ref[0].transpose(1, 0, 2)), (W, S, b)
    base = O.fwd_varlen(q, k, v, cu, W=5, scale=0.4)
    k2, v2 = k.copy(), v.copy()
    k2[cu[2]:cu[3]] += 3.0
    v2[cu[2]:cu[3]] -= 2.0
    got = O.fwd_varlen(q, k2, v2, cu, W=5, scale=0.4)
    keep = np.ones(total, dtype=bool)
    keep[cu[2]:cu[3]] = False
    assert np.array_equal(got[keep], base[keep])
    assert not np.array_equal(got[~keep], base[~keep])


def pin_cache_dense_example(O):
    """[Blog §2.1] prints the dense KV cache of a 32-layer, 32-head, d=128
    fp16 model at t=8192: one K about 67 MB, K+V about 134 MB per layer,
    about 4.3 GB over the layers.  Dense layers are global layers of the
    estimate ([Ch10 §10.2] with L_s = 0)."""
    g = gold("blog_dense_kv_cache.json")
    B, G, d, s, T, L = (g[k] for k in ("B", "heads", "head_dim", "bytes_per_element", "t",
                                       "layers"))
    one_layer = O.cache_bytes(B, G, d, s, T, 1, 0, 1)
    assert round(one_layer / 2 / 1e6) == g["one_K_MB"], one_layer
    assert round(one_layer / 1e6) == g["K_plus_V_per_layer_MB"], one_layer
    total = O.cache_bytes(B, G, d, s, T, 1, 0, L)
    assert round(total / 1e9, 1) == g["all_layers_GB"], total
    assert O.cache_bytes_layers(B, G, d, s, T, [-1] * L) == total
    # a window at least as long as the text changes nothing [Ch10 §10.2]
    assert O.cache_bytes(B, G, d, s, T, T, L, 0) == total
    assert O.cache_bytes_layers(B, G, d, s, T, [T + 5] * L) == total


def pin_cache_window_bound(O):
    """[Ch10 §10.2]: a windowed layer keeps at most its last W positions, a
    per-layer bound of 2BWGds bytes once T >= W.  Checked against the byte
    size of the ring cache tensors themselves (numpy nbytes of [B,G,W,d]
    arrays, K and V): at B=64, G=8, W=4096, d=128 in bf16 that is the
    1 073 741 824 bytes one decode step reads.  Below W tokens the layer
    holds only T rows, like a global layer."""
    B, G, W, d = 64, 8, 4096, 128
    ring = 2 * np.zeros((B, G, W, d), dtype=np.float16).nbytes
    assert ring == 1073741824
    for T in (W, W + 1, 131072):
        assert O.cache_bytes(B, G, d, 2, T, W, 1, 0) == ring
        assert O.cache_bytes_layers(B, G, d, 2, T, [W]) == ring
    for T in (0, 1, 77, W - 1):
        part = 2 * np.zeros((B, G, T, d), dtype=np.float16).nbytes
        assert O.cache_bytes(B, G, d, 2, T, W, 1, 0) == part
        assert O.cache_bytes(B, G, d, 2, T, W, 0, 1) == part
        assert O.cache_bytes_layers(B, G, d, 2, T, [W, -1]) == 2 * part
    # linear in each of B, G, d, s and in the layer counts
    base = O.cache_bytes(3, 5, 7, 1, 1000, 300, 2, 3)
    assert base == 2 * O.cache_bytes(3, 5, 7, 1, 1000, 300, 1, 0) + \
        3 * O.cache_bytes(3, 5, 7, 1, 1000, 300, 0, 1)
    assert O.cache_bytes(3, 5, 7, 4, 1000, 300, 2, 3) == 4 * base
    assert O.cache_bytes(6, 5, 7, 1, 1000, 300, 2, 3) == 2 * base


def pin_layer_plan(O):
    """[Ch10 §10.2]: a local:global ratio is resolved into whole layers.
    The pattern is checked against numpy's tile of one period; the counts
    against L*a/(a+b) when the period divides L, and against the example of
    26 layers at 5:1 (22 + 4, where 26*5/6 is not a whole number)."""
    for L, a, b in [(26, 5, 1), (12, 1, 1), (32, 3, 1), (7, 2, 3), (5, 0, 1), (5, 1, 0),
                    (1, 5, 1), (0, 2, 2), (40, 1, 7)]:
        flags, ns, nf = O.layer_plan(L, a, b)
        ref = np.tile(np.array([1] * a + [0] * b, dtype=np.uint8), L // (a + b) + 1)[:L]
        assert np.array_equal(flags, ref), (L, a, b)
        assert ns + nf == L and ns == int(ref.sum())
        if L % (a + b) == 0:
            assert ns * (a + b) == L * a
    assert O.layer_plan(26, 5, 1)[1:] == (22, 4)
    # the plan's counts in the one-W estimate equal the per-layer sum
    flags, ns, nf = O.layer_plan(26, 5, 1)
    W_layer = np.where(flags == 1, 1024, -1)
    for T in (100, 1024, 5000):
        assert O.cache_bytes_layers(2, 8, 128, 2, T, W_layer) == \
            O.cache_bytes(2, 8, 128, 2, T, 1024, ns, nf)
    # [Blog §3.1]: per-layer windows (12 layers at 256, 8 at 512, 12 at 1024)
    # are the sum of three single-window stacks
    bands = [256] * 12 + [512] * 8 + [1024] * 12
    for T in (200, 700, 4096):
        assert O.cache_bytes_layers(1, 32, 128, 2, T, bands) == sum(
            O.cache_bytes(1, 32, 128, 2, T, w, n, 0) for w, n in ((256, 12), (512, 8),
                                                                   (1024, 12)))


PINS = [
    pin_window_visible_sets,
    pin_pair_counts,
    pin_block_coverage,
    pin_blockmask_by_aggregation,
    pin_zero_scores,
    pin_dense_causal_reduction,
    pin_window_mask_sdpa,
    pin_dense_table_with_mask,
    pin_padding_rows,
    pin_causality_and_window_locality,
    pin_normalisation,
    pin_large_scores_stable,
    pin_chunked_equals_full,
    pin_chunk_against_full_sequence,
    pin_chunk_union,
    pin_decode_against_full_sequence,
    pin_decode_rotation_invariance,
    pin_bwd_finite_differences,
    pin_bwd_window_mask_autograd,
    pin_bwd_closed_forms,
    pin_bwd_selection_matches,
    pin_fwd_rows_matches,
    pin_sink_visible_sets,
    pin_sink_pair_counts_and_blocks,
    pin_sink_ring_metadata,
    pin_sink_mask_sdpa,
    pin_sink_decode_streams_like_full,
    pin_sink_chunk_streams_like_full,
    pin_sink_bwd,
    pin_varlen_equals_per_sequence,
    pin_cache_dense_example,
    pin_cache_window_bound,
    pin_layer_plan,
]
