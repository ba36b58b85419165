"""GPU edge cases through the C ABI against the fp64 oracle: scores large
enough to leave the fixed softmax reference's range (the kernels' rescale
path, both overflow and underflow), empty and one-token sequences, empty
sequences inside a packed batch, a decode step on an empty ring, a chunk as
long as the ring, and the backward of an empty sequence.  Bars as in
test_gpu_parity (bf16 max-abs 2e-2, mean-abs 2e-3; fp32 1e-4).
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


def f64(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def check(got, ref, bf16, where):
    got = f64(got) if torch.is_tensor(got) else got
    assert np.all(np.isfinite(got)), "non-finite " + where
    err = np.abs(got - ref)
    if bf16:
        assert err.max() <= 2e-2, (where, float(err.max()))
        assert err.mean() <= 2e-3, (where, float(err.mean()))
    else:
        assert err.max() <= 1e-4, (where, float(err.max()))


def _qkv(B, H, Hkv, N, d, seed, qk_std, bias, tdt):
    """q, k with a large common direction (scores of magnitude ~ qk_std^2 * d
    * scale, positive for bias > 0, negative for bias < 0), v small."""
    g = torch.Generator().manual_seed(seed)
    u = torch.randn(d, generator=g)
    u = u / u.norm()
    q = torch.randn(B, H, N, d, generator=g) * 0.3 + qk_std * math.sqrt(d) * u
    k = torch.randn(B, Hkv, N, d, generator=g) * 0.3 + bias * qk_std * math.sqrt(d) * u
    k = k + torch.randn(B, Hkv, N, 1, generator=g) * qk_std * math.sqrt(d) * 0.2 * u
    v = torch.randn(B, Hkv, N, d, generator=g) * 0.5
    return q.to(tdt), k.to(tdt), v.to(tdt)


def _fwd(q, k, v, W, tq, tk, q_len=None, lse=False):
    B, H, N, d = q.shape
    L = None if q_len is None else np.asarray(q_len, dtype=np.int32)
    meta = swa.swa_blockmask_build(B, N, N, W, tq, tk, q_len=L, k_len=L)
    md = swa.meta_to_device(meta, DEV)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    od = torch.full_like(qd, float("nan"))
    ls = torch.full((B, H, N), float("nan"), device=DEV) if lse else None
    qld = None if L is None else torch.from_numpy(L).to(DEV)
    swa.swa_fwd(qd, kd, vd, od, W, md, q_len=qld, lse=ls)
    torch.cuda.synchronize()
    return od, ls


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("qk_std,bias", [(1.5, 1.0), (3.0, 1.0), (1.5, -1.0), (3.0, -1.0)])
@pytest.mark.parametrize("W", [64, 600])
def test_fwd_large_scores(dtype, qk_std, bias, W):
    """Scores far above (bias > 0) or below (bias < 0) the fixed reference 0:
    row sums of a tile leave [2^-32, 2^32], so the kernel takes a real maximum
    and rescales O and the row sum; the result must not change."""
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    d = 128 if dtype == "bf16" else 32
    tq, tk = (128, 64) if dtype == "bf16" else (32, 16)
    q, k, v = _qkv(2, 4, 2, 700, d, seed=int(qk_std * 10) + W, qk_std=qk_std, bias=bias,
                   tdt=tdt)
    sc = 1 / math.sqrt(d)
    o, ls = _fwd(q, k, v, W, tq, tk, lse=True)
    ref = oracle.fwd(f64(q), f64(k), f64(v), W, sc)
    check(o, ref, dtype == "bf16", "large scores %s std=%g bias=%g W=%d" % (dtype, qk_std, bias, W))
    # the row log-sum-exp of those scores, against a direct fp64 evaluation
    # on a few rows (relative: the values are in the hundreds)
    qq, kk = f64(q), f64(k)
    for (b, h, i) in [(0, 0, 0), (1, 3, 699), (0, 2, 333), (1, 1, W - 1)]:
        j0 = max(0, i - W + 1)
        s = qq[b, h, i] @ kk[b, h // 2, j0:i + 1].T * sc
        want = s.max() + math.log(np.exp(s - s.max()).sum())
        got = float(ls[b, h, i])
        assert abs(got - want) <= 1e-3 * max(1.0, abs(want)), (b, h, i, got, want)


@pytest.mark.parametrize("bias", [1.0, -1.0])
def test_chunk_and_decode_large_scores(bias):
    """The chunk (tile kernel over the ring) and decode (split softmax) with
    scores far from the fixed reference."""
    W, Tq, d = 256, 100, 128
    B, H, Hkv = 2, 8, 2
    q, k, v = _qkv(B, H, Hkv, W + Tq, d, seed=77, qk_std=3.0, bias=bias, tdt=torch.bfloat16)
    inp = dict(q=q[:, :, W:].contiguous(), k_new=k[:, :, W:].contiguous(),
               v_new=v[:, :, W:].contiguous(), k_cache=k[:, :, :W].contiguous(),
               v_cache=v[:, :, :W].contiguous(),
               ring_start=torch.zeros(B, dtype=torch.int32),
               cache_len=torch.full((B,), W, dtype=torch.int32),
               next_pos=torch.full((B,), W, dtype=torch.int32))
    p = inp["next_pos"].numpy()
    meta = swa.swa_blockmask_build(B, Tq, Tq, W, 128, 64, q_start=p, k_start=p, W_ring=W,
                                   ring_start=inp["ring_start"].numpy(),
                                   cache_len=inp["cache_len"].numpy(), next_pos=p)
    md = swa.meta_to_device(meta, DEV)
    dev = {x: inp[x].to(DEV) for x in inp}
    o = torch.full_like(dev["q"], float("nan"))
    swa.swa_prefill_chunk(dev["q"], dev["k_new"], dev["v_new"], dev["k_cache"], dev["v_cache"],
                          dev["ring_start"], dev["cache_len"], dev["next_pos"], o, W, md)
    torch.cuda.synchronize()
    ref = oracle.chunk(f64(inp["q"]), f64(inp["k_new"]), f64(inp["v_new"]),
                       f64(inp["k_cache"]), f64(inp["v_cache"]), inp["ring_start"].numpy(),
                       inp["cache_len"].numpy(), inp["next_pos"].numpy(), W, 1 / math.sqrt(d))
    check(o, ref[0], True, "chunk large scores bias=%g" % bias)
    # one decode step after the chunk, on the updated rings
    g = torch.Generator().manual_seed(5)
    qn = (q[:, :, -1] + 0.01 * torch.randn(B, H, d, generator=g)).to(torch.bfloat16)
    kn, vn = k[:, :, -1].contiguous(), v[:, :, -1].contiguous()
    ws = torch.empty(swa.swa_decode_workspace_size(B, H, d, W) // 4 + 4, dtype=torch.float32,
                     device=DEV)
    od = torch.full((B, H, d), float("nan"), dtype=torch.bfloat16, device=DEV)
    swa.swa_decode(qn.to(DEV), kn.to(DEV), vn.to(DEV), dev["k_cache"], dev["v_cache"],
                   dev["ring_start"], dev["cache_len"], dev["next_pos"], od, ws, W)
    torch.cuda.synchronize()
    refd = oracle.decode(f64(qn), f64(kn), f64(vn), ref[1], ref[2], ref[3], ref[4], ref[5], W,
                         1 / math.sqrt(d))
    check(od, refd[0], True, "decode large scores bias=%g" % bias)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_fwd_empty_and_one_token_sequences(dtype):
    """Lengths 0 (every row padding: output 0, log-sum-exp -inf), 1 and a
    ragged one; also N = 1."""
    tdt = "bf16" if dtype == "bf16" else "f32"
    d = 128 if dtype == "bf16" else 12
    tq, tk = (128, 64) if dtype == "bf16" else (16, 8)
    inp = synth.gen_fwd(3, 4, 2, 129, d, seed=91, dtype=tdt)
    L = np.array([0, 1, 77], dtype=np.int32)
    for b, l in enumerate(L):
        for x in ("q", "k", "v"):
            inp[x][b, :, l:] = 0
    o, ls = _fwd(inp["q"], inp["k"], inp["v"], 20, tq, tk, q_len=L, lse=True)
    ref = oracle.fwd(f64(inp["q"]), f64(inp["k"]), f64(inp["v"]), 20, 1 / math.sqrt(d),
                     q_len=L)
    check(o, ref, dtype == "bf16", "lengths 0/1/77 " + dtype)
    assert torch.all(o[0] == 0) and torch.all(torch.isneginf(ls[0]))
    assert torch.all(torch.isneginf(ls[1, :, 1:])) and torch.all(torch.isfinite(ls[1, :, 0]))
    one = synth.gen_fwd(2, 4, 4, 1, d, seed=92, dtype=tdt)
    for W in (1, 5):
        o1, _ = _fwd(one["q"], one["k"], one["v"], W, tq, tk)
        # a single visible key: the output is its V row
        check(o1, f64(one["v"]), dtype == "bf16", "N=1 W=%d %s" % (W, dtype))


def test_varlen_with_empty_sequences():
    lens = [0, 100, 0, 65, 1]
    d, H, Hkv, W = 128, 4, 2, 48
    total, mx = sum(lens), max(lens)
    g = torch.Generator().manual_seed(93)
    q = (torch.randn(total, H, d, generator=g) * 0.5).to(torch.bfloat16)
    k = (torch.randn(total, Hkv, d, generator=g) * 0.5).to(torch.bfloat16)
    v = (torch.randn(total, Hkv, d, generator=g) * 0.5).to(torch.bfloat16)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    meta = swa.swa_blockmask_build(len(lens), mx, mx, W, 128, 64, q_len=np.array(lens),
                                   k_len=np.array(lens))
    md = swa.meta_to_device(meta, DEV)
    o = torch.full((total, H, d), float("nan"), dtype=torch.bfloat16, device=DEV)
    swa.swa_fwd_varlen(q.to(DEV), k.to(DEV), v.to(DEV), o, W, md, torch.from_numpy(cu).to(DEV))
    torch.cuda.synchronize()
    ref = oracle.fwd_varlen(f64(q), f64(k), f64(v), cu, W, 1 / math.sqrt(d))
    check(o, ref, True, "varlen with empty sequences")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_decode_first_token_and_full_chunk(dtype):
    """A decode step on an empty ring sees only its own token (output = its V
    row); a chunk as long as the ring on an empty ring."""
    tdt = "bf16" if dtype == "bf16" else "f32"
    d = 128 if dtype == "bf16" else 16
    W, B, H, Hkv = 64, 2, 8, 2
    inp = synth.gen_decode(B, H, Hkv, W, d, seed=94, dtype=tdt, pos_lo=0, pos_hi=0)
    inp["cache_len"][:] = 0
    inp["next_pos"][:] = 0
    dev = {x: inp[x].to(DEV).contiguous() for x in inp}
    ws = torch.empty(swa.swa_decode_workspace_size(B, H, d, W) // 4 + 4, dtype=torch.float32,
                     device=DEV)
    o = torch.full_like(dev["q"], float("nan"))
    swa.swa_decode(dev["q"], dev["k_new"], dev["v_new"], dev["k_cache"], dev["v_cache"],
                   dev["ring_start"], dev["cache_len"], dev["next_pos"], o, ws, W)
    torch.cuda.synchronize()
    want = np.repeat(f64(inp["v_new"]), H // Hkv, axis=1)
    check(o, want, dtype == "bf16", "first token " + dtype)
    assert np.array_equal(dev["cache_len"].cpu().numpy(), [1, 1])
    # a chunk of W tokens on an empty ring
    ch = synth.gen_chunk(B, H, Hkv, W, W, d, seed=95, dtype=tdt, p=[0, 0])
    ch["cache_len"][:] = 0
    ch["ring_start"][:] = torch.tensor([0, 17], dtype=torch.int32)
    p = ch["next_pos"].numpy()
    tq, tk = (128, 64) if dtype == "bf16" else (32, 16)
    meta = swa.swa_blockmask_build(B, W, W, W, tq, tk, q_start=p, k_start=p, W_ring=W,
                                   ring_start=ch["ring_start"].numpy(),
                                   cache_len=ch["cache_len"].numpy(), next_pos=p)
    md = swa.meta_to_device(meta, DEV)
    dv = {x: ch[x].to(DEV).contiguous() for x in ch}
    oc = torch.full_like(dv["q"], float("nan"))
    swa.swa_prefill_chunk(dv["q"], dv["k_new"], dv["v_new"], dv["k_cache"], dv["v_cache"],
                          dv["ring_start"], dv["cache_len"], dv["next_pos"], oc, W, md)
    torch.cuda.synchronize()
    ref = oracle.chunk(f64(ch["q"]), f64(ch["k_new"]), f64(ch["v_new"]), f64(ch["k_cache"]),
                       f64(ch["v_cache"]), ch["ring_start"].numpy(), ch["cache_len"].numpy(),
                       ch["next_pos"].numpy(), W, 1 / math.sqrt(d))
    check(oc, ref[0], dtype == "bf16", "full chunk on empty ring " + dtype)
    assert np.array_equal(f64(dv["k_cache"]), ref[1])
    assert np.array_equal(dv["ring_start"].cpu().numpy(), ref[3])


def test_bwd_empty_sequence():
    """Backward with a sequence of length 0 beside a ragged one: zero
    gradients for the empty sequence, parity for the other."""
    inp = synth.gen_bwd(2, 4, 2, 200, 128, seed=96)
    L = np.array([0, 131], dtype=np.int32)
    for b, l in enumerate(L):
        for x in ("q", "k", "v", "dout"):
            inp[x][b, :, l:] = 0
    B, H, N, d = inp["q"].shape
    meta = swa.swa_blockmask_build(B, N, N, 40, 128, 64, q_len=L, k_len=L)
    md = swa.meta_to_device(meta, DEV)
    q, k, v, do = (inp[x].to(DEV) for x in ("q", "k", "v", "dout"))
    qld = torch.from_numpy(L).to(DEV)
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=DEV)
    swa.swa_fwd(q, k, v, o, 40, md, q_len=qld, lse=lse)
    dq, dk, dv = (torch.full_like(t, float("nan")) for t in (q, k, v))
    ws = torch.empty(swa.swa_bwd_workspace_size(B, H, N) // 4, dtype=torch.float32, device=DEV)
    swa.swa_bwd(q, k, v, o, do, lse, dq, dk, dv, ws, 40, md, q_len=qld)
    torch.cuda.synchronize()
    rq, rk, rv, _ = oracle.bwd(f64(inp["q"]), f64(inp["k"]), f64(inp["v"]), f64(inp["dout"]), 40,
                               1 / math.sqrt(d), q_len=L)
    for got, ref, name in ((dq, rq, "dq"), (dk, rk, "dk"), (dv, rv, "dv")):
        assert torch.all(got[0] == 0), name
        check(got, ref, True, "bwd empty sequence " + name)


@pytest.mark.parametrize("bias", [1.0, -1.0])
def test_varlen_large_scores(bias):
    """The packed layout through the reference-moving path."""
    lens = [300, 0, 129, 77]
    d, H, Hkv, W = 128, 4, 2, 96
    total, mx = sum(lens), max(lens)
    q, k, v = _qkv(1, H, Hkv, total, d, seed=97, qk_std=3.0, bias=bias, tdt=torch.bfloat16)
    # token-major [total, heads, d]
    q, k, v = (x[0].transpose(0, 1).contiguous() for x in (q, k, v))
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    meta = swa.swa_blockmask_build(len(lens), mx, mx, W, 128, 64, q_len=np.array(lens),
                                   k_len=np.array(lens))
    md = swa.meta_to_device(meta, DEV)
    o = torch.full((total, H, d), float("nan"), dtype=torch.bfloat16, device=DEV)
    swa.swa_fwd_varlen(q.to(DEV), k.to(DEV), v.to(DEV), o, W, md, torch.from_numpy(cu).to(DEV))
    torch.cuda.synchronize()
    ref = oracle.fwd_varlen(f64(q), f64(k), f64(v), cu, W, 1 / math.sqrt(d))
    check(o, ref, True, "varlen large scores bias=%g" % bias)


@pytest.mark.parametrize("bias", [1.0, -1.0])
def test_bwd_large_scores(bias):
    """Gradients where the softmax is nearly one-hot (scaled scores ~ +-25
    with a spread of +-5): P = exp(s - lse) from the forward's lse."""
    q, k, v = _qkv(1, 4, 2, 300, 128, seed=98, qk_std=1.5, bias=bias, tdt=torch.bfloat16)
    g = torch.Generator().manual_seed(99)
    dout = (torch.randn(q.shape, generator=g) * 0.5).to(torch.bfloat16)
    B, H, N, d = q.shape
    W = 100
    md = swa.meta_to_device(swa.swa_blockmask_build(B, N, N, W, 128, 64), DEV)
    qd, kd, vd, dod = (x.to(DEV) for x in (q, k, v, dout))
    o = torch.empty_like(qd)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=DEV)
    swa.swa_fwd(qd, kd, vd, o, W, md, lse=lse)
    dq, dk, dv = torch.empty_like(qd), torch.empty_like(kd), torch.empty_like(vd)
    ws = torch.empty(swa.swa_bwd_workspace_size(B, H, N) // 4, dtype=torch.float32, device=DEV)
    swa.swa_bwd(qd, kd, vd, o, dod, lse, dq, dk, dv, ws, W, md)
    torch.cuda.synchronize()
    rq, rk, rv, rl = oracle.bwd(f64(q), f64(k), f64(v), f64(dout), W, 1 / math.sqrt(d))
    # the forward's lse bar for bf16 (the row sum is taken over bf16-rounded P)
    lerr = np.abs(f64(lse) - rl)
    assert lerr.max() <= 4e-3, float(lerr.max())
    for got, ref, name in ((dq, rq, "dq"), (dk, rk, "dk"), (dv, rv, "dv")):
        gg = f64(got)
        scale = max(1.0, float(np.abs(ref).max()))
        err = np.abs(gg - ref) / scale
        assert np.all(np.isfinite(gg)), name
        assert err.max() <= 2e-2 and err.mean() <= 2e-3, (name, float(err.max()),
                                                          float(err.mean()))


@pytest.mark.parametrize("bias", [1.0, -1.0])
def test_chunk_sinks_large_scores(bias):
    """A chunk with 4 attention sinks (the sink segment of the key axis) and
    scores far from the fixed reference."""
    W, Tq, d, S = 128, 64, 128, 4
    B, H, Hkv = 2, 8, 2
    P = 300  # next position: the ring holds 172 .. 299, the sinks 0 .. 3
    q, k, v = _qkv(B, H, Hkv, P + Tq, d, seed=100, qk_std=3.0, bias=bias, tdt=torch.bfloat16)
    rs = np.array([P % W, P % W], dtype=np.int32)
    kc = torch.empty(B, Hkv, W, d, dtype=torch.bfloat16)
    vc = torch.empty_like(kc)
    for s_ in range(W):  # slot s holds position P - W + ((s - rs) mod W)
        pos = P - W + ((s_ - int(rs[0])) % W)
        kc[:, :, s_], vc[:, :, s_] = k[:, :, pos], v[:, :, pos]
    sk, sv = k[:, :, :S].contiguous(), v[:, :, :S].contiguous()
    state = [None, None, rs, np.full(B, W, dtype=np.int32), np.full(B, P, dtype=np.int32)]
    md = _chunk_meta_local(state, Tq, W, S)
    qn, kn, vn = (x[:, :, P:].contiguous() for x in (q, k, v))
    dev = [t.to(DEV).contiguous() for t in (qn, kn, vn, kc, vc, sk, sv)]
    st = [torch.from_numpy(x.copy()).to(DEV) for x in state[2:]]
    o = torch.full_like(dev[0], float("nan"))
    swa.swa_prefill_chunk(dev[0], dev[1], dev[2], dev[3], dev[4], st[0], st[1], st[2], o, W, md,
                          sink_k=dev[5], sink_v=dev[6])
    torch.cuda.synchronize()
    ref = oracle.chunk(f64(qn), f64(kn), f64(vn), f64(kc), f64(vc), rs, state[3], state[4], W,
                       1 / math.sqrt(d), n_sink=S, sink_k=f64(sk), sink_v=f64(sv))
    check(o, ref[0], True, "chunk sinks large scores bias=%g" % bias)
    # the same rows of the full-sequence forward with sinks, positions P .. P+Tq-1
    full = oracle.fwd_rows(f64(q), f64(k), f64(v), W, 1 / math.sqrt(d),
                           [(b, h, P + i) for b in range(B) for h in range(H) for i in (0, 31, 63)],
                           n_sink=S)
    got = f64(o)[:, :, [0, 31, 63]].reshape(-1, d)
    assert np.abs(got - full).max() <= 2e-2


def _chunk_meta_local(state, Tq, W, S):
    rs, cl, npos = state[2], state[3], state[4]
    m = swa.swa_blockmask_build(len(npos), Tq, Tq, W, 128, 64, q_start=npos, k_start=npos,
                                W_ring=W, ring_start=rs, cache_len=cl, next_pos=npos, n_sink=S)
    return swa.meta_to_device(m, DEV)


@pytest.mark.parametrize("N", [4096, 4224])
def test_every_tile_written_at_scale(N):
    """More than 512 logical tiles, so that workgroups are dealt to XCDs in
    chunks (N = 4096: 512 tiles exactly; 4224: 528, a tail of 16 taking the
    contiguous path): the forward and the backward write every element (all
    outputs start as NaN), and sampled rows match the oracle."""
    B, H, Hkv, d, W = 2, 8, 8, 128, 300
    inp = synth.gen_bwd(B, H, Hkv, N, d, seed=101)
    q, k, v, do = (inp[x].to(DEV) for x in ("q", "k", "v", "dout"))
    md = swa.meta_to_device(swa.swa_blockmask_build(B, N, N, W, 128, 64), DEV)
    o = torch.full_like(q, float("nan"))
    lse = torch.full((B, H, N), float("nan"), device=DEV)
    swa.swa_fwd(q, k, v, o, W, md, lse=lse)
    dq, dk, dv = (torch.full_like(t, float("nan")) for t in (q, k, v))
    ws = torch.empty(swa.swa_bwd_workspace_size(B, H, N) // 4, dtype=torch.float32, device=DEV)
    swa.swa_bwd(q, k, v, o, do, lse, dq, dk, dv, ws, W, md)
    torch.cuda.synchronize()
    for t, name in ((o, "o"), (lse, "lse"), (dq, "dq"), (dk, "dk"), (dv, "dv")):
        assert torch.isfinite(t).all(), name
    rows = [(b, h, i) for b in range(B) for h in range(H) for i in (0, 127, 128, N // 2, N - 1)]
    ref = oracle.fwd_rows(f64(inp["q"]), f64(inp["k"]), f64(inp["v"]), W, 1 / math.sqrt(d), rows)
    got = np.stack([f64(o[b, h, i]) for b, h, i in rows])
    assert np.abs(got - ref).max() <= 2e-2
    keys = [(b, g, j) for b in range(B) for g in range(Hkv) for j in (0, 63, 64, N // 2, N - 1)]
    rq, rk, rv = oracle.bwd_sel(f64(inp["q"]), f64(inp["k"]), f64(inp["v"]), f64(inp["dout"]), W,
                                1 / math.sqrt(d), rows, keys)
    scale = lambda r: max(1.0, float(np.abs(r).max()))
    gq = np.stack([f64(dq[b, h, i]) for b, h, i in rows])
    gk = np.stack([f64(dk[b, g, j]) for b, g, j in keys])
    gv = np.stack([f64(dv[b, g, j]) for b, g, j in keys])
    assert np.abs(gq - rq).max() / scale(rq) <= 2e-2
    assert np.abs(gk - rk).max() / scale(rk) <= 2e-2
    assert np.abs(gv - rv).max() / scale(rv) <= 2e-2
