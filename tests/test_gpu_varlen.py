"""GPU parity of the packed variable-length forward (swa_fwd_varlen) against
the fp64 oracle on the same seeded inputs ("Dense vs sliding-window sparse
attention" §3.3 cu_seqlens, §5.2 per-sequence windows).  Bars as for the
padded forward (bf16 max-abs 2e-2, mean-abs 2e-3; fp32 1e-4; lse 4e-3 / 1e-5).
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


def packed_inputs(lens, H, Hkv, d, seed, dtype="bf16", std=0.5):
    """Draw a padded batch with these lengths, then pack its valid rows."""
    B, N = len(lens), max(lens)
    inp = synth.gen_fwd(B, H, Hkv, N, d, seed=seed, std=std, dtype=dtype)
    q = torch.cat([inp["q"][b, :, :L].transpose(0, 1) for b, L in enumerate(lens)]).contiguous()
    k = torch.cat([inp["k"][b, :, :L].transpose(0, 1) for b, L in enumerate(lens)]).contiguous()
    v = torch.cat([inp["v"][b, :, :L].transpose(0, 1) for b, L in enumerate(lens)]).contiguous()
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lens)]), dtype=torch.int32)
    return q, k, v, cu, inp


def run_varlen(q, k, v, cu, lens, W, S, tq, tk, lse=False):
    B, N = len(lens), max(lens)
    meta = swa.swa_blockmask_build(B, N, N, W, tq, tk, q_len=lens, k_len=lens, n_sink=S)
    md = swa.meta_to_device(meta, DEV)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    od = torch.full_like(qd, float("nan"))
    ls = torch.full((q.shape[0], q.shape[1]), float("nan"), device=DEV) if lse else None
    swa.swa_fwd_varlen(qd, kd, vd, od, W, md, cu.to(DEV), lse=ls)
    torch.cuda.synchronize()
    return od, ls


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("tq", [128, 64])
@pytest.mark.parametrize("W,S", [(1, 0), (17, 0), (100, 4), (400, 0)])
def test_varlen_bf16(d, tq, W, S):
    lens = [333, 1, 64, 200, 129]
    q, k, v, cu, inp = packed_inputs(lens, 4, 2, d, seed=700 + W)
    o, lse = run_varlen(q, k, v, cu, lens, W, S, tq, 64, lse=True)
    sc = 1 / math.sqrt(d)
    ref = oracle.fwd_varlen(f64(q), f64(k), f64(v), cu.numpy(), W, sc, n_sink=S)
    check(o, ref, True, "varlen d=%d tq=%d W=%d S=%d" % (d, tq, W, S))
    # row log-sum-exp against the oracle's padded run, mapped to packed order
    L = np.array(lens, dtype=np.int32)
    _, _, _, rl = oracle.bwd(f64(inp["q"]), f64(inp["k"]), f64(inp["v"]),
                             np.zeros(tuple(inp["q"].shape)), W, sc, q_len=L, n_sink=S)
    want = np.concatenate([rl[b, :, :n].T for b, n in enumerate(lens)])
    assert np.max(np.abs(f64(lse) - want)) <= 4e-3


def test_varlen_fp32():
    lens = [70, 3, 41]
    q, k, v, cu, _ = packed_inputs(lens, 4, 4, 20, seed=71, dtype="f32", std=1.0)
    for W, S, tq, tk in ((5, 0, 8, 8), (13, 3, 7, 5), (80, 0, 16, 16)):
        o, _ = run_varlen(q, k, v, cu, lens, W, S, tq, tk)
        ref = oracle.fwd_varlen(f64(q), f64(k), f64(v), cu.numpy(), W, 1 / math.sqrt(20),
                                n_sink=S)
        check(o, ref, False, "varlen fp32 W=%d S=%d" % (W, S))


def test_varlen_gqa_workload_sampled():
    """The GQA workload's sequences (B=4, H=32, Hkv=8, W=4096, lengths in
    [8192, 32768]) packed without padding; sampled rows against the oracle."""
    inp = synth.make("prefill_gqa")
    lens = [int(x) for x in inp["q_len"]]
    q = torch.cat([inp["q"][b, :, :L].transpose(0, 1) for b, L in enumerate(lens)]).contiguous()
    k = torch.cat([inp["k"][b, :, :L].transpose(0, 1) for b, L in enumerate(lens)]).contiguous()
    v = torch.cat([inp["v"][b, :, :L].transpose(0, 1) for b, L in enumerate(lens)]).contiguous()
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    o, _ = run_varlen(q, k, v, torch.from_numpy(cu), lens, 4096, 0, 128, 64)
    rng = np.random.default_rng(12)
    rows = []
    for b, L in enumerate(lens):
        rows += [[b, int(h), int(i)] for h, i in zip(rng.integers(0, 32, 48),
                                                     rng.integers(0, L, 48))]
        rows += [[b, 0, 0], [b, 31, L - 1], [b, 5, 4095], [b, 6, 4096]]
    ref = oracle.fwd_rows(f64(inp["q"]), f64(inp["k"]), f64(inp["v"]), 4096, 1 / math.sqrt(128),
                          rows, q_len=np.array(lens, dtype=np.int32))
    got = np.stack([f64(o[cu[b] + i, h]) for b, h, i in rows])
    check(got, ref, True, "varlen GQA workload sampled")


def run_bwd_varlen(lens, H, Hkv, d, W, S, tq, seed):
    """Packed forward then packed backward on the GPU; returns the packed
    gradients and the padded fp64 inputs they came from."""
    B, N = len(lens), max(lens)
    inp = synth.gen_bwd(B, H, Hkv, N, d, seed=seed)
    pack = lambda x: torch.cat([x[b, :, :L].transpose(0, 1) for b, L in enumerate(lens)]
                               ).contiguous()
    q, k, v, do = (pack(inp[n]).to(DEV) for n in ("q", "k", "v", "dout"))
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lens)]), dtype=torch.int32, device=DEV)
    meta = swa.swa_blockmask_build(B, N, N, W, tq, 64, q_len=lens, k_len=lens, n_sink=S)
    md = swa.meta_to_device(meta, DEV)
    total = q.shape[0]
    o = torch.empty_like(q)
    lse = torch.full((total, H), float("nan"), device=DEV)
    swa.swa_fwd_varlen(q, k, v, o, W, md, cu, lse=lse)
    # NaN-filled outputs: every packed row must be written
    dq, dk, dv = (torch.full_like(x, float("nan")) for x in (q, k, v))
    ws = torch.empty(swa.swa_bwd_workspace_size(1, H, total) // 4, device=DEV)
    swa.swa_bwd_varlen(q, k, v, o, do, lse, dq, dk, dv, ws, W, md, cu)
    torch.cuda.synchronize()
    return dq, dk, dv, inp


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("tq", [128, 64])
@pytest.mark.parametrize("W,S", [(1, 0), (17, 0), (100, 4), (400, 0)])
def test_bwd_varlen_bf16(d, tq, W, S):
    """Packed backward against the oracle's padded backward of the same
    sequences, mapped to packed order (grouped heads, H=4 over Hkv=2)."""
    lens = [333, 1, 64, 200, 129]
    dq, dk, dv, inp = run_bwd_varlen(lens, 4, 2, d, W, S, tq, seed=900 + W + d)
    L = np.array(lens, dtype=np.int32)
    rq, rk, rv, _ = oracle.bwd(f64(inp["q"]), f64(inp["k"]), f64(inp["v"]), f64(inp["dout"]),
                               W, 1 / math.sqrt(d), q_len=L, n_sink=S)
    packed = lambda r: np.concatenate([r[b, :, :n].transpose(1, 0, 2) for b, n in enumerate(lens)])
    where = "bwd varlen d=%d tq=%d W=%d S=%d" % (d, tq, W, S)
    for got, ref, nm in ((dq, rq, "dq"), (dk, rk, "dk"), (dv, rv, "dv")):
        ref = packed(ref)
        got = f64(got)
        assert np.all(np.isfinite(got)), "unwritten or non-finite rows, " + where + " " + nm
        err = np.abs(got - ref) / max(1.0, float(np.abs(ref).max()))
        assert err.max() <= 2e-2 and err.mean() <= 2e-3, (where, nm, float(err.max()))


def test_bwd_varlen_empty_sequences_mha():
    """Zero-length sequences among the packed ones (one head per group)."""
    lens = [0, 97, 1, 0, 190]
    dq, dk, dv, inp = run_bwd_varlen(lens, 2, 2, 128, 64, 0, 128, seed=955)
    L = np.array(lens, dtype=np.int32)
    rq, rk, rv, _ = oracle.bwd(f64(inp["q"]), f64(inp["k"]), f64(inp["v"]), f64(inp["dout"]),
                               64, 1 / math.sqrt(128), q_len=L)
    packed = lambda r: np.concatenate([r[b, :, :n].transpose(1, 0, 2) for b, n in enumerate(lens)])
    for got, ref, nm in ((dq, rq, "dq"), (dk, rk, "dk"), (dv, rv, "dv")):
        ref = packed(ref)
        got = f64(got)
        assert got.shape == ref.shape and np.all(np.isfinite(got)), nm
        err = np.abs(got - ref) / max(1.0, float(np.abs(ref).max()))
        assert err.max() <= 2e-2 and err.mean() <= 2e-3, (nm, float(err.max()))


def test_bwd_varlen_gqa_workload_sampled():
    """The packed backward at the size the benchmark times: the GQA workload's
    four sequences (H=32, Hkv=8, W=4096, 76 563 tokens) packed token-major,
    sampled dq rows and dk/dv keys against the oracle's selected-entry
    gradients of the same sequences in padded form."""
    inp = synth.make("prefill_gqa")
    lens = [int(x) for x in inp["q_len"]]
    B, H, N, d = inp["q"].shape
    Hkv, W = inp["k"].shape[1], 4096
    pack = lambda x: torch.cat([x[b, :, :n].transpose(0, 1) for b, n in enumerate(lens)]
                               ).contiguous()
    q, k, v = (pack(inp[n]).to(DEV) for n in ("q", "k", "v"))
    total = q.shape[0]
    gen = torch.Generator(device="cpu").manual_seed(2024)
    do_cpu = (torch.randn((total, H, d), generator=gen) * 0.5).to(torch.bfloat16)
    do = do_cpu.to(DEV)
    cu_np = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    cu = torch.from_numpy(cu_np).to(DEV)
    meta = swa.swa_blockmask_build(B, N, N, W, 128, 64, q_len=lens, k_len=lens)
    md = swa.meta_to_device(meta, DEV)
    o = torch.empty_like(q)
    lse = torch.empty((total, H), dtype=torch.float32, device=DEV)
    swa.swa_fwd_varlen(q, k, v, o, W, md, cu, lse=lse)
    dq, dk, dv = (torch.full_like(x, float("nan")) for x in (q, k, v))
    ws = torch.empty(swa.swa_bwd_workspace_size(1, H, total) // 4, device=DEV)
    swa.swa_bwd_varlen(q, k, v, o, do, lse, dq, dk, dv, ws, W, md, cu)
    torch.cuda.synchronize()
    del q, k, v, o, do, lse, ws
    # the output gradient in the oracle's padded layout (zero past each length)
    dout = np.zeros((B, H, N, d))
    for b, n in enumerate(lens):
        dout[b, :, :n] = f64(do_cpu[cu_np[b]:cu_np[b + 1]]).transpose(1, 0, 2)
    rng = np.random.default_rng(31)
    rows, keys = [], []
    for b, n in enumerate(lens):
        rows += [[b, int(h), int(i)] for h, i in zip(rng.integers(0, H, 12), rng.integers(0, n, 12))]
        rows += [[b, 0, 0], [b, H - 1, n - 1], [b, 5, W - 1], [b, 6, W]]
        # a key is costly for the oracle in proportion to the rows that see it
        # (up to G*W): random keys near the end, and two that W rows see
        keys += [[b, int(g), int(j)] for g, j in zip(rng.integers(0, Hkv, 2),
                                                     rng.integers(n - 300, n, 2))]
        keys += [[b, 0, 0], [b, Hkv - 1, n - 1], [b, 3, n - W]]
    rq, rk, rv = oracle.bwd_sel(f64(inp["q"]), f64(inp["k"]), f64(inp["v"]), dout, W,
                                1 / math.sqrt(d), rows, keys, q_len=np.array(lens, dtype=np.int32))
    gq = np.stack([f64(dq[cu_np[b] + i, h]) for b, h, i in rows])
    gk = np.stack([f64(dk[cu_np[b] + j, g]) for b, g, j in keys])
    gv = np.stack([f64(dv[cu_np[b] + j, g]) for b, g, j in keys])
    assert all(np.all(np.isfinite(t)) for t in (f64(dq), f64(dk), f64(dv))), "unwritten rows"
    for got, ref, nm in ((gq, rq, "dq"), (gk, rk, "dk"), (gv, rv, "dv")):
        err = np.abs(got - ref) / max(1.0, float(np.abs(ref).max()))
        assert err.max() <= 2e-2 and err.mean() <= 2e-3, ("GQA packed " + nm, float(err.max()))


def test_bwd_varlen_fp32():
    """The fp32 packed backward (fp32-arithmetic kernels) with odd tiles and
    head dim, grouped heads, sinks and a zero-length sequence, against the
    oracle's padded backward in packed order at the fp32 bar."""
    lens = [70, 0, 3, 41]
    B, N, H, Hkv, d = len(lens), max(lens), 4, 2, 20
    inp = synth.gen_bwd(B, H, Hkv, N, d, seed=77, std=1.0, dtype="f32")
    pack = lambda x: torch.cat([x[b, :, :L].transpose(0, 1) for b, L in enumerate(lens)]
                               ).contiguous()
    q, k, v, do = (pack(inp[n]).to(DEV) for n in ("q", "k", "v", "dout"))
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lens)]), dtype=torch.int32, device=DEV)
    total = q.shape[0]
    L = np.array(lens, dtype=np.int32)
    for W, S, tq, tk in ((5, 0, 8, 8), (13, 3, 7, 5), (80, 2, 16, 16)):
        meta = swa.swa_blockmask_build(B, N, N, W, tq, tk, q_len=lens, k_len=lens, n_sink=S)
        md = swa.meta_to_device(meta, DEV)
        o = torch.empty_like(q)
        lse = torch.empty((total, H), dtype=torch.float32, device=DEV)
        swa.swa_fwd_varlen(q, k, v, o, W, md, cu, lse=lse)
        dq, dk, dv = (torch.full_like(x, float("nan")) for x in (q, k, v))
        ws = torch.empty(swa.swa_bwd_workspace_size(1, H, total) // 4, device=DEV)
        swa.swa_bwd_varlen(q, k, v, o, do, lse, dq, dk, dv, ws, W, md, cu)
        torch.cuda.synchronize()
        rq, rk, rv, _ = oracle.bwd(f64(inp["q"]), f64(inp["k"]), f64(inp["v"]),
                                   f64(inp["dout"]), W, 1 / math.sqrt(d), q_len=L, n_sink=S)
        packed = lambda r: np.concatenate([r[b, :, :n].transpose(1, 0, 2)
                                           for b, n in enumerate(lens)])
        for got, ref, nm in ((dq, rq, "dq"), (dk, rk, "dk"), (dv, rv, "dv")):
            ref, got = packed(ref), f64(got)
            assert np.all(np.isfinite(got)), ("unwritten rows", W, S, nm)
            err = np.abs(got - ref) / max(1.0, float(np.abs(ref).max()))
            assert err.max() <= 1e-4, ("fp32 packed bwd", W, S, nm, float(err.max()))


@pytest.mark.parametrize("dtype,d,W,S,tq,tk", [("bf16", 128, 100, 4, 128, 64),
                                               ("bf16", 64, 33, 0, 64, 64),
                                               ("f32", 20, 13, 3, 7, 5)])
def test_bwd_varlen_equals_padded(dtype, d, W, S, tq, tk):
    """The packed backward changes only addressing: on the same sequences its
    gradients equal the padded backward's (with q_len) bit for bit, rows past
    each sequence excepted."""
    lens = [150, 1, 0, 97, 64]
    B, N, H, Hkv = len(lens), max(lens), 4, 2
    inp = synth.gen_bwd(B, H, Hkv, N, d, seed=31 + d, dtype=dtype)
    L = torch.tensor(lens, dtype=torch.int32)
    meta = swa.swa_blockmask_build(B, N, N, W, tq, tk, q_len=lens, k_len=lens, n_sink=S)
    md = swa.meta_to_device(meta, DEV)
    # padded
    q, k, v, do = (inp[n].to(DEV) for n in ("q", "k", "v", "dout"))
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=DEV)
    swa.swa_fwd(q, k, v, o, W, md, q_len=L.to(DEV), lse=lse)
    gq, gk, gv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws = torch.empty(swa.swa_bwd_workspace_size(B, H, N) // 4, device=DEV)
    swa.swa_bwd(q, k, v, o, do, lse, gq, gk, gv, ws, W, md, q_len=L.to(DEV))
    # packed
    pack = lambda x: torch.cat([x[b, :, :n].transpose(0, 1) for b, n in enumerate(lens)]
                               ).contiguous()
    qp, kp, vp, dop = (pack(x) for x in (q, k, v, do))
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lens)]), dtype=torch.int32, device=DEV)
    op = torch.empty_like(qp)
    lsp = torch.empty((qp.shape[0], H), dtype=torch.float32, device=DEV)
    swa.swa_fwd_varlen(qp, kp, vp, op, W, md, cu, lse=lsp)
    pq, pk_, pv = (torch.full_like(x, float("nan")) for x in (qp, kp, vp))
    wsp = torch.empty(swa.swa_bwd_workspace_size(1, H, qp.shape[0]) // 4, device=DEV)
    swa.swa_bwd_varlen(qp, kp, vp, op, dop, lsp, pq, pk_, pv, wsp, W, md, cu)
    torch.cuda.synchronize()
    assert torch.equal(op, pack(o)), "packed forward differs from padded"
    for got, ref, nm in ((pq, gq, "dq"), (pk_, gk, "dk"), (pv, gv, "dv")):
        assert torch.equal(got, pack(ref)), nm
