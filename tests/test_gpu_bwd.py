"""GPU parity of the backward (swa_bwd) and of the forward's row log-sum-exp,
through the C ABI, against the fp64 oracle on the same seeded inputs.

Bars, from the arithmetic (bf16 operands in every product, fp32 accumulation):
gradients are compared after dividing by their reference's largest magnitude
(at least 1): bf16 inputs
max-abs <= 2e-2 and mean-abs <= 2e-3, fp32 path max-abs <= 1e-4; lse abs
<= 4e-3 (bf16: the row sum is taken over bf16-rounded P) or 1e-5 (fp32);
padded rows and keys exactly 0.
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


def check_grad(got, ref, bf16, where):
    got = f64(got) if torch.is_tensor(got) else got
    assert np.all(np.isfinite(got)), "non-finite " + where
    scale = max(1.0, float(np.abs(ref).max()))
    err = np.abs(got - ref) / scale
    if bf16:
        assert err.max() <= 2e-2, (where, float(err.max()))
        assert err.mean() <= 2e-3, (where, float(err.mean()))
    else:
        assert err.max() <= 1e-4, (where, float(err.max()))


def run(inp, W, tq, tk, scale=None):
    q, k, v, do, ql = inp["q"], inp["k"], inp["v"], inp["dout"], inp["q_len"]
    B, H, N, d = q.shape
    L = None if ql is None else ql.numpy()
    meta = swa.swa_blockmask_build(B, N, N, W, tq, tk, q_len=L, k_len=L)
    md = swa.meta_to_device(meta, DEV)
    qd, kd, vd, dod = (x.to(DEV) for x in (q, k, v, do))
    qld = None if ql is None else ql.to(DEV)
    od = torch.empty_like(qd)
    lse = torch.full((B, H, N), float("nan"), device=DEV)
    swa.swa_fwd(qd, kd, vd, od, W, md, q_len=qld, lse=lse, scale=scale)
    dq = torch.full_like(qd, float("nan"))
    dk = torch.full_like(kd, float("nan"))
    dv = torch.full_like(vd, float("nan"))
    ws = torch.empty(swa.swa_bwd_workspace_size(B, H, N) // 4, dtype=torch.float32, device=DEV)
    swa.swa_bwd(qd, kd, vd, od, dod, lse, dq, dk, dv, ws, W, md, q_len=qld, scale=scale)
    torch.cuda.synchronize()
    return dq, dk, dv, lse


def compare_full(inp, W, tq, tk, where):
    d = inp["q"].shape[-1]
    scale = 1 / math.sqrt(d)
    dq, dk, dv, lse = run(inp, W, tq, tk)
    L = None if inp["q_len"] is None else inp["q_len"].numpy()
    rq, rk, rv, rl = oracle.bwd(f64(inp["q"]), f64(inp["k"]), f64(inp["v"]), f64(inp["dout"]),
                                W, scale, q_len=L)
    bf = inp["q"].dtype == torch.bfloat16
    check_grad(dq, rq, bf, where + " dq")
    check_grad(dk, rk, bf, where + " dk")
    check_grad(dv, rv, bf, where + " dv")
    got_l = f64(lse)
    fin = np.isfinite(rl)
    assert np.array_equal(np.isfinite(got_l), fin), where + " lse finiteness"
    assert np.max(np.abs(got_l[fin] - rl[fin])) <= (4e-3 if bf else 1e-5), where + " lse"
    if L is not None:
        for b, l in enumerate(L):
            assert torch.all(dq[b, :, int(l):] == 0) and torch.all(dk[b, :, int(l):] == 0)
            assert torch.all(dv[b, :, int(l):] == 0)


@pytest.mark.parametrize("d", [4, 36, 128])
def test_bwd_fp32(d):
    inp = synth.gen_bwd(2, 4, 2, 70, d, seed=300 + d, std=1.0, dtype="f32", len_lo=20,
                        len_hi=70)
    for W, tq, tk in ((1, 8, 8), (9, 16, 8), (33, 7, 5), (100, 64, 64)):
        compare_full(inp, W, tq, tk, "fp32 d=%d W=%d" % (d, W))


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("tq", [128, 64])
@pytest.mark.parametrize("W", [1, 17, 100, 333])
def test_bwd_bf16(d, tq, W):
    inp = synth.gen_bwd(2, 4, 2, 333, d, seed=400 + W, std=0.5, len_lo=150, len_hi=333)
    inp["q_len"][0] = 333
    compare_full(inp, W, tq, 64, "bf16 d=%d tq=%d W=%d" % (d, tq, W))


def test_bwd_prefill_workload_full():
    """The prefill workload's shape (B=1, H=32, N=8192, W=512, d=128): every
    entry of dq, dk, dv and the forward's lse against the oracle's backward of
    the whole workload."""
    inp = synth.gen_bwd(1, 32, 32, 8192, 128, seed=11, std=0.5)
    compare_full(inp, 512, 128, 64, "prefill workload")


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("tq", [128, 64])
@pytest.mark.parametrize("W", [17, 333])
def test_bwd_bf16_tk128(d, tq, W):
    """Metadata with 128-key tiles (which the forward takes): the backward
    runs its fp32-arithmetic kernels on bf16 data (the MFMA kernels take
    64-key tiles), against the same oracle and bars."""
    inp = synth.gen_bwd(2, 4, 2, 333, d, seed=700 + W, std=0.5, len_lo=150, len_hi=333)
    inp["q_len"][0] = 333
    compare_full(inp, W, tq, 128, "bf16 tk128 d=%d tq=%d W=%d" % (d, tq, W))
