"""Seeded synthetic inputs shaped like the workloads of the SWA pages.

This module holds no attention arithmetic: it only draws random tensors and
integers in a fixed order from a seeded CPU generator, so that the GPU library
and the fp64 oracle receive byte-identical inputs.  Values are drawn in fp32
(``randn * std``) and rounded to bf16 on the host where the workload is bf16.

Workloads (sizes as named; "prefill" stands in for the 8192-token prompt with a
512-token window of the dense-vs-SWA blog, "decode" for the long-context decode
step whose KV read the sparse-attention taxonomy page estimates):

  tiny         B=1  H=Hkv=1  N=8      W=3    d=4    fp32
  prefill      B=1  H=Hkv=32 N=8192   W=512  d=128  bf16
  prefill_gqa  B=4  H=32 Hkv=8 N=32768 W=4096 d=128 bf16, lengths U[8192, 32768]
  chunk        B=8  H=32 Hkv=8 Tq=512 W=4096 d=128 bf16, p U[4096, 65536]
  decode       B=64 H=32 Hkv=8 W=4096 d=128 bf16, query position U[4096, 131072]
"""
from __future__ import annotations

import torch

WORKLOADS = {
    "tiny": dict(kind="fwd", B=1, H=1, Hkv=1, N=8, W=3, d=4, dtype="f32", seed=1, std=1.0),
    "prefill": dict(kind="fwd", B=1, H=32, Hkv=32, N=8192, W=512, d=128, dtype="bf16",
                    seed=2, std=0.5),
    "prefill_gqa": dict(kind="fwd", B=4, H=32, Hkv=8, N=32768, W=4096, d=128,
                        dtype="bf16", seed=3, std=0.5, len_lo=8192, len_hi=32768),
    "chunk": dict(kind="chunk", B=8, H=32, Hkv=8, Tq=512, W=4096, d=128, dtype="bf16",
                  seed=4, std=0.5, p_lo=4096, p_hi=65536),
    "decode": dict(kind="decode", B=64, H=32, Hkv=8, W=4096, d=128, dtype="bf16", seed=5,
                   std=0.5, pos_lo=4096, pos_hi=131072),
}

_DT = {"f32": torch.float32, "bf16": torch.bfloat16}


def _randn(gen, shape, std, dtype):
    x = torch.randn(*shape, generator=gen, dtype=torch.float32)
    if std != 1.0:
        x = x * std
    return x.to(_DT[dtype])


def _randint(gen, lo, hi_inclusive, n):
    return torch.randint(lo, hi_inclusive + 1, (n,), generator=gen, dtype=torch.int64).to(
        torch.int32)


def gen_fwd(B, H, Hkv, N, d, seed, std=0.5, dtype="bf16", len_lo=None, len_hi=None):
    """Q [B,H,N,d], K/V [B,Hkv,N,d]; optional per-sequence lengths drawn after the
    tensors, with rows at or past each length zero-filled (padding)."""
    gen = torch.Generator(device="cpu").manual_seed(seed)
    q = _randn(gen, (B, H, N, d), std, dtype)
    k = _randn(gen, (B, Hkv, N, d), std, dtype)
    v = _randn(gen, (B, Hkv, N, d), std, dtype)
    q_len = None
    if len_lo is not None:
        q_len = _randint(gen, len_lo, len_hi, B)
        for b in range(B):
            L = int(q_len[b])
            q[b, :, L:] = 0
            k[b, :, L:] = 0
            v[b, :, L:] = 0
    return dict(q=q, k=k, v=v, q_len=q_len)


def gen_bwd(B, H, Hkv, N, d, seed, std=0.5, dtype="bf16", len_lo=None, len_hi=None):
    """The forward inputs of gen_fwd (same seed gives the same q, k, v, q_len)
    plus an output gradient dout [B,H,N,d] drawn after them, zero on padded rows."""
    inp = gen_fwd(B, H, Hkv, N, d, seed, std, dtype, len_lo, len_hi)
    gen = torch.Generator(device="cpu").manual_seed(seed + 7919)
    dout = _randn(gen, (B, H, N, d), std, dtype)
    if inp["q_len"] is not None:
        for b in range(B):
            dout[b, :, int(inp["q_len"][b]):] = 0
    inp["dout"] = dout
    return inp


def gen_chunk(B, H, Hkv, Tq, W, d, seed, std=0.5, dtype="bf16", p_lo=None, p_hi=None,
              p=None):
    """A chunk of Tq new tokens per request plus a full ring cache of W slots.

    The ring's physical slots get independent random rows; the request's next
    position p is drawn (or given) and the ring start index is p mod W, the
    fill count W.  Which logical position each slot stands for is not decided
    here."""
    gen = torch.Generator(device="cpu").manual_seed(seed)
    q = _randn(gen, (B, H, Tq, d), std, dtype)
    k_new = _randn(gen, (B, Hkv, Tq, d), std, dtype)
    v_new = _randn(gen, (B, Hkv, Tq, d), std, dtype)
    k_cache = _randn(gen, (B, Hkv, W, d), std, dtype)
    v_cache = _randn(gen, (B, Hkv, W, d), std, dtype)
    if p is None:
        p = _randint(gen, p_lo, p_hi, B)
    else:
        p = torch.as_tensor(p, dtype=torch.int32).reshape(B)
    ring_start = torch.remainder(p, W).to(torch.int32)
    cache_len = torch.full((B,), W, dtype=torch.int32)
    return dict(q=q, k_new=k_new, v_new=v_new, k_cache=k_cache, v_cache=v_cache,
                ring_start=ring_start, cache_len=cache_len, next_pos=p.clone())


def gen_decode(B, H, Hkv, W, d, seed, std=0.5, dtype="bf16", pos_lo=None, pos_hi=None):
    """One query token per request, its new K/V row, and a full ring of W slots
    with a random start index.  next_pos is the query's logical position."""
    gen = torch.Generator(device="cpu").manual_seed(seed)
    q = _randn(gen, (B, H, d), std, dtype)
    k_new = _randn(gen, (B, Hkv, d), std, dtype)
    v_new = _randn(gen, (B, Hkv, d), std, dtype)
    k_cache = _randn(gen, (B, Hkv, W, d), std, dtype)
    v_cache = _randn(gen, (B, Hkv, W, d), std, dtype)
    pos = _randint(gen, pos_lo, pos_hi, B)
    ring_start = _randint(gen, 0, W - 1, B)
    cache_len = torch.full((B,), W, dtype=torch.int32)
    return dict(q=q, k_new=k_new, v_new=v_new, k_cache=k_cache, v_cache=v_cache,
                ring_start=ring_start, cache_len=cache_len, next_pos=pos)


def make(name: str, **overrides):
    """Inputs of a named workload; keyword overrides change sizes or the seed."""
    cfg = dict(WORKLOADS[name])
    cfg.update(overrides)
    kind = cfg.pop("kind")
    cfg.pop("W", None) if kind == "fwd" else None
    if kind == "fwd":
        keys = ("B", "H", "Hkv", "N", "d", "seed", "std", "dtype", "len_lo", "len_hi")
        return gen_fwd(**{k: cfg[k] for k in keys if k in cfg})
    if kind == "chunk":
        keys = ("B", "H", "Hkv", "Tq", "W", "d", "seed", "std", "dtype", "p_lo", "p_hi", "p")
        return gen_chunk(**{k: cfg[k] for k in keys if k in cfg})
    keys = ("B", "H", "Hkv", "W", "d", "seed", "std", "dtype", "pos_lo", "pos_hi")
    return gen_decode(**{k: cfg[k] for k in keys if k in cfg})
