"""Causal sliding-window attention for MI355X (gfx950): Python binding of libswa.so.

Thin ctypes marshalling over the C ABI declared in ``include/swa.h``; every step
of the computation runs in the library (host metadata builder, HIP kernels).
PyTorch supplies device memory and streams only.  There is no fallback: when
``libswa.so`` is missing or a call fails, a ``SwaError`` is raised.

Functions keep the ABI's names:

    swa_blockmask_size(B, nq, nk, tile_q, tile_k)          -> (cls_elems, max_nnz)
    swa_blockmask_build(B, nq, nk_lin, W, tile_q, tile_k, ..., n_sink=0) -> dict (host numpy)
    swa_fwd(q, k, v, o, W, meta, q_len=None, lse=None, scale=None)
    swa_fwd_varlen(q, k, v, o, W, meta, cu_seqlens, lse=None, scale=None)
    swa_bwd_workspace_size(B, H, N)
    swa_bwd(q, k, v, o, dout, lse, dq, dk, dv, workspace, W, meta, q_len=None, scale=None)
    swa_bwd_varlen(q, k, v, o, dout, lse, dq, dk, dv, workspace, W, meta, cu_seqlens, scale=None)
    swa_prefill_chunk(q, k_new, v_new, k_cache, v_cache, ring_start, cache_len,
                      next_pos, o, W, meta, tile_q, tile_k, scale=None)
    swa_decode_workspace_size(B, H, d, W)
    swa_decode(q, k_new, v_new, k_cache, v_cache, ring_start, cache_len, next_pos,
               o, workspace, W, scale=None, n_sink=0, sink_k=None, sink_v=None)
    swa_last_error()

``meta`` is the device copy of a build (``meta_to_device``); it carries the
build's tiles and attention-sink count, which swa_fwd and swa_bwd pass on.  Calls are enqueued
on torch's current stream of the tensors' device.
"""
from __future__ import annotations

import ctypes
import math
import os
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libswa.so")

SWA_OK, SWA_EINVAL, SWA_EUNSUPPORTED, SWA_EHIP = 0, 1, 2, 3
SWA_BF16, SWA_F32 = 0, 1
STAT_NAMES = ("valid_pairs", "covered_coords", "keys_touched", "n_live", "n_full",
              "n_partial")

# Symbols declared in include/swa.h (checked by the CPU tests).
EXPORTS = ("swa_blockmask_size", "swa_blockmask_build", "swa_fwd", "swa_prefill_chunk",
           "swa_decode_workspace_size", "swa_decode", "swa_bwd_workspace_size", "swa_bwd",
           "swa_fwd_varlen", "swa_bwd_varlen", "swa_layer_plan", "swa_cache_bytes",
           "swa_last_error", "swa_decode_noalloc", "swa_chunk_blockmask_dev")


class SwaError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__("swa status %d: %s" % (code, msg))
        self.code = code


class MaskStats(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int64) for n in STAT_NAMES]


_lock = threading.Lock()
_lib = None


def lib():
    """The loaded libswa.so (raises SwaError if it has not been built)."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise SwaError(-1, "%s is missing: build it with "
                               "`python -m causal_sliding_window_swa_amd.build`" % LIB_PATH)
            L = ctypes.CDLL(LIB_PATH)
            P, I, F = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
            L.swa_blockmask_size.argtypes = [I, I, I, I, I, ctypes.POINTER(ctypes.c_size_t),
                                             ctypes.POINTER(ctypes.c_size_t)]
            L.swa_blockmask_build.argtypes = [I, I, I, I, I, I, I, P, P, P, P, I, P, P, P,
                                              P, P, P, P, ctypes.POINTER(MaskStats)]
            L.swa_fwd.argtypes = [I, I, I, I, I, I, I, I, I, I, P, P, P, P, P, P, P, P, P, F, P]
            L.swa_fwd_varlen.argtypes = [I, I, I, I, I, I, I, I, I, I, I, P, P, P, P, P, P, P, P,
                                         P, F, P]
            L.swa_bwd_workspace_size.argtypes = [I, I, I]
            L.swa_bwd_workspace_size.restype = ctypes.c_size_t
            L.swa_bwd.argtypes = [I, I, I, I, I, I, I, I, I, I, P, P, P, P, P, P, P, P, P, P, P, P,
                                  P, P, ctypes.c_size_t, F, P]
            L.swa_bwd_varlen.argtypes = [I] * 11 + [P] * 14 + [ctypes.c_size_t, F, P]
            L.swa_prefill_chunk.argtypes = [I, I, I, I, I, I, I, I, P, P, I, I, P, P, P, P, P, P,
                                            P, P, P, P, P, P, F, P]
            L.swa_decode_workspace_size.argtypes = [I, I, I, I]
            L.swa_decode_workspace_size.restype = ctypes.c_size_t
            L.swa_decode.argtypes = [I, I, I, I, I, I, I, P, P, P, P, P, P, P, P, P, P, P, P,
                                     ctypes.c_size_t, F, P]
            L.swa_decode_noalloc.argtypes = [I, I, I, I, I, I, I, P, P, P, P, P, P, P, P, P, P,
                                             P, F, P]
            L.swa_chunk_blockmask_dev.argtypes = [I, I, I, I, I, I, P, P, P, P, P, P, P, P, P]
            L.swa_layer_plan.argtypes = [I, I, I, I, P, P, P]
            L.swa_cache_bytes.argtypes = [I, I, I, I, ctypes.c_int64, I, P, P]
            L.swa_last_error.argtypes = []
            L.swa_last_error.restype = ctypes.c_char_p
            for n in ("swa_blockmask_size", "swa_blockmask_build", "swa_fwd",
                      "swa_prefill_chunk", "swa_decode", "swa_bwd", "swa_fwd_varlen",
                      "swa_bwd_varlen", "swa_decode_noalloc", "swa_chunk_blockmask_dev",
                      "swa_layer_plan", "swa_cache_bytes"):
                getattr(L, n).restype = ctypes.c_int
            _lib = L
    return _lib


def swa_last_error() -> str:
    return lib().swa_last_error().decode()


def _check(rc):
    if rc != SWA_OK:
        raise SwaError(rc, swa_last_error())


def _np_i32(x):
    if x is None:
        return None
    if hasattr(x, "cpu"):
        x = x.cpu().numpy()
    return np.ascontiguousarray(np.asarray(x, dtype=np.int32))


def _hp(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def swa_blockmask_size(B, nq, nk, tile_q, tile_k):
    c, n = ctypes.c_size_t(), ctypes.c_size_t()
    _check(lib().swa_blockmask_size(B, nq, nk, tile_q, tile_k, ctypes.byref(c), ctypes.byref(n)))
    return c.value, n.value


def swa_blockmask_build(B, nq, nk_lin, W, tile_q, tile_k, q_start=None, k_start=None,
                        q_len=None, k_len=None, W_ring=0, ring_start=None, cache_len=None,
                        next_pos=None, n_sink=0):
    """Host metadata build.  Returns dict: cls [B,nqt,nkt] uint8, row_ptr int32,
    col int32 [nnz], col_cls uint8 [nnz], plus the six statistics.  A ring axis
    with n_sink > 0 starts with n_sink rounded up to tile_k sink slots."""
    ns = -(-n_sink // tile_k) * tile_k if (W_ring > 0 and n_sink > 0) else 0
    nk = ns + W_ring + nk_lin
    cls_n, max_nnz = swa_blockmask_size(B, nq, nk, tile_q, tile_k)
    nqt = -(-nq // tile_q)
    nkt = -(-nk // tile_k)
    cls = np.zeros(max(1, cls_n), dtype=np.uint8)
    row_ptr = np.zeros(B * nqt + 1, dtype=np.int32)
    col = np.zeros(max(1, max_nnz), dtype=np.int32)
    col_cls = np.zeros(max(1, max_nnz), dtype=np.uint8)
    st = MaskStats()
    args = [_np_i32(x) for x in (q_start, k_start, q_len, k_len, ring_start, cache_len,
                                 next_pos)]
    _check(lib().swa_blockmask_build(B, nq, nk_lin, W, n_sink, tile_q, tile_k,
                                     *[_hp(a) for a in args[:4]],
                                     W_ring, *[_hp(a) for a in args[4:]], _hp(cls),
                                     _hp(row_ptr), _hp(col), _hp(col_cls), ctypes.byref(st)))
    nnz = int(row_ptr[-1])
    out = {"cls": cls[:cls_n].reshape(B, nqt, nkt), "row_ptr": row_ptr,
           "col": col[:nnz].copy(), "col_cls": col_cls[:nnz].copy(),
           "tile_q": tile_q, "tile_k": tile_k, "n_sink": n_sink, "max_len": nq,
           "B": B, "nq": nq, "nk_lin": nk_lin, "W": W, "W_ring": W_ring}
    out.update({n: int(getattr(st, n)) for n in STAT_NAMES})
    return out


def chunk_meta_buffers(B, Tq, W, tile_q, tile_k, device, n_sink=0, stats=True):
    """Device arrays for swa_chunk_blockmask_dev of these shapes (allocated once,
    rebuilt in place every step), as a metadata dict swa_prefill_chunk takes;
    stats=False: no statistics (one kernel fewer per build)."""
    import torch
    ns = -(-n_sink // tile_k) * tile_k if n_sink > 0 else 0
    nk = ns + W + Tq
    cls_n, max_nnz = swa_blockmask_size(B, Tq, nk, tile_q, tile_k)
    nqt = -(-Tq // tile_q)
    dev = torch.device(device)
    return {"row_ptr": torch.zeros(B * nqt + 1, dtype=torch.int32, device=dev),
            "col": torch.zeros(max(1, max_nnz), dtype=torch.int32, device=dev),
            "col_cls": torch.zeros(max(1, max_nnz), dtype=torch.uint8, device=dev),
            "cls": torch.zeros(max(1, cls_n), dtype=torch.uint8, device=dev),
            "stats": torch.zeros(6, dtype=torch.int64, device=dev) if stats else None,
            "tile_q": tile_q, "tile_k": tile_k, "n_sink": n_sink, "max_len": Tq,
            "B": B, "nq": Tq, "nk_lin": Tq, "W": W, "W_ring": W}


def swa_chunk_blockmask_dev(meta, ring_start, cache_len, next_pos, stream=None):
    """Rebuild, on the device and in stream order, the metadata of the next
    swa_prefill_chunk step from the device ring state (int32 [B] tensors);
    `meta` comes from chunk_meta_buffers and is filled in place."""
    for t in (ring_start, cache_len, next_pos):
        _require(t.is_contiguous() and t.numel() == meta["B"], "ring state must be int32 [B]")
    _check(lib().swa_chunk_blockmask_dev(meta["B"], meta["nq"], meta["W"], meta["n_sink"],
                                         meta["tile_q"], meta["tile_k"], _dptr(ring_start),
                                         _dptr(cache_len), _dptr(next_pos), _dptr(meta["cls"]),
                                         _dptr(meta["row_ptr"]), _dptr(meta["col"]),
                                         _dptr(meta["col_cls"]), _dptr(meta["stats"]),
                                         _stream(ring_start, stream)))
    return meta


def swa_layer_plan(L, ratio, W):
    """Per-layer windows of an L-layer stack for a local:global ratio given as
    "a:b" or (a, b).  Returns (W_layer int32 [L] with -1 for global layers,
    L_s, L_f)."""
    if isinstance(ratio, str):
        parts = ratio.split(":")
        if len(parts) != 2:
            raise ValueError("ratio must look like 'a:b', got %r" % (ratio,))
        ratio = parts
    a, b = (int(x) for x in ratio)
    w = np.zeros(max(1, L), dtype=np.int32)
    ns, nf = ctypes.c_int32(0), ctypes.c_int32(0)
    _check(lib().swa_layer_plan(L, a, b, W, _hp(w), ctypes.byref(ns), ctypes.byref(nf)))
    return w[:L].copy(), ns.value, nf.value


def swa_cache_bytes(B, G, d, elem_bytes, T, W_layer):
    """Bytes of the persistent K/V caches of a stack with windows W_layer
    (-1 = global) after T tokens."""
    w = _np_i32(W_layer)
    if w is None or w.size == 0:
        w = np.zeros(1, dtype=np.int32)
        L = 0
    else:
        L = int(w.size)
    out = ctypes.c_int64(0)
    _check(lib().swa_cache_bytes(B, G, d, elem_bytes, ctypes.c_int64(T), L, _hp(w),
                                 ctypes.byref(out)))
    return int(out.value)


def meta_to_device(meta, device):
    """Device copies of a build's CSR arrays (what the kernels read)."""
    import torch
    dev = torch.device(device)
    col = meta["col"] if meta["col"].size else np.zeros(1, dtype=np.int32)
    ccls = meta["col_cls"] if meta["col_cls"].size else np.zeros(1, dtype=np.uint8)
    return {"row_ptr": torch.from_numpy(meta["row_ptr"]).to(dev),
            "col": torch.from_numpy(col).to(dev),
            "col_cls": torch.from_numpy(ccls).to(dev),
            "cls": torch.from_numpy(np.ascontiguousarray(meta["cls"]).reshape(-1)).to(dev),
            "tile_q": meta["tile_q"], "tile_k": meta["tile_k"],
            "n_sink": meta.get("n_sink", 0), "max_len": meta.get("max_len", 0),
            **{k: meta[k] for k in _SHAPE_KEYS}}


_SHAPE_KEYS = ("B", "nq", "nk_lin", "W", "W_ring")


def _check_meta(meta, fn, **want):
    """The kernels index the device metadata without bounds checks, so it must
    come from a swa_blockmask_build with the call's shape; a mismatch is
    rejected here, before anything is enqueued."""
    for key in _SHAPE_KEYS:
        if key not in meta:
            raise SwaError(SWA_EINVAL, "%s: metadata lacks %r (use swa_blockmask_build and "
                           "meta_to_device)" % (fn, key))
    for key, v in want.items():
        if meta[key] != v:
            raise SwaError(SWA_EINVAL, "%s: metadata built for %s=%d, the call has %s=%d"
                           % (fn, key, meta[key], key, v))
    nqt = -(-meta["nq"] // meta["tile_q"])
    if meta["row_ptr"].numel() != meta["B"] * nqt + 1:
        raise SwaError(SWA_EINVAL, "%s: row_ptr has %d entries, the build's shape needs %d"
                       % (fn, meta["row_ptr"].numel(), meta["B"] * nqt + 1))


def _dptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _dtype_code(t):
    import torch
    if t.dtype == torch.bfloat16:
        return SWA_BF16
    if t.dtype == torch.float32:
        return SWA_F32
    raise SwaError(SWA_EUNSUPPORTED, "dtype %s not supported" % t.dtype)


def _stream(t, stream):
    import torch
    if stream is not None:
        return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else stream)
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _require(cond, msg):
    if not cond:
        raise SwaError(SWA_EINVAL, msg)


def swa_fwd(q, k, v, o, W, meta, q_len=None, lse=None, scale=None, stream=None):
    """Full-sequence forward.  q,o [B,H,N,d], k,v [B,Hkv,N,d] device tensors;
    lse: optional fp32 [B,H,N] device tensor for the row log-sum-exp."""
    for t in (q, k, v, o):
        _require(t.is_contiguous(), "tensors must be contiguous")
    B, H, N, d = q.shape
    Hkv = k.shape[1]
    _require(tuple(k.shape) == (B, Hkv, N, d) and tuple(v.shape) == (B, Hkv, N, d) and
             tuple(o.shape) == (B, H, N, d), "shape mismatch")
    _require(k.dtype == q.dtype == v.dtype == o.dtype, "dtype mismatch")
    _check_meta(meta, "swa_fwd", B=B, nq=N, nk_lin=N, W=W, W_ring=0)
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    _check(lib().swa_fwd(_dtype_code(q), B, H, Hkv, N, d, W, meta.get("n_sink", 0),
                         meta["tile_q"], meta["tile_k"],
                         _dptr(q), _dptr(k), _dptr(v), _dptr(o), _dptr(q_len),
                         _dptr(meta["row_ptr"]), _dptr(meta["col"]), _dptr(meta["col_cls"]),
                         _dptr(lse), ctypes.c_float(scale), _stream(q, stream)))
    return o


def swa_fwd_varlen(q, k, v, o, W, meta, cu_seqlens, lse=None, scale=None, stream=None):
    """Packed variable-length forward.  q,o [total,H,d], k,v [total,Hkv,d]
    token-major device tensors; cu_seqlens int32 [B+1] device tensor; meta
    built with nq = nk_lin = max_len and q_len = k_len = the lengths;
    lse: optional fp32 [total,H] device tensor."""
    for t in (q, k, v, o):
        _require(t.is_contiguous(), "tensors must be contiguous")
    total, H, d = q.shape
    Hkv = k.shape[1]
    _require(tuple(k.shape) == (total, Hkv, d) and tuple(v.shape) == (total, Hkv, d) and
             tuple(o.shape) == (total, H, d), "shape mismatch")
    _require(k.dtype == q.dtype == v.dtype == o.dtype, "dtype mismatch")
    B = cu_seqlens.numel() - 1
    _check_meta(meta, "swa_fwd_varlen", B=B, W=W, W_ring=0)
    _require(meta["nk_lin"] == meta["nq"], "swa_fwd_varlen: metadata must be built with "
             "nq = nk_lin = max_len")
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    _check(lib().swa_fwd_varlen(_dtype_code(q), B, H, Hkv, total, meta["max_len"], d, W,
                                meta.get("n_sink", 0), meta["tile_q"], meta["tile_k"],
                                _dptr(q), _dptr(k), _dptr(v), _dptr(o), _dptr(cu_seqlens),
                                _dptr(meta["row_ptr"]), _dptr(meta["col"]),
                                _dptr(meta["col_cls"]), _dptr(lse), ctypes.c_float(scale),
                                _stream(q, stream)))
    return o


def swa_bwd_workspace_size(B, H, N) -> int:
    return int(lib().swa_bwd_workspace_size(B, H, N))


def swa_bwd(q, k, v, o, dout, lse, dq, dk, dv, workspace, W, meta, q_len=None, scale=None,
            stream=None):
    """Gradients of swa_fwd for output gradient dout.  q,o,dout,dq [B,H,N,d];
    k,v,dk,dv [B,Hkv,N,d]; lse fp32 [B,H,N] from swa_fwd; workspace: device
    tensor of at least swa_bwd_workspace_size(B, H, N) bytes."""
    for t in (q, k, v, o, dout, lse, dq, dk, dv):
        _require(t.is_contiguous(), "tensors must be contiguous")
    B, H, N, d = q.shape
    Hkv = k.shape[1]
    _require(tuple(k.shape) == (B, Hkv, N, d) and tuple(v.shape) == (B, Hkv, N, d) and
             tuple(o.shape) == (B, H, N, d) and tuple(dout.shape) == (B, H, N, d) and
             tuple(dq.shape) == (B, H, N, d) and tuple(dk.shape) == (B, Hkv, N, d) and
             tuple(dv.shape) == (B, Hkv, N, d) and tuple(lse.shape) == (B, H, N),
             "shape mismatch")
    _require(len({t.dtype for t in (q, k, v, o, dout, dq, dk, dv)}) == 1, "dtype mismatch")
    _check_meta(meta, "swa_bwd", B=B, nq=N, nk_lin=N, W=W, W_ring=0)
    nkt = -(-N // meta["tile_k"])
    _require(meta["cls"].numel() == B * (-(-N // meta["tile_q"])) * nkt,
             "swa_bwd: class grid size does not match the call")
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    ws_bytes = workspace.numel() * workspace.element_size()
    _check(lib().swa_bwd(_dtype_code(q), B, H, Hkv, N, d, W, meta.get("n_sink", 0),
                         meta["tile_q"], meta["tile_k"],
                         _dptr(q), _dptr(k), _dptr(v), _dptr(o), _dptr(dout), _dptr(lse),
                         _dptr(q_len), _dptr(meta["row_ptr"]), _dptr(meta["col"]),
                         _dptr(meta["cls"]), _dptr(dq), _dptr(dk), _dptr(dv), _dptr(workspace),
                         ctypes.c_size_t(ws_bytes), ctypes.c_float(scale), _stream(q, stream)))
    return dq, dk, dv


def swa_bwd_varlen(q, k, v, o, dout, lse, dq, dk, dv, workspace, W, meta, cu_seqlens,
                   scale=None, stream=None):
    """Gradients of swa_fwd_varlen.  q,o,dout,dq [total,H,d]; k,v,dk,dv
    [total,Hkv,d] token-major; lse fp32 [total,H] from swa_fwd_varlen; meta and
    cu_seqlens as for swa_fwd_varlen; workspace: device tensor of at least
    swa_bwd_workspace_size(1, H, total) bytes."""
    for t in (q, k, v, o, dout, lse, dq, dk, dv):
        _require(t.is_contiguous(), "tensors must be contiguous")
    total, H, d = q.shape
    Hkv = k.shape[1]
    _require(tuple(k.shape) == (total, Hkv, d) and tuple(v.shape) == (total, Hkv, d) and
             tuple(o.shape) == (total, H, d) and tuple(dout.shape) == (total, H, d) and
             tuple(dq.shape) == (total, H, d) and tuple(dk.shape) == (total, Hkv, d) and
             tuple(dv.shape) == (total, Hkv, d) and tuple(lse.shape) == (total, H),
             "shape mismatch")
    _require(len({t.dtype for t in (q, k, v, o, dout, dq, dk, dv)}) == 1, "dtype mismatch")
    B = cu_seqlens.numel() - 1
    _check_meta(meta, "swa_bwd_varlen", B=B, W=W, W_ring=0)
    _require(meta["nk_lin"] == meta["nq"], "swa_bwd_varlen: metadata must be built with "
             "nq = nk_lin = max_len")
    n = meta["max_len"]
    _require(meta["cls"].numel() == B * (-(-n // meta["tile_q"])) * (-(-n // meta["tile_k"])),
             "swa_bwd_varlen: class grid size does not match the call")
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    ws_bytes = workspace.numel() * workspace.element_size()
    _check(lib().swa_bwd_varlen(_dtype_code(q), B, H, Hkv, total, n, d, W,
                                meta.get("n_sink", 0), meta["tile_q"], meta["tile_k"],
                                _dptr(q), _dptr(k), _dptr(v), _dptr(o), _dptr(dout), _dptr(lse),
                                _dptr(cu_seqlens), _dptr(meta["row_ptr"]), _dptr(meta["col"]),
                                _dptr(meta["cls"]), _dptr(dq), _dptr(dk), _dptr(dv),
                                _dptr(workspace), ctypes.c_size_t(ws_bytes),
                                ctypes.c_float(scale), _stream(q, stream)))
    return dq, dk, dv


def swa_prefill_chunk(q, k_new, v_new, k_cache, v_cache, ring_start, cache_len, next_pos, o,
                      W, meta, scale=None, stream=None, n_sink=None, sink_k=None, sink_v=None):
    """Chunked prefill; q,o [B,H,Tq,d], k_new,v_new [B,Hkv,Tq,d], caches [B,Hkv,W,d],
    ring state int32 [B] device tensors (updated in place on the stream).
    Attention sinks: the metadata's n_sink (or n_sink given here) with sink
    caches sink_k, sink_v [B,Hkv,n_sink,d] (updated in place)."""
    n_sink = meta.get("n_sink", 0) if n_sink is None else n_sink
    if n_sink > 0:
        _require(sink_k is not None and sink_v is not None, "sink caches required")
        _require(tuple(sink_k.shape) == (q.shape[0], k_new.shape[1], n_sink, q.shape[3]) and
                 tuple(sink_v.shape) == tuple(sink_k.shape), "sink cache shape")
        _require(sink_k.is_contiguous() and sink_v.is_contiguous() and
                 sink_k.dtype == q.dtype and sink_v.dtype == q.dtype, "sink cache layout")
    for t in (q, k_new, v_new, k_cache, v_cache, o, ring_start, cache_len, next_pos):
        _require(t.is_contiguous(), "tensors must be contiguous")
    B, H, Tq, d = q.shape
    Hkv = k_new.shape[1]
    _require(tuple(k_cache.shape) == (B, Hkv, W, d) and tuple(v_cache.shape) == (B, Hkv, W, d),
             "cache shape must be [B,Hkv,W,d]")
    _require(tuple(k_new.shape) == (B, Hkv, Tq, d) and tuple(v_new.shape) == (B, Hkv, Tq, d)
             and tuple(o.shape) == (B, H, Tq, d), "shape mismatch")
    _check_meta(meta, "swa_prefill_chunk", B=B, nq=Tq, nk_lin=Tq, W=W, W_ring=W)
    _require(n_sink == meta.get("n_sink", 0), "swa_prefill_chunk: metadata built for "
             "n_sink=%d, the call has %d" % (meta.get("n_sink", 0), n_sink))
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    _check(lib().swa_prefill_chunk(_dtype_code(q), B, H, Hkv, Tq, d, W, n_sink,
                                   _dptr(sink_k) if n_sink > 0 else None,
                                   _dptr(sink_v) if n_sink > 0 else None, meta["tile_q"],
                                   meta["tile_k"], _dptr(q), _dptr(k_new), _dptr(v_new),
                                   _dptr(k_cache), _dptr(v_cache), _dptr(ring_start),
                                   _dptr(cache_len), _dptr(next_pos), _dptr(meta["row_ptr"]),
                                   _dptr(meta["col"]), _dptr(meta["col_cls"]), _dptr(o),
                                   ctypes.c_float(scale), _stream(q, stream)))
    return o


def swa_decode_workspace_size(B, H, d, W) -> int:
    return int(lib().swa_decode_workspace_size(B, H, d, W))


def swa_decode(q, k_new, v_new, k_cache, v_cache, ring_start, cache_len, next_pos, o,
               workspace, W, scale=None, stream=None, n_sink=0, sink_k=None, sink_v=None):
    """One decode step; q,o [B,H,d], k_new,v_new [B,Hkv,d], caches [B,Hkv,W,d];
    with n_sink > 0 the sink caches sink_k, sink_v [B,Hkv,n_sink,d] (in/out)."""
    for t in (q, k_new, v_new, k_cache, v_cache, o, ring_start, cache_len, next_pos):
        _require(t.is_contiguous(), "tensors must be contiguous")
    B, H, d = q.shape
    Hkv = k_new.shape[1]
    _require(tuple(k_cache.shape) == (B, Hkv, W, d) and tuple(v_cache.shape) == (B, Hkv, W, d),
             "cache shape must be [B,Hkv,W,d]")
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    if n_sink:
        _require(sink_k is not None and sink_v is not None and
                 tuple(sink_k.shape) == (B, Hkv, n_sink, d) and
                 tuple(sink_v.shape) == (B, Hkv, n_sink, d) and sink_k.is_contiguous() and
                 sink_v.is_contiguous(), "sink caches must be contiguous [B,Hkv,n_sink,d]")
    _check(lib().swa_decode(_dtype_code(q), B, H, Hkv, d, W, n_sink,
                            _dptr(sink_k if n_sink else None), _dptr(sink_v if n_sink else None),
                            _dptr(q), _dptr(k_new),
                            _dptr(v_new), _dptr(k_cache), _dptr(v_cache), _dptr(ring_start),
                            _dptr(cache_len), _dptr(next_pos), _dptr(o), _dptr(workspace),
                            ctypes.c_size_t(ws_bytes), ctypes.c_float(scale),
                            _stream(q, stream)))
    return o


def swa_decode_noalloc(q, k_new, v_new, k_cache, v_cache, ring_start, cache_len, next_pos, o,
                       W, scale=None, stream=None, n_sink=0, sink_k=None, sink_v=None):
    """swa_decode without a workspace: the library's own scratch array holds
    the partials (for callers that cannot allocate).  Runs on q's device."""
    for t in (q, k_new, v_new, k_cache, v_cache, o, ring_start, cache_len, next_pos):
        _require(t.is_contiguous(), "tensors must be contiguous")
    B, H, d = q.shape
    Hkv = k_new.shape[1]
    _require(tuple(k_cache.shape) == (B, Hkv, W, d) and tuple(v_cache.shape) == (B, Hkv, W, d),
             "cache shape must be [B,Hkv,W,d]")
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    if n_sink:
        _require(sink_k is not None and sink_v is not None and
                 tuple(sink_k.shape) == (B, Hkv, n_sink, d) and
                 tuple(sink_v.shape) == (B, Hkv, n_sink, d) and sink_k.is_contiguous() and
                 sink_v.is_contiguous(), "sink caches must be contiguous [B,Hkv,n_sink,d]")
    import torch
    with torch.cuda.device(q.device):
        _check(lib().swa_decode_noalloc(_dtype_code(q), B, H, Hkv, d, W, n_sink,
                                        _dptr(sink_k if n_sink else None),
                                        _dptr(sink_v if n_sink else None), _dptr(q),
                                        _dptr(k_new), _dptr(v_new), _dptr(k_cache),
                                        _dptr(v_cache), _dptr(ring_start), _dptr(cache_len),
                                        _dptr(next_pos), _dptr(o), ctypes.c_float(scale),
                                        _stream(q, stream)))
    return o
