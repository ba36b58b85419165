"""fp64 CPU oracle for causal sliding-window attention (TEST INFRASTRUCTURE).

Only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product library never does, and this
package never imports the product: the two share no code.

The arithmetic lives in ``swa_oracle.c`` (plain loops, fp64, OpenMP over rows);
this module only compiles it with gcc and marshals numpy arrays through ctypes.
Every function takes and returns float64 arrays in the layout the C file
documents ([B][heads][rows][d], d fastest).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(_HERE, "swa_oracle.c")
LIB = os.path.join(_HERE, "libswa_oracle.so")
_lock = threading.Lock()
_default = None

STAT_NAMES = ("valid_pairs", "covered_coords", "keys_touched", "n_live", "n_full",
              "n_partial")


def build(force: bool = False, src: str = SRC, out: str = LIB) -> str:
    """Compile the oracle with gcc (OpenMP, -O2, strict IEEE: no fast-math, no
    FMA contraction).  Rebuilds when the source is newer than the library."""
    if force or not os.path.exists(out) or os.path.getmtime(out) < os.path.getmtime(src):
        tmp = out + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-std=c99", "-fopenmp", "-fPIC", "-shared", "-Wall",
               "-fno-fast-math", "-ffp-contract=off", src, "-o", tmp, "-lm"]
        subprocess.check_call(cmd)
        os.replace(tmp, out)
    return out


def _f64(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _i32(a):
    if a is None:
        return None
    return np.ascontiguousarray(np.asarray(a, dtype=np.int32))


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


class Oracle:
    """ctypes front of one compiled oracle library (float64 numpy in and out)."""

    def __init__(self, lib_path: str):
        lib = ctypes.CDLL(lib_path)
        P = ctypes.c_void_p
        i = ctypes.c_int
        d = ctypes.c_double
        lib.orc_fwd_sink.argtypes = [i, i, i, i, i, i, i, P, P, P, P, d, P]
        lib.orc_fwd_sink.restype = None
        lib.orc_fwd_rows_sink.argtypes = [i, i, i, i, i, i, i, P, P, P, P, d, i, P, P, P, P]
        lib.orc_fwd_rows_sink.restype = None
        lib.orc_chunk.argtypes = [i, i, i, i, i, i, P, P, P, P, P, P, P, P, d, P]
        lib.orc_chunk.restype = None
        lib.orc_chunk_sink.argtypes = [i, i, i, i, i, i, i, P, P, P, P, P, P, P, P, P, P, d, P]
        lib.orc_chunk_sink.restype = None
        lib.orc_decode_sink.argtypes = [i, i, i, i, i, i, P, P, P, P, P, P, P, P, P, P, d, P]
        lib.orc_decode_sink.restype = None
        lib.orc_blockmask_sink.argtypes = [i, i, i, i, i, i, i, P, P, P, P, i, P, P, P,
                                           P, P, P, P, P]
        lib.orc_blockmask_sink.restype = ctypes.c_int64
        lib.orc_bwd_sink.argtypes = [i, i, i, i, i, i, i, P, P, P, P, P, d, P, P, P, P]
        lib.orc_bwd_sink.restype = None
        lib.orc_bwd_sel_sink.argtypes = [i, i, i, i, i, i, i, P, P, P, P, P, d, i, P, P, P, P,
                                         i, P, P, P, P, P]
        lib.orc_bwd_sel_sink.restype = None
        lib.orc_fwd_varlen.argtypes = [i, i, i, P, i, i, i, P, P, P, d, P]
        lib.orc_fwd_varlen.restype = None
        L = ctypes.c_int64
        lib.orc_layer_plan.argtypes = [i, i, i, P, P, P]
        lib.orc_layer_plan.restype = None
        lib.orc_cache_bytes.argtypes = [L] * 8
        lib.orc_cache_bytes.restype = L
        lib.orc_cache_bytes_layers.argtypes = [L, L, L, L, L, i, P]
        lib.orc_cache_bytes_layers.restype = L
        lib.orc_num_threads.argtypes = []
        lib.orc_num_threads.restype = ctypes.c_int
        lib.orc_set_num_threads.argtypes = [i]
        lib.orc_set_num_threads.restype = None
        self.lib = lib
        self.path = lib_path

    def num_threads(self) -> int:
        return self.lib.orc_num_threads()

    def set_num_threads(self, n: int) -> None:
        """Thread count of later calls (for timing at one thread)."""
        self.lib.orc_set_num_threads(int(n))

    def fwd(self, q, k, v, W: int, scale: float, q_len=None, n_sink: int = 0) -> np.ndarray:
        """Full-sequence SWA forward.  q [B,H,N,d], k/v [B,Hkv,N,d] -> o [B,H,N,d];
        n_sink > 0 keeps the first n_sink positions visible as attention sinks."""
        q, k, v = _f64(q), _f64(k), _f64(v)
        B, H, N, dd = q.shape
        Hkv = k.shape[1]
        ql = _i32(q_len)
        o = np.empty_like(q)
        self.lib.orc_fwd_sink(B, H, Hkv, N, dd, W, n_sink, _ptr(q), _ptr(k), _ptr(v), _ptr(ql),
                              float(scale), _ptr(o))
        return o

    def fwd_rows(self, q, k, v, W: int, scale: float, rows, q_len=None,
                 n_sink: int = 0) -> np.ndarray:
        """Forward for selected rows only.  rows: int array [n,3] of (b, h, i)."""
        q, k, v = _f64(q), _f64(k), _f64(v)
        B, H, N, dd = q.shape
        Hkv = k.shape[1]
        rows = np.asarray(rows, dtype=np.int32).reshape(-1, 3)
        rb, rh, ri = (np.ascontiguousarray(rows[:, c]) for c in range(3))
        ql = _i32(q_len)
        out = np.empty((rows.shape[0], dd), dtype=np.float64)
        self.lib.orc_fwd_rows_sink(B, H, Hkv, N, dd, W, n_sink, _ptr(q), _ptr(k), _ptr(v),
                                   _ptr(ql), float(scale), rows.shape[0], _ptr(rb), _ptr(rh),
                                   _ptr(ri), _ptr(out))
        return out

    def layer_plan(self, L: int, a: int, b: int):
        """Windowed (1) / global (0) flag per layer for the repeating a:b
        pattern, and the counts (L_s, L_f)."""
        flags = np.zeros(max(1, L), dtype=np.uint8)
        ns, nf = ctypes.c_int(0), ctypes.c_int(0)
        self.lib.orc_layer_plan(L, a, b, _ptr(flags), ctypes.byref(ns), ctypes.byref(nf))
        return flags[:L].copy(), ns.value, nf.value

    def cache_bytes(self, B, G, d, s, T, W, L_s, L_f) -> int:
        """The pages' estimate 2BGds[L_s min(T,W) + L_f T] in bytes."""
        return int(self.lib.orc_cache_bytes(B, G, d, s, T, W, L_s, L_f))

    def cache_bytes_layers(self, B, G, d, s, T, W_layer) -> int:
        """Sum over layers of 2BGds min(T, W_l), W_l = -1 for a global layer."""
        w = np.ascontiguousarray(np.asarray(W_layer, dtype=np.int32))
        return int(self.lib.orc_cache_bytes_layers(B, G, d, s, T, w.size, _ptr(w)))

    def fwd_varlen(self, q, k, v, cu_seqlens, W: int, scale: float, n_sink: int = 0):
        """Packed batch: q [total,H,d], k/v [total,Hkv,d] token-major, sequence b
        owning tokens cu_seqlens[b] .. cu_seqlens[b+1]-1 -> o [total,H,d]."""
        q, k, v = _f64(q), _f64(k), _f64(v)
        cu = _i32(cu_seqlens)
        total, H, dd = q.shape
        Hkv = k.shape[1]
        o = np.zeros_like(q)
        self.lib.orc_fwd_varlen(len(cu) - 1, H, Hkv, _ptr(cu), dd, W, n_sink, _ptr(q), _ptr(k),
                                _ptr(v), float(scale), _ptr(o))
        return o

    def bwd(self, q, k, v, dout, W: int, scale: float, q_len=None, n_sink: int = 0):
        """Gradients of the full-sequence forward for output gradient dout.
        Returns (dq [B,H,N,d], dk [B,Hkv,N,d], dv [B,Hkv,N,d], lse [B,H,N]); lse is
        the natural-log log-sum-exp of each row's allowed scores (-inf if none)."""
        q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(dout)
        B, H, N, dd = q.shape
        Hkv = k.shape[1]
        ql = _i32(q_len)
        dq, dk, dv = np.empty_like(q), np.empty_like(k), np.empty_like(v)
        lse = np.empty((B, H, N), dtype=np.float64)
        self.lib.orc_bwd_sink(B, H, Hkv, N, dd, W, n_sink, _ptr(q), _ptr(k), _ptr(v), _ptr(do),
                              _ptr(ql), float(scale), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(lse))
        return dq, dk, dv, lse

    def bwd_sel(self, q, k, v, dout, W: int, scale: float, qrows, keys, q_len=None,
                n_sink: int = 0):
        """Gradients for selected entries: dq of rows qrows [n,3] (b, h, i) and
        dk, dv of keys keys [m,3] (b, g, j).  Returns (dq [n,d], dk [m,d], dv [m,d])."""
        q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(dout)
        B, H, N, dd = q.shape
        Hkv = k.shape[1]
        ql = _i32(q_len)
        qrows = np.asarray(qrows, dtype=np.int32).reshape(-1, 3)
        keys = np.asarray(keys, dtype=np.int32).reshape(-1, 3)
        qc = [np.ascontiguousarray(qrows[:, c]) for c in range(3)]
        kc = [np.ascontiguousarray(keys[:, c]) for c in range(3)]
        dq = np.empty((qrows.shape[0], dd))
        dk = np.empty((keys.shape[0], dd))
        dv = np.empty((keys.shape[0], dd))
        self.lib.orc_bwd_sel_sink(B, H, Hkv, N, dd, W, n_sink, _ptr(q), _ptr(k), _ptr(v),
                                  _ptr(do), _ptr(ql), float(scale), qrows.shape[0],
                                  *[_ptr(x) for x in qc], _ptr(dq), keys.shape[0],
                                  *[_ptr(x) for x in kc], _ptr(dk), _ptr(dv))
        return dq, dk, dv

    def chunk(self, q, k_new, v_new, k_cache, v_cache, ring_start, cache_len, next_pos,
              W: int, scale: float, n_sink: int = 0, sink_k=None, sink_v=None):
        """Chunked prefill against a ring cache.  Returns (o, k_cache', v_cache',
        ring_start', cache_len', next_pos'); with n_sink > 0 also sink_k', sink_v'
        ([B,Hkv,n_sink,d] sink caches).  The inputs are not modified."""
        q, kn, vn = _f64(q), _f64(k_new), _f64(v_new)
        kc, vc = _f64(k_cache).copy(), _f64(v_cache).copy()
        rs, cl, npos = (_i32(x).copy() for x in (ring_start, cache_len, next_pos))
        B, H, Tq, dd = q.shape
        Hkv = kn.shape[1]
        o = np.empty_like(q)
        if n_sink > 0:
            sk, sv = _f64(sink_k).copy(), _f64(sink_v).copy()
            self.lib.orc_chunk_sink(B, H, Hkv, Tq, dd, W, n_sink, _ptr(q), _ptr(kn), _ptr(vn),
                                    _ptr(kc), _ptr(vc), _ptr(sk), _ptr(sv), _ptr(rs), _ptr(cl),
                                    _ptr(npos), float(scale), _ptr(o))
            return o, kc, vc, rs, cl, npos, sk, sv
        self.lib.orc_chunk(B, H, Hkv, Tq, dd, W, _ptr(q), _ptr(kn), _ptr(vn), _ptr(kc),
                           _ptr(vc), _ptr(rs), _ptr(cl), _ptr(npos), float(scale), _ptr(o))
        return o, kc, vc, rs, cl, npos

    def decode(self, q, k_new, v_new, k_cache, v_cache, ring_start, cache_len, next_pos,
               W: int, scale: float, n_sink: int = 0, sink_k=None, sink_v=None):
        """One decode step (append, then attend).  q [B,H,d], k_new/v_new [B,Hkv,d].
        Returns (o, k_cache', v_cache', ring_start', cache_len', next_pos'); with
        n_sink > 0 also sink_k', sink_v' ([B,Hkv,n_sink,d] sink caches)."""
        q, kn, vn = _f64(q), _f64(k_new), _f64(v_new)
        kc, vc = _f64(k_cache).copy(), _f64(v_cache).copy()
        rs, cl, npos = (_i32(x).copy() for x in (ring_start, cache_len, next_pos))
        B, H, dd = q.shape
        Hkv = kn.shape[1]
        o = np.empty_like(q)
        sk = sv = None
        if n_sink > 0:
            sk, sv = _f64(sink_k).copy(), _f64(sink_v).copy()
        self.lib.orc_decode_sink(B, H, Hkv, dd, W, n_sink, _ptr(q), _ptr(kn), _ptr(vn), _ptr(kc),
                                 _ptr(vc), _ptr(sk), _ptr(sv), _ptr(rs), _ptr(cl), _ptr(npos),
                                 float(scale), _ptr(o))
        if n_sink > 0:
            return o, kc, vc, rs, cl, npos, sk, sv
        return o, kc, vc, rs, cl, npos

    def blockmask(self, B, nq, nk_lin, W, tile_q, tile_k, q_start=None, k_start=None,
                  q_len=None, k_len=None, W_ring=0, ring_start=None, cache_len=None,
                  next_pos=None, n_sink=0):
        """Brute-force block metadata.  Returns a dict with cls [B,nqt,nkt] uint8,
        row_ptr [B*nqt+1] int32, col [nnz] int32, col_cls [nnz] uint8 and the six
        statistics named in STAT_NAMES.  With a ring and n_sink > 0 the key axis
        starts with n_sink rounded up to tile_k sink slots."""
        ns = -(-n_sink // tile_k) * tile_k if (W_ring > 0 and n_sink > 0) else 0
        nk = ns + W_ring + nk_lin
        nqt = -(-nq // tile_q)
        nkt = -(-nk // tile_k)
        cls = np.zeros((B, nqt, nkt), dtype=np.uint8)
        row_ptr = np.zeros(B * nqt + 1, dtype=np.int32)
        cap = max(1, B * nqt * nkt)
        col = np.zeros(cap, dtype=np.int32)
        col_cls = np.zeros(cap, dtype=np.uint8)
        stats = np.zeros(6, dtype=np.int64)
        qs, ks, ql, kl, rs, cl, npos = (_i32(x) for x in (
            q_start, k_start, q_len, k_len, ring_start, cache_len, next_pos))
        nnz = self.lib.orc_blockmask_sink(B, nq, nk_lin, W, n_sink, tile_q, tile_k, _ptr(qs),
                                          _ptr(ks), _ptr(ql), _ptr(kl), W_ring, _ptr(rs),
                                          _ptr(cl), _ptr(npos), _ptr(cls), _ptr(row_ptr),
                                          _ptr(col), _ptr(col_cls), _ptr(stats))
        out = {"cls": cls, "row_ptr": row_ptr, "col": col[:nnz].copy(),
               "col_cls": col_cls[:nnz].copy()}
        out.update({n: int(stats[i]) for i, n in enumerate(STAT_NAMES)})
        return out


def default() -> Oracle:
    """The oracle built from swa_oracle.c next to this file."""
    global _default
    with _lock:
        if _default is None:
            _default = Oracle(build())
    return _default


def num_threads() -> int:
    return default().num_threads()


def set_num_threads(n: int) -> None:
    default().set_num_threads(n)


def fwd(*a, **kw):
    return default().fwd(*a, **kw)


def fwd_rows(*a, **kw):
    return default().fwd_rows(*a, **kw)


def chunk(*a, **kw):
    return default().chunk(*a, **kw)


def bwd(*a, **kw):
    return default().bwd(*a, **kw)


def fwd_varlen(*a, **kw):
    return default().fwd_varlen(*a, **kw)


def bwd_sel(*a, **kw):
    return default().bwd_sel(*a, **kw)


def decode(*a, **kw):
    return default().decode(*a, **kw)


def blockmask(*a, **kw):
    return default().blockmask(*a, **kw)


def layer_plan(*a, **kw):
    return default().layer_plan(*a, **kw)


def cache_bytes(*a, **kw):
    return default().cache_bytes(*a, **kw)


def cache_bytes_layers(*a, **kw):
    return default().cache_bytes_layers(*a, **kw)
