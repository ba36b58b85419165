"""The C-ABI library on the CPU: it loads, exports every declared symbol, and
rejects bad arguments with the documented status before launching anything."""
import ctypes
import os
import re

import pytest

import causal_sliding_window_swa_amd as swa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    with open(os.path.join(ROOT, "include", "swa.h")) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(swa_\w+)\s*\(", text)))


def test_exports_every_declared_symbol():
    names = declared_functions()
    assert set(names) == set(swa.EXPORTS)
    L = swa.lib()
    for n in names:
        assert hasattr(L, n), n


def test_blockmask_rejects_bad_arguments():
    with pytest.raises(swa.SwaError) as e:
        swa.swa_blockmask_build(1, 8, 8, 0, 2, 2)
    assert e.value.code == swa.SWA_EINVAL and "W" in str(e.value)
    with pytest.raises(swa.SwaError):
        swa.swa_blockmask_build(1, 8, 8, 3, 0, 2)
    with pytest.raises(swa.SwaError):  # ring size not a multiple of tile_k
        swa.swa_blockmask_build(1, 4, 4, 6, 4, 4, q_start=[6], k_start=[6], W_ring=6,
                                ring_start=[0], cache_len=[6], next_pos=[6])
    with pytest.raises(swa.SwaError):  # ring start out of range
        swa.swa_blockmask_build(1, 4, 4, 8, 4, 4, q_start=[8], k_start=[8], W_ring=8,
                                ring_start=[8], cache_len=[8], next_pos=[8])
    with pytest.raises(swa.SwaError):  # next_pos below cache_len
        swa.swa_blockmask_build(1, 4, 4, 8, 4, 4, q_start=[3], k_start=[3], W_ring=8,
                                ring_start=[0], cache_len=[8], next_pos=[3])
    with pytest.raises(swa.SwaError):  # length past the rows
        swa.swa_blockmask_build(1, 8, 8, 3, 2, 2, q_len=[9], k_len=[9])
    with pytest.raises(swa.SwaError):  # positions overflowing int32
        swa.swa_blockmask_build(1, 8, 8, 3, 2, 2, q_start=[2**31 - 5], k_start=[0])
    with pytest.raises(swa.SwaError):  # negative sink count
        swa.swa_blockmask_build(1, 8, 8, 3, 2, 2, n_sink=-1)
    # sinks with a ring key axis: a sink segment of whole key tiles in front
    m = swa.swa_blockmask_build(1, 4, 4, 8, 4, 4, q_start=[8], k_start=[8], W_ring=8,
                                ring_start=[0], cache_len=[8], next_pos=[8], n_sink=2)
    assert m["cls"].shape == (1, 1, (4 + 8 + 4) // 4)


P = ctypes.c_void_p


def _fwd(dt=0, B=1, H=4, Hkv=2, N=128, d=128, W=16, tq=128, tk=64, ptr=16, sink=0):
    p = ctypes.c_void_p(ptr)
    return swa.lib().swa_fwd(dt, B, H, Hkv, N, d, W, sink, tq, tk, p, p, p, p, None, p, p, p,
                             None, ctypes.c_float(0.1), None)


def test_fwd_validation_codes():
    assert _fwd(W=0) == swa.SWA_EINVAL
    assert _fwd(H=3, Hkv=2) == swa.SWA_EINVAL
    assert _fwd(N=0) == swa.SWA_EINVAL
    assert _fwd(d=96) == swa.SWA_EUNSUPPORTED
    assert _fwd(dt=1, d=6) == swa.SWA_EUNSUPPORTED
    assert _fwd(tq=32) == swa.SWA_EUNSUPPORTED
    assert _fwd(tk=32) == swa.SWA_EUNSUPPORTED
    assert _fwd(tk=256) == swa.SWA_EUNSUPPORTED
    # 256-row query tiles: head dim 128 and 64-key tiles only
    assert _fwd(tq=256, d=64) == swa.SWA_EUNSUPPORTED
    assert _fwd(tq=256, tk=128) == swa.SWA_EUNSUPPORTED
    assert "tile_q = 256" in swa.swa_last_error()
    assert _fwd(tq=512) == swa.SWA_EUNSUPPORTED
    assert _fwd(ptr=0) == swa.SWA_EINVAL
    assert _fwd(ptr=8) == swa.SWA_EINVAL  # misaligned
    assert _fwd(dt=7) == swa.SWA_EINVAL
    assert _fwd(sink=-1) == swa.SWA_EINVAL
    assert "window" in swa.swa_last_error() or True


def _bwd(dt=0, B=1, H=4, Hkv=2, N=128, d=128, W=16, ptr=16, ws=None, cls=True):
    p = ctypes.c_void_p(ptr)
    need = swa.swa_bwd_workspace_size(B, H, N)
    wsb = need if ws is None else ws
    return swa.lib().swa_bwd(dt, B, H, Hkv, N, d, W, 0, 128, 64, p, p, p, p, p, p, None, p, p,
                             p if cls else None, p, p, p, p, ctypes.c_size_t(wsb),
                             ctypes.c_float(0.1), None)


def test_bwd_validation_codes():
    assert swa.swa_bwd_workspace_size(2, 3, 5) == 2 * 3 * 5 * 4
    assert swa.swa_bwd_workspace_size(0, 3, 5) == 0
    assert _bwd(W=0) == swa.SWA_EINVAL
    assert _bwd(H=3, Hkv=2) == swa.SWA_EINVAL
    assert _bwd(N=0) == swa.SWA_EINVAL
    assert _bwd(d=96) == swa.SWA_EUNSUPPORTED
    assert _bwd(dt=1, d=6) == swa.SWA_EUNSUPPORTED
    assert _bwd(ptr=0) == swa.SWA_EINVAL
    assert _bwd(ptr=8) == swa.SWA_EINVAL
    assert _bwd(ws=100) == swa.SWA_EINVAL
    assert "workspace" in swa.swa_last_error()
    assert _bwd(cls=False) == swa.SWA_EINVAL


def _varlen(total=100, max_len=60, cu=True, d=128, W=16):
    p = ctypes.c_void_p(16)
    return swa.lib().swa_fwd_varlen(0, 2, 4, 2, total, max_len, d, W, 0, 128, 64, p, p, p, p,
                                    p if cu else None, p, p, p, None, ctypes.c_float(0.1), None)


def test_varlen_validation_codes():
    assert _varlen(total=0) == swa.SWA_EINVAL
    assert _varlen(max_len=0) == swa.SWA_EINVAL
    assert _varlen(max_len=101) == swa.SWA_EINVAL
    assert _varlen(cu=False) == swa.SWA_EINVAL
    assert _varlen(W=0) == swa.SWA_EINVAL
    assert _varlen(d=96) == swa.SWA_EUNSUPPORTED


def _bwd_varlen(dt=0, total=100, max_len=60, d=128, W=16, tq=128, tk=64, cu=True, cls=True,
                ws=None, H=4, n_sink=0):
    p = ctypes.c_void_p(16)
    if ws is None:
        ws = swa.swa_bwd_workspace_size(1, H, total)
    return swa.lib().swa_bwd_varlen(dt, 2, H, 2, total, max_len, d, W, n_sink, tq, tk,
                                    p, p, p, p, p, p, p if cu else None, p, p,
                                    p if cls else None, p, p, p, p, ctypes.c_size_t(ws),
                                    ctypes.c_float(0.1), None)


def test_bwd_varlen_validation_codes():
    """Every refusal happens before a launch (the pointers are never touched)."""
    assert _bwd_varlen(total=0) == swa.SWA_EINVAL
    assert _bwd_varlen(max_len=0) == swa.SWA_EINVAL
    assert _bwd_varlen(max_len=101) == swa.SWA_EINVAL
    assert _bwd_varlen(W=0) == swa.SWA_EINVAL
    assert _bwd_varlen(n_sink=-1) == swa.SWA_EINVAL
    assert _bwd_varlen(cu=False) == swa.SWA_EINVAL
    assert _bwd_varlen(cls=False) == swa.SWA_EINVAL
    # fp32 takes any d % 4 == 0 up to 128 (and any tiles), bf16 d in {64, 128}
    assert _bwd_varlen(dt=1, d=130) == swa.SWA_EUNSUPPORTED
    assert _bwd_varlen(dt=1, d=6) == swa.SWA_EUNSUPPORTED
    assert _bwd_varlen(d=96) == swa.SWA_EUNSUPPORTED
    assert _bwd_varlen(tq=32) == swa.SWA_EUNSUPPORTED
    assert _bwd_varlen(tk=128) == swa.SWA_EUNSUPPORTED
    assert _bwd_varlen(tq=256) == swa.SWA_EUNSUPPORTED  # a forward-only tile shape
    # workspace: fp32 row values [total][H]
    assert _bwd_varlen(ws=100 * 4 * 4 - 1) == swa.SWA_EINVAL
    assert "workspace" in swa.swa_last_error()
    # query rows H * d * 2 bytes apart: max_len = 2^20, H = 8, d = 128 spans 2^31
    assert _bwd_varlen(total=1 << 20, max_len=1 << 20, H=8) == swa.SWA_EUNSUPPORTED
    assert "span" in swa.swa_last_error()


def _chunk(Tq=64, W=128, tk=64, d=128, nullstate=False, sink=0, sink_ptr=16):
    p = ctypes.c_void_p(16)
    st = None if nullstate else p
    sp = ctypes.c_void_p(sink_ptr) if sink_ptr else None
    return swa.lib().swa_prefill_chunk(0, 1, 4, 2, Tq, d, W, sink, sp, sp, 128, tk, p, p, p, p,
                                       p, st, st, st, p, p, p, p, ctypes.c_float(0.1), None)


def test_chunk_validation_codes():
    assert _chunk(Tq=0) == swa.SWA_EINVAL
    assert _chunk(Tq=129) == swa.SWA_EINVAL
    assert _chunk(W=96) == swa.SWA_EINVAL  # W not a multiple of tile_k
    assert _chunk(nullstate=True) == swa.SWA_EINVAL
    assert _chunk(d=80) == swa.SWA_EUNSUPPORTED
    assert _chunk(sink=-1) == swa.SWA_EINVAL
    assert _chunk(sink=4, sink_ptr=0) == swa.SWA_EINVAL     # sinks need their caches
    assert _chunk(sink=4, sink_ptr=24) == swa.SWA_EINVAL    # misaligned sink cache
    assert _chunk(sink=0, sink_ptr=0, nullstate=True) == swa.SWA_EINVAL  # still checks the rest


def _decode(H=32, Hkv=8, d=128, W=4096, ws=None, ws_bytes=0, dt=0, sink=0, sink_ptr=16):
    p = ctypes.c_void_p(16)
    sp = ctypes.c_void_p(sink_ptr) if sink_ptr else None
    return swa.lib().swa_decode(dt, 2, H, Hkv, d, W, sink, sp, sp, p, p, p, p, p, p, p, p, p,
                                ws, ctypes.c_size_t(ws_bytes), ctypes.c_float(0.1), None)


def test_decode_validation_codes():
    need = swa.swa_decode_workspace_size(2, 32, 128, 4096)
    assert need > 0
    assert _decode(ws=None) == swa.SWA_EINVAL
    assert _decode(ws=ctypes.c_void_p(16), ws_bytes=need - 1) == swa.SWA_EINVAL
    assert _decode(H=48, Hkv=3) == swa.SWA_EUNSUPPORTED  # group of 16
    assert _decode(W=0) == swa.SWA_EINVAL
    assert _decode(sink=-1) == swa.SWA_EINVAL
    assert _decode(sink=4, sink_ptr=0) == swa.SWA_EINVAL  # sink caches required
    assert _decode(sink=4, sink_ptr=8) == swa.SWA_EINVAL  # misaligned
    assert swa.swa_decode_workspace_size(0, 32, 128, 4096) == 0


def _decode_noalloc(B=2, H=32, Hkv=8, d=128, W=4096, dt=0, sink=0, sink_ptr=16):
    p = ctypes.c_void_p(16)
    sp = ctypes.c_void_p(sink_ptr) if sink_ptr else None
    return swa.lib().swa_decode_noalloc(dt, B, H, Hkv, d, W, sink, sp, sp, p, p, p, p, p, p, p,
                                        p, p, ctypes.c_float(0.1), None)


def test_decode_noalloc_validation_codes():
    """The allocation-free decode checks what swa_decode checks, and refuses
    shapes whose one-range partials exceed its 32 MiB scratch (only with
    attention sinks), all before touching the device."""
    assert _decode_noalloc(W=0) == swa.SWA_EINVAL
    assert _decode_noalloc(H=48, Hkv=3) == swa.SWA_EUNSUPPORTED
    assert _decode_noalloc(d=80) == swa.SWA_EUNSUPPORTED
    assert _decode_noalloc(sink=-1) == swa.SWA_EINVAL
    assert _decode_noalloc(sink=4, sink_ptr=0) == swa.SWA_EINVAL
    # 1024 * 64 * (128 + 2) * 4 bytes > 32 MiB
    assert _decode_noalloc(B=1024, H=64, Hkv=8, sink=4) == swa.SWA_EINVAL
    assert b"scratch" in swa.lib().swa_last_error()


def test_bf16_span_limit():
    """The bf16 tile kernels address one head's K/V rows with 32-bit offsets:
    longer spans are refused before any launch (no device memory needed)."""
    L = swa.lib()
    P = ctypes.c_void_p(16)
    # N * d * 2 = 2^31 for N = 2^23, d = 128
    rc = L.swa_fwd(0, 1, 1, 1, 1 << 23, 128, 64, 0, 128, 64, P, P, P, P, None, P, P, P, None,
                   ctypes.c_float(0.1), None)
    assert rc == 2 and b"span" in L.swa_last_error()
    # varlen: max_len * Hkv * d * 2 = 2^31 for max_len = 2^20, Hkv = 8
    rc = L.swa_fwd_varlen(0, 1, 8, 8, 1 << 20, 1 << 20, 128, 64, 0, 128, 64, P, P, P, P, P, P, P,
                          P, None, ctypes.c_float(0.1), None)
    assert rc == 2 and b"span" in L.swa_last_error()
    # fp32 has no such limit at this check (it reaches other validation instead)
    rc = L.swa_fwd(1, 1, 1, 1, 1 << 23, 128, 64, 0, 128, 64, P, P, P, P, None, P, P, P, None,
                   ctypes.c_float(0.1), None)
    assert b"span" not in L.swa_last_error()


def test_binding_rejects_mismatched_metadata():
    """The kernels index the device metadata without bounds checks; the
    binding refuses metadata built for another shape before any launch
    (CPU tensors: nothing reaches the library)."""
    import torch
    bf = torch.bfloat16
    meta = swa.meta_to_device(swa.swa_blockmask_build(1, 128, 128, 16, 128, 64), "cpu")
    q = torch.zeros(1, 4, 256, 128, dtype=bf)
    k = torch.zeros(1, 2, 256, 128, dtype=bf)
    with pytest.raises(swa.SwaError, match="nq=128"):
        swa.swa_fwd(q, k, k.clone(), q.clone(), 16, meta)  # N = 256 against a build for 128
    q, k = q[:, :, :128].contiguous(), k[:, :, :128].contiguous()
    with pytest.raises(swa.SwaError, match="W=16"):
        swa.swa_fwd(q, k, k.clone(), q.clone(), 32, meta)
    q2, k2 = torch.cat([q, q]), torch.cat([k, k])
    with pytest.raises(swa.SwaError, match="B=1"):
        swa.swa_fwd(q2, k2, k2.clone(), q2.clone(), 16, meta)
    lse = torch.zeros(1, 4, 128)
    ws = torch.zeros(swa.swa_bwd_workspace_size(1, 4, 128) // 4)
    with pytest.raises(swa.SwaError, match="W=16"):
        swa.swa_bwd(q, k, k.clone(), q.clone(), q.clone(), lse, q.clone(), k.clone(), k.clone(),
                    ws, 8, meta)
    # a chunk needs ring metadata of its own W and Tq
    with pytest.raises(swa.SwaError, match="W_ring=0"):
        swa.swa_prefill_chunk(torch.zeros(1, 4, 64, 128, dtype=bf),
                              torch.zeros(1, 2, 64, 128, dtype=bf),
                              torch.zeros(1, 2, 64, 128, dtype=bf),
                              torch.zeros(1, 2, 128, 128, dtype=bf),
                              torch.zeros(1, 2, 128, 128, dtype=bf),
                              torch.zeros(1, dtype=torch.int32), torch.zeros(1, dtype=torch.int32),
                              torch.zeros(1, dtype=torch.int32),
                              torch.zeros(1, 4, 64, 128, dtype=bf), 128,
                              swa.meta_to_device(swa.swa_blockmask_build(1, 64, 64, 128, 128, 64),
                                                 "cpu"))
    # varlen: a build for another batch size
    cu = torch.tensor([0, 50, 100], dtype=torch.int32)
    mv = swa.meta_to_device(swa.swa_blockmask_build(3, 60, 60, 16, 128, 64), "cpu")
    t = torch.zeros(100, 4, 128, dtype=bf)
    kv = torch.zeros(100, 2, 128, dtype=bf)
    with pytest.raises(swa.SwaError, match="B=3"):
        swa.swa_fwd_varlen(t, kv, kv.clone(), t.clone(), 16, mv, cu)
    wsv = torch.zeros(100 * 4)
    with pytest.raises(swa.SwaError, match="B=3"):
        swa.swa_bwd_varlen(t, kv, kv.clone(), t.clone(), t.clone(), torch.zeros(100, 4),
                           t.clone(), kv.clone(), kv.clone(), wsv, 16, mv, cu)
    # packed backward with a build for a padded (nq != nk_lin) shape
    mp = swa.meta_to_device(swa.swa_blockmask_build(2, 60, 64, 16, 128, 64), "cpu")
    with pytest.raises(swa.SwaError, match="nq = nk_lin"):
        swa.swa_bwd_varlen(t, kv, kv.clone(), t.clone(), t.clone(), torch.zeros(100, 4),
                           t.clone(), kv.clone(), kv.clone(), wsv, 16, mp, cu)
    # a hand-made dict without the build's shape is refused too
    bad = {x: meta[x] for x in ("row_ptr", "col", "col_cls", "cls", "tile_q", "tile_k")}
    with pytest.raises(swa.SwaError, match="lacks"):
        swa.swa_fwd(q, k, k.clone(), q.clone(), 16, bad)


def test_chunk_blockmask_dev_validation_codes():
    """The device metadata builder checks its arguments before touching the
    device (no GPU needed for these)."""
    L = swa.lib()
    p = ctypes.c_void_p(16)

    def call(B=2, Tq=64, W=256, S=0, tq=128, tk=64, ptr=p):
        return L.swa_chunk_blockmask_dev(B, Tq, W, S, tq, tk, ptr, ptr, ptr, ptr, ptr, ptr, ptr,
                                         None, None)
    assert call(W=0) == swa.SWA_EINVAL
    assert call(B=0) == swa.SWA_EINVAL
    assert call(Tq=0) == swa.SWA_EINVAL
    assert call(tk=0) == swa.SWA_EINVAL
    assert call(S=-1) == swa.SWA_EINVAL
    assert call(W=96) == swa.SWA_EINVAL  # W not a multiple of tile_k
    assert call(ptr=None) == swa.SWA_EINVAL
    assert call(B=65535, Tq=1 << 20, W=1 << 20, tq=1, tk=1) == swa.SWA_EINVAL  # grid beyond int32
