// swa_api.cpp -- the C ABI of include/swa.h: argument checks, kernel choice and
// launches.  Nothing here allocates, frees or synchronises; every check runs
// before anything is enqueued.
#include <hip/hip_runtime.h>
#include <limits.h>

#include "../../include/swa.h"
#include "swa_internal.h"

namespace {

using swa::fail;

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

int check_ptrs(const char *fn, const void *const *ptrs, const char *const *names, int n) {
    for (int i = 0; i < n; i++) {
        if (!ptrs[i]) return fail(SWA_EINVAL, "%s: %s is NULL", fn, names[i]);
        if (!aligned16(ptrs[i]))
            return fail(SWA_EINVAL, "%s: %s is not 16-byte aligned", fn, names[i]);
    }
    return SWA_OK;
}

int check_heads(const char *fn, int B, int H, int Hkv, int d, int W) {
    if (W < 1) return fail(SWA_EINVAL, "%s: window W=%d must be >= 1", fn, W);
    if (B < 1 || B > 65535) return fail(SWA_EINVAL, "%s: B=%d out of range [1, 65535]", fn, B);
    if (H < 1 || H > 65535 || Hkv < 1 || H % Hkv != 0)
        return fail(SWA_EINVAL, "%s: need 1 <= Hkv, H %% Hkv == 0 (H=%d Hkv=%d)", fn, H, Hkv);
    if (d < 1) return fail(SWA_EINVAL, "%s: d=%d must be >= 1", fn, d);
    return SWA_OK;
}

int check_dtype_d(const char *fn, swa_dtype dt, int d) {
    if (dt == SWA_BF16) {
        if (d != 64 && d != 128)
            return fail(SWA_EUNSUPPORTED, "%s: bf16 path needs d in {64, 128}, got %d", fn, d);
    } else if (dt == SWA_F32) {
        if (d % 4 != 0 || d > 128)
            return fail(SWA_EUNSUPPORTED, "%s: fp32 path needs d %% 4 == 0 and d <= 128, got %d",
                        fn, d);
    } else {
        return fail(SWA_EINVAL, "%s: unknown dtype %d", fn, (int)dt);
    }
    return SWA_OK;
}

// The bf16 tile kernels address one (request, KV head) run of K/V rows with
// 32-bit buffer offsets: `rows` rows `row_bytes` apart must span < 2^31 bytes.
int check_span(const char *fn, swa_dtype dt, long long rows, long long row_bytes) {
    if (dt == SWA_BF16 && rows * row_bytes > (long long)INT_MAX)
        return fail(SWA_EUNSUPPORTED, "%s: bf16 K/V rows of one head span %lld bytes (limit 2^31)",
                    fn, rows * row_bytes);
    return SWA_OK;
}

// bf16 forward tiles: (64 or 128) x (64 or 128), or 256 x 64 at d = 128
int check_tiles(const char *fn, swa_dtype dt, int d, int tile_q, int tile_k) {
    if (tile_q < 1 || tile_k < 1)
        return fail(SWA_EINVAL, "%s: tiles must be >= 1 (%d, %d)", fn, tile_q, tile_k);
    if (dt == SWA_BF16 && tile_q == 256) {
        if (d != 128 || tile_k != 64)
            return fail(SWA_EUNSUPPORTED, "%s: bf16 tile_q = 256 takes d = 128 and tile_k = 64, "
                        "got d=%d tile_k=%d", fn, d, tile_k);
        return SWA_OK;
    }
    if (dt == SWA_BF16 && !((tile_q == 128 || tile_q == 64) && (tile_k == 64 || tile_k == 128)))
        return fail(SWA_EUNSUPPORTED, "%s: bf16 kernels take tile_q in {64, 128, 256} and tile_k "
                    "in {64, 128}, got (%d, %d)", fn, tile_q, tile_k);
    return SWA_OK;
}

// the MFMA backward kernels take 64- or 128-row and 64-key tiles only
int check_tiles_bwd(const char *fn, swa_dtype dt, int d, int tile_q, int tile_k) {
    int rc = check_tiles(fn, dt, d, tile_q, tile_k);
    if (rc == SWA_OK && dt == SWA_BF16 && (tile_k != 64 || tile_q == 256))
        return fail(SWA_EUNSUPPORTED, "%s: bf16 backward takes tile_q in {64, 128} and "
                    "tile_k = 64, got (%d, %d)", fn, tile_q, tile_k);
    return rc;
}

// the bf16 forward kernel for the tile shape (256-row tiles: swa_pp_bf16.hip)
hipError_t launch_fwd_bf16(const swa::AttnArgs &a, hipStream_t s) {
    return a.tile_q == 256 ? swa::launch_pp_bf16(a, s) : swa::launch_tile_bf16(a, s);
}

int launched(const char *fn, hipError_t e) {
    if (e != hipSuccess) return fail(SWA_EHIP, "%s: launch failed: %s", fn, hipGetErrorString(e));
    return SWA_OK;
}

}  // namespace

extern "C" int swa_fwd(swa_dtype dt, int B, int H, int Hkv, int N, int d, int W, int n_sink,
                       int tile_q, int tile_k, const void *q, const void *k, const void *v, void *o,
                       const int32_t *q_len_dev, const int32_t *row_ptr_dev,
                       const int32_t *col_dev, const uint8_t *col_cls_dev, float *lse_dev,
                       float scale, void *stream) {
    static const char *fn = "swa_fwd";
    swa::clear_error();
    int rc;
    if ((rc = check_heads(fn, B, H, Hkv, d, W))) return rc;
    if (n_sink < 0) return fail(SWA_EINVAL, "%s: n_sink=%d < 0", fn, n_sink);
    if (N < 1) return fail(SWA_EINVAL, "%s: N=%d must be >= 1", fn, N);
    if (N > INT_MAX - W) return fail(SWA_EINVAL, "%s: positions overflow int32", fn);
    if ((rc = check_dtype_d(fn, dt, d))) return rc;
    if ((rc = check_tiles(fn, dt, d, tile_q, tile_k))) return rc;
    if ((rc = check_span(fn, dt, N, 2LL * d))) return rc;
    const void *ptrs[] = {q, k, v, o, row_ptr_dev, col_dev};
    const char *names[] = {"q", "k", "v", "o", "row_ptr", "col"};
    if ((rc = check_ptrs(fn, ptrs, names, 6))) return rc;
    if (!col_cls_dev) return fail(SWA_EINVAL, "%s: col_cls is NULL", fn);
    if (!(scale > 0.f) || scale == INFINITY)
        return fail(SWA_EINVAL, "%s: scale must be positive and finite", fn);

    swa::AttnArgs a = {};
    a.mode = 0;
    a.B = B; a.H = H; a.Hkv = Hkv; a.nq = N; a.d = d; a.W = W;
    a.tile_q = tile_q; a.tile_k = tile_k;
    a.q = q; a.k = k; a.v = v; a.o = o;
    a.q_len = q_len_dev;
    a.row_ptr = row_ptr_dev; a.col = col_dev; a.col_cls = col_cls_dev;
    a.lse = lse_dev;
    a.n_sink = n_sink;
    a.scale = scale;
    hipStream_t s = (hipStream_t)stream;
    return launched(fn, dt == SWA_BF16 ? launch_fwd_bf16(a, s) : swa::launch_tile_f32(a, s));
}

extern "C" int swa_fwd_varlen(swa_dtype dt, int B, int H, int Hkv, int total, int max_len,
                              int d, int W, int n_sink, int tile_q, int tile_k, const void *q,
                              const void *k, const void *v, void *o,
                              const int32_t *cu_seqlens_dev, const int32_t *row_ptr_dev,
                              const int32_t *col_dev, const uint8_t *col_cls_dev,
                              float *lse_dev, float scale, void *stream) {
    static const char *fn = "swa_fwd_varlen";
    swa::clear_error();
    int rc;
    if ((rc = check_heads(fn, B, H, Hkv, d, W))) return rc;
    if (n_sink < 0) return fail(SWA_EINVAL, "%s: n_sink=%d < 0", fn, n_sink);
    if (total < 1 || max_len < 1 || max_len > total)
        return fail(SWA_EINVAL, "%s: need 1 <= max_len <= total (total=%d max_len=%d)", fn,
                    total, max_len);
    if (max_len > INT_MAX - W) return fail(SWA_EINVAL, "%s: positions overflow int32", fn);
    if ((rc = check_dtype_d(fn, dt, d))) return rc;
    if ((rc = check_tiles(fn, dt, d, tile_q, tile_k))) return rc;
    if ((rc = check_span(fn, dt, max_len, 2LL * d * Hkv))) return rc;
    const void *ptrs[] = {q, k, v, o, row_ptr_dev, col_dev};
    const char *names[] = {"q", "k", "v", "o", "row_ptr", "col"};
    if ((rc = check_ptrs(fn, ptrs, names, 6))) return rc;
    if (!col_cls_dev || !cu_seqlens_dev)
        return fail(SWA_EINVAL, "%s: col_cls and cu_seqlens are required", fn);
    if (!(scale > 0.f) || scale == INFINITY)
        return fail(SWA_EINVAL, "%s: scale must be positive and finite", fn);

    swa::AttnArgs a = {};
    a.mode = 0;
    a.B = B; a.H = H; a.Hkv = Hkv; a.nq = max_len; a.d = d; a.W = W;
    a.tile_q = tile_q; a.tile_k = tile_k;
    a.q = q; a.k = k; a.v = v; a.o = o;
    a.cu = cu_seqlens_dev;
    a.row_ptr = row_ptr_dev; a.col = col_dev; a.col_cls = col_cls_dev;
    a.lse = lse_dev;
    a.n_sink = n_sink;
    a.scale = scale;
    hipStream_t s = (hipStream_t)stream;
    return launched(fn, dt == SWA_BF16 ? launch_fwd_bf16(a, s) : swa::launch_tile_f32(a, s));
}

extern "C" size_t swa_bwd_workspace_size(int B, int H, int N) {
    if (B < 1 || H < 1 || N < 1) return 0;
    return (size_t)B * H * N * sizeof(float);
}

extern "C" int swa_bwd(swa_dtype dt, int B, int H, int Hkv, int N, int d, int W, int n_sink,
                       int tile_q, int tile_k, const void *q, const void *k, const void *v, const void *o,
                       const void *dout, const float *lse_dev, const int32_t *q_len_dev,
                       const int32_t *row_ptr_dev, const int32_t *col_dev,
                       const uint8_t *cls_dev, void *dq, void *dk, void *dv, void *workspace,
                       size_t ws_bytes, float scale, void *stream) {
    static const char *fn = "swa_bwd";
    swa::clear_error();
    int rc;
    if ((rc = check_heads(fn, B, H, Hkv, d, W))) return rc;
    if (n_sink < 0) return fail(SWA_EINVAL, "%s: n_sink=%d < 0", fn, n_sink);
    if (N < 1) return fail(SWA_EINVAL, "%s: N=%d must be >= 1", fn, N);
    if (N > INT_MAX - W) return fail(SWA_EINVAL, "%s: positions overflow int32", fn);
    if ((rc = check_dtype_d(fn, dt, d))) return rc;
    if (tile_q < 1 || tile_k < 1)
        return fail(SWA_EINVAL, "%s: tiles must be positive (tile_q=%d tile_k=%d)", fn, tile_q,
                    tile_k);
    if ((rc = check_span(fn, dt, N, 2LL * d))) return rc;
    const void *ptrs[] = {q, k, v, o, dout, lse_dev, dq, dk, dv, workspace, row_ptr_dev, col_dev};
    const char *names[] = {"q", "k", "v", "o", "dout", "lse", "dq", "dk", "dv", "workspace",
                           "row_ptr", "col"};
    if ((rc = check_ptrs(fn, ptrs, names, 12))) return rc;
    if (!cls_dev) return fail(SWA_EINVAL, "%s: cls is NULL", fn);
    if (ws_bytes < swa_bwd_workspace_size(B, H, N))
        return fail(SWA_EINVAL, "%s: workspace of %zu bytes is below the %zu required", fn,
                    ws_bytes, swa_bwd_workspace_size(B, H, N));
    if (!(scale > 0.f) || scale == INFINITY)
        return fail(SWA_EINVAL, "%s: scale must be positive and finite", fn);

    swa::BwdArgs a = {};
    a.B = B; a.H = H; a.Hkv = Hkv; a.N = N; a.d = d; a.W = W;
    a.tile_q = tile_q; a.tile_k = tile_k;
    a.q = q; a.k = k; a.v = v; a.o = o; a.dout = dout; a.lse = lse_dev;
    a.q_len = q_len_dev;
    a.row_ptr = row_ptr_dev; a.col = col_dev; a.cls = cls_dev;
    a.dq = dq; a.dk = dk; a.dv = dv;
    a.dvec = (float *)workspace;
    a.n_sink = n_sink;
    a.scale = scale;
    a.bf16 = dt == SWA_BF16;
    return launched(fn, swa::launch_bwd(a, (hipStream_t)stream));
}

extern "C" int swa_bwd_varlen(swa_dtype dt, int B, int H, int Hkv, int total, int max_len,
                              int d, int W, int n_sink, int tile_q, int tile_k, const void *q,
                              const void *k, const void *v, const void *o, const void *dout,
                              const float *lse_dev, const int32_t *cu_seqlens_dev,
                              const int32_t *row_ptr_dev, const int32_t *col_dev,
                              const uint8_t *cls_dev, void *dq, void *dk, void *dv,
                              void *workspace, size_t ws_bytes, float scale, void *stream) {
    static const char *fn = "swa_bwd_varlen";
    swa::clear_error();
    int rc;
    if ((rc = check_heads(fn, B, H, Hkv, d, W))) return rc;
    if (n_sink < 0) return fail(SWA_EINVAL, "%s: n_sink=%d < 0", fn, n_sink);
    if (total < 1 || max_len < 1 || max_len > total)
        return fail(SWA_EINVAL, "%s: need 1 <= max_len <= total (total=%d max_len=%d)", fn,
                    total, max_len);
    if (max_len > INT_MAX - W) return fail(SWA_EINVAL, "%s: positions overflow int32", fn);
    if ((rc = check_dtype_d(fn, dt, d))) return rc;
    if ((rc = check_tiles_bwd(fn, dt, d, tile_q, tile_k))) return rc;
    // query-side rows are H * d elements apart (the wider of the two strides)
    if ((rc = check_span(fn, dt, max_len, 2LL * d * H))) return rc;
    const void *ptrs[] = {q, k, v, o, dout, lse_dev, dq, dk, dv, workspace, row_ptr_dev, col_dev};
    const char *names[] = {"q", "k", "v", "o", "dout", "lse", "dq", "dk", "dv", "workspace",
                           "row_ptr", "col"};
    if ((rc = check_ptrs(fn, ptrs, names, 12))) return rc;
    if (!cls_dev || !cu_seqlens_dev)
        return fail(SWA_EINVAL, "%s: cls and cu_seqlens are required", fn);
    if (ws_bytes < swa_bwd_workspace_size(1, H, total))
        return fail(SWA_EINVAL, "%s: workspace of %zu bytes is below the %zu required", fn,
                    ws_bytes, swa_bwd_workspace_size(1, H, total));
    if (!(scale > 0.f) || scale == INFINITY)
        return fail(SWA_EINVAL, "%s: scale must be positive and finite", fn);

    swa::BwdArgs a = {};
    a.B = B; a.H = H; a.Hkv = Hkv; a.N = max_len; a.d = d; a.W = W;
    a.tile_q = tile_q; a.tile_k = tile_k;
    a.q = q; a.k = k; a.v = v; a.o = o; a.dout = dout; a.lse = lse_dev;
    a.cu = cu_seqlens_dev;
    a.row_ptr = row_ptr_dev; a.col = col_dev; a.cls = cls_dev;
    a.dq = dq; a.dk = dk; a.dv = dv;
    a.dvec = (float *)workspace;
    a.n_sink = n_sink;
    a.scale = scale;
    a.bf16 = dt == SWA_BF16;
    return launched(fn, swa::launch_bwd(a, (hipStream_t)stream));
}

extern "C" int swa_prefill_chunk(swa_dtype dt, int B, int H, int Hkv, int Tq, int d, int W,
                                 int n_sink, void *sink_k, void *sink_v, int tile_q,
                                 int tile_k, const void *q, const void *k_new,
                                 const void *v_new, void *k_cache, void *v_cache,
                                 int32_t *ring_start_dev, int32_t *cache_len_dev,
                                 int32_t *next_pos_dev, const int32_t *row_ptr_dev,
                                 const int32_t *col_dev, const uint8_t *col_cls_dev, void *o,
                                 float scale, void *stream) {
    static const char *fn = "swa_prefill_chunk";
    swa::clear_error();
    int rc;
    if ((rc = check_heads(fn, B, H, Hkv, d, W))) return rc;
    if (Tq < 1 || Tq > W) return fail(SWA_EINVAL, "%s: need 1 <= Tq <= W (Tq=%d W=%d)", fn, Tq, W);
    if (n_sink < 0) return fail(SWA_EINVAL, "%s: n_sink=%d < 0", fn, n_sink);
    if ((rc = check_dtype_d(fn, dt, d))) return rc;
    if ((rc = check_tiles(fn, dt, d, tile_q, tile_k))) return rc;
    if (W % tile_k != 0)
        return fail(SWA_EINVAL, "%s: W=%d must be a multiple of tile_k=%d", fn, W, tile_k);
    if ((rc = check_span(fn, dt, W, 2LL * d))) return rc;
    if ((rc = check_span(fn, dt, n_sink, 2LL * d))) return rc;
    if ((int64_t)n_sink + tile_k + W > INT_MAX)
        return fail(SWA_EINVAL, "%s: n_sink=%d too large", fn, n_sink);
    const void *ptrs[] = {q, k_new, v_new, k_cache, v_cache, o, row_ptr_dev, col_dev};
    const char *names[] = {"q", "k_new", "v_new", "k_cache", "v_cache", "o", "row_ptr", "col"};
    if ((rc = check_ptrs(fn, ptrs, names, 8))) return rc;
    if (n_sink > 0) {
        const void *sp[] = {sink_k, sink_v};
        const char *sn[] = {"sink_k", "sink_v"};
        if ((rc = check_ptrs(fn, sp, sn, 2))) return rc;
    }
    if (!col_cls_dev || !ring_start_dev || !cache_len_dev || !next_pos_dev)
        return fail(SWA_EINVAL, "%s: col_cls and the ring state arrays are required", fn);
    if (!(scale > 0.f) || scale == INFINITY)
        return fail(SWA_EINVAL, "%s: scale must be positive and finite", fn);

    swa::AttnArgs a = {};
    a.mode = 1;
    a.B = B; a.H = H; a.Hkv = Hkv; a.nq = Tq; a.d = d; a.W = W;
    a.tile_q = tile_q; a.tile_k = tile_k;
    a.q = q; a.k = k_new; a.v = v_new; a.o = o;
    a.kc = k_cache; a.vc = v_cache;
    a.ring_start = ring_start_dev; a.cache_len = cache_len_dev; a.next_pos = next_pos_dev;
    a.row_ptr = row_ptr_dev; a.col = col_dev; a.col_cls = col_cls_dev;
    a.n_sink = n_sink;
    a.sk = sink_k; a.sv = sink_v;
    a.scale = scale;
    hipStream_t s = (hipStream_t)stream;
    swa::CommitArgs c = {};
    c.B = B; c.Hkv = Hkv; c.Tq = Tq; c.d = d; c.W = W;
    c.elem_bytes = dt == SWA_BF16 ? 2 : 4;
    c.k_new = k_new; c.v_new = v_new; c.kc = k_cache; c.vc = v_cache;
    c.ring_start = ring_start_dev; c.cache_len = cache_len_dev; c.next_pos = next_pos_dev;
    c.n_sink = n_sink; c.sk = sink_k; c.sv = sink_v;
    // new rows below n_sink go to the sink caches first (the attention reads
    // every position below n_sink there); the ring commit runs after the
    // attention, which reads the old ring
    if (n_sink > 0 && (rc = launched(fn, swa::launch_sink_write(c, s)))) return rc;
    if ((rc = launched(fn, dt == SWA_BF16 ? launch_fwd_bf16(a, s)
                                          : swa::launch_tile_f32(a, s))))
        return rc;
    return launched(fn, swa::launch_commit(c, s));
}

extern "C" size_t swa_decode_workspace_size(int B, int H, int d, int W) {
    if (B < 1 || H < 1 || d < 1 || W < 1) return 0;
    return (size_t)B * H * swa::decode_max_splits(W) * (size_t)(d + 2) * sizeof(float);
}

extern "C" int swa_chunk_blockmask_dev(int B, int Tq, int W, int n_sink, int tile_q, int tile_k,
                                       const int32_t *ring_start_dev,
                                       const int32_t *cache_len_dev,
                                       const int32_t *next_pos_dev, uint8_t *cls_dev,
                                       int32_t *row_ptr_dev, int32_t *col_dev,
                                       uint8_t *col_cls_dev, int64_t *stats_dev, void *stream) {
    static const char *fn = "swa_chunk_blockmask_dev";
    swa::clear_error();
    if (W < 1) return fail(SWA_EINVAL, "%s: window W=%d must be >= 1", fn, W);
    if (B < 1 || Tq < 1 || tile_q < 1 || tile_k < 1)
        return fail(SWA_EINVAL, "%s: need B, Tq, tiles >= 1 (B=%d Tq=%d tile_q=%d tile_k=%d)",
                    fn, B, Tq, tile_q, tile_k);
    if (n_sink < 0) return fail(SWA_EINVAL, "%s: n_sink=%d < 0", fn, n_sink);
    if (W % tile_k != 0)
        return fail(SWA_EINVAL, "%s: W=%d must be a multiple of tile_k=%d", fn, W, tile_k);
    const long long NS = n_sink > 0 ? ((long long)n_sink + tile_k - 1) / tile_k * tile_k : 0;
    const long long nk = NS + W + Tq;
    const long long nqt = (Tq + tile_q - 1) / tile_q, nkt = (nk + tile_k - 1) / tile_k;
    if (nk > INT_MAX || (long long)B * nqt * nkt > INT_MAX)
        return fail(SWA_EINVAL, "%s: key axis or block grid too large", fn);
    if (!ring_start_dev || !cache_len_dev || !next_pos_dev || !cls_dev || !row_ptr_dev ||
        !col_dev || !col_cls_dev)
        return fail(SWA_EINVAL, "%s: ring state and output arrays are required", fn);
    swa::ChunkMetaArgs a = {};
    a.B = B; a.Tq = Tq; a.W = W; a.n_sink = n_sink; a.tile_q = tile_q; a.tile_k = tile_k;
    a.ring_start = ring_start_dev; a.cache_len = cache_len_dev; a.next_pos = next_pos_dev;
    a.cls = cls_dev; a.row_ptr = row_ptr_dev; a.col = col_dev; a.col_cls = col_cls_dev;
    a.stats = stats_dev;
    return launched(fn, swa::launch_chunk_meta(a, (hipStream_t)stream));
}

// Shared by swa_decode (caller's workspace) and swa_decode_noalloc (the
// library's scratch array; workspace == NULL there).
static int decode_call(const char *fn, bool noalloc, swa_dtype dt, int B, int H, int Hkv, int d,
                       int W, int n_sink, void *sink_k, void *sink_v, const void *q,
                       const void *k_new, const void *v_new, void *k_cache, void *v_cache,
                       int32_t *ring_start_dev, int32_t *cache_len_dev, int32_t *next_pos_dev,
                       void *o, void *workspace, size_t ws_bytes, float scale, void *stream) {
    swa::clear_error();
    int rc;
    if ((rc = check_heads(fn, B, H, Hkv, d, W))) return rc;
    if ((rc = check_dtype_d(fn, dt, d))) return rc;
    const int G = H / Hkv;
    if (dt == SWA_BF16 && !(G == 1 || G == 2 || G == 4 || G == 8))
        return fail(SWA_EUNSUPPORTED, "%s: bf16 path needs H/Hkv in {1, 2, 4, 8}, got %d", fn, G);
    const void *ptrs[] = {q, k_new, v_new, k_cache, v_cache, o};
    const char *names[] = {"q", "k_new", "v_new", "k_cache", "v_cache", "o"};
    if ((rc = check_ptrs(fn, ptrs, names, 6))) return rc;
    if (!ring_start_dev || !cache_len_dev || !next_pos_dev)
        return fail(SWA_EINVAL, "%s: the ring state arrays are required", fn);
    if (!(scale > 0.f) || scale == INFINITY)
        return fail(SWA_EINVAL, "%s: scale must be positive and finite", fn);
    if (n_sink < 0) return fail(SWA_EINVAL, "%s: n_sink=%d < 0", fn, n_sink);
    if (n_sink > 0) {
        const void *sp[] = {sink_k, sink_v};
        const char *sn[] = {"sink_k", "sink_v"};
        if ((rc = check_ptrs(fn, sp, sn, 2))) return rc;
    }
    swa::DecodeArgs a = {};
    a.n_sink = n_sink;
    a.sk = sink_k;
    a.sv = sink_v;
    a.B = B; a.H = H; a.Hkv = Hkv; a.d = d; a.W = W;
    a.q = q; a.k_new = k_new; a.v_new = v_new; a.kc = k_cache; a.vc = v_cache;
    a.ring_start = ring_start_dev; a.cache_len = cache_len_dev; a.next_pos = next_pos_dev;
    a.o = o;
    a.scale = scale;
    hipStream_t s = (hipStream_t)stream;
    if (dt == SWA_F32) return launched(fn, swa::launch_decode_f32(a, s));
    a.n_split = swa::decode_bf16_splits(B, Hkv, W);
    if (noalloc) {
        // the ranges' partials go to the library's scratch array: fewer ranges
        // when those of swa_decode would not fit (one range without sinks
        // writes O directly and needs none)
        const size_t per_range = (size_t)B * H * (size_t)(d + 2) * sizeof(float);
        while (a.n_split > 1 && per_range * a.n_split > swa::kDecodeScratchBytes) a.n_split >>= 1;
        if ((a.n_split > 1 || n_sink > 0) && per_range * a.n_split > swa::kDecodeScratchBytes)
            return fail(SWA_EINVAL,
                        "%s: B*H*(d+2)*4 = %zu bytes of partials exceed the %zu-byte scratch "
                        "(with attention sinks one range needs them)", fn, per_range,
                        swa::kDecodeScratchBytes);
        float *scr = nullptr;
        if ((rc = swa::decode_scratch(&scr))) return rc;
        a.ws = scr;
        return launched(fn, swa::launch_decode_bf16(a, s));
    }
    const size_t need = swa_decode_workspace_size(B, H, d, W);
    if (!workspace || !aligned16(workspace) || ws_bytes < need)
        return fail(SWA_EINVAL, "%s: workspace of %zu bytes (16-byte aligned) required, got %zu",
                    fn, need, ws_bytes);
    a.ws = (float *)workspace;
    return launched(fn, swa::launch_decode_bf16(a, s));
}

extern "C" int swa_decode(swa_dtype dt, int B, int H, int Hkv, int d, int W, int n_sink,
                          void *sink_k, void *sink_v, const void *q,
                          const void *k_new, const void *v_new, void *k_cache, void *v_cache,
                          int32_t *ring_start_dev, int32_t *cache_len_dev,
                          int32_t *next_pos_dev, void *o, void *workspace, size_t ws_bytes,
                          float scale, void *stream) {
    return decode_call("swa_decode", false, dt, B, H, Hkv, d, W, n_sink, sink_k, sink_v, q,
                       k_new, v_new, k_cache, v_cache, ring_start_dev, cache_len_dev,
                       next_pos_dev, o, workspace, ws_bytes, scale, stream);
}

extern "C" int swa_decode_noalloc(swa_dtype dt, int B, int H, int Hkv, int d, int W, int n_sink,
                                  void *sink_k, void *sink_v, const void *q, const void *k_new,
                                  const void *v_new, void *k_cache, void *v_cache,
                                  int32_t *ring_start_dev, int32_t *cache_len_dev,
                                  int32_t *next_pos_dev, void *o, float scale, void *stream) {
    return decode_call("swa_decode_noalloc", true, dt, B, H, Hkv, d, W, n_sink, sink_k, sink_v,
                       q, k_new, v_new, k_cache, v_cache, ring_start_dev, cache_len_dev,
                       next_pos_dev, o, nullptr, 0, scale, stream);
}
