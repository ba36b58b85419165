/*
 * swa.h -- C ABI of the MI355X (gfx950) causal sliding-window attention library.
 *
 * The operation (cited by page title and section):
 *   [M003] "Weight sparsity vs attention sparsity" (AI-infra KB), §03-§08
 *   [Ch10] "LLMs from scratch, chapter 10: SWA and DSA", §10.1-§10.2
 *   [Blog] "Dense attention vs sliding-window sparse attention", §3.1-§3.3, §5.2
 *   [Taxonomy] "Sparse attention taxonomy: what to read, what not to read",
 *           §1.1, §3.2
 *
 *   A query at logical position t reads exactly the keys at logical positions
 *   max(0, t-W+1) .. t (W counts the current token) [M003 §03], [Ch10 §10.1];
 *   scores are scale * <q, k>; softmax is normalised over that set only and
 *   weights the V rows of that set.  A query with no visible key (a padded
 *   row) is written as 0.  Grouped KV heads: query head h reads KV head
 *   h / (H / Hkv) (contiguous groups).
 *
 * Conventions shared by every entry point
 *   - Tensors are dense row-major, d fastest: Q and O [B][H][rows][d],
 *     K and V [B][Hkv][rows][d], ring caches [B][Hkv][W][d].
 *   - Device pointers are caller-owned device memory (16-byte aligned) and
 *     host pointers caller-owned host memory.  The library never allocates,
 *     frees or synchronises: device work is enqueued on `stream` (NULL = the
 *     default stream) and its faults surface at the caller's next sync.
 *   - Every call returns a swa_status.  On anything but SWA_OK nothing was
 *     enqueued (except SWA_EHIP after a failed launch) and swa_last_error()
 *     describes the problem.  No exception crosses the ABI.
 *   - Padded rows, keys past a valid length and unfilled ring slots must hold
 *     finite values (zeros are fine): they are masked, and 0 * NaN is NaN.
 *   - bf16 inputs are accumulated in fp32 (softmax in fp32, probabilities
 *     rounded to bf16 before the PV product, output rounded to bf16).
 */
#ifndef SWA_H
#define SWA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    SWA_OK = 0,
    SWA_EINVAL = 1,       /* an argument is out of range, inconsistent or NULL */
    SWA_EUNSUPPORTED = 2, /* valid, but no kernel for this dtype / d / tile */
    SWA_EHIP = 3          /* the HIP runtime refused a launch */
} swa_status;

typedef enum { SWA_BF16 = 0, SWA_F32 = 1 } swa_dtype;

/* Classes of a (query tile, key tile) block [M003 §04]: no visible pair,
 * every in-range pair visible, or some visible. */
typedef enum { SWA_BLOCK_SKIP = 0, SWA_BLOCK_FULL = 1, SWA_BLOCK_PARTIAL = 2 } swa_block_class;

/* Work statistics of one metadata build, each summed over the batch. */
typedef struct {
    int64_t valid_pairs;    /* visible (query, key) pairs between valid rows/keys [M003 §03] */
    int64_t covered_coords; /* in-range coordinates of all live blocks [M003 §04] */
    int64_t keys_touched;   /* distinct keys visible to at least one valid query
                               (W+Tq-1 for a chunk after a full ring [Ch10 §10.2]) */
    int64_t n_live;         /* full + partial blocks (= CSR entries) */
    int64_t n_full;
    int64_t n_partial;
} swa_mask_stats;

/* Sizes of the metadata buffers for a build with these shapes.
 * nk is the whole key axis (ring slots + linear keys).  Host only.
 * cls_elems = B * ceil(nq/tile_q) * ceil(nk/tile_k) (bytes of `cls`);
 * max_nnz   = an upper bound on CSR entries (elements of `col`, `col_cls`);
 * the row_ptr array has B * ceil(nq/tile_q) + 1 elements.
 * Errors: SWA_EINVAL for B < 1, nq < 0, nk < 0, tile < 1, NULL outputs. */
int swa_blockmask_size(int B, int nq, int nk, int tile_q, int tile_k,
                       size_t *cls_elems, size_t *max_nnz);

/* Block metadata (host, integer, exact) [M003 §04]: classifies every
 * (query tile, key tile) by counting its visible pairs: 0 -> skip, equal to
 * the tile's in-range area -> full, else partial, and lists the live key
 * tiles of each query tile in ascending order (CSR over rows b*nqt + qt).
 *
 * Query i of sequence b sits at logical position q_start[b] + i and is
 * valid iff i < q_len[b].  The key axis is [W_ring ring slots | nk_lin
 * linear keys]: linear key t sits at k_start[b] + t, valid iff t < k_len[b];
 * ring slot s (when W_ring > 0) holds the logical position
 *   next_pos[b] - cache_len[b] + ((s - ring_start[b]) mod W_ring)
 * and is valid iff (s - ring_start[b]) mod W_ring < cache_len[b]: slots keep
 * their logical positions after being overwritten [M003 §06], [Ch10 §10.2].
 * NULL q_start/k_start mean 0, NULL q_len/k_len mean "all valid"; the ring
 * arrays are ignored when W_ring == 0 and required otherwise.
 *
 * n_sink >= 0 attention sinks [Taxonomy §3.2, the StreamingLLM rule]: keys
 * at logical positions below n_sink stay visible to every query at or after
 * them, besides the window (a key in both counts once); 0 is the plain
 * window.  With W_ring > 0 the key axis gains a sink segment in front:
 * [NS sink slots | W_ring ring slots | nk_lin linear keys], NS = n_sink
 * rounded up to a multiple of tile_k; sink slot s stands for position s
 * (valid iff s < n_sink) and is visible to every query at or after s, and
 * ring or linear keys below n_sink are then not counted (the chunk reads
 * those positions from its sink cache), so each position counts once.
 *
 * For swa_fwd: q_start = k_start = NULL, nq = nk_lin = N, q_len = k_len =
 *   the per-sequence valid lengths (or NULL), W_ring = 0, the call's n_sink.
 * For swa_prefill_chunk: nq = nk_lin = Tq, q_start = k_start = next_pos,
 *   k_len = NULL, W_ring = W, the ring state the call will see and the
 *   call's n_sink; swa_blockmask_size then takes nk = NS + W + Tq.
 *
 * Outputs (caller-owned host memory, sizes from swa_blockmask_size):
 * cls [B][nqt][nkt] uint8, row_ptr [B*nqt+1] int32, col [nnz] int32 (key
 * tile index), col_cls [nnz] uint8 (1 full, 2 partial); stats may be NULL.
 * Errors: SWA_EINVAL for W < 1 [Blog §5.1: the window has to be at least
 * one token], bad sizes, W_ring % tile_k != 0, ring state out of range
 * (ring_start not in [0, W_ring), cache_len not in [0, W_ring],
 * next_pos < cache_len), a negative length, or positions that overflow int32. */
int swa_blockmask_build(int B, int nq, int nk_lin, int W, int n_sink, int tile_q, int tile_k,
                        const int32_t *q_start, const int32_t *k_start,
                        const int32_t *q_len, const int32_t *k_len,
                        int W_ring, const int32_t *ring_start, const int32_t *cache_len,
                        const int32_t *next_pos,
                        uint8_t *cls, int32_t *row_ptr, int32_t *col, uint8_t *col_cls,
                        swa_mask_stats *stats);

/* Full-sequence SWA forward (prefill) [M003 §03-§04].
 * q, o [B][H][N][d]; k, v [B][Hkv][N][d]; query row i and key row j sit at
 * logical positions i and j.  q_len_dev: device int32 [B] valid lengths or
 * NULL (= N); rows at or past the length are written as 0.
 * n_sink: attention sinks as in swa_blockmask_build (0: plain window).
 * row_ptr_dev / col_dev / col_cls_dev: device copies of a swa_blockmask_build
 * with the same B, N, W, n_sink, tile_q, tile_k and lengths; only listed key tiles
 * are read, and only partial ones are masked per element.  The kernel does
 * not re-check the metadata: metadata of other shapes is a caller error.
 * Supported: SWA_BF16 with d in {64, 128}, tile_q in {64, 128}, tile_k in
 * {64, 128} (a 128-key tile is streamed as two 64-key halves; coarser tiles
 * halve the metadata but can cover more masked pairs, "Weight sparsity vs
 * attention sparsity" (AI-infra KB) §04), or tile_q = 256 with d = 128 and
 * tile_k = 64 (one eight-wave workgroup per query tile whose two wave groups
 * alternate matrix and vector work; the same outputs as (128, 64) bit for
 * bit), and N * d * 2 < 2^31 (one head's K rows are addressed with 32-bit
 * offsets); SWA_F32 with d a multiple of 4 in [4, 128] and any tiles.
 * Other bf16 tiles: SWA_EUNSUPPORTED.
 * W >= N is legal (dense causal).
 * lse_dev: NULL, or device fp32 [B][H][N] that receives each row's natural-log
 * log-sum-exp of its visible scaled scores (-inf for rows that see no key),
 * which swa_bwd needs.
 * Errors: SWA_EINVAL (W < 1, H % Hkv != 0, N < 1, NULL or misaligned
 * pointers), SWA_EUNSUPPORTED, SWA_EHIP. */
int swa_fwd(swa_dtype dt, int B, int H, int Hkv, int N, int d, int W, int n_sink,
            int tile_q, int tile_k,
            const void *q, const void *k, const void *v, void *o,
            const int32_t *q_len_dev,
            const int32_t *row_ptr_dev, const int32_t *col_dev, const uint8_t *col_cls_dev,
            float *lse_dev, float scale, void *stream);

/* Full-sequence forward of a packed variable-length batch [Blog §3.3 passes
 * cu_seqlens to the varlen kernel; §5.2: the window is per sequence, and a
 * wrong split lets windows leak across sequences].  Sequence b owns tokens
 * cu_seqlens[b] .. cu_seqlens[b+1]-1 of the packed axis (token i of it at
 * logical position i); layout is token-major: q, o [total][H][d], k, v
 * [total][Hkv][d]; lse_dev (may be NULL) [total][H].  cu_seqlens_dev: device
 * int32 [B+1] with cu[0] = 0, non-decreasing, cu[B] = total and every length
 * at most max_len.  Metadata: swa_blockmask_build with nq = nk_lin = max_len,
 * q_len = k_len = the lengths (host copy), the call's W, n_sink and tiles.
 * No padding is read or written.  The kernel does not re-check cu_seqlens
 * against the metadata: inconsistent ones are a caller error.
 * Supported and errors: as swa_fwd (max_len * Hkv * d * 2 < 2^31 in place of
 * N * d * 2 for bf16), plus SWA_EINVAL for total < 1, max_len outside
 * [1, total] or NULL cu_seqlens_dev. */
int swa_fwd_varlen(swa_dtype dt, int B, int H, int Hkv, int total, int max_len, int d, int W,
                   int n_sink, int tile_q, int tile_k,
                   const void *q, const void *k, const void *v, void *o,
                   const int32_t *cu_seqlens_dev,
                   const int32_t *row_ptr_dev, const int32_t *col_dev, const uint8_t *col_cls_dev,
                   float *lse_dev, float scale, void *stream);

/* Bytes of device workspace swa_bwd needs (fp32 row values [B][H][N]);
 * 0 for non-positive sizes. */
size_t swa_bwd_workspace_size(int B, int H, int N);

/* Gradients of swa_fwd [M003 §07 asks for the Q/K/V gradients of the masked
 * attention, checked by finite differences].  For output gradient dout, with
 * P the softmax of s = scale q.k over each row's visible keys and o = P v:
 *   D_i = <dout_i, o_i>, dS_ij = P_ij (<dout_i, v_j> - D_i),
 *   dq_i = scale sum_j dS_ij k_j, dk_j = scale sum_i dS_ij q_i,
 *   dv_j = sum_i P_ij dout_i  (visible pairs only; grouped heads summed).
 * q, o, dout, dq [B][H][N][d]; k, v, dk, dv [B][Hkv][N][d], all of dtype dt
 * (fp32 arithmetic inside); lse_dev: the fp32 [B][H][N] that swa_fwd wrote
 * for this q, k, v and n_sink; q_len_dev as for swa_fwd.  row_ptr_dev / col_dev: the
 * block metadata of swa_fwd (query rows visit their tile's key tiles);
 * cls_dev: its class grid [B][nqt][nkt] (keys visit the query tiles whose
 * entry for their key tile is live).  Padded rows and keys get 0.  The
 * caller owns every buffer, including workspace (ws_bytes >=
 * swa_bwd_workspace_size(B, H, N)); the outputs are overwritten, not summed.
 * Supported: as swa_fwd for d; any positive tiles matching the metadata.
 * Errors: SWA_EINVAL (as swa_fwd, small workspace), SWA_EUNSUPPORTED,
 * SWA_EHIP. */
int swa_bwd(swa_dtype dt, int B, int H, int Hkv, int N, int d, int W, int n_sink,
            int tile_q, int tile_k,
            const void *q, const void *k, const void *v, const void *o, const void *dout,
            const float *lse_dev, const int32_t *q_len_dev,
            const int32_t *row_ptr_dev, const int32_t *col_dev, const uint8_t *cls_dev,
            void *dq, void *dk, void *dv, void *workspace, size_t ws_bytes,
            float scale, void *stream);

/* Gradients of swa_fwd_varlen: the quantities of swa_bwd for a packed
 * variable-length batch [M003 §07 for the gradients; Blog §3.3 and §5.2 for
 * the packed layout with per-sequence windows].  Sequence b owns tokens
 * cu_seqlens[b] .. cu_seqlens[b+1]-1 (token i of it at logical position i,
 * positions below n_sink are its attention sinks).  Layout is token-major:
 * q, o, dout, dq [total][H][d]; k, v, dk, dv [total][Hkv][d]; lse_dev the
 * fp32 [total][H] that swa_fwd_varlen wrote for this q, k, v and n_sink.
 * Metadata: that of swa_fwd_varlen (nq = nk_lin = max_len, q_len = k_len =
 * the lengths), with cls_dev its class grid [B][nqt][nkt].  workspace: fp32
 * row values [total][H], ws_bytes >= swa_bwd_workspace_size(1, H, total).
 * Every output row is written; no padding is read or written.  The kernels
 * do not re-check cu_seqlens against the metadata: inconsistent ones are a
 * caller error.
 * Supported: as swa_fwd_varlen for dt and d (bf16: d in {64, 128}, tile_q in
 * {64, 128} and tile_k = 64, on the MFMA kernels, with
 * max_len * H * d * 2 < 2^31; fp32: d % 4 == 0, d <= 128, any positive tiles,
 * on the fp32-arithmetic kernels); anything else is SWA_EUNSUPPORTED.
 * Errors: SWA_EINVAL (as swa_fwd_varlen, NULL cls_dev, small workspace),
 * SWA_EUNSUPPORTED, SWA_EHIP. */
int swa_bwd_varlen(swa_dtype dt, int B, int H, int Hkv, int total, int max_len, int d, int W,
                   int n_sink, int tile_q, int tile_k,
                   const void *q, const void *k, const void *v, const void *o, const void *dout,
                   const float *lse_dev, const int32_t *cu_seqlens_dev,
                   const int32_t *row_ptr_dev, const int32_t *col_dev, const uint8_t *cls_dev,
                   void *dq, void *dk, void *dv, void *workspace, size_t ws_bytes,
                   float scale, void *stream);

/* Chunked prefill of Tq new tokens against a ring-buffer cache [Ch10 §10.2],
 * [Blog §3.2], [M003 §06].
 * q, o [B][H][Tq][d]; k_new, v_new [B][Hkv][Tq][d]; k_cache, v_cache
 * [B][Hkv][W][d] (in/out); ring state ring_start_dev, cache_len_dev,
 * next_pos_dev: device int32 [B] (in/out), meaning as in swa_blockmask_build.
 * New token t sits at logical position next_pos + t.  Every query attends
 * over the union of the old ring and the chunk (up to W+Tq-1 keys), read
 * before anything is overwritten; then the last min(Tq, W) new rows are
 * written into the ring (the slot of logical position P is the one whose
 * formula above yields P) and the state becomes next_pos += Tq,
 * cache_len = min(W, cache_len + Tq), ring_start = slot of the oldest kept
 * position.  Metadata: swa_blockmask_build with W_ring = W, nq = nk_lin = Tq,
 * q_start = k_start = next_pos, the same n_sink and the same tiles.
 * n_sink > 0 [Taxonomy §3.2]: sink_k, sink_v [B][Hkv][n_sink][d] (in/out,
 * dtype dt) hold the rows of logical positions 0 .. n_sink-1 (as swa_decode
 * keeps them); new tokens at positions below n_sink are copied there first,
 * and every query also sees each position below n_sink (at or before its
 * own) once, from the sink cache.  n_sink == 0: the sink pointers are ignored.
 * The ring state lives on the device, so the host cannot check it: the
 * kernels do, per request.  A request whose state is unusable (ring_start
 * outside [0, W), cache_len outside [0, W], next_pos < 0, or next_pos + Tq
 * beyond INT32_MAX) writes nothing to its ring, sink cache or
 * state, and its output is zero; the other requests are unaffected.
 * Supported: as swa_fwd (W * d * 2 < 2^31 for bf16), plus W % tile_k == 0
 * and 1 <= Tq <= W.
 * Errors: as swa_fwd, plus SWA_EINVAL for n_sink < 0 or NULL / misaligned
 * sink pointers with n_sink > 0. */
int swa_prefill_chunk(swa_dtype dt, int B, int H, int Hkv, int Tq, int d, int W,
                      int n_sink, void *sink_k, void *sink_v, int tile_q, int tile_k,
                      const void *q, const void *k_new, const void *v_new,
                      void *k_cache, void *v_cache,
                      int32_t *ring_start_dev, int32_t *cache_len_dev, int32_t *next_pos_dev,
                      const int32_t *row_ptr_dev, const int32_t *col_dev,
                      const uint8_t *col_cls_dev,
                      void *o, float scale, void *stream);

/* Block metadata of one swa_prefill_chunk step, built on the device from the
 * ring state in device memory [M003 §07: a pattern that moves with the input
 * is rebuilt each step, and that cost counts], so that consecutive chunk
 * steps chain on one stream with no host copy of the ring state.  Enqueued on
 * `stream`; it reads ring_start_dev, cache_len_dev, next_pos_dev as they are
 * when it runs (after earlier work on the stream), so enqueue it before each
 * swa_prefill_chunk of the same (B, Tq, W, n_sink, tile_q, tile_k).
 * Outputs (device memory, caller-owned, sizes as swa_blockmask_size with
 * nq = Tq and nk = NS + W + Tq, NS = n_sink rounded up to tile_k): cls_dev
 * [B][nqt][nkt], row_ptr_dev [B*nqt+1], col_dev and col_cls_dev [max_nnz];
 * stats_dev: NULL or device int64[6] in swa_mask_stats order.  The arrays
 * equal those swa_blockmask_build writes for that step (nq = nk_lin = Tq,
 * q_start = k_start = next_pos, k_len = NULL, W_ring = W, the same n_sink).
 * The ring state must be one swa_blockmask_build accepts (ring_start in
 * [0, W), cache_len in [0, W], next_pos >= cache_len, positions within int32);
 * it is not re-checked on the device.
 * Errors: SWA_EINVAL for W < 1, B, Tq or a tile < 1, n_sink < 0,
 * W % tile_k != 0, a grid beyond int32, NULL arrays; SWA_EHIP. */
int swa_chunk_blockmask_dev(int B, int Tq, int W, int n_sink, int tile_q, int tile_k,
                            const int32_t *ring_start_dev, const int32_t *cache_len_dev,
                            const int32_t *next_pos_dev, uint8_t *cls_dev, int32_t *row_ptr_dev,
                            int32_t *col_dev, uint8_t *col_cls_dev, int64_t *stats_dev,
                            void *stream);

/* Bytes of device workspace swa_decode needs for these shapes. */
size_t swa_decode_workspace_size(int B, int H, int d, int W);

/* One decode step per request against its ring cache [Blog §3.2],
 * [Taxonomy §1.1: decode streams the whole KV it reads].
 * q, o [B][H][d] (one token each); k_new, v_new [B][Hkv][d]; caches and ring
 * state as swa_prefill_chunk.  The new row is appended first (the next free
 * slot (ring_start + cache_len) mod W while filling, else the oldest slot
 * ring_start, which then advances), then the query at logical position
 * next_pos (the old value) attends over the ring's valid slots; next_pos
 * grows by one.  workspace: device memory of swa_decode_workspace_size bytes
 * (ws_bytes), no initialisation needed.
 * n_sink > 0 [Taxonomy §3.2]: sink_k, sink_v [B][Hkv][n_sink][d] (in/out,
 * dtype dt) hold the rows of logical positions 0 .. n_sink-1; a token
 * appended at position p < n_sink is also copied to sink slot p, and the
 * query also attends over the sink positions the ring no longer holds
 * (below next_pos + 1 - cache_len after the append).  n_sink == 0: the sink
 * pointers are ignored.
 * Device ring state as swa_prefill_chunk with Tq = 1: a request whose state is
 * unusable (including next_pos == INT32_MAX) appends nothing, keeps its state
 * and gets a zero output.
 * Supported: SWA_BF16 with d in {64, 128}, H / Hkv in {1, 2, 4, 8}; SWA_F32 with d a
 * multiple of 4 in [4, 128].
 * Errors: as swa_fwd, plus SWA_EINVAL when ws_bytes is too small. */
int swa_decode(swa_dtype dt, int B, int H, int Hkv, int d, int W, int n_sink,
               void *sink_k, void *sink_v,
               const void *q, const void *k_new, const void *v_new,
               void *k_cache, void *v_cache,
               int32_t *ring_start_dev, int32_t *cache_len_dev, int32_t *next_pos_dev,
               void *o, void *workspace, size_t ws_bytes, float scale, void *stream);

/* Allocation-free variant of swa_decode, for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc.  Arguments and results are those of swa_decode
 * without the workspace: the bf16 path keeps its per-range partials in a
 * scratch array inside the library, 32 MiB on each GPU it runs on (held until
 * the process ends), at the current device's address of it, so the stream
 * must belong to the current device.  It uses swa_decode's number of W ranges
 * when their partials (B * H * ranges * (d + 2) * 4 bytes) fit, else halves
 * it until they do; one range without attention sinks writes O directly and
 * needs none.  Nothing in the scratch needs clearing (each range writes its
 * partial before the merge reads it).  Calls that overlap on one GPU (other
 * streams, other threads) share that scratch and race; calls ordered on one
 * stream do not.  The fp32 path needs no scratch.
 * Errors: as swa_decode, plus SWA_EINVAL when one range's partials do not fit
 * (only with n_sink > 0 and B * H * (d + 2) * 4 > 32 MiB), SWA_EHIP when the
 * scratch's address cannot be looked up. */
int swa_decode_noalloc(swa_dtype dt, int B, int H, int Hkv, int d, int W, int n_sink,
                       void *sink_k, void *sink_v,
                       const void *q, const void *k_new, const void *v_new,
                       void *k_cache, void *v_cache,
                       int32_t *ring_start_dev, int32_t *cache_len_dev, int32_t *next_pos_dev,
                       void *o, float scale, void *stream);

/* Which layers of a stack use the window ("LLMs from scratch, chapter 10:
 * SWA and DSA", §10.2: a local:global ratio has to be resolved into whole
 * layers; a stride option picks the windowed layers).  Host only.
 * The stack repeats a period of n_local windowed layers followed by n_global
 * global (full-history) layers, from layer 0 upward; L layers take the first
 * L of that pattern (e.g. 26 layers at 5:1 give 22 windowed and 4 global).
 * Writes W_layer[l] = W for a windowed layer and -1 for a global one (the
 * (-1, -1) window of "Dense attention vs sliding-window sparse attention",
 * §3.3, meaning dense), and the counts *L_s (windowed), *L_f (global).
 * A windowed layer runs swa_fwd / swa_decode with W; a global layer is the
 * same call with W >= the sequence length (dense causal).
 * Errors: SWA_EINVAL for L < 0, a negative ratio part or 0:0, W < 1, NULL
 * outputs (W_layer may be NULL only when L == 0). */
int swa_layer_plan(int L, int n_local, int n_global, int W, int32_t *W_layer,
                   int32_t *L_s, int32_t *L_f);

/* Bytes of the persistent K and V caches of a layer stack after T tokens
 * ("LLMs from scratch, chapter 10", §10.2): a layer with window W_layer[l]
 * keeps min(T, W_layer[l]) rows per KV head, a global layer (-1) keeps T, so
 *   *bytes = 2 * B * G * d * elem_bytes * sum_l kept_l
 * which is the chapter's 2BGds[L_s min(T,W) + L_f T] when every windowed
 * layer has the same W, and 2BWGds per windowed layer once T >= W (the ring
 * cache swa_decode reads).  B requests, G KV heads of width d, elem_bytes
 * bytes per element (2 for bf16).  Host only.
 * Errors: SWA_EINVAL for B, G, d or elem_bytes < 1, T < 0, L < 0, a window
 * that is neither >= 1 nor -1, a result beyond int64, NULL pointers
 * (W_layer may be NULL only when L == 0). */
int swa_cache_bytes(int B, int G, int d, int elem_bytes, int64_t T, int L,
                    const int32_t *W_layer, int64_t *bytes);

/* Message for the last non-OK status returned on this thread ("" if none). */
const char *swa_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* SWA_H */
