// swa_internal.h -- declarations shared by the library's translation units.
// Not part of the ABI (include/swa.h is).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace swa {

// Records a message for swa_last_error() and returns `code`.
int fail(int code, const char *fmt, ...) __attribute__((format(printf, 2, 3)));
void clear_error();

// Everything a tile-loop kernel (full-sequence forward or chunked prefill)
// needs.  mode 0: forward, keys are rows 0..nq-1 of k/v at positions 0..nq-1,
// q_len valid lengths.  mode 1: chunk, key axis = [W ring slots of kc/vc |
// nq new rows of k/v], ring state read from the device arrays.
struct AttnArgs {
    int mode;
    int B, H, Hkv, nq, d, W, tile_q, tile_k;
    const void *q, *k, *v;
    void *o;
    const void *kc, *vc;
    const int32_t *q_len;
    const int32_t *ring_start, *cache_len, *next_pos;
    const int32_t *row_ptr, *col;
    const uint8_t *col_cls;
    float *lse;  // mode 0, may be null: [B][H][nq] natural-log row log-sum-exp
    int n_sink;  // mode 0: keys at positions < n_sink stay visible (attention sinks)
    const int32_t *cu;  // mode 0, may be null: packed batch, sequence b = tokens
                        // cu[b] .. cu[b+1]-1 of token-major q, o [tokens][H][d],
                        // k, v [tokens][Hkv][d]; nq is then the longest sequence
    // mode 1 with n_sink > 0: sink caches [B][Hkv][n_sink][d]; the key axis is
    // then [n_sink rounded up to tile_k sink slots | W ring slots | nq new rows]
    const void *sk, *sv;
    float scale;
};

struct DecodeArgs {
    int B, H, Hkv, d, W;
    const void *q, *k_new, *v_new;
    void *kc, *vc;
    int32_t *ring_start, *cache_len, *next_pos;
    void *o;
    float *ws;
    int n_split;
    int n_sink;     // attention sinks: sink caches [B][Hkv][n_sink][d] (sk, sv)
    void *sk, *sv;
    float scale;
};

struct CommitArgs {
    int B, Hkv, Tq, d, W, elem_bytes;
    const void *k_new, *v_new;
    void *kc, *vc;
    int32_t *ring_start, *cache_len, *next_pos;
    int n_sink;     // sink caches [B][Hkv][n_sink][d] (sk, sv), for launch_sink_write
    void *sk, *sv;
};

// bf16 MFMA tile loop (swa_tile_bf16.hip): d in {64,128}, tile_q in {64,128},
// tile_k in {64,128} (a 128-key tile is staged as two 64-key halves).
hipError_t launch_tile_bf16(const AttnArgs &a, hipStream_t s);
// 256-row query tiles, head dim 128, 64-key tiles (swa_pp_bf16.hip)
hipError_t launch_pp_bf16(const AttnArgs &a, hipStream_t s);
// fp32 reference-grade kernels (swa_f32.hip): any tiles, d % 4 == 0, d <= 128.
hipError_t launch_tile_f32(const AttnArgs &a, hipStream_t s);
hipError_t launch_decode_f32(const DecodeArgs &a, hipStream_t s);
// bf16 split decode + combine (swa_decode_bf16.hip).
hipError_t launch_decode_bf16(const DecodeArgs &a, hipStream_t s);
int decode_bf16_splits(int B, int Hkv, int W);
int decode_max_splits(int W);
// Scratch array of swa_decode_noalloc (a file-scope __device__ array in
// swa_decode_bf16.hip, one per GPU, held until the process ends) and the
// current device's address of it, looked up once per device.
constexpr size_t kDecodeScratchBytes = (size_t)32 << 20;
int decode_scratch(float **ptr);
// Backward of the full-sequence forward (swa_bwd.hip).
struct BwdArgs {
    int B, H, Hkv, N, d, W, tile_q, tile_k;
    const void *q, *k, *v, *o, *dout;
    const float *lse;
    const int32_t *q_len;
    const int32_t *row_ptr, *col;
    const uint8_t *cls;  // [B][nqt][nkt] class grid
    void *dq, *dk, *dv;
    float *dvec;  // workspace: [B][H][N] fp32 row values D = <dout, o>
    int n_sink;
    float scale;
    int bf16;
    // may be null: packed batch, sequence b = tokens cu[b] .. cu[b+1]-1 of
    // token-major q, o, dout, dq [tokens][H][d], k, v, dk, dv [tokens][Hkv][d],
    // lse and dvec [tokens][H]; N is then the longest sequence
    const int32_t *cu;
};
hipError_t launch_bwd(const BwdArgs &a, hipStream_t s);
// bf16 MFMA kernels (swa_bwd_bf16.hip): d in {64, 128}, tile_k 64, tile_q in {64, 128}.
bool bwd_bf16_supported(const BwdArgs &a);
hipError_t launch_bwd_bf16(const BwdArgs &a, hipStream_t s);

// Block metadata of a chunked-prefill step built on the device from the
// device ring state (swa_chunk_meta.hip); same arrays and statistics as
// swa_blockmask_build for that step.
struct ChunkMetaArgs {
    int B, Tq, W, n_sink, tile_q, tile_k;
    const int32_t *ring_start, *cache_len, *next_pos;
    uint8_t *cls;
    int32_t *row_ptr, *col;
    uint8_t *col_cls;
    int64_t *stats;  // may be null: the six swa_mask_stats fields
};
hipError_t launch_chunk_meta(const ChunkMetaArgs &a, hipStream_t s);

// Ring bookkeeping (swa_ring.hip): write the new rows into their slots, then
// advance the state; launch_commit does both (after a chunk's attention).
hipError_t launch_ring_write(const CommitArgs &a, hipStream_t s);
hipError_t launch_ring_state(const CommitArgs &a, hipStream_t s);
hipError_t launch_commit(const CommitArgs &a, hipStream_t s);
// Copy the new rows at logical positions below n_sink into the sink caches
// (before the chunk's attention reads them there).
hipError_t launch_sink_write(const CommitArgs &a, hipStream_t s);

}  // namespace swa
