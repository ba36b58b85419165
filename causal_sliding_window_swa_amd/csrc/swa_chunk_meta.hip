// swa_chunk_meta.hip -- the block metadata of a chunked-prefill step, built on
// the device from the ring state the previous step left there.
//
// "Weight sparsity vs attention sparsity" (AI-infra KB) §04 classifies each
// (query tile, key tile) as skip / full / partial by its visible pairs; §07
// notes that a pattern which changes with the input (here the ring moves every
// step) must be rebuilt each time, and that this cost counts.  Building it in
// the stream lets consecutive swa_prefill_chunk calls chain with no host copy
// of the ring state.
//
// The key axis is that of swa_blockmask_build for a chunk ("LLMs from
// scratch" ch.10 §10.2; "Dense vs sliding-window sparse attention" §3.2):
// [NS sink slots | W ring slots | Tq new rows], NS = n_sink rounded up to the
// key tile.  Query row i sits at position next_pos + i.  A key is counted by
// the range of query positions that see it: a sink slot s (< n_sink) by every
// query at s or later; a ring slot (valid iff its offset r = (s - ring_start)
// mod W is below cache_len, position next_pos - cache_len + r) and a new row
// j (position next_pos + j) by the queries at p .. p+W-1, and, with sinks,
// only when p >= n_sink (positions below n_sink are read from the sink
// segment).  A pair count per key and tile is the length of that range within
// the tile's query positions; this is a different formulation from the host
// builder's runs of positions, and both are checked against the oracle's
// brute force.
//
// Two kernels: the first classifies every (batch, query tile, key tile), one
// workgroup per query tile, four lanes per key tile; the second, one workgroup,
// walks the class grid in row-major order, 1024 entries per round, and a
// block-wide prefix count of the live ones places them in the CSR arrays in ascending
// key tile, the first entry of each row writing its row pointer.  With
// statistics requested, a third, tiny kernel clears them first and the
// classifier adds its sums with atomics.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "swa_internal.h"

namespace swa {
namespace {

constexpr int NT = 1024;  // threads of the one workgroup

struct ChunkKey {
    int64_t lo, hi;  // query positions that see the key (empty when hi < lo)
};

// Ring state of one batch entry, loaded once per workgroup.
struct Ring {
    int64_t np, rs, cl;
};

// The query positions that see key slot j of a batch entry's key axis.
__device__ __forceinline__ ChunkKey key_range(const ChunkMetaArgs &a, int64_t NS, Ring g,
                                              int64_t j) {
    const int64_t W = a.W, S = a.n_sink;
    ChunkKey k{1, 0};
    if (j < NS) {  // sink slot: position j
        if (j < S) {
            k.lo = j;
            k.hi = INT64_MAX;
        }
        return k;
    }
    int64_t p;
    const int64_t jr = j - NS;
    if (jr < W) {  // ring slot
        int64_t r = jr - g.rs;
        if (r < 0) r += W;
        if (r >= g.cl) return k;
        p = g.np - g.cl + r;
    } else {  // new row
        p = g.np + (jr - W);
    }
    if (S > 0 && p < S) return k;
    k.lo = p;
    k.hi = p + W - 1;
    return k;
}

__device__ __forceinline__ int64_t overlap(ChunkKey k, int64_t t0, int64_t t1) {
    const int64_t lo = k.lo > t0 ? k.lo : t0, hi = k.hi < t1 ? k.hi : t1;
    return hi >= lo ? hi - lo + 1 : 0;
}

struct Grid {
    int64_t NS, nk;
    int nqt, nkt;
};

__device__ __forceinline__ Grid grid_of(const ChunkMetaArgs &a) {
    Grid g;
    g.NS = a.n_sink > 0 ? ((int64_t)a.n_sink + a.tile_k - 1) / a.tile_k * a.tile_k : 0;
    g.nk = g.NS + a.W + a.Tq;
    g.nqt = (a.Tq + a.tile_q - 1) / a.tile_q;
    g.nkt = (int)((g.nk + a.tile_k - 1) / a.tile_k);
    return g;
}

constexpr int CT = 256;  // threads of a classifying workgroup

__device__ __forceinline__ int64_t block_sum(int64_t x, int64_t *red) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off, 64);
    __syncthreads();  // red may still be read from a previous call
    if (lane == 0) red[wave] = x;
    __syncthreads();
    int64_t s = 0;
    for (int w = 0; w < CT / 64; w++) s += red[w];
    return s;
}

// One workgroup per (batch entry, query tile): the class of each key tile of
// the row, and (with statistics) the row's sums and the touched keys of a
// share of the batch entry's key axis.
__global__ __launch_bounds__(CT) void chunk_classify_kernel(ChunkMetaArgs a) {
    __shared__ int64_t red[CT / 64];
    const Grid G = grid_of(a);
    const int row = blockIdx.x, qt = row % G.nqt, b = row / G.nqt;
    const int i0 = qt * a.tile_q, i1 = min(a.Tq, i0 + a.tile_q);
    const Ring g{a.next_pos[b], a.ring_start[b], a.cache_len[b]};
    const int64_t np = g.np;
    const int64_t t0 = np + i0, t1 = np + i1 - 1;
    int64_t pairs = 0, cov = 0, live = 0, full = 0, part = 0, touched = 0;
    // four consecutive lanes share a key tile, a quarter of its keys each; the
    // quarter sums are added across them (every lane runs every round)
    for (int base = 0; base < G.nkt * 4; base += CT) {
        const int item = base + threadIdx.x, kt = item >> 2, qu = item & 3;
        int64_t count = 0, j0 = 0, j1 = 0;
        if (kt < G.nkt) {
            j0 = (int64_t)kt * a.tile_k;
            j1 = min(G.nk, j0 + a.tile_k);
            const int64_t span = (a.tile_k + 3) / 4;
            const int64_t q0 = j0 + qu * span, q1 = min(j1, q0 + span);
            for (int64_t j = q0; j < q1; j++) count += overlap(key_range(a, G.NS, g, j), t0, t1);
        }
        count += __shfl_xor(count, 1, 64);
        count += __shfl_xor(count, 2, 64);
        if (kt < G.nkt && qu == 0) {
            const int64_t area = (int64_t)(i1 - i0) * (j1 - j0);
            const int c = count == 0 ? 0 : (count == area ? 1 : 2);
            a.cls[(int64_t)row * G.nkt + kt] = (uint8_t)c;
            pairs += count;
            if (c) {
                cov += area;
                live++;
                full += c == 1;
                part += c == 2;
            }
        }
    }
    if (!a.stats) return;
    // keys of this batch entry's axis seen by some query of the chunk: each
    // query tile of the entry takes a contiguous share
    const int64_t share = (G.nk + G.nqt - 1) / G.nqt;
    const int64_t k0 = qt * share, k1 = min(G.nk, k0 + share);
    for (int64_t j = k0 + threadIdx.x; j < k1; j += CT)
        touched += overlap(key_range(a, G.NS, g, j), np, np + a.Tq - 1) > 0;
    const int64_t v[6] = {pairs, cov, touched, live, full, part};
#pragma unroll
    for (int s = 0; s < 6; s++) {
        const int64_t tot = block_sum(v[s], red);
        if (threadIdx.x == 0 && tot)
            atomicAdd((unsigned long long *)(a.stats + s), (unsigned long long)tot);
    }
}

__global__ void chunk_stats_clear_kernel(int64_t *stats) {
    if (threadIdx.x < 6) stats[threadIdx.x] = 0;
}

// One workgroup: the CSR arrays from the class grid, in row-major order.
__global__ __launch_bounds__(NT) void chunk_compact_kernel(ChunkMetaArgs a) {
    __shared__ int wsum[NT / 64];
    const Grid G = grid_of(a);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int64_t M = (int64_t)a.B * G.nqt * G.nkt;
    int running = 0;  // live entries before this round
    for (int64_t base = 0; base < M; base += NT) {
        const int64_t idx = base + tid;
        const int c = idx < M ? a.cls[idx] : 0;
        const uint64_t bal = __ballot(c != 0);
        const int before = __builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32),
                                                    __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0));
        if (lane == 0) wsum[wave] = __builtin_popcountll(bal);
        __syncthreads();
        int woff = 0, total = 0;
        for (int w = 0; w < NT / 64; w++) {
            woff += w < wave ? wsum[w] : 0;
            total += wsum[w];
        }
        const int pos = running + woff + before;
        if (idx < M) {
            const int kt = (int)(idx % G.nkt);
            if (c) {
                a.col[pos] = kt;
                a.col_cls[pos] = (uint8_t)c;
            }
            if (kt == 0) a.row_ptr[idx / G.nkt] = pos;
        }
        running += total;
        __syncthreads();  // wsum is rewritten next round
    }
    if (tid == 0) a.row_ptr[(int64_t)a.B * G.nqt] = running;
}

}  // namespace

hipError_t launch_chunk_meta(const ChunkMetaArgs &a, hipStream_t s) {
    hipError_t e;
    if (a.stats) {
        hipLaunchKernelGGL(chunk_stats_clear_kernel, dim3(1), dim3(64), 0, s, a.stats);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    const int nqt = (a.Tq + a.tile_q - 1) / a.tile_q;
    hipLaunchKernelGGL(chunk_classify_kernel, dim3((unsigned)(a.B * nqt)), dim3(CT), 0, s, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(chunk_compact_kernel, dim3(1), dim3(NT), 0, s, a);
    return hipGetLastError();
}

}  // namespace swa
