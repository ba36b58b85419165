// swa_ring.hip -- ring-buffer cache bookkeeping on the device.
//
// The cache of one request is [Hkv][W][d] plus (ring_start, cache_len,
// next_pos) ("Dense vs sliding-window sparse attention" blog, §3.2: a start
// index marks the oldest slot; rows are written to the next free slot while
// filling, then over the oldest one).  The r-th oldest row (r < cache_len)
// lives in slot (ring_start + r) mod W at logical position
// next_pos - cache_len + r, so slots keep their logical positions after being
// overwritten ("Weight sparsity vs attention sparsity" §06; "LLMs from
// scratch" ch.10 §10.2).  Appending Tq rows one by one under that rule puts
// the row of position next_pos + t into slot (ring_start + cache_len + t)
// mod W; when Tq > W only the last W rows survive.
#include <hip/hip_runtime.h>

#include "ring_state.h"
#include "swa_internal.h"

namespace swa {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Copy new rows t in [t0, Tq) of k_new/v_new into their ring slots.  One
// thread per 16-byte piece of a row (rows are d * elem_bytes long, a multiple
// of 16 for every supported d and dtype, and the buffers are 16-byte
// aligned); consecutive threads take consecutive pieces of rows (b, g, t) in
// k_new order, so reads and writes coalesce.
__global__ __launch_bounds__(256) void ring_write_kernel(CommitArgs a, int t0) {
    const int P = (int)((size_t)a.d * a.elem_bytes / 16);  // pieces per row
    const int nt = a.Tq - t0;
    const long idx = (long)blockIdx.x * 256 + threadIdx.x;
    if (idx >= (long)nt * a.Hkv * a.B * P) return;
    const int pc = (int)(idx % P);
    const long r = idx / P;
    const int t = t0 + (int)(r % nt);
    const int g = (int)((r / nt) % a.Hkv);
    const int b = (int)(r / ((long)nt * a.Hkv));
    const int W = a.W;
    if (!ring_state_ok(a.ring_start[b], a.cache_len[b], a.next_pos[b], W, a.Tq)) return;
    const int slot = (int)(((int64_t)a.ring_start[b] + a.cache_len[b] + t) % W);
    const size_t kvh = (size_t)b * a.Hkv + g;
    const size_t src = (kvh * a.Tq + t) * P + pc, dst = (kvh * W + slot) * P + pc;
    ((u32x4 *)a.kc)[dst] = ((const u32x4 *)a.k_new)[src];
    ((u32x4 *)a.vc)[dst] = ((const u32x4 *)a.v_new)[src];
}

// State after appending Tq rows: next_pos += Tq, cache_len = min(W, len+Tq),
// ring_start = slot of the oldest kept position.
__global__ void ring_state_kernel(int32_t *ring_start, int32_t *cache_len, int32_t *next_pos,
                                  int B, int W, int Tq) {
    const int b = blockIdx.x * blockDim.x + threadIdx.x;
    if (b >= B) return;
    const int64_t rs = ring_start[b], cl = cache_len[b], np = next_pos[b];
    if (!ring_state_ok((int)rs, (int)cl, (int)np, W, Tq)) return;
    const int64_t cl2 = (cl + Tq < W) ? cl + Tq : W;
    ring_start[b] = (int32_t)((rs + Tq + cl - cl2) % W);
    cache_len[b] = (int32_t)cl2;
    next_pos[b] = (int32_t)(np + Tq);
}

// New row t of a chunk sits at logical position next_pos + t; rows below
// n_sink are also attention sinks ("Sparse attention taxonomy" §3.2) and are
// copied to sink slot next_pos + t.  grid (min(Tq, n_sink), Hkv, B).
__global__ void sink_write_kernel(CommitArgs a) {
    const int t = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
    if (!ring_state_ok(a.ring_start[b], a.cache_len[b], a.next_pos[b], a.W, a.Tq)) return;
    const int64_t pos = (int64_t)a.next_pos[b] + t;
    if (pos >= a.n_sink) return;
    const size_t row_bytes = (size_t)a.d * a.elem_bytes;
    const size_t kvh = (size_t)b * a.Hkv + g;
    const char *ks = (const char *)a.k_new + (kvh * a.Tq + t) * row_bytes;
    const char *vs = (const char *)a.v_new + (kvh * a.Tq + t) * row_bytes;
    char *kd = (char *)a.sk + (kvh * a.n_sink + pos) * row_bytes;
    char *vd = (char *)a.sv + (kvh * a.n_sink + pos) * row_bytes;
    for (size_t off = threadIdx.x * 4; off < row_bytes; off += blockDim.x * 4) {
        *(uint32_t *)(kd + off) = *(const uint32_t *)(ks + off);
        *(uint32_t *)(vd + off) = *(const uint32_t *)(vs + off);
    }
}

}  // namespace

hipError_t launch_sink_write(const CommitArgs &a, hipStream_t s) {
    if (a.n_sink <= 0) return hipSuccess;
    dim3 grid(a.Tq < a.n_sink ? a.Tq : a.n_sink, a.Hkv, a.B);
    hipLaunchKernelGGL(sink_write_kernel, grid, dim3(64), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_ring_write(const CommitArgs &a, hipStream_t s) {
    const int t0 = a.Tq > a.W ? a.Tq - a.W : 0;
    if ((size_t)a.d * a.elem_bytes % 16 != 0) return hipErrorInvalidValue;
    const long pieces = (long)(a.Tq - t0) * a.Hkv * a.B * (long)((size_t)a.d * a.elem_bytes / 16);
    const long blocks = (pieces + 255) / 256;
    if (blocks < 1) return hipSuccess;
    if (blocks > 0x7fffffffL) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(ring_write_kernel, dim3((unsigned)blocks), dim3(256), 0, s, a, t0);
    return hipGetLastError();
}

hipError_t launch_ring_state(const CommitArgs &a, hipStream_t s) {
    hipLaunchKernelGGL(ring_state_kernel, dim3((a.B + 63) / 64), dim3(64), 0, s, a.ring_start,
                       a.cache_len, a.next_pos, a.B, a.W, a.Tq);
    return hipGetLastError();
}

hipError_t launch_commit(const CommitArgs &a, hipStream_t s) {
    hipError_t e = launch_ring_write(a, s);
    if (e != hipSuccess) return e;
    return launch_ring_state(a, s);
}

}  // namespace swa
