// swa_bwd.hip -- gradients of the full-sequence sliding-window forward.
//
// For a scalar loss with output gradient dO ("Weight sparsity vs attention
// sparsity" §07 asks for the Q/K/V gradients of the masked attention), with
// P the softmax of s = scale q.k over each row's visible keys and O = P V:
//   D_i   = <dO_i, O_i>                  (= sum_j P_ij <dO_i, v_j>)
//   dS_ij = P_ij (<dO_i, v_j> - D_i)
//   dQ_i  = scale sum_j dS_ij k_j,  dK_j = scale sum_i dS_ij q_i,
//   dV_j  = sum_i P_ij dO_i,
// sums over visible pairs only; P_ij = exp(s_ij - lse_i) from the row
// log-sum-exp the forward wrote.  Grouped heads: dK and dV of kv head g sum
// over its query heads.  Padded rows and keys (past q_len) get 0.
//
// Work is driven by the block metadata ("Weight sparsity vs attention
// sparsity" §04): a query row visits the key tiles of its query tile's CSR
// row; a key visits the query tiles whose class-grid entry for its key tile
// is live.  This is the fp32-arithmetic path for both dtypes: one wave per
// query row (dQ) or per key (dK, dV), the head dim spread over the lanes and
// dot products reduced across the wave.  A packed batch (cu set) runs over
// the same padded index space of longest-sequence length, with rows and keys
// past a sequence's end skipped and every access mapped to the token-major
// layout (qrow, krow).
#include <hip/hip_runtime.h>
#include <math.h>

#include "swa_internal.h"

namespace swa {
namespace {

constexpr float LOG2E = 1.4426950408889634f;

template <typename T>
__device__ __forceinline__ float ld(const T *p, size_t i) {
    return (float)p[i];
}
template <typename T>
__device__ __forceinline__ void st(T *p, size_t i, float x) {
    p[i] = (T)x;
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) x += __shfl_xor(x, m, 64);
    return x;
}

// Rows of request b that exist: N when padded, its own length when packed.
__device__ __forceinline__ int rows_of(const BwdArgs &a, int b) {
    return a.cu ? a.cu[b + 1] - a.cu[b] : a.N;
}
// Index of row i of head h of request b in the query-side row arrays (q, o,
// dout, dq in units of d; lse, dvec): [B][H][N] padded, [tokens][H] packed.
__device__ __forceinline__ size_t qrow(const BwdArgs &a, int b, int h, int i) {
    return a.cu ? (size_t)(a.cu[b] + i) * a.H + h : ((size_t)b * a.H + h) * a.N + i;
}
// Index of key j of kv head g of request b in k, v, dk, dv (units of d).
__device__ __forceinline__ size_t krow(const BwdArgs &a, int b, int g, int j) {
    return a.cu ? (size_t)(a.cu[b] + j) * a.Hkv + g : ((size_t)b * a.Hkv + g) * a.N + j;
}

// D_i = <dO_i, O_i>: one wave per row, lanes over the head dim.
template <typename T>
__global__ __launch_bounds__(256) void bwd_dvec_kernel(BwdArgs a) {
    const long lrow = (long)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const long rows = (long)a.B * a.H * a.N;
    if (lrow >= rows) return;
    const int i = (int)(lrow % a.N);
    const int h = (int)((lrow / a.N) % a.H);
    const int b = (int)(lrow / ((long)a.N * a.H));
    if (i >= rows_of(a, b)) return;
    const size_t row = qrow(a, b, h, i);
    const T *o = (const T *)a.o + row * a.d;
    const T *dO = (const T *)a.dout + row * a.d;
    float acc = 0.f;
    for (int c = lane; c < a.d; c += 64) acc += ld(o, c) * ld(dO, c);
    acc = wave_sum(acc);
    if (lane == 0) a.dvec[row] = acc;
}

// dQ: one wave per query row (b, h, i); keys from the CSR row of its tile.
template <typename T>
__global__ __launch_bounds__(256) void bwd_dq_kernel(BwdArgs a) {
    const long lrow = (long)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const long rows = (long)a.B * a.H * a.N;
    if (lrow >= rows) return;
    const int N = a.N, d = a.d, W = a.W;
    const int i = (int)(lrow % N);
    const int h = (int)((lrow / N) % a.H);
    const int b = (int)(lrow / ((long)N * a.H));
    const int g = h / (a.H / a.Hkv);
    if (i >= rows_of(a, b)) return;  // past a packed sequence: another sequence's row
    const int qlen = a.cu ? rows_of(a, b) : (a.q_len ? a.q_len[b] : N);
    const size_t row = qrow(a, b, h, i);
    T *dq = (T *)a.dq + row * d;
    float qv[2] = {0.f, 0.f}, dov[2] = {0.f, 0.f}, acc[2] = {0.f, 0.f};
    if (i < qlen && a.lse[row] != -INFINITY) {
        const T *q = (const T *)a.q + row * d;
        const T *dO = (const T *)a.dout + row * d;
#pragma unroll
        for (int u = 0; u < 2; u++)
            if (lane + 64 * u < d) {
                qv[u] = ld(q, lane + 64 * u);
                dov[u] = ld(dO, lane + 64 * u);
            }
        const float c2 = a.scale * LOG2E, lse2 = a.lse[row] * LOG2E, Dr = a.dvec[row];
        // key j of this row's kv head at kb + j * ks (ks = d, or Hkv*d packed)
        const size_t ks = a.cu ? (size_t)a.Hkv * d : (size_t)d;
        const T *kb = (const T *)a.k + krow(a, b, g, 0) * d;
        const T *vb = (const T *)a.v + krow(a, b, g, 0) * d;
        const int nqt = (N + a.tile_q - 1) / a.tile_q;
        const int qt = i / a.tile_q;
        const int e0 = a.row_ptr[b * nqt + qt], e1 = a.row_ptr[b * nqt + qt + 1];
        for (int e = e0; e < e1; e++) {
            const int kt = a.col[e];
            // window keys, plus the attention sinks below n_sink
            const int j0 = max(kt * a.tile_k, (kt * a.tile_k < a.n_sink) ? 0 : i - W + 1);
            const int j1 = min(min((kt + 1) * a.tile_k - 1, i), qlen - 1);
            for (int j = j0; j <= j1; j++) {
                if (j < i - W + 1 && j >= a.n_sink) continue;
                float s = 0.f, dp = 0.f, kv[2] = {0.f, 0.f};
#pragma unroll
                for (int u = 0; u < 2; u++)
                    if (lane + 64 * u < d) {
                        kv[u] = ld(kb, (size_t)j * ks + lane + 64 * u);
                        s += qv[u] * kv[u];
                        dp += dov[u] * ld(vb, (size_t)j * ks + lane + 64 * u);
                    }
                s = wave_sum(s);
                dp = wave_sum(dp);
                const float p = exp2f(s * c2 - lse2);
                const float ds = p * (dp - Dr);
#pragma unroll
                for (int u = 0; u < 2; u++) acc[u] += ds * kv[u];
            }
        }
    }
#pragma unroll
    for (int u = 0; u < 2; u++)
        if (lane + 64 * u < d) st(dq, lane + 64 * u, acc[u] * a.scale);
}

// dK, dV: one wave per key (b, g, j); rows of every query head of the group
// in the query tiles whose class-grid entry for the key's tile is live.
template <typename T>
__global__ __launch_bounds__(256) void bwd_dkdv_kernel(BwdArgs a) {
    const long lkey = (long)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const long keys = (long)a.B * a.Hkv * a.N;
    if (lkey >= keys) return;
    const int N = a.N, d = a.d, W = a.W;
    const int j = (int)(lkey % N);
    const int g = (int)((lkey / N) % a.Hkv);
    const int b = (int)(lkey / ((long)N * a.Hkv));
    const int G = a.H / a.Hkv;
    if (j >= rows_of(a, b)) return;  // past a packed sequence: another sequence's key
    const int qlen = a.cu ? rows_of(a, b) : (a.q_len ? a.q_len[b] : N);
    const size_t key = krow(a, b, g, j);
    T *dk = (T *)a.dk + key * d;
    T *dv = (T *)a.dv + key * d;
    float kv[2] = {0.f, 0.f}, vv[2] = {0.f, 0.f}, ak[2] = {0.f, 0.f}, av[2] = {0.f, 0.f};
    if (j < qlen) {
        const T *kr = (const T *)a.k + key * d;
        const T *vr = (const T *)a.v + key * d;
#pragma unroll
        for (int u = 0; u < 2; u++)
            if (lane + 64 * u < d) {
                kv[u] = ld(kr, lane + 64 * u);
                vv[u] = ld(vr, lane + 64 * u);
            }
        const float c2 = a.scale * LOG2E;
        const int nqt = (N + a.tile_q - 1) / a.tile_q;
        const int nkt = (N + a.tile_k - 1) / a.tile_k;
        const int kt = j / a.tile_k;
        // query tiles that can reach this key tile: rows kt*tk .. kt*tk+tk-1+W-1,
        // or every later row for a tile holding attention sinks
        const int qt0 = (kt * a.tile_k) / a.tile_q;
        const long last = (long)kt * a.tile_k + a.tile_k - 2 + W;
        const int qt1 = (kt * a.tile_k < a.n_sink) ? nqt - 1
                                                   : (int)min((long)nqt - 1, last / a.tile_q);
        for (int qt = qt0; qt <= qt1; qt++) {
            if (a.cls[((size_t)b * nqt + qt) * nkt + kt] == 0) continue;
            const int i0 = max(qt * a.tile_q, j);
            const int i1 = min(min((qt + 1) * a.tile_q - 1, (j < a.n_sink) ? qlen - 1 : j + W - 1),
                               qlen - 1);
            for (int h = g * G; h < (g + 1) * G; h++) {
                for (int i = i0; i <= i1; i++) {
                    const size_t row = qrow(a, b, h, i);
                    const T *q = (const T *)a.q + row * d;
                    const T *dO = (const T *)a.dout + row * d;
                    float s = 0.f, dp = 0.f, qv[2] = {0.f, 0.f}, dov[2] = {0.f, 0.f};
#pragma unroll
                    for (int u = 0; u < 2; u++)
                        if (lane + 64 * u < d) {
                            qv[u] = ld(q, lane + 64 * u);
                            dov[u] = ld(dO, lane + 64 * u);
                            s += qv[u] * kv[u];
                            dp += dov[u] * vv[u];
                        }
                    s = wave_sum(s);
                    dp = wave_sum(dp);
                    const float p = exp2f(s * c2 - a.lse[row] * LOG2E);
                    const float ds = p * (dp - a.dvec[row]);
#pragma unroll
                    for (int u = 0; u < 2; u++) {
                        av[u] += p * dov[u];
                        ak[u] += ds * qv[u];
                    }
                }
            }
        }
    }
#pragma unroll
    for (int u = 0; u < 2; u++)
        if (lane + 64 * u < d) {
            st(dk, lane + 64 * u, ak[u] * a.scale);
            st(dv, lane + 64 * u, av[u]);
        }
}

template <typename T>
hipError_t launch_t(const BwdArgs &a, hipStream_t s) {
    hipError_t e;
    const long rows = (long)a.B * a.H * a.N, keys = (long)a.B * a.Hkv * a.N;
    if ((rows + 3) / 4 > 0x7fffffffL || (keys + 3) / 4 > 0x7fffffffL)
        return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(bwd_dvec_kernel<T>, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, s, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(bwd_dq_kernel<T>, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, s, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(bwd_dkdv_kernel<T>, dim3((unsigned)((keys + 3) / 4)), dim3(256), 0, s, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd(const BwdArgs &a, hipStream_t s) {
    if (!a.bf16) return launch_t<float>(a, s);
    if (!bwd_bf16_supported(a)) return launch_t<__bf16>(a, s);
    // the MFMA dq kernel computes the row values D itself
    return launch_bwd_bf16(a, s);
}

}  // namespace swa
