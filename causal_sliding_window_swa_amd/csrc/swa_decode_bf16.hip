// swa_decode_bf16.hip -- one decode step against a ring-buffer KV cache, bf16.
//
// A decode step must stream every K/V row it reads from HBM ("Sparse
// attention taxonomy" §1.1), so the kernel is built to read each ring row of a
// request exactly once and keep many bytes in flight:
//   * grid (n_split, Hkv, B): the W slots of one (request, KV head) are split
//     into n_split ranges, each range into 4 per-wave quarters;
//   * all G = H/Hkv query heads of the KV group are scored together, so a K/V
//     row is loaded once for the whole group: S^T (16 keys x 16 head slots)
//     = K Q^T with v_mfma_f32_16x16x32_bf16 (K rows straight from HBM);
//   * fp32 online softmax per head (exp2, scale folded into one FMA);
//   * probabilities go through a small per-wave LDS table to the lanes that
//     hold V rows (16 lanes x 16 bytes per row), which accumulate P V in fp32;
//   * each wave walks its quarter in 32-key steps with two register buffers,
//     so the next step's K/V loads are in flight while one step computes;
//   * the waves merge in LDS; a single range writes O directly (a tiny kernel
//     then advances the ring state), otherwise each range writes (max, sum,
//     unnormalised O) to the workspace and a second kernel merges the ranges
//     by log-sum-exp and advances the state.
//
// Append first ("Dense vs sliding-window sparse attention" blog §3.2 rule):
// the new row goes to slot (ring_start + cache_len) mod W while the ring is
// filling, else over the oldest slot ring_start.  The range owning that slot
// reads the new row from k_new/v_new and writes it into the ring; no other
// block reads that slot.  The ring state itself is advanced by a second
// kernel, after every range has read it.
#include <hip/hip_runtime.h>
#include <math.h>

#include <mutex>

#include "../../include/swa.h"
#include "ring_state.h"
#include "swa_internal.h"

namespace swa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr float LOG2E = 1.4426950408889634f;
constexpr int CH = 32;    // keys per wave iteration (two register buffers in flight)
constexpr int PST = 20;   // LDS probability row stride (floats): conflict-free writes

__device__ __forceinline__ u32x4 ld16(const void *p) { return *(const u32x4 *)p; }

// Combine lane l with lane l^16 / l^32 without an LDS round trip.
__device__ __forceinline__ float swap16_max(float x) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                    false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float swap32_max(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                    false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float swap16_sum(float x) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                    false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float swap32_sum(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                    false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
// lane-xor sum for the end-of-range merge (offsets 8, 16 or 32)
__device__ __forceinline__ float xor_sum(float x, int off) {
    if (off == 16) return swap16_sum(x);
    if (off == 32) return swap32_sum(x);
    return x + __shfl_xor(x, off);
}

__device__ __forceinline__ float bf_lo(uint32_t x) { return __uint_as_float(x << 16); }
__device__ __forceinline__ float bf_hi(uint32_t x) { return __uint_as_float(x & 0xffff0000u); }

// Orders this wave's LDS accesses for the compiler; LDS operations of one
// wave are executed in issue order by the hardware.
__device__ __forceinline__ void wave_lds_order() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

struct RingView {
    int W, rs2, cl2, np2, s_new;
    // valid slot of the ring after the append, and its logical position
    __device__ __forceinline__ bool valid(int s, int &pos) const {
        int r = s - rs2;
        r += (r < 0) ? W : 0;
        pos = np2 - cl2 + r;
        return r < cl2;
    }
};

template <int D, int G, int NWV>
__global__ __launch_bounds__(NWV * 64) void decode_split_kernel(DecodeArgs a) {
    constexpr int KSTEP = D / 32;  // 32-wide k-steps of the QK product
    constexpr int LPR = D / 8;     // lanes per V row (16 bytes each)
    constexpr int RPI = 64 / LPR;  // V rows per wave instruction
    constexpr int NRR = CH / RPI;  // V row rounds per iteration

    __shared__ __attribute__((aligned(16))) float Pl[NWV][CH * PST];
    __shared__ float wm[NWV][16], wl[NWV][16];
    __shared__ float wo[NWV][G][D];

    const int split = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int lh = lane & 15, lg = lane >> 4;
    const int W = a.W;

    // ring state before and after the append
    const int rs = a.ring_start[b], cl = a.cache_len[b], np = a.next_pos[b];
    const bool st_ok = ring_state_ok(rs, cl, np, W, 1);  // else: no append, no key
    RingView rv;
    rv.W = W;
    const bool full = cl == W;
    rv.s_new = full ? rs : (rs + cl) % W;
    rv.rs2 = full ? (rs + 1 == W ? 0 : rs + 1) : rs;
    rv.cl2 = full ? W : cl + 1;
    rv.np2 = np + 1;
    const int qpos = np;

    // slot ranges: split -> [s0, s1), wave -> [w0, w1)
    const int S = (W + a.n_split - 1) / a.n_split;
    const int s0 = split * S, s1 = min(W, s0 + S);
    const int SW = (S + NWV - 1) / NWV;
    const int w0 = s0 + wave * SW, w1 = min(s1, w0 + SW);
    const int niter = (SW + CH - 1) / CH;  // same for every wave of the block

    const size_t kvh = (size_t)b * a.Hkv + g;
    const __bf16 *kring = (const __bf16 *)a.kc + kvh * (size_t)W * D;
    const __bf16 *vring = (const __bf16 *)a.vc + kvh * (size_t)W * D;
    const __bf16 *knew = (const __bf16 *)a.k_new + kvh * D;
    const __bf16 *vnew = (const __bf16 *)a.v_new + kvh * D;

    // the range owning the new slot stores the new row into the ring
    if (st_ok && rv.s_new >= s0 && rv.s_new < s1 && tid < LPR) {
        *(u32x4 *)((__bf16 *)a.kc + (kvh * W + rv.s_new) * D + tid * 8) = ld16(knew + tid * 8);
        *(u32x4 *)((__bf16 *)a.vc + (kvh * W + rv.s_new) * D + tid * 8) = ld16(vnew + tid * 8);
    }

    // Q of the group as the B operand: column lh = head (zero past G).  The MFMA
    // k index lg*8 + t of k-step ks stands for d = ks*32 + lg*8 + t in both
    // operands, so the 4 lanes of one K row read 64 contiguous bytes per load.
    bf16x8 qf[KSTEP];
    {
        const __bf16 *qp = (const __bf16 *)a.q + ((size_t)b * a.H + g * G + lh) * D + lg * 8;
#pragma unroll
        for (int ks = 0; ks < KSTEP; ks++) {
            u32x4 x = (lh < G) ? ld16(qp + ks * 32) : u32x4{0, 0, 0, 0};
            qf[ks] = __builtin_bit_cast(bf16x8, x);
        }
    }

    const float c2 = a.scale * LOG2E;
    float m_run = -INFINITY, l_run = 0.f;  // per head lh (replicated over lg)
    float o[G][8];
#pragma unroll
    for (int hq = 0; hq < G; hq++)
#pragma unroll
        for (int e = 0; e < 8; e++) o[hq][e] = 0.f;
    float *P = Pl[wave];

    // one iteration's loads: K in the MFMA A layout, V as 16-byte row pieces
    struct Buf {
        u32x4 k[2][KSTEP];
        u32x4 v[NRR];
    };
    auto load = [&](Buf &bf, int c0) {
#pragma unroll
        for (int kb = 0; kb < 2; kb++) {
            const int s = c0 + kb * 16 + lh;
            const __bf16 *src = (s == rv.s_new) ? knew : kring + (size_t)s * D;
#pragma unroll
            for (int ks = 0; ks < KSTEP; ks++)
                bf.k[kb][ks] = (s < w1) ? ld16(src + ks * 32 + lg * 8) : u32x4{0, 0, 0, 0};
        }
#pragma unroll
        for (int rr = 0; rr < NRR; rr++) {
            const int s = c0 + rr * RPI + lane / LPR;
            const __bf16 *src = (s == rv.s_new) ? vnew : vring + (size_t)s * D;
            bf.v[rr] = (s < w1) ? ld16(src + (lane % LPR) * 8) : u32x4{0, 0, 0, 0};
        }
    };
    auto compute = [&](const Buf &bf, int c0) {
        // scores: sacc[kb][j] = S[key c0 + kb*16 + lg*4 + j][head lh]
        f32x4 sacc[2];
#pragma unroll
        for (int kb = 0; kb < 2; kb++) {
            sacc[kb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < KSTEP; ks++)
                sacc[kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                    __builtin_bit_cast(bf16x8, bf.k[kb][ks]), qf[ks], sacc[kb], 0, 0, 0);
        }
        float mloc = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < 2; kb++)
#pragma unroll
            for (int j = 0; j < 4; j++) {
                const int s = c0 + kb * 16 + lg * 4 + j;
                int pos;
                const bool ok =
                    st_ok && s < w1 && rv.valid(s, pos) && pos <= qpos && pos >= qpos - W + 1;
                if (!ok) sacc[kb][j] = -INFINITY;
                mloc = fmaxf(mloc, sacc[kb][j]);
            }
        mloc = swap32_max(swap16_max(mloc));
        const float m_new = fmaxf(m_run, mloc * c2);
        const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
        float psum = 0.f;
#pragma unroll
        for (int kb = 0; kb < 2; kb++)
#pragma unroll
            for (int j = 0; j < 4; j++) {
                const float p = __builtin_amdgcn_exp2f(fmaf(sacc[kb][j], c2, -m_use));
                psum += p;
                P[(kb * 16 + lg * 4 + j) * PST + lh] = p;
            }
        psum = swap32_sum(swap16_sum(psum));
        l_run = l_run * alpha + psum;
        m_run = m_new;
        // rescale O by each head's alpha (held by lane hq)
#pragma unroll
        for (int hq = 0; hq < G; hq++) {
            const float ah = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(alpha), hq));
#pragma unroll
            for (int e = 0; e < 8; e++) o[hq][e] *= ah;
        }
        wave_lds_order();
        // O += P V over this iteration's rows
#pragma unroll
        for (int rr = 0; rr < NRR; rr++) {
            const int row = rr * RPI + lane / LPR;
            float pr[G];
            if (G >= 4) {
#pragma unroll
                for (int q4 = 0; q4 < G / 4; q4++) {
                    const f32x4 t = *(const f32x4 *)(P + row * PST + q4 * 4);
#pragma unroll
                    for (int e = 0; e < 4; e++) pr[q4 * 4 + e] = t[e];
                }
            } else {
#pragma unroll
                for (int hq = 0; hq < G; hq++) pr[hq] = P[row * PST + hq];
            }
            float v[8];
#pragma unroll
            for (int e = 0; e < 4; e++) {
                v[2 * e] = bf_lo(bf.v[rr][e]);
                v[2 * e + 1] = bf_hi(bf.v[rr][e]);
            }
#pragma unroll
            for (int hq = 0; hq < G; hq++)
#pragma unroll
                for (int e = 0; e < 8; e++) o[hq][e] = fmaf(pr[hq], v[e], o[hq][e]);
        }
        wave_lds_order();
    };
    // two buffers: the next iteration's loads are in flight while one computes
    Buf b0, b1;
    if (niter > 0) load(b0, w0);
    for (int it = 0; it < niter; it += 2) {
        if (it + 1 < niter) load(b1, w0 + (it + 1) * CH);
        compute(b0, w0 + it * CH);
        if (it + 1 < niter) {
            if (it + 2 < niter) load(b0, w0 + (it + 2) * CH);
            compute(b1, w0 + (it + 1) * CH);
        }
    }

    // sum the row groups of the wave (lanes with equal lane % LPR)
#pragma unroll
    for (int off = LPR; off < 64; off <<= 1)
#pragma unroll
        for (int hq = 0; hq < G; hq++)
#pragma unroll
            for (int e = 0; e < 8; e++) o[hq][e] = xor_sum(o[hq][e], off);
    if (lane < 16) {
        wm[wave][lane] = m_run;
        wl[wave][lane] = l_run;
    }
    if (lane < LPR) {
#pragma unroll
        for (int hq = 0; hq < G; hq++)
#pragma unroll
            for (int e = 0; e < 8; e++) wo[wave][hq][lane * 8 + e] = o[hq][e];
    }
    __syncthreads();
    // merge the waves; with one range per (request, KV head) write O itself,
    // else this range's (max, sum, unnormalised O)
    const int nsp = a.n_split;
    for (int idx = tid; idx < G * D; idx += NWV * 64) {
        const int hq = idx / D, dd = idx % D;
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < NWV; w++) M = fmaxf(M, wm[w][hq]);
        const float Mu = (M == -INFINITY) ? 0.f : M;
        float L = 0.f, O = 0.f;
#pragma unroll
        for (int w = 0; w < NWV; w++) {
            const float f = __builtin_amdgcn_exp2f(wm[w][hq] - Mu);
            L += f * wl[w][hq];
            O += f * wo[w][hq][dd];
        }
        if (nsp == 1 && a.n_sink == 0) {
            ((__bf16 *)a.o)[((size_t)b * a.H + g * G + hq) * D + dd] =
                (__bf16)((L > 0.f) ? O / L : 0.f);
            continue;
        }
        const size_t hidx = ((size_t)b * a.H + g * G + hq) * nsp + split;
        a.ws[hidx * D + dd] = O;
        if (dd == 0) {
            float *ml = a.ws + (size_t)a.B * a.H * nsp * D;
            ml[2 * hidx] = M;
            ml[2 * hidx + 1] = L;
        }
    }
}

// Sum over the D threads of a block (D = 64 or 128).
template <int D>
__device__ __forceinline__ float block_sum(float x, float *red) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) x += __shfl_xor(x, m, 64);
    if (D == 64) return x;
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = x;
    __syncthreads();
    const float r = red[0] + red[1];
    __syncthreads();
    return r;
}

// grid (B*H), D threads: log-sum-exp merge of the NSP ranges, O = sum / l as
// bf16; block (b, head 0) then advances the ring state of request b by one
// token.  NSP is a compile-time constant so every (max, sum) pair (uniform
// across the block, hence scalar loads) and partial row is loaded before any
// is used.  SINK: the attention sinks ("Sparse attention taxonomy" §3.2) the
// ring no longer holds join the merge as one more partial, a token appended
// at a sink position is copied to the sink cache, and the ring state is left
// to decode_state_kernel (every block reads it here).
template <int D, int NSP, bool SINK>
__global__ __launch_bounds__(D) void decode_combine_kernel(DecodeArgs a) {
    const int bh = blockIdx.x, b = bh / a.H, h = bh % a.H;
    float msk = -INFINITY, lsk = 0.f, osk = 0.f;  // sink partial (log2 units)
    if (SINK) {
        __shared__ float red[2];
        const int W = a.W, cl = a.cache_len[b], np = a.next_pos[b];
        const bool st_ok = ring_state_ok(a.ring_start[b], cl, np, W, 1);
        const int cl2 = (cl == W) ? W : cl + 1;
        const int nsink = st_ok ? min(a.n_sink, np + 1 - cl2) : 0;
        const int G = a.H / a.Hkv, g = h / G, c = threadIdx.x;
        const float qc = (float)((const __bf16 *)a.q)[(size_t)bh * D + c];
        const float c2 = a.scale * 1.4426950408889634f;
        const size_t sbase = ((size_t)b * a.Hkv + g) * a.n_sink;
        for (int p = 0; p < nsink; p++) {
            const float kc = (float)((const __bf16 *)a.sk)[(sbase + p) * D + c];
            const float vc = (float)((const __bf16 *)a.sv)[(sbase + p) * D + c];
            const float s2 = block_sum<D>(qc * kc, red) * c2;
            const float mn = fmaxf(msk, s2);
            const float f = __builtin_amdgcn_exp2f(msk - mn), e = __builtin_amdgcn_exp2f(s2 - mn);
            lsk = lsk * f + e;
            osk = osk * f + e * vc;
            msk = mn;
        }
        if (st_ok && np < a.n_sink && h % G == 0) {  // slot np is not read in this step
            ((__bf16 *)a.sk)[(sbase + np) * D + c] = ((const __bf16 *)a.k_new)[((size_t)b * a.Hkv + g) * D + c];
            ((__bf16 *)a.sv)[(sbase + np) * D + c] = ((const __bf16 *)a.v_new)[((size_t)b * a.Hkv + g) * D + c];
        }
    }
    const float *ml = a.ws + (size_t)a.B * a.H * NSP * D + (size_t)bh * NSP * 2;
    const float *op = a.ws + (size_t)bh * NSP * D + threadIdx.x;
    float m[NSP], l[NSP], o[NSP];
#pragma unroll
    for (int s = 0; s < NSP; s++) {
        m[s] = ml[2 * s];
        l[s] = ml[2 * s + 1];
        o[s] = op[(size_t)s * D];
    }
    float M = msk;
#pragma unroll
    for (int s = 0; s < NSP; s++) M = fmaxf(M, m[s]);
    const float Mu = (M == -INFINITY) ? 0.f : M;
    float L = 0.f, O = 0.f;
#pragma unroll
    for (int s = 0; s < NSP; s++) {
        const float f = __builtin_amdgcn_exp2f(m[s] - Mu);
        L += f * l[s];
        O += f * o[s];
    }
    if (SINK) {
        const float f = __builtin_amdgcn_exp2f(msk - Mu);
        L += f * lsk;
        O += f * osk;
    }
    ((__bf16 *)a.o)[(size_t)bh * D + threadIdx.x] = (__bf16)((L > 0.f) ? O / L : 0.f);
    if (!SINK && h == 0 && threadIdx.x == 0) {
        const int W = a.W, rs = a.ring_start[b], cl = a.cache_len[b];
        if (!ring_state_ok(rs, cl, a.next_pos[b], W, 1)) return;
        const bool full = cl == W;
        a.ring_start[b] = full ? (rs + 1) % W : rs;
        a.cache_len[b] = full ? W : cl + 1;
        a.next_pos[b] = a.next_pos[b] + 1;
    }
}

// Advances the ring state of every request by one token (after the single-
// range kernel, which writes O itself).
__global__ void decode_state_kernel(int32_t *ring_start, int32_t *cache_len, int32_t *next_pos,
                                    int B, int W) {
    const int b = blockIdx.x * blockDim.x + threadIdx.x;
    if (b >= B) return;
    const int rs = ring_start[b], cl = cache_len[b];
    if (!ring_state_ok(rs, cl, next_pos[b], W, 1)) return;
    const bool full = cl == W;
    ring_start[b] = full ? (rs + 1) % W : rs;
    cache_len[b] = full ? W : cl + 1;
    next_pos[b] = next_pos[b] + 1;
}

// One range per (request, KV head): the waves merge in LDS and write O, then
// the ring state advances.  Several ranges: the log-sum-exp combine follows.
template <int D, bool SINK>
hipError_t launch_combine(const DecodeArgs &a, hipStream_t s) {
    const dim3 grid(a.B * a.H), blk(D);
    switch (a.n_split) {
        case 1: hipLaunchKernelGGL((decode_combine_kernel<D, 1, SINK>), grid, blk, 0, s, a); break;
        case 2: hipLaunchKernelGGL((decode_combine_kernel<D, 2, SINK>), grid, blk, 0, s, a); break;
        case 4: hipLaunchKernelGGL((decode_combine_kernel<D, 4, SINK>), grid, blk, 0, s, a); break;
        case 8: hipLaunchKernelGGL((decode_combine_kernel<D, 8, SINK>), grid, blk, 0, s, a); break;
        case 16: hipLaunchKernelGGL((decode_combine_kernel<D, 16, SINK>), grid, blk, 0, s, a); break;
        case 32: hipLaunchKernelGGL((decode_combine_kernel<D, 32, SINK>), grid, blk, 0, s, a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

// One range per (request, KV head) and no sinks: the waves merge in LDS and
// write O, then the ring state advances.  Otherwise each range writes its
// partial and the log-sum-exp combine follows (with sinks, then the state).
template <int D, int G>
hipError_t launch_dg(const DecodeArgs &a, hipStream_t s) {
    hipError_t e;
    hipLaunchKernelGGL((decode_split_kernel<D, G, 4>), dim3(a.n_split, a.Hkv, a.B), dim3(256), 0,
                       s, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if (a.n_split == 1 && a.n_sink == 0) {
        hipLaunchKernelGGL(decode_state_kernel, dim3((a.B + 63) / 64), dim3(64), 0, s,
                           a.ring_start, a.cache_len, a.next_pos, a.B, a.W);
        return hipGetLastError();
    }
    if (a.n_sink == 0) return launch_combine<D, false>(a, s);
    if ((e = launch_combine<D, true>(a, s)) != hipSuccess) return e;
    hipLaunchKernelGGL(decode_state_kernel, dim3((a.B + 63) / 64), dim3(64), 0, s, a.ring_start,
                       a.cache_len, a.next_pos, a.B, a.W);
    return hipGetLastError();
}

template <int D>
hipError_t launch_d(const DecodeArgs &a, hipStream_t s) {
    switch (a.H / a.Hkv) {
        case 1: return launch_dg<D, 1>(a, s);
        case 2: return launch_dg<D, 2>(a, s);
        case 4: return launch_dg<D, 4>(a, s);
        default: return launch_dg<D, 8>(a, s);
    }
}

}  // namespace

// Ranges per (request, KV head): a power of two, each range at least 256
// slots (64 per wave), at most 32 (the combine kernel's instantiations); the
// workspace is sized for this maximum.
int decode_max_splits(int W) {
    int m = 1;
    while (m < 32 && 2 * m * 256 <= W) m <<= 1;
    return m;
}

// Enough ranges for about 8192 workgroups (many short workgroups keep the
// CUs fuller than a few long ones), never more than the workspace holds.
int decode_bf16_splits(int B, int Hkv, int W) {
    const long pairs = (long)B * Hkv;
    const int cap = decode_max_splits(W);
    int n = 1;
    while (pairs * n < 8192 && n < cap) n <<= 1;
    return n;
}

// Partials of swa_decode_noalloc: each GPU holds its own copy of this array.
// Host code must not pass the array's name to a kernel (on the host it names
// a stand-in, not device memory): decode_scratch() looks up the current
// device's address once and every launch uses that.  Nothing in it needs to
// start at zero (each range writes its partial before the merge reads it).
static __device__ __align__(256) float scratch[kDecodeScratchBytes / sizeof(float)];

int decode_scratch(float **ptr) {
    constexpr int MAXDEV = 64;
    static std::mutex mu;
    static float *addr[MAXDEV];
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return fail(SWA_EHIP, "swa_decode_noalloc: hipGetDevice failed: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= MAXDEV)
        return fail(SWA_EUNSUPPORTED, "swa_decode_noalloc: device %d beyond the %d supported",
                    dev, MAXDEV);
    std::lock_guard<std::mutex> lock(mu);
    if (!addr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p)
            return fail(SWA_EHIP, "swa_decode_noalloc: hipGetSymbolAddress(scratch) failed: %s",
                        hipGetErrorString(e));
        addr[dev] = (float *)p;
    }
    *ptr = addr[dev];
    return SWA_OK;
}

hipError_t launch_decode_bf16(const DecodeArgs &a, hipStream_t s) {
    return a.d == 128 ? launch_d<128>(a, s) : launch_d<64>(a, s);
}

}  // namespace swa
