// swa_tile_bf16.hip -- bf16 MFMA tile loop for causal sliding-window attention
// on gfx950: the full-sequence forward and the chunked prefill over a ring cache.
//
// What it computes ("Weight sparsity vs attention sparsity" (AI-infra KB) §03;
// "LLMs from scratch" ch.10 §10.1-§10.2): the query at logical position t
// attends over keys at positions t-W+1 .. t, softmax normalised over exactly
// those keys.  Execution follows §04 of the AI-infra page: a workgroup owns one
// query tile and visits only the key tiles its metadata row lists; only
// partial tiles are masked per element.
//
// Work split (tile_q = 32 * NW query rows, tile_k = 64 keys, head dim D):
//   * one workgroup per (query tile, head, batch); NW waves, 32 query rows each;
//   * K tile staged in LDS row-major [key][d]; V tile staged transposed
//     [d][key] so that PV operands are key-contiguous;
//   * S^T = K Q^T with v_mfma_f32_32x32x16_bf16 (A = K rows from LDS, B = the
//     wave's Q rows kept in registers).  The transposed product leaves each
//     lane with one query column, so row max / sum need one cross-half swap;
//   * fp32 online softmax with exp2 and the scale folded into one FMA; a row
//     whose running max is still -inf uses 0 instead (no -inf - -inf);
//   * P rounded to bf16 feeds O^T += V^T P^T directly from the S registers
//     (keys are permuted consistently between the two operands);
//   * inside a partial tile a wave skips a 32-key half in which none of its
//     32 rows sees any key (finer than the metadata, same result);
//   * the next tile's K/V are loaded into registers while this one computes.
#include <hip/hip_runtime.h>
#include <math.h>

#include "swa_internal.h"

namespace swa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int BN = 64;                 // keys per tile
constexpr float LOG2E = 1.4426950408889634f;

__device__ __forceinline__ u32x4 ld16(const void *p) { return *(const u32x4 *)p; }

__device__ __forceinline__ float wave_xor32_max(float x) {
    return fmaxf(x, __shfl_xor(x, 32));
}
__device__ __forceinline__ float wave_xor32_sum(float x) { return x + __shfl_xor(x, 32); }

// Logical position and validity of key `j` (0..BN-1) of key tile kt.
struct KeyPos {
    int mode, nq, W, nrt, qlen;
    int rs, cl;
    int np;
    __device__ __forceinline__ void at(int kt, int j, int &pos, bool &ok) const {
        if (mode == 0) {
            pos = kt * BN + j;
            ok = pos < qlen;
        } else if (kt < nrt) {
            const int s = kt * BN + j;
            int r = s - rs;
            r += (r < 0) ? W : 0;
            ok = r < cl;
            pos = np - cl + r;
        } else {
            const int t = (kt - nrt) * BN + j;
            ok = t < nq;
            pos = np + t;
        }
    }
};

template <int MODE, int D, int NW>
__global__ __launch_bounds__(NW * 64) void tile_kernel(AttnArgs a) {
    constexpr int NT = NW * 64;
    constexpr int KS = D / 16;    // k-steps of the QK product
    constexpr int DB = D / 32;    // 32-wide d blocks of the output
    constexpr int DC = D / 8;     // 16-byte chunks per row
    constexpr int KROW = D + 8;   // LDS K row stride (bf16 elements)
    constexpr int VROW = BN + 4;  // LDS V^T row stride (bf16 elements)
    constexpr int KLD = BN * DC / NT;        // 16-byte K loads per thread per tile
    constexpr int VLD = (BN / 2) * DC / NT;  // (key pair, chunk) tasks per thread
    static_assert(KLD >= 1 && VLD >= 1, "tile too small for the block");

    __shared__ __attribute__((aligned(16))) __bf16 Ks[BN * KROW];
    __shared__ __attribute__((aligned(16))) __bf16 Vt[D * VROW];

    const int qt = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int lq = lane & 31, hh = lane >> 5;
    const int G = a.H / a.Hkv;
    const int g = h / G;
    const int nq = a.nq;
    const int nqt = (nq + 32 * NW - 1) / (32 * NW);

    KeyPos kp;
    kp.mode = MODE;
    kp.nq = nq;
    kp.W = a.W;
    kp.nrt = (MODE == 1) ? a.W / BN : 0;
    kp.qlen = (MODE == 0) ? (a.q_len ? a.q_len[b] : nq) : nq;
    kp.rs = (MODE == 1) ? a.ring_start[b] : 0;
    kp.cl = (MODE == 1) ? a.cache_len[b] : 0;
    kp.np = (MODE == 1) ? a.next_pos[b] : 0;
    const int qlen = kp.qlen;
    const int qbase = (MODE == 1) ? kp.np : 0;  // logical position of query row 0

    // ---- this wave's 32 query rows in registers (B operand of S^T = K Q^T)
    const int row0 = qt * 32 * NW + wave * 32;
    const int myrow = row0 + lq;
    const __bf16 *qp = (const __bf16 *)a.q + (((size_t)b * a.H + h) * nq + myrow) * D;
    bf16x8 qf[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ks++) {
        u32x4 x = (myrow < nq) ? ld16(qp + ks * 16 + hh * 8) : u32x4{0, 0, 0, 0};
        qf[ks] = __builtin_bit_cast(bf16x8, x);
    }

    // ---- key/value sources
    const size_t kvh = (size_t)b * a.Hkv + g;
    const __bf16 *klin = (const __bf16 *)a.k + kvh * (size_t)nq * D;
    const __bf16 *vlin = (const __bf16 *)a.v + kvh * (size_t)nq * D;
    const __bf16 *kring = (MODE == 1) ? (const __bf16 *)a.kc + kvh * (size_t)a.W * D : nullptr;
    const __bf16 *vring = (MODE == 1) ? (const __bf16 *)a.vc + kvh * (size_t)a.W * D : nullptr;
    auto krow_ptr = [&](int kt, int j, const __bf16 *lin, const __bf16 *ring) -> const __bf16 * {
        if (MODE == 1 && kt < kp.nrt) return ring + (size_t)(kt * BN + j) * D;
        const int t = (kt - kp.nrt) * BN + j;
        return (t < nq) ? lin + (size_t)t * D : nullptr;
    };

    u32x4 kreg[KLD];
    u32x4 vreg[VLD][2];
    auto gload = [&](int kt) {
#pragma unroll
        for (int it = 0; it < KLD; it++) {
            const int c = tid + NT * it;
            const int j = c / DC, dc = c % DC;
            const __bf16 *p = krow_ptr(kt, j, klin, kring);
            kreg[it] = p ? ld16(p + dc * 8) : u32x4{0, 0, 0, 0};
        }
#pragma unroll
        for (int it = 0; it < VLD; it++) {
            const int T = tid + NT * it;
            const int kpi = (T & 15) + 16 * (T / (16 * DC));
            const int dc = (T >> 4) % DC;
            const __bf16 *p0 = krow_ptr(kt, 2 * kpi, vlin, vring);
            const __bf16 *p1 = krow_ptr(kt, 2 * kpi + 1, vlin, vring);
            vreg[it][0] = p0 ? ld16(p0 + dc * 8) : u32x4{0, 0, 0, 0};
            vreg[it][1] = p1 ? ld16(p1 + dc * 8) : u32x4{0, 0, 0, 0};
        }
    };
    auto lstore = [&]() {
#pragma unroll
        for (int it = 0; it < KLD; it++) {
            const int c = tid + NT * it;
            const int j = c / DC, dc = c % DC;
            *(u32x4 *)(Ks + j * KROW + dc * 8) = kreg[it];
        }
#pragma unroll
        for (int it = 0; it < VLD; it++) {
            const int T = tid + NT * it;
            const int kpi = (T & 15) + 16 * (T / (16 * DC));
            const int dc = (T >> 4) % DC;
#pragma unroll
            for (int e = 0; e < 8; e++) {
                const uint32_t lo = (vreg[it][0][e >> 1] >> ((e & 1) * 16)) & 0xffffu;
                const uint32_t hi = (vreg[it][1][e >> 1] >> ((e & 1) * 16)) & 0xffffu;
                *(uint32_t *)(Vt + (dc * 8 + e) * VROW + 2 * kpi) = lo | (hi << 16);
            }
        }
    };

    // ---- running softmax state: lanes l and l^32 share query column lq
    const float c2 = a.scale * LOG2E;
    float m_run = -INFINITY, l_run = 0.f;
    f32x16 oacc[DB];
#pragma unroll
    for (int db = 0; db < DB; db++)
#pragma unroll
        for (int e = 0; e < 16; e++) oacc[db][e] = 0.f;

    const int mrow = b * nqt + qt;
    const int e0 = a.row_ptr[mrow], e1 = a.row_ptr[mrow + 1];
    const int qpos = qbase + myrow;
    const bool qvalid = myrow < qlen;
    // ragged key tiles (beyond the array) always take the element mask
    const int nlin_tiles_full = nq / BN;

    if (e1 > e0) gload(a.col[e0]);
    for (int e = e0; e < e1; e++) {
        const int kt = a.col[e];
        const bool ragged = (kt - kp.nrt) >= nlin_tiles_full;
        const bool partial = (a.col_cls[e] == 2) || ragged;
        __syncthreads();
        lstore();
        __syncthreads();
        if (e + 1 < e1) gload(a.col[e + 1]);

        // element mask of this lane's 32 scores (bit kb*16 + i*4 + j)
        uint32_t vis = 0xffffffffu;
        bool live[2] = {true, true};
        if (partial) {
            vis = 0;
#pragma unroll
            for (int kb = 0; kb < 2; kb++)
#pragma unroll
                for (int i = 0; i < 4; i++)
#pragma unroll
                    for (int j = 0; j < 4; j++) {
                        int pos;
                        bool ok;
                        kp.at(kt, kb * 32 + 8 * i + 4 * hh + j, pos, ok);
                        ok = ok && qvalid && pos <= qpos && pos >= qpos - a.W + 1;
                        vis |= (ok ? 1u : 0u) << (kb * 16 + i * 4 + j);
                    }
            live[0] = __ballot((vis & 0xffffu) != 0) != 0;
            live[1] = __ballot((vis >> 16) != 0) != 0;
        }

        // S^T = K Q^T: rows = keys (A from LDS), columns = this wave's queries
        f32x16 sacc[2];
#pragma unroll
        for (int kb = 0; kb < 2; kb++) {
#pragma unroll
            for (int e2 = 0; e2 < 16; e2++) sacc[kb][e2] = 0.f;
            if (!live[kb]) continue;
            const __bf16 *kr = Ks + (kb * 32 + lq) * KROW + hh * 8;
#pragma unroll
            for (int ks = 0; ks < KS; ks++) {
                bf16x8 af = __builtin_bit_cast(bf16x8, *(const u32x4 *)(kr + ks * 16));
                sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, qf[ks], sacc[kb], 0, 0, 0);
            }
        }

        // online softmax over this tile
        float mloc = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < 2; kb++)
#pragma unroll
            for (int e2 = 0; e2 < 16; e2++) {
                if (partial && !((vis >> (kb * 16 + e2)) & 1u)) sacc[kb][e2] = -INFINITY;
                mloc = fmaxf(mloc, sacc[kb][e2]);
            }
        mloc = wave_xor32_max(mloc);
        const float m_new = fmaxf(m_run, mloc * c2);
        const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
        float psum = 0.f;
#pragma unroll
        for (int kb = 0; kb < 2; kb++)
#pragma unroll
            for (int e2 = 0; e2 < 16; e2++) {
                const float pv = __builtin_amdgcn_exp2f(fmaf(sacc[kb][e2], c2, -m_use));
                sacc[kb][e2] = pv;
                psum += pv;
            }
        psum = wave_xor32_sum(psum);
        l_run = l_run * alpha + psum;
        m_run = m_new;
#pragma unroll
        for (int db = 0; db < DB; db++)
#pragma unroll
            for (int e2 = 0; e2 < 16; e2++) oacc[db][e2] *= alpha;

        // O^T += V^T P^T, 16 keys per step; the k index hh*8+t of both operands
        // stands for key 16*s + 4*hh + t (t < 4) or 16*s + 8 + 4*hh + (t-4).
#pragma unroll
        for (int kb = 0; kb < 2; kb++) {
            if (!live[kb]) continue;
#pragma unroll
            for (int s = 0; s < 2; s++) {
                bf16x8 pf;
#pragma unroll
                for (int t = 0; t < 4; t++) {
                    pf[t] = (__bf16)sacc[kb][(2 * s) * 4 + t];
                    pf[4 + t] = (__bf16)sacc[kb][(2 * s + 1) * 4 + t];
                }
                const int kbase = kb * 32 + 16 * s + 4 * hh;
#pragma unroll
                for (int db = 0; db < DB; db++) {
                    const __bf16 *vr = Vt + (db * 32 + lq) * VROW + kbase;
                    const u32x2 lo = *(const u32x2 *)(vr);
                    const u32x2 hi = *(const u32x2 *)(vr + 8);
                    const u32x4 vv = {lo[0], lo[1], hi[0], hi[1]};
                    oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                        __builtin_bit_cast(bf16x8, vv), pf, oacc[db], 0, 0, 0);
                }
            }
        }
    }

    // ---- epilogue: O = O / l; rows without any visible key (padding) get 0
    if (myrow < nq) {
        const float inv = (l_run > 0.f) ? 1.f / l_run : 0.f;
        __bf16 *op = (__bf16 *)a.o + (((size_t)b * a.H + h) * nq + myrow) * D;
#pragma unroll
        for (int db = 0; db < DB; db++)
#pragma unroll
            for (int i = 0; i < 4; i++) {
                bf16x4 w;
#pragma unroll
                for (int j = 0; j < 4; j++) w[j] = (__bf16)(oacc[db][i * 4 + j] * inv);
                *(bf16x4 *)(op + db * 32 + 8 * i + 4 * hh) = w;
            }
    }
}

template <int MODE, int D, int NW>
hipError_t launch_one(const AttnArgs &a, hipStream_t s) {
    const int nqt = (a.nq + 32 * NW - 1) / (32 * NW);
    dim3 grid(nqt, a.H, a.B);
    hipLaunchKernelGGL((tile_kernel<MODE, D, NW>), grid, dim3(NW * 64), 0, s, a);
    return hipGetLastError();
}

template <int MODE>
hipError_t launch_mode(const AttnArgs &a, hipStream_t s) {
    if (a.d == 128) {
        if (a.tile_q == 128) return launch_one<MODE, 128, 4>(a, s);
        return launch_one<MODE, 128, 2>(a, s);
    }
    if (a.tile_q == 128) return launch_one<MODE, 64, 4>(a, s);
    return launch_one<MODE, 64, 2>(a, s);
}

}  // namespace

hipError_t launch_tile_bf16(const AttnArgs &a, hipStream_t s) {
    return a.mode == 0 ? launch_mode<0>(a, s) : launch_mode<1>(a, s);
}

}  // namespace swa
