// swa_bwd_bf16.hip -- bf16 MFMA kernels for the gradients of the full-sequence
// sliding-window forward (d in {64, 128}, tile_k = 64).  Same quantities as
// swa_bwd.hip ("Weight sparsity vs attention sparsity" §07); with the row
// log-sum-exp of the forward, P = exp(s - lse) <= 1, so no running max is
// needed.  Fragment layouts of v_mfma_f32_32x32x16_bf16 as in the forward:
// A lane l = A[l%32][(l/32)*8 .. +8], B lane l = B[(l/32)*8 .. +8][l%32],
// C element 4i+j of lane l = C[8i + 4(l/32) + j][l%32].
//
// dq_kernel: one workgroup per (query tile, head, request), 32 query rows per
// wave, visiting the key tiles of its metadata row (K and V tiles staged in
// LDS, double-buffered).  Per tile: S^T = K Q^T and dP^T = V dO^T (A = K or
// V rows read from LDS, B = the wave's Q or dO rows in registers), then
// dS^T = P^T (dP^T - D) and dQ^T += K^T dS^T with K^T read by transposing
// LDS reads, one 32-key half after the other (so that two waves fit per
// SIMD).  Each lane holds one query column: lse and D are per lane.
//
// dkdv_kernel: one workgroup of four waves per (key tile of 64, kv head,
// request), visiting 64-row steps of every query head of the group in the
// query tiles whose class-grid entry for the key tile is live (Q, dO, lse and
// D rows staged in LDS, double-buffered).  The waves split the work by role,
// two per role, one per 32-key half: role 0 holds its keys' K rows and
// computes S = Q K^T, P (masked) and dV^T += dO^T P; role 1 holds the V rows
// and computes dP = dO V^T, then dS = P (dP - D) and dK^T += Q^T dS.  P goes
// from role 0 to role 1 through LDS, once per step, across a barrier that
// waits for LDS writes only.  A wave then holds one operand row set and one
// accumulator set (252 registers at D = 128), so two waves run per SIMD, where
// one wave holding K, V, dK and dV needed 316 and ran alone.  Each lane holds
// one key column; A operands are Q or dO rows from LDS, and dO^T, Q^T come
// from transposing LDS reads.
//
// PK (packed batch): the same kernels over token-major tensors, sequence b
// being tokens cu[b] .. cu[b+1]-1; rows are then H*D (Q side) or Hkv*D (K
// side) elements apart and lse / D are [tokens][H].  The grid is sized by
// the longest sequence; work items past a sequence's end find empty metadata
// rows and write nothing, and no row past it is read or written.
#include <hip/hip_runtime.h>
#include <math.h>

#include "swa_internal.h"

namespace swa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

constexpr int BN = 64;  // keys per key tile; rows per dkdv step
constexpr float LOG2E = 1.4426950408889634f;

__device__ __forceinline__ u32x4 ld16(const void *p) { return *(const u32x4 *)p; }

// Workgroup p of T runs logical item L: XCD x = p % 8 gets a contiguous range.
__device__ __forceinline__ int xcd_remap(int p, int T) {
    const int x = p & 7, i = p >> 3, q = T >> 3, r = T & 7;
    return x * q + (x < r ? x : r) + i;
}

// Workgroups go to the XCDs round-robin, about 64 per XCD at a time.  The
// logical order is cut into 64-item chunks and runs of 4 chunks; in rounds
// 4R .. 4R+3 XCD x runs the chunks of run 8R + (x + R) % 8 in order, so the
// items an XCD runs together, and its successive chunks, are neighbours
// (shared tiles in its L2), and every XCD draws from all parts of the order
// (even work when sequence lengths differ).  The tail of T mod 2048 items
// keeps contiguous ranges.  A bijection.
__device__ __forceinline__ int xcd_deal(int p, int T) {
    constexpr int C = 64, S = 4;
    const int Tm = T / (8 * C * S) * (8 * C * S);
    if (p < Tm) {
        const int x = p & 7, i = p >> 3, r = i / C, o = i % C;
        const int R = r / S, sub = r % S;
        return ((R * 8 + ((x + R) & 7)) * S + sub) * C + o;
    }
    return Tm + xcd_remap(p - Tm, T - Tm);
}

// 16-byte chunk c of row r sits at physical chunk c ^ swz(r).  The staged Q,
// dO and K tiles are read both ways, as rows (16 lanes: 16 consecutive rows,
// one chunk) and by transposing reads (32 lanes: 4 consecutive rows, 4
// consecutive chunks), so the swizzle must spread both over the 64 four-byte
// banks (256 bytes).  D = 128 (16 chunks, one row per 256 bytes): the two
// 2-bit fields of r % 16 swapped, distinct over 16 rows and distinct in its
// top bits over 4 rows.  D = 64 (8 chunks, two rows per 256 bytes): rows of
// one parity get distinct values, and rows r, r + 2 differ in bit 2.  (r % 16
// alone left the transposing reads with 4-way bank conflicts at D = 128.)
template <int CPR>
__device__ __forceinline__ int swz(int r) {
    if (CPR == 16) return ((r & 3) << 2) | ((r >> 2) & 3);
    return (((r >> 1) & 1) << 2) | ((r >> 2) & 3);
}

// 8 bf16 of a transposing read pair: lanes' 4-element pieces of rows
// kk*16 + 8r + tr_row, columns db*32 + tr_col .. +3 of a row-major tile.
template <int D>
__device__ __forceinline__ bf16x8 tr_frag(const char *base, int kk, int db, int tr_row,
                                          int tr_col) {
    constexpr int ROWB = D * 2, CPR = D / 8;
    i16x4 v2[2];
#pragma unroll
    for (int r = 0; r < 2; r++) {
        const int row = kk * 16 + 8 * r + tr_row;
        const int col = db * 32 + tr_col;
        const int c = (col >> 3) ^ swz<CPR>(row);
        v2[r] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_i16x4 *)(base + row * ROWB + c * 16 + (col & 7) * 2));
    }
    const u32x2 lo = __builtin_bit_cast(u32x2, v2[0]);
    const u32x2 hi = __builtin_bit_cast(u32x2, v2[1]);
    const u32x4 vv = {lo[0], lo[1], hi[0], hi[1]};
    return __builtin_bit_cast(bf16x8, vv);
}

// A fragment of rows r0 .. r0+31 (lane row r0 + lq), k-step ks of a row-major tile.
template <int D>
__device__ __forceinline__ bf16x8 row_frag(const char *base, int r0, int lq, int hh, int ks) {
    constexpr int ROWB = D * 2, CPR = D / 8;
    const int r = r0 + lq;
    const int c = (2 * ks + hh) ^ swz<CPR>(r);
    return __builtin_bit_cast(bf16x8, *(const u32x4 *)(base + r * ROWB + c * 16));
}

typedef __attribute__((address_space(3))) void lds_void;

// Buffer resource over `bytes` bytes at `base`: raw loads past the end return 0.
#define SWA_RSRC(base, bytes) \
    __builtin_amdgcn_make_buffer_rsrc((void *)(base), 0, (bytes), 0x00020000)

// Copy 64 rows x D of a bf16 matrix of nrows rows, rsb bytes apart (rows
// row0..; rows past the data read as zeros: finite, and masked) into an LDS
// tile, swizzled; NW waves share the work.  The buffer (MUBUF) form of the LDS DMA
// keeps the compiler's LDS-read waits partial (the FLAT global_load_lds form
// makes every wait lgkmcnt(0)).
template <int D, int NW>
__device__ __forceinline__ void stage_rows(const __bf16 *src, int row0, int nrows, int rsb,
                                           char *dst, int wave, int lane) {
#if defined(__HIP_DEVICE_COMPILE__)  // the buffer builtins exist for the device only
    constexpr int ROWB = D * 2, CPR = D / 8, RPL = 64 / CPR, LPW = BN / RPL / NW;
    // the range ends with the last row's own bytes: a row past it starts at or
    // beyond the end and reads as zeros
    const auto rs = SWA_RSRC(src, nrows > 0 ? (nrows - 1) * rsb + ROWB : 0);
#pragma unroll
    for (int i = 0; i < LPW; i++) {
        const int ins = wave * LPW + i;
        const int r = ins * RPL + lane / CPR;
        const int pch = lane % CPR;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void *)(dst + ins * 1024), 16,
                                                 (row0 + r) * rsb + (pch ^ swz<CPR>(r)) * 16, 0,
                                                 0, 0);
    }
#endif
}

// One fp32 value per lane (element i of an n-element array whose elements
// are `stride` floats apart; zero past the end) into 64 consecutive LDS words.
__device__ __forceinline__ void stage_vals(const float *src, int i, int n, int stride,
                                           char *dst) {
#if defined(__HIP_DEVICE_COMPILE__)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(SWA_RSRC(src, n > 0 ? ((n - 1) * stride + 1) * 4 : 0),
                                             (lds_void *)dst, 4, i * stride * 4, 0, 0, 0);
#endif
}

// ---------------------------------------------------------------------------
// SK: attention sinks may be present; without them the second key interval of
// the per-element mask folds away (a call without sinks runs SK = false)
template <int D, int NW, bool PK, bool SK>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(2)))
void dq_kernel(BwdArgs a) {
    constexpr int KS = D / 16, DB = D / 32, ROWB = D * 2, TILEB = BN * ROWB;
    __shared__ __attribute__((aligned(1024))) char stage0[2 * TILEB];
    __shared__ __attribute__((aligned(1024))) char stage1[2 * TILEB];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lq = lane & 31, hh = lane >> 5;
    const int N = a.N;
    const int nqt = (N + 32 * NW - 1) / (32 * NW);
    const int L = xcd_deal(blockIdx.x, gridDim.x);
    const int G = a.H / a.Hkv;
    const int h_in = L % G, qt = (L / G) % nqt, g = (L / (G * nqt)) % a.Hkv;
    const int b = L / (G * nqt * a.Hkv);
    const int h = g * G + h_in;
    // rows of this request that exist (all N when padded)
    const int cub = PK ? a.cu[b] : 0;
    const int nrows = PK ? a.cu[b + 1] - cub : N;
    const int qlen = PK ? nrows : (a.q_len ? a.q_len[b] : N);

    const int myrow = qt * 32 * NW + wave * 32 + lq;
    const bool qvalid = myrow < qlen;
    // index of this row in the [.][H][N] (or [tokens][H]) row arrays
    const size_t rowidx = PK ? (size_t)(cub + myrow) * a.H + h : ((size_t)b * a.H + h) * N + myrow;
    bf16x8 qf[KS], dof[KS];
    {
        const __bf16 *qp = (const __bf16 *)a.q + rowidx * D;
        const __bf16 *dp = (const __bf16 *)a.dout + rowidx * D;
#pragma unroll
        for (int ks = 0; ks < KS; ks++) {
            const u32x4 z = {0, 0, 0, 0};
            qf[ks] = __builtin_bit_cast(bf16x8, (myrow < nrows) ? ld16(qp + ks * 16 + hh * 8) : z);
            dof[ks] = __builtin_bit_cast(bf16x8, (myrow < nrows) ? ld16(dp + ks * 16 + hh * 8) : z);
        }
    }
    // D = <dO, O> of this row: each lane of the pair (l, l^32) holds half of
    // the row; the dk/dv kernel (launched after this one) reads it back
    float Dr;
    {
        const __bf16 *op = (const __bf16 *)a.o + rowidx * D;
        float acc = 0.f;
#pragma unroll
        for (int ks = 0; ks < KS; ks++) {
            const u32x4 z = {0, 0, 0, 0};
            const bf16x8 of =
                __builtin_bit_cast(bf16x8, (myrow < nrows) ? ld16(op + ks * 16 + hh * 8) : z);
#pragma unroll
            for (int t = 0; t < 8; t++) acc = fmaf((float)of[t], (float)dof[ks][t], acc);
        }
        const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(acc), __float_as_uint(acc),
                                                        false, false);
        Dr = __uint_as_float(r[0]) + __uint_as_float(r[1]);
        if (myrow < nrows && hh == 0) a.dvec[rowidx] = Dr;
        if (!qvalid) Dr = 0.f;
    }
    const float c2 = a.scale * LOG2E;
    const float lse2 = qvalid ? a.lse[rowidx] * LOG2E : 0.f;

    const size_t kvo = PK ? ((size_t)cub * a.Hkv + g) * D : ((size_t)b * a.Hkv + g) * N * D;
    const __bf16 *kb = (const __bf16 *)a.k + kvo;
    const __bf16 *vb = (const __bf16 *)a.v + kvo;
    const int krsb = PK ? a.Hkv * ROWB : ROWB;  // bytes between key rows
    auto issue = [&](int kt, char *dst) __attribute__((always_inline)) {
        stage_rows<D, NW>(kb, kt * BN, nrows, krsb, dst, wave, lane);
        stage_rows<D, NW>(vb, kt * BN, nrows, krsb, dst + TILEB, wave, lane);
    };

    f32x16 dqacc[DB];
#pragma unroll
    for (int db = 0; db < DB; db++)
#pragma unroll
        for (int e = 0; e < 16; e++) dqacc[db][e] = 0.f;

    const int e0 = a.row_ptr[b * nqt + qt], e1 = a.row_ptr[b * nqt + qt + 1];
    const int tr_j = lane & 15;
    const int tr_row = 4 * hh + (tr_j >> 2);
    const int tr_col = ((lane >> 4) & 1) * 16 + 4 * (tr_j & 3);

    // CSR columns travel one tile ahead of their use, in vector registers
    // (loaded at an address the compiler cannot prove uniform, lz an opaque
    // 0), so that no tile waits at its barrier for a global load; see the
    // forward tile kernel
    int lz;
    asm volatile("v_mov_b32 %0, 0" : "=v"(lz));
    int v_col = 0, v_col1 = 0;
    if (e1 > e0) {
        v_col = a.col[e0 + lz];
        v_col1 = (e0 + 1 < e1) ? a.col[e0 + 1 + lz] : 0;
    }
    auto tile = [&](int e, const char *cur, char *nxt) __attribute__((always_inline)) {
        const int kt = __builtin_amdgcn_readfirstlane(v_col);
        const int kt1 = __builtin_amdgcn_readfirstlane(v_col1);
        __syncthreads();
        if (e + 1 < e1) issue(kt1, nxt);
        v_col = v_col1;
        v_col1 = (e + 2 < e1) ? a.col[e + 2 + lz] : 0;
        const char *ksm = cur;
        const char *vsm = cur + TILEB;
        // visible keys of this lane's row inside the tile: [a1, b1] (tile-local)
        const int base = kt * BN;
        int a1 = myrow - a.W + 1 - base, b1 = min(myrow, qlen - 1) - base;
        if (!qvalid) b1 = -1;
        a1 = max(a1, 0);
        b1 = min(b1, BN - 1);
        const bool empty = b1 < a1;
        const int L1 = empty ? -(1 << 20) : a1 - 4 * hh;
        const uint32_t n1 = empty ? 0u : (uint32_t)(b1 - a1);
        // attention sinks: keys 0 .. n_sink-1 (a second interval)
        int a2 = -base, b2 = min(a.n_sink - 1, min(myrow, qlen - 1)) - base;
        if (!qvalid || a.n_sink <= base) b2 = -1;
        a2 = max(a2, 0);
        b2 = min(b2, BN - 1);
        const bool empty2 = b2 < a2;
        const int L2 = (!SK || empty2) ? -(1 << 20) : a2 - 4 * hh;
        const uint32_t n2 = (!SK || empty2) ? 0u : (uint32_t)(b2 - a2);

        // the two 32-key halves one after the other (a loop, not unrolled): S,
        // dP and dS of one half are live at a time, which keeps the kernel
        // within the 256 registers of two waves per SIMD
#pragma unroll 1
        for (int kb2 = 0; kb2 < 2; kb2++) {
            f32x16 s, dp;
#pragma unroll
            for (int e2 = 0; e2 < 16; e2++) {
                s[e2] = 0.f;
                dp[e2] = 0.f;
            }
#pragma unroll
            for (int ks = 0; ks < KS; ks++) {
                s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(row_frag<D>(ksm, kb2 * 32, lq, hh, ks),
                                                            qf[ks], s, 0, 0, 0);
                dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(row_frag<D>(vsm, kb2 * 32, lq, hh, ks),
                                                             dof[ks], dp, 0, 0, 0);
            }
            // dS^T packed as B operands: dsk[s2] for 16-key step 2*kb2 + s2
            // (key 16kk + 8r + 4hh + t)
            bf16x8 dsk[2];
#pragma unroll
            for (int s2 = 0; s2 < 2; s2++)
#pragma unroll
                for (int r = 0; r < 2; r++)
#pragma unroll
                    for (int t = 0; t < 4; t++) {
                        const int e2 = (2 * s2 + r) * 4 + t;
                        const int c = kb2 * 32 + 8 * (2 * s2 + r) + t;  // minus 4hh, see L1
                        const bool vis = ((uint32_t)(c - L1) <= n1) | ((uint32_t)(c - L2) <= n2);
                        const float p =
                            vis ? __builtin_amdgcn_exp2f(fmaf(s[e2], c2, -lse2)) : 0.f;
                        dsk[s2][4 * r + t] = (__bf16)(p * (dp[e2] - Dr));
                    }
            // every K^T fragment of this half's dQ MFMAs before the first of them
            // (left to itself the compiler reads each pair just before its MFMA,
            // which then waits out the LDS latency)
            bf16x8 ktf[2][DB];
#pragma unroll
            for (int s2 = 0; s2 < 2; s2++)
#pragma unroll
                for (int db = 0; db < DB; db++)
                    ktf[s2][db] = tr_frag<D>(ksm, 2 * kb2 + s2, db, tr_row, tr_col);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int s2 = 0; s2 < 2; s2++)
#pragma unroll
                for (int db = 0; db < DB; db++)
                    dqacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ktf[s2][db], dsk[s2],
                                                                        dqacc[db], 0, 0, 0);
        }
    };
    if (e1 > e0) issue(__builtin_amdgcn_readfirstlane(v_col), stage0);
    for (int e = e0; e < e1; e += 2) {
        tile(e, stage0, stage1);
        if (e + 1 < e1) tile(e + 1, stage1, stage0);
    }

    if (myrow < nrows) {
        __bf16 *op = (__bf16 *)a.dq + rowidx * D;
#pragma unroll
        for (int db = 0; db < DB; db++)
#pragma unroll
            for (int i = 0; i < 4; i++) {
                bf16x4 w;
#pragma unroll
                for (int j = 0; j < 4; j++) w[j] = (__bf16)(dqacc[db][i * 4 + j] * a.scale);
                *(bf16x4 *)(op + db * 32 + 8 * i + 4 * hh) = w;
            }
    }
}

// ---------------------------------------------------------------------------
// Barrier for a hand-off through LDS only: waits for this wave's LDS writes,
// not for its global loads in flight (the next step's staging continues).
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

template <int D, bool PK>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2)))
void dkdv_kernel(BwdArgs a) {
    constexpr int NW = 4, KS = D / 16, DB = D / 32, ROWB = D * 2, TILEB = BN * ROWB;
    // stage: [Q rows | dO rows | lse[64] | D[64]]
    __shared__ __attribute__((aligned(1024))) char stage0[2 * TILEB + 512];
    __shared__ __attribute__((aligned(1024))) char stage1[2 * TILEB + 512];
    // P of the current step, from the waves that compute it to the waves that
    // need it for dS: [key half][32-row block][lane][16 bf16]
    __shared__ __attribute__((aligned(16))) u32x4 xch[2][2][64][2];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    // role 0 waves hold K and compute S, P and dV; role 1 waves hold V and
    // compute dP, dS and dK; kh: which 32 keys of the tile
    const int role = wave >> 1, kh = wave & 1;
    const int lq = lane & 31, hh = lane >> 5;
    const int N = a.N, W = a.W;
    const int nkt = (N + BN - 1) / BN;
    const int L = xcd_deal(blockIdx.x, gridDim.x);
    const int kt = L % nkt, g = (L / nkt) % a.Hkv, b = L / (nkt * a.Hkv);
    const int G = a.H / a.Hkv;
    // rows (and keys) of this request that exist (all N when padded)
    const int cub = PK ? a.cu[b] : 0;
    const int nrows = PK ? a.cu[b + 1] - cub : N;
    const int qlen = PK ? nrows : (a.q_len ? a.q_len[b] : N);
    const int tq = a.tile_q;
    const int nqt = (N + tq - 1) / tq;

    const int mykey = kt * BN + kh * 32 + lq;
    // index of this key in the [.][Hkv][N] (or [tokens][Hkv]) row arrays
    const size_t keyidx =
        PK ? (size_t)(cub + mykey) * a.Hkv + g : ((size_t)b * a.Hkv + g) * N + mykey;
    bf16x8 op[KS];  // this lane's K row (role 0) or V row (role 1)
    {
        const __bf16 *src = (const __bf16 *)(role == 0 ? a.k : a.v) + keyidx * D;
#pragma unroll
        for (int ks = 0; ks < KS; ks++) {
            const u32x4 z = {0, 0, 0, 0};
            op[ks] = __builtin_bit_cast(bf16x8, (mykey < nrows) ? ld16(src + ks * 16 + hh * 8) : z);
        }
    }
    // visible query rows of this lane's key: [ka, kb_] (every later row for an
    // attention sink); empty if the key is padding
    const int ka = mykey, kb_ = (mykey < a.n_sink) ? qlen - 1 : min(mykey + W - 1, qlen - 1);
    const bool kempty = mykey >= qlen || kb_ < ka;
    const float c2 = a.scale * LOG2E;

    f32x16 acc[DB];  // dV^T (role 0) or dK^T (role 1) of this lane's key
#pragma unroll
    for (int db = 0; db < DB; db++)
#pragma unroll
        for (int e = 0; e < 16; e++) acc[db][e] = 0.f;

    // steps: (query head h, 64-row block s0) over query tiles whose class-grid
    // entry for this key tile is live, rows kt*64 .. kt*64+63+W-1 at most
    const int qt_lo = (kt * BN) / tq;
    const int qt_hi = (kt * BN < a.n_sink) ? nqt - 1
                                           : (int)min((long)nqt - 1, ((long)kt * BN + BN - 2 + W) / tq);
    const int spt = (tq + BN - 1) / BN;  // 64-row steps per query tile
    const uint8_t *clsb = a.cls + (size_t)b * nqt * nkt;
    const int qtn = qt_hi - qt_lo + 1;
    // the class-grid column of this key tile over [qt_lo, qt_hi], read once
    // into two wave-wide masks (live, partial) when it spans at most 64 query
    // tiles; the step loop then never waits on a global load for it
    const bool inmask = qtn <= 64;
    uint64_t m_live = 0, m_part = 0;
    if (inmask) {
        const int c = lane < qtn ? clsb[(size_t)(qt_lo + lane) * nkt + kt] : 0;
        m_live = __ballot(c != 0);
        m_part = __ballot(c == 2);
    }
    auto cls_of = [&](int qt) __attribute__((always_inline)) -> int {
        if (inmask) {
            const int r = qt - qt_lo;
            return ((m_live >> r) & 1) ? (((m_part >> r) & 1) ? 2 : 1) : 0;
        }
        return clsb[(size_t)qt * nkt + kt];
    };
    // a step's position: head h of the group, query tile qt_lo + q, 64-row
    // block s of it (s fastest, then q, then h); advanced by increments, so
    // that the scalar code divides by nothing
    struct Pos {
        int h, q, s;
    };
    auto next = [&](Pos p) __attribute__((always_inline)) -> Pos {
        if (++p.s == spt) {
            p.s = 0;
            if (++p.q == qtn) {
                p.q = 0;
                p.h++;
            }
        }
        return p;
    };
    auto live_from = [&](Pos p) __attribute__((always_inline)) -> Pos {
        for (; p.h < G; p = next(p)) {
            const int qt = qt_lo + p.q;
            if (cls_of(qt) != 0 && qt * tq + p.s * BN < nrows) break;
        }
        return p;
    };
    auto step_rows = [&](Pos p, int &hq, int &s0, bool &part) __attribute__((always_inline)) {
        const int qt = qt_lo + p.q;
        hq = g * G + p.h;
        s0 = qt * tq + p.s * BN;
        // a full class counts only in-range pairs: steps or key tiles cut by
        // the array edge are masked too
        part = cls_of(qt) == 2 || s0 + BN > nrows || kt * BN + BN > nrows;
    };
    auto issue = [&](Pos t, char *dst) __attribute__((always_inline)) {
        int hq, s0;
        bool part;
        step_rows(t, hq, s0, part);
        // row 0 of head hq in the row arrays; rows are H apart when packed
        const size_t rb = PK ? (size_t)cub * a.H + hq : ((size_t)b * a.H + hq) * N;
        const int rst = PK ? a.H : 1;
        stage_rows<D, NW>((const __bf16 *)a.q + rb * D, s0, nrows, rst * ROWB, dst, wave, lane);
        stage_rows<D, NW>((const __bf16 *)a.dout + rb * D, s0, nrows, rst * ROWB, dst + TILEB,
                          wave, lane);
        // row values of the 64 rows (zeros past the data, which is masked)
        if (wave < 2) {
            const float *src = (wave == 0) ? (a.lse + rb) : (a.dvec + rb);
            stage_vals(src, s0 + lane, nrows, rst, dst + 2 * TILEB + wave * 256);
        }
    };

    const int tr_j = lane & 15;
    const int tr_row = 4 * hh + (tr_j >> 2);
    const int tr_col = ((lane >> 4) & 1) * 16 + 4 * (tr_j & 3);

    auto step = [&](Pos t, const char *cur, char *nxt, Pos tnext) {
        __syncthreads();
        if (tnext.h < G) issue(tnext, nxt);
        int hq, s0;
        bool part;
        step_rows(t, hq, s0, part);
        (void)hq;
        const char *qsm = cur;
        const char *dsm = cur + TILEB;
        const float *lsm = (const float *)(cur + 2 * TILEB);
        const float *Dsm = lsm + 64;
        // lane constants of the LDS addresses, made opaque per step (lzs is an
        // opaque 0) so that the compiler recomputes each fragment address near
        // its read instead of keeping dozens of them live across the loop
        int lzs;
        asm volatile("v_mov_b32 %0, 0" : "=v"(lzs));
        const int lqs = lq + lzs, trr = tr_row + lzs, trc = tr_col + lzs;
        // carried across the hand-off, 16 dwords of bf16 pairs: role 0 its P of
        // both 32-row blocks, role 1 its dP - D of both blocks (rounded to bf16
        // like the dS it becomes: a relative error of the same size)
        f32x16 hold;
        if (role == 0) {
            // S = Q K^T, P = exp(S - lse) (0 where masked), handed to role 1
#pragma unroll
            for (int rb = 0; rb < 2; rb++) {
                __builtin_amdgcn_sched_barrier(0);
                f32x16 s;
#pragma unroll
                for (int e2 = 0; e2 < 16; e2++) s[e2] = 0.f;
#pragma unroll
                for (int ks = 0; ks < KS; ks++)
                {
                    s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(row_frag<D>(qsm, rb * 32, lqs, hh, ks),
                                                                op[ks], s, 0, 0, 0);
                    if (ks & 1) __builtin_amdgcn_sched_barrier(0);
                }
                // rows of C element 4i+j: q = s0 + rb*32 + 8i + 4hh + j
                const int qb = s0 + rb * 32 + 4 * hh;
                const int L1 = kempty ? -(1 << 20) : ka - qb;
                const uint32_t n1 = kempty ? 0u : (uint32_t)(kb_ - ka);
                bf16x8 pk[2];
#pragma unroll
                for (int i = 0; i < 4; i++) {
                    const f32x4 lse4 = *(const f32x4 *)(lsm + rb * 32 + 8 * i + 4 * hh);
#pragma unroll
                    for (int j = 0; j < 4; j++) {
                        const int c = 8 * i + j;
                        const bool vis = !part || ((uint32_t)(c - L1) <= n1);
                        const float p =
                            vis ? __builtin_amdgcn_exp2f(fmaf(s[4 * i + j], c2, -lse4[j] * LOG2E))
                                : 0.f;
                        // k index hh*8 + 4r + t of 16-row step kk = q 16kk + 8r + 4hh + t
                        pk[i >> 1][4 * (i & 1) + j] = (__bf16)p;
                    }
                }
                const u32x4 w0 = __builtin_bit_cast(u32x4, pk[0]);
                const u32x4 w1 = __builtin_bit_cast(u32x4, pk[1]);
                xch[kh][rb][lane][0] = w0;
                xch[kh][rb][lane][1] = w1;
#pragma unroll
                for (int e2 = 0; e2 < 4; e2++) {
                    hold[rb * 8 + e2] = __uint_as_float(w0[e2]);
                    hold[rb * 8 + 4 + e2] = __uint_as_float(w1[e2]);
                }
            }
        } else {
            // dP = dO V^T
#pragma unroll
            for (int rb = 0; rb < 2; rb++) {
                __builtin_amdgcn_sched_barrier(0);
                f32x16 dp;
#pragma unroll
                for (int e2 = 0; e2 < 16; e2++) dp[e2] = 0.f;
#pragma unroll
                for (int ks = 0; ks < KS; ks++)
                {
                    dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                        row_frag<D>(dsm, rb * 32, lqs, hh, ks), op[ks], dp, 0, 0, 0);
                    if (ks & 1) __builtin_amdgcn_sched_barrier(0);
                }
                bf16x8 dd[2];
#pragma unroll
                for (int i = 0; i < 4; i++) {
                    const f32x4 D4 = *(const f32x4 *)(Dsm + rb * 32 + 8 * i + 4 * hh);
#pragma unroll
                    for (int j = 0; j < 4; j++) dd[i >> 1][4 * (i & 1) + j] = (__bf16)(dp[4 * i + j] - D4[j]);
                }
                const u32x4 w0 = __builtin_bit_cast(u32x4, dd[0]);
                const u32x4 w1 = __builtin_bit_cast(u32x4, dd[1]);
#pragma unroll
                for (int e2 = 0; e2 < 4; e2++) {
                    hold[rb * 8 + e2] = __uint_as_float(w0[e2]);
                    hold[rb * 8 + 4 + e2] = __uint_as_float(w1[e2]);
                }
            }
        }
        lds_barrier();
        if (role == 0) {
            // dV^T += dO^T P
#pragma unroll
            for (int rb = 0; rb < 2; rb++) {
                u32x4 w0, w1;
#pragma unroll
                for (int e2 = 0; e2 < 4; e2++) {
                    w0[e2] = __float_as_uint(hold[rb * 8 + e2]);
                    w1[e2] = __float_as_uint(hold[rb * 8 + 4 + e2]);
                }
                const bf16x8 pk[2] = {__builtin_bit_cast(bf16x8, w0), __builtin_bit_cast(bf16x8, w1)};
#pragma unroll
                for (int kk = 0; kk < 2; kk++)
#pragma unroll
                    for (int db = 0; db < DB; db++) {
                        acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                            tr_frag<D>(dsm + rb * 32 * ROWB, kk, db, trr, trc), pk[kk],
                            acc[db], 0, 0, 0);
                        if (db & 1) __builtin_amdgcn_sched_barrier(0);
                    }
            }
        } else {
            // dS = P (dP - D), dK^T += Q^T dS
#pragma unroll
            for (int rb = 0; rb < 2; rb++) {
                const bf16x8 pk[2] = {__builtin_bit_cast(bf16x8, xch[kh][rb][lane][0]),
                                      __builtin_bit_cast(bf16x8, xch[kh][rb][lane][1])};
                u32x4 w0, w1;
#pragma unroll
                for (int e2 = 0; e2 < 4; e2++) {
                    w0[e2] = __float_as_uint(hold[rb * 8 + e2]);
                    w1[e2] = __float_as_uint(hold[rb * 8 + 4 + e2]);
                }
                const bf16x8 dd[2] = {__builtin_bit_cast(bf16x8, w0), __builtin_bit_cast(bf16x8, w1)};
                bf16x8 dsk[2];
#pragma unroll
                for (int x = 0; x < 2; x++)
#pragma unroll
                    for (int t = 0; t < 8; t++)
                        dsk[x][t] = (__bf16)((float)pk[x][t] * (float)dd[x][t]);
#pragma unroll
                for (int kk = 0; kk < 2; kk++)
#pragma unroll
                    for (int db = 0; db < DB; db++) {
                        acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                            tr_frag<D>(qsm + rb * 32 * ROWB, kk, db, trr, trc), dsk[kk],
                            acc[db], 0, 0, 0);
                        if (db & 1) __builtin_amdgcn_sched_barrier(0);
                    }
            }
        }
    };
    Pos t = live_from(Pos{0, 0, 0});
    if (t.h < G) issue(t, stage0);
    while (t.h < G) {
        const Pos t1 = live_from(next(t));
        step(t, stage0, stage1, t1);
        if (t1.h >= G) break;
        const Pos t2 = live_from(next(t1));
        step(t1, stage1, stage0, t2);
        t = t2;
    }

    if (mykey < nrows) {
        // role 0 writes dV, role 1 dK (scaled)
        __bf16 *dst = (__bf16 *)(role == 0 ? a.dv : a.dk) + keyidx * D;
        const float f = role == 0 ? 1.f : a.scale;
#pragma unroll
        for (int db = 0; db < DB; db++)
#pragma unroll
            for (int i = 0; i < 4; i++) {
                bf16x4 w;
#pragma unroll
                for (int j = 0; j < 4; j++) w[j] = (__bf16)(acc[db][i * 4 + j] * f);
                *(bf16x4 *)(dst + db * 32 + 8 * i + 4 * hh) = w;
            }
    }
}

template <int D, bool PK>
hipError_t launch_d(const BwdArgs &a, hipStream_t s) {
    hipError_t e;
    const int NWq = a.tile_q == 128 ? 4 : 2;
    const long nqt = (a.N + 32L * NWq - 1) / (32L * NWq);
    const long nkt = (a.N + BN - 1) / BN;
    const long gq = nqt * a.H * a.B, gk = nkt * a.Hkv * a.B;
    if (gq > 0x7fffffffL || gk > 0x7fffffffL) return hipErrorInvalidConfiguration;
    if (NWq == 4 && a.n_sink > 0)
        hipLaunchKernelGGL((dq_kernel<D, 4, PK, true>), dim3((unsigned)gq), dim3(256), 0, s, a);
    else if (NWq == 4)
        hipLaunchKernelGGL((dq_kernel<D, 4, PK, false>), dim3((unsigned)gq), dim3(256), 0, s, a);
    else if (a.n_sink > 0)
        hipLaunchKernelGGL((dq_kernel<D, 2, PK, true>), dim3((unsigned)gq), dim3(128), 0, s, a);
    else
        hipLaunchKernelGGL((dq_kernel<D, 2, PK, false>), dim3((unsigned)gq), dim3(128), 0, s, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL((dkdv_kernel<D, PK>), dim3((unsigned)gk), dim3(256), 0, s, a);
    return hipGetLastError();
}

}  // namespace

bool bwd_bf16_supported(const BwdArgs &a) {
    return a.bf16 && (a.d == 64 || a.d == 128) && a.tile_k == BN &&
           (a.tile_q == 64 || a.tile_q == 128);
}

hipError_t launch_bwd_bf16(const BwdArgs &a, hipStream_t s) {
    if (a.cu) return a.d == 128 ? launch_d<128, true>(a, s) : launch_d<64, true>(a, s);
    return a.d == 128 ? launch_d<128, false>(a, s) : launch_d<64, false>(a, s);
}

}  // namespace swa
