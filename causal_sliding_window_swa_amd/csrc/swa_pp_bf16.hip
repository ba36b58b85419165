// swa_pp_bf16.hip -- bf16 forward of causal sliding-window attention for
// 256-row query tiles (head dim 128, 64-key tiles) on gfx950: the full-sequence
// forward and the chunked prefill over a ring cache, with the same results as
// the 128-row tile loop.
//
// What it computes ("Weight sparsity vs attention sparsity" (AI-infra KB) §03;
// "LLMs from scratch" ch.10 §10.1-§10.2): the query at logical position t
// attends over keys at positions t-W+1 .. t, softmax normalised over exactly
// those keys; a workgroup visits only the key tiles its metadata row lists
// and masks per element only inside partial tiles (§04 of the AI-infra page).
//
// Schedule.  One workgroup of eight waves per (256-row query tile, head,
// request); waves 0-3 (group 0) own rows 0-127, waves 4-7 (group 1) rows
// 128-255, 32 rows per wave, so each SIMD runs one wave of each group.  Every
// wave walks the same key tiles; step j of a wave is
//   MFMA part:  the loads of its share of K tile j+2 and V tile j+1, then
//               O^T += V^T P^T of tile j-1 and S^T = K Q^T of tile j
//   VALU part:  P = exp2(S c - m_ref) of tile j (the softmax) and the
//               masking state of tile j+1
// with one workgroup barrier per step: group 0 meets it after its VALU part,
// group 1 after its MFMA part.  Between two barriers group 0 runs MFMA part
// j+1 and then VALU part j+1 while group 1 runs VALU part j and then MFMA
// part j+1, so one wave of each SIMD issues matrix work while the other
// issues the softmax's vector work, which the SIMD overlaps (with two
// independent workgroups per CU the two waves' phases drift into line and
// overlap little); the point where the two swap floats, so a part that runs
// long on one SIMD does not hold up the other seven waves.
// The per-wave order of the work (QK, softmax, PV, tile after tile) is that of
// the 128-row loop, so are the fragments, the swizzles, the reference-max
// softmax with its rare-case rescale and the masking; only the placement of
// the barriers and the staging depth differ.
//
// Staging.  K and V tiles go from HBM straight to LDS (buffer_load_dwordx4 ...
// lds) into four stages each (K tile t in stage t % 4, V likewise; 128 KB,
// one workgroup per CU).  Group g loads rows 32g .. 32g+31 of each tile.
// Between barriers p and p+1 both groups run MFMA part p, which reads K tile
// p and V tile p-1 and loads K tile p+2 (the stage of K tile p-2) and V tile
// p+1 (that of V tile p-3); K tile p is also read by the rare-case recompute
// of VALU part p (group 0 in the same interval, group 1 in the next).  So a
// stage is written only after every read of its previous tile has passed a
// barrier.  Each wave waits for its loads of step p-1 (vmcnt, leaving those
// of step p in flight) before the barrier that ends its step p, so every
// tile is in LDS one barrier before the first MFMA part that reads it.  The
// barriers carry no memory fence (a fence would wait for every load in
// flight); these waits and the program order of each wave's LDS reads before
// its barrier are what the staging relies on.  Every step issues its loads,
// past the last tile from an offset the buffer range check turns into zeros,
// so that the number of loads in flight is the same on every path.
//
// Metadata.  The row's tile columns and classes are read with scalar loads at
// the end of a VALU part for the next step (their wait then falls on the first
// LDS wait of the MFMA part, which waits anyway).  The masking intervals of a
// partial tile j+1 are formed at the end of the VALU part of step j; a half
// that every row of the wave sees whole is left unmasked, and one that no row
// of it sees is computed and masked like the rest (straight-line code
// schedules better than the skip, and P is exactly 0 there), while a tile
// none of its rows sees is skipped whole.
#include <hip/hip_runtime.h>
#include <math.h>

#include "ring_state.h"
#include "swa_internal.h"

namespace swa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef __attribute__((address_space(3))) void lds_void;

constexpr int BN = 64;    // keys per tile
constexpr int D = 128;    // head dim
constexpr int KS = D / 16, DB = D / 32, ROWB = D * 2, TILEB = BN * ROWB;
constexpr int HALFB = TILEB / 2;  // the 32 rows one group loads
constexpr float LOG2E = 1.4426950408889634f;
constexpr float P_HI = 4294967296.0f;            // 2^32: tile sums above this rescale
constexpr float P_LO = 2.3283064365386963e-10f;  // 2^-32: below this, before a real max

__device__ __forceinline__ u32x4 ld16(const void *p) { return *(const u32x4 *)p; }

// Combine lane l with lane l^32 (v_permlane32_swap: no LDS round trip).
__device__ __forceinline__ float half_swap_max(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                    false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float half_swap_sum(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                    false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Workgroup barrier without a memory fence (see the header): the compiler
// keeps memory operations on their side of it, the hardware only waits for
// the other waves.
__device__ __forceinline__ void step_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// Workgroup p of T runs logical tile L: XCD x = p % 8 gets the contiguous
// logical range [start_x, start_x + count_x) in dispatch order.
__device__ __forceinline__ int xcd_remap(int p, int T) {
    const int x = p & 7, i = p >> 3, q = T >> 3, r = T & 7;
    return x * q + (x < r ? x : r) + i;
}

// The dealing of the 128-row loop with chunks of 32 workgroups (one
// workgroup per CU, 32 CUs per XCD): in rounds 4R .. 4R+3 XCD x runs the
// chunks of run 8R + (x + R) % 8, so the workgroups an XCD runs together are
// neighbours in the logical order (shared K/V tiles in its L2) and every XCD
// draws its work from all parts of the order.  A tail of T mod 1024 keeps
// contiguous ranges.  A bijection on [0, T).
__device__ __forceinline__ int xcd_deal(int p, int T) {
    constexpr int C = 32, S = 4;
    const int Tm = T / (8 * C * S) * (8 * C * S);
    if (p < Tm) {
        const int x = p & 7, i = p >> 3, r = i / C, o = i % C;
        const int R = r / S, sub = r % S;
        return ((R * 8 + ((x + R) & 7)) * S + sub) * C + o;
    }
    return Tm + xcd_remap(p - Tm, T - Tm);
}

// Per-request ring/metadata constants.
struct KeyPos {
    int nq, W, nst, nrt, qlen, rs, cl, np;
};

// Visibility of one tile for this lane's query: the tile keys it sees form
// one interval [a1, b1] of tile-local indices, plus [a2, b2] in a tile that
// holds the ring's wrap point or the attention sinks (empty when b < a).
struct TileMask {
    int L1, L2;           // interval starts relative to the lane's first key (masked offsets)
    uint32_t n1, n2;      // interval lengths - 1 (unsigned compare)
    int a1, b1, a2, b2;   // clamped intervals (for the whole-half test)
    bool two;
};

template <int MODE, bool PK>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2)))
void pp_kernel(AttnArgs a) {
    __shared__ __attribute__((aligned(1024))) char K0[TILEB];
    __shared__ __attribute__((aligned(1024))) char K1[TILEB];
    __shared__ __attribute__((aligned(1024))) char K2[TILEB];
    __shared__ __attribute__((aligned(1024))) char K3[TILEB];
    __shared__ __attribute__((aligned(1024))) char V0[TILEB];
    __shared__ __attribute__((aligned(1024))) char V1[TILEB];
    __shared__ __attribute__((aligned(1024))) char V2[TILEB];
    __shared__ __attribute__((aligned(1024))) char V3[TILEB];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int grp = wave >> 2, wg = wave & 3;
    const int lq = lane & 31, hh = lane >> 5;
    const int nq = a.nq;
    const int nqt = (nq + 255) / 256;
    const int L = xcd_deal(blockIdx.x, gridDim.x);
    const int G = a.H / a.Hkv;
    const int h_in = L % G, qt = (L / G) % nqt, g = (L / (G * nqt)) % a.Hkv;
    const int b = L / (G * nqt * a.Hkv);
    const int h = g * G + h_in;

    KeyPos kp;
    kp.nq = nq;
    kp.W = a.W;
    kp.nst = (MODE == 1 && a.n_sink > 0) ? (a.n_sink + BN - 1) / BN : 0;
    kp.nrt = (MODE == 1) ? a.W / BN : 0;
    const int cub = PK ? a.cu[b] : 0;
    const int nrows = PK ? a.cu[b + 1] - cub : nq;
    kp.qlen = PK ? nrows : ((MODE == 0) ? (a.q_len ? a.q_len[b] : nq) : nq);
    kp.rs = (MODE == 1) ? a.ring_start[b] : 0;
    kp.cl = (MODE == 1) ? a.cache_len[b] : 0;
    kp.np = (MODE == 1) ? a.next_pos[b] : 0;
    const int qlen = kp.qlen;
    const int qbase = (MODE == 1) ? kp.np : 0;

    // ---- K/V sources (rows past the data read as zeros through the buffer
    // range check: finite, and always masked)
    const size_t kvh = (size_t)b * a.Hkv + g;
    const int RSB = PK ? a.Hkv * ROWB : ROWB;
    const __bf16 *klin = (const __bf16 *)a.k + (PK ? ((size_t)cub * a.Hkv + g) * D
                                                   : kvh * (size_t)nq * D);
    const __bf16 *vlin = (const __bf16 *)a.v + (PK ? ((size_t)cub * a.Hkv + g) * D
                                                   : kvh * (size_t)nq * D);
    const __bf16 *kring = (MODE == 1) ? (const __bf16 *)a.kc + kvh * (size_t)a.W * D : nullptr;
    const __bf16 *vring = (MODE == 1) ? (const __bf16 *)a.vc + kvh * (size_t)a.W * D : nullptr;
    // logical 16-byte chunk c of row r sits at physical chunk c ^ swz(r): K is
    // read as rows, V by transposing reads; both patterns conflict-free
    auto kswz = [](int r) { return r & 15; };
    auto vswz = [](int r) { return (r & 3) << 2; };

    // this wave's two 1 KB loads of its group's 32 rows of a tile
    uint32_t koff[2], voff[2];
    int lds_off[2];
#pragma unroll
    for (int i = 0; i < 2; i++) {
        const int ins = grp * 8 + wg * 2 + i;  // 4 rows per load
        const int r = ins * 4 + lane / 16, pch = lane % 16;
        koff[i] = (uint32_t)(r * RSB + (pch ^ kswz(r)) * 16);
        voff[i] = (uint32_t)(r * RSB + (pch ^ vswz(r)) * 16);
        lds_off[i] = ins * 1024;
    }
    const int lin_bytes = nrows > 0 ? (nrows - 1) * RSB + ROWB : 0;
    const __amdgpu_buffer_rsrc_t klr =
        __builtin_amdgcn_make_buffer_rsrc((void *)klin, 0, lin_bytes, 0x00020000);
    const __amdgpu_buffer_rsrc_t vlr =
        __builtin_amdgcn_make_buffer_rsrc((void *)vlin, 0, lin_bytes, 0x00020000);
    __amdgpu_buffer_rsrc_t krr = klr, vrr = vlr, ksr = klr, vsr = vlr;
    if (MODE == 1) {
        krr = __builtin_amdgcn_make_buffer_rsrc((void *)kring, 0, a.W * ROWB, 0x00020000);
        vrr = __builtin_amdgcn_make_buffer_rsrc((void *)vring, 0, a.W * ROWB, 0x00020000);
        if (a.n_sink > 0) {
            const size_t sko = kvh * (size_t)a.n_sink * D;
            ksr = __builtin_amdgcn_make_buffer_rsrc((void *)((const __bf16 *)a.sk + sko), 0,
                                                    a.n_sink * ROWB, 0x00020000);
            vsr = __builtin_amdgcn_make_buffer_rsrc((void *)((const __bf16 *)a.sv + sko), 0,
                                                    a.n_sink * ROWB, 0x00020000);
        }
    }
    auto ld2 = [&](__amdgpu_buffer_rsrc_t r, const uint32_t *off, int base, char *dst)
        __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < 2; i++)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void *)(dst + lds_off[i]), 16,
                                                     base + (int)off[i], 0, 0, 0);
    };
    // key tile kt (-1: none, zeros from past the linear rows) into dst; one
    // uniform branch per segment (selecting descriptors by value would put
    // them in scratch memory)
    auto load_k = [&](int kt, char *dst) __attribute__((always_inline)) {
        const int kr = kt - kp.nst;
        if (kt < 0)
            ld2(klr, koff, lin_bytes, dst);
        else if (MODE == 1 && kt < kp.nst)
            ld2(ksr, koff, kt * BN * ROWB, dst);
        else if (MODE == 1 && kr < kp.nrt)
            ld2(krr, koff, kr * BN * ROWB, dst);
        else
            ld2(klr, koff, (kr - kp.nrt) * BN * RSB, dst);
    };
    auto load_v = [&](int kt, char *dst) __attribute__((always_inline)) {
        const int kr = kt - kp.nst;
        if (kt < 0)
            ld2(vlr, voff, lin_bytes, dst);
        else if (MODE == 1 && kt < kp.nst)
            ld2(vsr, voff, kt * BN * ROWB, dst);
        else if (MODE == 1 && kr < kp.nrt)
            ld2(vrr, voff, kr * BN * ROWB, dst);
        else
            ld2(vlr, voff, (kr - kp.nrt) * BN * RSB, dst);
    };

    // ---- the row's key tiles
    // (read through the constant address space: the metadata does not change
    // during the launch, so the compiler may use scalar loads, which keep the
    // vector-memory count free for the K/V loads)
    typedef const __attribute__((address_space(4))) int32_t cint;
    const cint *rowp = (const cint *)a.row_ptr;
    const cint *colp = (const cint *)a.col;
    const int mrow = b * nqt + qt;
    const bool st_ok = MODE == 0 || ring_state_ok(kp.rs, kp.cl, kp.np, a.W, nq);
    const int e0 = rowp[mrow];
    const int T = st_ok ? rowp[mrow + 1] - e0 : 0;
    auto col_of = [&](int j) __attribute__((always_inline)) { return j < T ? colp[e0 + j] : -1; };
    // class byte of entry j, from the aligned dword that holds it (a dword
    // never crosses a page, so this reads no unmapped memory)
    const cint *clsp = (const cint *)((uintptr_t)a.col_cls & ~(uintptr_t)3);
    const int cls_sh = (int)((uintptr_t)a.col_cls & 3);
    // the dword holding the class of entry j (entries past the row: the last
    // one's) and the class taken from it
    auto cls_word = [&](int j) __attribute__((always_inline)) {
        return T > 0 ? clsp[(e0 + min(j, T - 1) + cls_sh) >> 2] : 0;
    };
    auto cls_from = [&](int w, int j) __attribute__((always_inline)) {
        return (w >> (((e0 + min(j, T - 1) + cls_sh) & 3) * 8)) & 0xff;
    };

    // ---- this wave's 32 query rows (B operand of S^T = K Q^T)
    const int row0 = qt * 256 + grp * 128 + wg * 32;
    const int myrow = row0 + lq;
    bf16x8 qf[KS];
    {
        const __bf16 *qp = (const __bf16 *)a.q +
                           (PK ? ((size_t)(cub + myrow) * a.H + h) * D
                               : (((size_t)b * a.H + h) * nq + myrow) * D);
#pragma unroll
        for (int ks = 0; ks < KS; ks++) {
            u32x4 x = (myrow < nrows) ? ld16(qp + ks * 16 + hh * 8) : u32x4{0, 0, 0, 0};
            qf[ks] = __builtin_bit_cast(bf16x8, x);
        }
    }

    // ---- prologue: this group's rows of K tiles 0 and 1 and V tile 0
    load_k(col_of(0), K0 + 0);
    load_k(col_of(1), K1);
    load_v(col_of(0), V0);

    // ---- running softmax state: lanes l and l^32 share query column lq
    const float c2 = a.scale * LOG2E;
    float m_ref = 0.f, l_run = 0.f;  // p = exp2(s*c2 - m_ref); O, l share m_ref
    bool guess = true;               // m_ref not yet taken from a real max
    f32x16 oacc[DB];
#pragma unroll
    for (int db = 0; db < DB; db++)
#pragma unroll
        for (int e = 0; e < 16; e++) oacc[db][e] = 0.f;
    const int qpos = qbase + myrow;
    const bool qvalid = myrow < qlen;

    const int kr_row = lq;
    const int tr_j = lane & 15;
    const int tr_row = 4 * hh + (tr_j >> 2);
    const int tr_col = ((lane >> 4) & 1) * 16 + 4 * (tr_j & 3);

    // Masking state of key tile kt (metadata class cls) for this wave: partial
    // (any masking), the lanes' intervals, and which 32-key halves any lane
    // of the wave sees.
    const int nlin_full = nrows / BN;  // linear tiles lying fully inside the data
    auto tile_state = [&](int kt, int cls, bool &partial, bool &live0, bool &live1, TileMask &m)
        __attribute__((always_inline)) {
        const int kr = kt - kp.nst;
        // a full tile (every row of the query tile sees every key) that lies
        // inside the data needs no intervals
        partial = (cls != 1) || (kr - kp.nrt) >= nlin_full;
        live0 = live1 = true;
        int a1 = 0, b1 = BN - 1, a2 = 0, b2 = -1;
        bool two = false;
        if (partial) {
            const int lo_pos = qpos - a.W + 1;
            if (MODE == 0) {
                const int base = kt * BN;
                a1 = lo_pos - base;
                b1 = min(qpos, qlen - 1) - base;
                if (a.n_sink > base) {
                    two = true;
                    a2 = -base;
                    b2 = min(a.n_sink - 1, min(qpos, qlen - 1)) - base;
                }
            } else if (kt < kp.nst) {
                a1 = -kt * BN;
                b1 = min(a.n_sink - 1, qpos) - kt * BN;
            } else if (kr < kp.nrt) {
                const int off = kp.np - kp.cl;
                const int rlo = max(0, max(lo_pos, a.n_sink) - off);
                const int rhi = min(kp.cl - 1, qpos - off);
                const int base = kr * BN - kp.rs;
                if (base < 0 && base + BN > 0) {
                    two = true;
                    a1 = rlo - base - a.W;
                    b1 = min(-base - 1, rhi - base - a.W);
                    a2 = max(-base, rlo - base);
                    b2 = rhi - base;
                } else {
                    const int rb = base < 0 ? base + a.W : base;
                    a1 = rlo - rb;
                    b1 = rhi - rb;
                }
            } else {
                const int t0 = (kr - kp.nrt) * BN;
                a1 = max(lo_pos, a.n_sink) - (kp.np + t0);
                b1 = min(qpos - kp.np, nq - 1) - t0;
            }
            if (!qvalid) {
                b1 = -1;
                b2 = -1;
            }
            a1 = max(a1, 0);
            b1 = min(b1, BN - 1);
            a2 = max(a2, 0);
            b2 = min(b2, BN - 1);
            bool lv[2];
#pragma unroll
            for (int kb = 0; kb < 2; kb++) {
                const bool o1 = a1 <= b1 && a1 <= kb * 32 + 31 && b1 >= kb * 32;
                const bool o2 = a2 <= b2 && a2 <= kb * 32 + 31 && b2 >= kb * 32;
                lv[kb] = __ballot(o1 || o2) != 0;
            }
            live0 = lv[0];
            live1 = lv[1];
            // a tile that every lane sees whole needs no mask
            bool whole = true;
#pragma unroll
            for (int kb = 0; kb < 2; kb++)
                whole = whole && ((a1 <= kb * 32 && b1 >= kb * 32 + 31) ||
                                  (two && a2 <= kb * 32 && b2 >= kb * 32 + 31));
            partial = __ballot(!whole) != 0;
        }
        const bool x1 = b1 < a1, x2 = !two || b2 < a2;
        m.L1 = x1 ? -(1 << 20) : a1 - 4 * hh;
        m.L2 = x2 ? -(1 << 20) : a2 - 4 * hh;
        m.n1 = x1 ? 0u : (uint32_t)(b1 - a1);
        m.n2 = x2 ? 0u : (uint32_t)(b2 - a2);
        m.a1 = a1;
        m.b1 = b1;
        m.a2 = a2;
        m.b2 = b2;
        m.two = two;
    };

    // S^T = K Q^T of the tile in ksm: rows = keys (A from LDS), columns = this
    // wave's queries; masked scores become -inf
    f32x16 sacc[2];
    auto scores = [&](const char *ksm, bool partial, const TileMask &m)
        __attribute__((always_inline)) {
        // both 32-key halves, also one that no row of the wave sees (it is
        // masked): straight-line code schedules better than skipping it
        bf16x8 kf[KS];
#pragma unroll
        for (int ks = 0; ks < KS; ks++) {
            const int c = (2 * ks + hh) ^ kswz(kr_row);
            kf[ks] = __builtin_bit_cast(bf16x8, ld16(ksm + kr_row * ROWB + c * 16));
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int ks = 0; ks < KS; ks++) {
            sacc[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[ks], qf[ks],
                                                              ks == 0 ? f32x16{} : sacc[0], 0, 0, 0);
            const int r = 32 + kr_row;
            const int c = (2 * ks + hh) ^ kswz(r);
            kf[ks] = __builtin_bit_cast(bf16x8, ld16(ksm + r * ROWB + c * 16));
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int ks = 0; ks < KS; ks++)
            sacc[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[ks], qf[ks],
                                                              ks == 0 ? f32x16{} : sacc[1], 0, 0, 0);
        if (partial) {
#pragma unroll
            for (int kb = 0; kb < 2; kb++) {
                // a half every row of the wave sees whole needs no mask
                const bool whole = (m.a1 <= kb * 32 && m.b1 >= kb * 32 + 31) ||
                                   (m.two && m.a2 <= kb * 32 && m.b2 >= kb * 32 + 31);
                if (__ballot(!whole) == 0) continue;
#pragma unroll
                for (int i = 0; i < 4; i++)
#pragma unroll
                    for (int j = 0; j < 4; j++) {
                        const int c = kb * 32 + 8 * i + j;
                        const bool vis = ((uint32_t)(c - m.L1) <= m.n1) |
                                         ((uint32_t)(c - m.L2) <= m.n2);
                        sacc[kb][4 * i + j] = vis ? sacc[kb][4 * i + j] : -INFINITY;
                    }
            }
        }
    };
    // P = exp2(S*c2 - m_ref) rounded to bf16 (pk[kk]: 16-key step kk) and the
    // tile's row sum of P
    bf16x8 pk[4];
    auto probs = [&]() __attribute__((always_inline)) -> float {
        float acc[4] = {0.f, 0.f, 0.f, 0.f};
        const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
        for (int kk = 0; kk < 4; kk++) {
            const int kb = kk >> 1, s2 = kk & 1;
#pragma unroll
            for (int t = 0; t < 4; t++) {
                pk[kk][t] = (__bf16)__builtin_amdgcn_exp2f(
                    fmaf(sacc[kb][(2 * s2) * 4 + t], c2, -m_ref));
                pk[kk][4 + t] = (__bf16)__builtin_amdgcn_exp2f(
                    fmaf(sacc[kb][(2 * s2 + 1) * 4 + t], c2, -m_ref));
            }
#pragma unroll
            for (int t = 0; t < 4; t++) {
                const bf16x2 pr = {pk[kk][2 * t], pk[kk][2 * t + 1]};
                acc[kk] = __builtin_amdgcn_fdot2_f32_bf16(pr, ones, acc[kk], false);
            }
        }
        return half_swap_sum((acc[0] + acc[1]) + (acc[2] + acc[3]));
    };
    // the softmax of the tile whose scores are in sacc (K still in ksm)
    auto softmax = [&](const char *ksm, bool partial, const TileMask &m)
        __attribute__((always_inline)) {
        float psum = probs();
        const bool lane_vis = !partial || (m.b1 >= m.a1) || (m.two && m.b2 >= m.a2);
        const bool rare = psum > P_HI || (guess && lane_vis && psum < P_LO);
        if (__ballot(rare) != 0) {
            // take the real max of this tile's scores and move the reference
            scores(ksm, partial, m);
            float mloc = -INFINITY;
#pragma unroll
            for (int kb = 0; kb < 2; kb++)
#pragma unroll
                for (int e2 = 0; e2 < 16; e2++) mloc = fmaxf(mloc, sacc[kb][e2]);
            mloc = half_swap_max(mloc) * c2;
            if (mloc != -INFINITY && (guess || mloc > m_ref)) {
                float mnew = mloc;
                if (guess && l_run > 0.f) mnew = fmaxf(mnew, m_ref + log2f(l_run));
                if (l_run > 0.f) {
                    const float alpha = __builtin_amdgcn_exp2f(m_ref - mnew);
                    l_run *= alpha;
#pragma unroll
                    for (int db = 0; db < DB; db++)
#pragma unroll
                        for (int e2 = 0; e2 < 16; e2++) oacc[db][e2] *= alpha;
                }
                m_ref = mnew;
                guess = false;
            }
            psum = probs();
        }
        l_run += psum;
    };
    // O^T += V^T P^T; the MFMA k index hh*8 + 4r + t of both operands stands
    // for tile key 16kk + 8r + 4hh + t
    // (all four key steps: P is exactly 0 on every masked key, so a half that
    // no row sees adds zeros)
    auto pv = [&](const char *vsm) __attribute__((always_inline)) {
#pragma unroll
        for (int kk = 0; kk < 4; kk++) {
#pragma unroll
            for (int db = 0; db < DB; db++) {
                i16x4 v2[2];
#pragma unroll
                for (int r = 0; r < 2; r++) {
                    const int row = kk * 16 + 8 * r + tr_row;
                    const int col = db * 32 + tr_col;
                    const int c = (col >> 3) ^ vswz(row);
                    const char *p = vsm + row * ROWB + c * 16 + (col & 7) * 2;
                    v2[r] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)p);
                }
                const u32x2 lo = __builtin_bit_cast(u32x2, v2[0]);
                const u32x2 hi = __builtin_bit_cast(u32x2, v2[1]);
                const u32x4 vv = {lo[0], lo[1], hi[0], hi[1]};
                oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, vv),
                                                                   pk[kk], oacc[db], 0, 0, 0);
            }
        }
    };

    // state of tile j (cur) and of tile j-1 (for its PV)
    bool cur_partial = false, cur_live0 = false, cur_live1 = false;
    TileMask cur_m;
    bool prv_run = false;
    if (T > 0)
        tile_state(col_of(0), cls_from(cls_word(0), 0), cur_partial, cur_live0, cur_live1, cur_m);
    // columns of the K tile and V tile the next MFMA part loads (the V tile
    // is also the one after the current tile) and that tile's class dword
    int colK = col_of(2), colV = col_of(1), clsN = cls_word(1);

    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();

    // step j: reads K tile j from Kc and V tile j-1 from Vp; loads K tile j+2
    // into Kd and V tile j+1 into Vd
    auto step = [&](int j, const char *Kc, const char *Vp, char *Kd, char *Vd)
        __attribute__((always_inline)) {
        // ---- MFMA part
        load_k(colK, Kd);
        load_v(colV, Vd);
        if (j > 0 && prv_run) pv(Vp);
        const bool run = j < T && (cur_live0 || cur_live1);
        if (run) scores(Kc, cur_partial, cur_m);
        if (grp == 1) {
            asm volatile("s_waitcnt vmcnt(4)" ::: "memory");  // loads of step j-1
            step_barrier();
        }
        // ---- VALU part
        __builtin_amdgcn_s_setprio(1);  // the softmax issues ahead of the other wave's MFMAs
        if (run) softmax(Kc, cur_partial, cur_m);
        __builtin_amdgcn_s_setprio(0);
        prv_run = run;
        // (the opaque copy keeps the compiler from deriving the class test
        // right after the load, a step early, where it would wait for it)
        int cls_now = clsN;
        asm volatile("" : "+s"(cls_now));
        if (j + 1 < T)
            tile_state(colV, cls_from(cls_now, j + 1), cur_partial, cur_live0, cur_live1, cur_m);
        colV = colK;
        colK = col_of(j + 3);
        clsN = cls_word(j + 2);
        if (grp == 0) {
            asm volatile("s_waitcnt vmcnt(4)" ::: "memory");  // loads of step j-1
            step_barrier();
        }
    };
    for (int j = 0; j <= T; j += 4) {
        step(j, K0, V3, K2, V1);
        if (j + 1 > T) break;
        step(j + 1, K1, V0, K3, V2);
        if (j + 2 > T) break;
        step(j + 2, K2, V1, K0, V3);
        if (j + 3 > T) break;
        step(j + 3, K3, V2, K1, V0);
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // loads into LDS past the last tile

    // ---- epilogue: O = O / l; rows without any visible key get 0.  The row
    // log-sum-exp (natural log) of the scaled scores is (m_ref + log2 l) ln 2.
    if (myrow < nrows) {
        const float inv = (l_run > 0.f) ? 1.f / l_run : 0.f;
        if (MODE == 0 && a.lse && hh == 0)
            a.lse[PK ? (size_t)(cub + myrow) * a.H + h : ((size_t)b * a.H + h) * nq + myrow] =
                (l_run > 0.f) ? (m_ref + log2f(l_run)) * 0.69314718055994531f : -INFINITY;
        __bf16 *op = (__bf16 *)a.o + (PK ? ((size_t)(cub + myrow) * a.H + h) * D
                                         : (((size_t)b * a.H + h) * nq + myrow) * D);
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

template <int MODE, bool PK>
hipError_t launch_pp(const AttnArgs &a, hipStream_t s) {
    const long nqt = (a.nq + 255) / 256;
    const long total = nqt * a.H * a.B;
    if (total > 0x7fffffffL) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((pp_kernel<MODE, PK>), dim3((unsigned)total), dim3(512), 0, s, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_pp_bf16(const AttnArgs &a, hipStream_t s) {
    if (a.mode == 1) return launch_pp<1, false>(a, s);
    return a.cu ? launch_pp<0, true>(a, s) : launch_pp<0, false>(a, s);
}

}  // namespace swa
