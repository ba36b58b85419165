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
// Work split (tile_q = 32 * NW query rows, head dim D; K/V staged 64 keys at a
// time; the metadata's key tile is 64 keys, or 128 keys streamed as two
// 64-key halves):
//   * one workgroup per (query tile, head, batch).  In the logical order the
//     query heads of one KV group are next to each other (they read identical
//     K/V tiles) and then the query tiles (neighbours share most of theirs);
//     chunks of 64 consecutive tiles are dealt to the XCDs so that the
//     workgroups one XCD runs together hit in its L2 and every XCD gets an
//     even share of the work (see xcd_deal);
//   * wave priority is raised over the MFMA sections (measured neutral, kept
//     as the intent: one wave issues matrix work while the other fills VALU);
//   * K and V tiles go straight from HBM to LDS (buffer_load_dwordx4 ... lds,
//     no register staging), double-buffered: the next tile streams in while
//     this one is computed; rows are XOR-swizzled in 16-byte chunks so that
//     both LDS read patterns below are free of bank conflicts.  The buffer
//     (MUBUF) form of the LDS DMA matters: with the FLAT-encoded
//     global_load_lds in flight the compiler can only wait for all LDS reads
//     at once (lgkmcnt(0)); with it, K fragments are read ahead with partial
//     waits.  The buffer range check returns zeros for rows past the data, so
//     the ragged last tile needs no clamping;
//   * S^T = K Q^T with v_mfma_f32_32x32x16_bf16: A = K rows read from LDS,
//     B = the wave's 32 query rows kept in registers.  Each lane then holds
//     one query column, so row max and sum need one swap across wave halves;
//   * fp32 online softmax in the exp2 domain with the scale folded into one
//     FMA, against a reference max m_ref (0 to start) instead of the running
//     max: p = exp2(s*c - m_ref) needs no max pass.  Only when a row's tile
//     sum leaves [2^-32, 2^32] (overflow risk, or underflow before the row has
//     seen a real max) does the wave recompute the tile's scores, take their
//     max and rescale O and l (exact: O and l share the reference); p <= 2^32
//     fits bf16 and fp32 with room to spare; the row sum is taken on the
//     bf16-rounded P with v_dot2_f32_bf16, so it matches what PV uses;
//   * O^T += V^T P^T: P comes straight from the S registers (rounded to bf16)
//     and V^T from LDS with ds_read_b64_tr_b16, which transposes 4x4 blocks of
//     16-bit values across lanes, so V stays row-major in LDS;
//   * inside a partial tile a wave skips a 32-key half in which none of its 32
//     rows sees any key, and leaves unmasked a half that all of them see
//     whole (finer than the metadata, same result); without attention sinks
//     the plain forward's mask tests one key interval per element (a
//     separate instantiation), with them two;
//   * the plain forward starts its first K/V load before the query rows and
//     the metadata row are read (the first key tile follows from the tile's
//     first row; the metadata's first entry is checked), and issues the next
//     tile's loads one per two QK MFMAs rather than all at once after the
//     barrier, where every wave's loads queued together in the memory pipe;
//   * the chunk checks its request's device ring state first; an unusable one
//     visits no key tile.
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

constexpr int BN = 64;  // keys per tile
constexpr float LOG2E = 1.4426950408889634f;
constexpr float P_HI = 4294967296.0f;       // 2^32: tile sums above this rescale
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

// Per-request ring/metadata constants of a tile kernel.
struct KeyPos {
    int nq, W, nst, nrt, qlen, rs, cl, np;
};

// Workgroup p of T runs logical tile L: XCD x = p % 8 gets the contiguous
// logical range [start_x, start_x + count_x) in dispatch order.
__device__ __forceinline__ int xcd_remap(int p, int T) {
    const int x = p & 7, i = p >> 3, q = T >> 3, r = T & 7;
    return x * q + (x < r ? x : r) + i;
}

// Workgroups go to the 8 XCDs round-robin (p % 8), each XCD running about 64
// at a time.  The logical order is cut into chunks of 64 tiles and runs of
// S = 4 consecutive chunks; in rounds 4R .. 4R+3 (its workgroups 256R ..
// 256R+255) XCD x runs the chunks of run 8R + (x + R) % 8, in order.  The 64
// workgroups an XCD runs together stay neighbours in the logical order (they
// share K/V tiles in its L2), and so do its successive chunks: with long
// windows the K/V span of a chunk overlaps the next chunk's by most of the
// window, which the XCD's L2 then still holds (one chunk per XCD per round
// fetched each K/V tile from HBM about 2.75 times on the GQA workload).
// Every XCD still draws its runs from all parts of the order, so work that
// varies along it (sequences of different lengths) is shared out evenly;
// contiguous ranges per XCD left one XCD with 1.7x the mean work on the GQA
// workload.  A tail of T mod 2048 tiles keeps contiguous ranges.  A
// bijection on [0, T).
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

// SK: attention sinks may be present (else the per-element mask of the plain
// forward tests one key interval instead of two)
template <int MODE, int D, int NW, bool PK, int SUB, bool SK>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(2)))
void tile_kernel(AttnArgs a) {
    constexpr int KS = D / 16;          // k-steps of the QK product
    constexpr int DB = D / 32;          // 32-wide d blocks of the output
    constexpr int CPR = D / 8;          // 16-byte chunks per row
    constexpr int RPL = 64 / CPR;       // rows per wave-wide 1 KB load
    constexpr int LPW = BN / RPL / NW;  // such loads per wave, per matrix, per tile
    constexpr int ROWB = D * 2;         // bytes per row
    constexpr int TILEB = BN * ROWB;    // bytes per K (or V) tile
    static_assert(LPW >= 1, "tile too small for the block");

    // two stages [K tile | V tile]; separate arrays so that the compiler can
    // tell the reads of one stage from the LDS-DMA writes into the other (else
    // it waits for the next tile's loads before every LDS read)
    __shared__ __attribute__((aligned(1024))) char stage0[2 * TILEB];
    __shared__ __attribute__((aligned(1024))) char stage1[2 * TILEB];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lq = lane & 31, hh = lane >> 5;
    const int nq = a.nq;
    const int nqt = (nq + 32 * NW - 1) / (32 * NW);
    // logical order: query heads of one KV group adjacent (they read the same
    // K/V tiles), then query tiles, then KV heads, then requests
    const int L = xcd_deal(blockIdx.x, gridDim.x);
    const int G = a.H / a.Hkv;
    const int h_in = L % G, qt = (L / G) % nqt, g = (L / (G * nqt)) % a.Hkv;
    const int b = L / (G * nqt * a.Hkv);
    const int h = g * G + h_in;

    // SUB = 64-key halves per metadata tile (tile_k 64 or 128); key tiles
    // below are counted in 64-key units
    constexpr int sub = SUB;
    KeyPos kp;
    kp.nq = nq;
    kp.W = a.W;
    // chunk key axis: [sink slots, n_sink rounded up to tile_k (with sinks) |
    // ring tiles | new rows]
    kp.nst = (MODE == 1 && a.n_sink > 0) ? (a.n_sink + a.tile_k - 1) / a.tile_k * sub : 0;
    kp.nrt = (MODE == 1) ? a.W / BN : 0;
    // packed batch (PK): sequence b owns tokens cu[b] .. cu[b+1]-1 of a
    // token-major [tokens][heads][D] layout; only its own rows exist
    const int cub = PK ? a.cu[b] : 0;
    const int nrows = PK ? a.cu[b + 1] - cub : nq;
    kp.qlen = PK ? nrows : ((MODE == 0) ? (a.q_len ? a.q_len[b] : nq) : nq);
    kp.rs = (MODE == 1) ? a.ring_start[b] : 0;
    kp.cl = (MODE == 1) ? a.cache_len[b] : 0;
    kp.np = (MODE == 1) ? a.next_pos[b] : 0;
    const int qlen = kp.qlen;
    const int qbase = (MODE == 1) ? kp.np : 0;  // logical position of query row 0

    // ---- key/value rows of a tile (rows past the data read as zeros through
    // the buffer range check below: finite, and always masked)
    const size_t kvh = (size_t)b * a.Hkv + g;
    // global row stride in bytes: D*2, or Hkv*D*2 in the packed layout
    const int RSB = PK ? a.Hkv * ROWB : ROWB;
    const __bf16 *klin = (const __bf16 *)a.k + (PK ? ((size_t)cub * a.Hkv + g) * D
                                                   : kvh * (size_t)nq * D);
    const __bf16 *vlin = (const __bf16 *)a.v + (PK ? ((size_t)cub * a.Hkv + g) * D
                                                   : kvh * (size_t)nq * D);
    const __bf16 *kring = (MODE == 1) ? (const __bf16 *)a.kc + kvh * (size_t)a.W * D : nullptr;
    const __bf16 *vring = (MODE == 1) ? (const __bf16 *)a.vc + kvh * (size_t)a.W * D : nullptr;
    // swizzles: logical 16-byte chunk c of row r sits at physical chunk c ^ swz(r).
    // K is read as rows (16 lanes: 16 consecutive rows, one chunk), V by
    // transposing reads (32 lanes: 4 consecutive rows, 4 consecutive chunks);
    // each swizzle spreads its pattern over the 64 four-byte banks.  At D = 64
    // two rows share 256 bytes, so rows of one parity must differ.
    auto kswz = [](int r) { return CPR == 16 ? (r & 15) : ((r >> 1) & 7); };
    auto vswz = [](int r) { return CPR == 16 ? ((r & 3) << 2) : (((r >> 1) & 1) << 2); };

    // byte offsets of this lane's 16-byte pieces inside a tile (tile-invariant)
    uint32_t koff[LPW], voff[LPW];
#pragma unroll
    for (int i = 0; i < LPW; i++) {
        const int r = (wave * LPW + i) * RPL + lane / CPR;
        const int pch = lane % CPR;
        koff[i] = (uint32_t)(r * RSB + (pch ^ kswz(r)) * 16);
        voff[i] = (uint32_t)(r * RSB + (pch ^ vswz(r)) * 16);
    }
    // buffer resources of the linear K/V rows (and the ring): loads past the
    // last row return zeros (raw buffer range check), so the ragged last tile
    // needs no clamping
    typedef __attribute__((address_space(3))) void lds_void;
    const int lin_bytes = nrows > 0 ? (nrows - 1) * RSB + ROWB : 0;
    const __amdgpu_buffer_rsrc_t klr =
        __builtin_amdgcn_make_buffer_rsrc((void *)klin, 0, lin_bytes, 0x00020000);
    const __amdgpu_buffer_rsrc_t vlr =
        __builtin_amdgcn_make_buffer_rsrc((void *)vlin, 0, lin_bytes, 0x00020000);
    __amdgpu_buffer_rsrc_t krr = klr, vrr = vlr, ksr = klr, vsr = vlr;
    if (MODE == 1) {
        krr = __builtin_amdgcn_make_buffer_rsrc((void *)kring, 0, a.W * ROWB, 0x00020000);
        vrr = __builtin_amdgcn_make_buffer_rsrc((void *)vring, 0, a.W * ROWB, 0x00020000);
        if (a.n_sink > 0) {  // sink slots past n_sink read as zeros (masked)
            const size_t sko = kvh * (size_t)a.n_sink * D;
            ksr = __builtin_amdgcn_make_buffer_rsrc((void *)((const __bf16 *)a.sk + sko), 0,
                                                    a.n_sink * ROWB, 0x00020000);
            vsr = __builtin_amdgcn_make_buffer_rsrc((void *)((const __bf16 *)a.sv + sko), 0,
                                                    a.n_sink * ROWB, 0x00020000);
        }
    }
    // (a uniform branch per segment: selecting buffer resources by value would
    // put them in scratch memory)
    auto load_tile = [&](__amdgpu_buffer_rsrc_t kq, __amdgpu_buffer_rsrc_t vq,
                         int base, char *kdst) __attribute__((always_inline)) {
        char *vdst = kdst + TILEB;
#pragma unroll
        for (int i = 0; i < LPW; i++) {
            const int ins = wave * LPW + i;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(kq, (lds_void *)(kdst + ins * 1024), 16,
                                                     base + (int)koff[i], 0, 0, 0);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(vq, (lds_void *)(vdst + ins * 1024), 16,
                                                     base + (int)voff[i], 0, 0, 0);
        }
    };
    auto issue = [&](int kt, char *kdst) {
        const int kr = kt - kp.nst;
        if (MODE == 1 && kt < kp.nst)
            load_tile(ksr, vsr, kt * BN * ROWB, kdst);
        else if (MODE == 1 && kr < kp.nrt)
            load_tile(krr, vrr, kr * BN * ROWB, kdst);
        else
            load_tile(klr, vlr, (kr - kp.nrt) * BN * RSB, kdst);
    };

    // The first key tile of the plain forward follows from the tile's first row
    // (tile 0 with sinks, else the one holding row0 - W + 1), so its K/V load
    // starts before the query rows and the metadata row are read: the
    // metadata's first entry is checked against it below (a mismatch, which a
    // metadata row built with another key length can give, waits for the
    // predicted load and issues the listed tile).
    const int row0_wg = qt * 32 * NW;
    int pred = -1;
    if (MODE == 0 && row0_wg < kp.qlen) {
        const int first = a.n_sink > 0 ? 0 : max(0, row0_wg - a.W + 1);
        pred = first / a.tile_k * sub;
        issue(pred, stage0);
    }

    // ---- this wave's 32 query rows in registers (B operand of S^T = K Q^T)
    const int row0 = qt * 32 * NW + wave * 32;
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

    // ---- running softmax state: lanes l and l^32 share query column lq
    const float c2 = a.scale * LOG2E;
    float m_ref = 0.f, l_run = 0.f;  // p = exp2(s*c2 - m_ref); O, l share m_ref
    bool guess = true;               // m_ref not yet taken from a real max
    f32x16 oacc[DB];
#pragma unroll
    for (int db = 0; db < DB; db++)
#pragma unroll
        for (int e = 0; e < 16; e++) oacc[db][e] = 0.f;

    const int mrow = b * nqt + qt;
    // a chunk over an unusable ring state visits no key tile (output 0)
    const bool st_ok = MODE == 0 || ring_state_ok(kp.rs, kp.cl, kp.np, a.W, nq);
    const int e0 = a.row_ptr[mrow], e1 = st_ok ? a.row_ptr[mrow + 1] : e0;
    const int qpos = qbase + myrow;
    const bool qvalid = myrow < qlen;
    const int nlin_full = nrows / BN;  // linear tiles lying fully inside the data

    // per-lane constants of the two LDS read patterns
    const int kr_row = lq;                       // + kb*32
    const int tr_j = lane & 15;
    const int tr_row = 4 * hh + (tr_j >> 2);     // + kk*16 + 8*r
    const int tr_col = ((lane >> 4) & 1) * 16 + 4 * (tr_j & 3);  // + db*32

    // one tile: compute on `cur` while the next tile streams into `nxt`
    // Metadata entries travel one tile ahead of their use: tile e's column and
    // class are loaded during tile e-1, the column of tile e+1 (whose K/V this
    // tile issues) one tile earlier still.  They are loaded per lane at an
    // address the compiler cannot prove uniform (lz is an opaque 0), so the
    // values stay in vector registers and the wait for them falls where
    // readfirstlane takes them, a tile later, instead of right after the load.
    int lz;
    asm volatile("v_mov_b32 %0, 0" : "=v"(lz));
    int v_col = 0, v_col1 = 0, v_cls = 0;
    if (e1 > e0) {
        v_col = a.col[e0 + lz];
        v_cls = a.col_cls[e0 + lz];
        v_col1 = (e0 + 1 < e1) ? a.col[e0 + 1 + lz] : 0;
    }
    // One 64-key step: key tile kt (64-key units) of class cls is in `cur`;
    // the K/V of step tile ktn (none when < 0) go to `nxt`; with next_meta,
    // the metadata of entry e + 2 (column) and e + 1 (class) is loaded.
    auto tile = [&](int e, int kt, int cls, int ktn, bool next_meta, const char *cur,
                    char *nxt) {
        const int kr = kt - kp.nst;  // index on the [ring | new rows] part
        const bool ragged = (kr - kp.nrt) >= nlin_full;
        const bool partial = (cls == 2) || ragged;
        __syncthreads();  // this tile is in LDS; every wave is done with the previous one
        // The plain forward spreads this wave's loads of the next tile over
        // the QK MFMAs below (ld_next) instead of issuing them together here:
        // issued at once by every wave after the barrier, they queue in the
        // memory pipe and hold up each wave's first MFMAs.  After the last
        // tile the loads still go out, from an offset past the data (zeros
        // into the unused stage; the buffer range check covers the whole
        // offset), so the MFMA blocks need no branch.  (With 128-key tiles and
        // attention sinks the extra registers spill, so that case issues here.)
        constexpr bool spread = MODE == 0 && (SUB == 1 || !SK);
        constexpr int NL = 2 * LPW;  // this wave's 1 KB loads of one K and V tile
        static_assert(NL <= 2 * KS, "at most one load per QK MFMA");
        const int ld_base = (ktn >= 0) ? ktn * BN * RSB : lin_bytes;
        auto ld_next = [&](int i) __attribute__((always_inline)) {  // K, V, K, V, ...
            const int j = i >> 1, ins = wave * LPW + j;
            if (i & 1)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(
                    vlr, (lds_void *)(nxt + TILEB + ins * 1024), 16, ld_base + (int)voff[j], 0,
                    0, 0);
            else
                __builtin_amdgcn_raw_ptr_buffer_load_lds(
                    klr, (lds_void *)(nxt + ins * 1024), 16, ld_base + (int)koff[j], 0, 0, 0);
        };
        // load i follows QK MFMA (i + 1) * 2KS / NL - 1 of the tile's 2KS
        auto ld_after = [&](int m) __attribute__((always_inline)) {
#pragma unroll
            for (int i = 0; i < NL; i++)
                if ((i + 1) * 2 * KS / NL - 1 == m) ld_next(i);
        };
        auto ld_count = [](int m) {
            int c = 0;
            for (int i = 0; i < NL; i++) c += ((i + 1) * 2 * KS / NL - 1 == m) ? 1 : 0;
            return c;
        };
        if (!spread && ktn >= 0) issue(ktn, nxt);
        // loads for the next tiles (after the barrier, so that its wait does
        // not include them)
        if (next_meta) {
            v_col = v_col1;
            v_col1 = (e + 2 < e1) ? a.col[e + 2 + lz] : 0;
            v_cls = (e + 1 < e1) ? a.col_cls[e + 1 + lz] : 0;
        }
        const char *ksm = cur;
        const char *vsm = cur + TILEB;

        // Partial tiles: the tile keys this lane's query sees form one interval
        // [a1, b1] of tile-local indices, plus a second one [a2, b2] only in a
        // ring tile that holds the ring's wrap point (empty when b < a).
        int a1 = 0, b1 = BN - 1, a2 = 0, b2 = -1;
        bool live[2] = {true, true};
        bool two = false;
        if (partial) {
            const int lo_pos = qpos - a.W + 1;  // visible positions [lo_pos, qpos]
            if (MODE == 0) {
                const int base = kt * BN;       // position of tile key 0
                a1 = lo_pos - base;
                b1 = min(qpos, qlen - 1) - base;
                if (SK && a.n_sink > base) {  // attention sinks: keys 0 .. n_sink-1
                    two = true;
                    a2 = -base;
                    b2 = min(a.n_sink - 1, min(qpos, qlen - 1)) - base;
                }
            } else if (kt < kp.nst) {  // sink slots: position = slot, every one <= qpos
                a1 = -kt * BN;
                b1 = min(a.n_sink - 1, qpos) - kt * BN;
            } else if (kr < kp.nrt) {
                const int off = kp.np - kp.cl;  // position of ring offset r = 0
                // with sinks, positions below n_sink come from the sink slots only
                const int rlo = max(0, max(lo_pos, a.n_sink) - off);
                const int rhi = min(kp.cl - 1, qpos - off);
                const int base = kr * BN - kp.rs;  // r of tile key 0, before wrapping
                if (base < 0 && base + BN > 0) {   // keys k < -base sit at r = base + k + W
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
                const int t0 = (kr - kp.nrt) * BN;  // new-row index of tile key 0
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
#pragma unroll
            for (int kb = 0; kb < 2; kb++) {
                const bool o1 = a1 <= b1 && a1 <= kb * 32 + 31 && b1 >= kb * 32;
                const bool o2 = a2 <= b2 && a2 <= kb * 32 + 31 && b2 >= kb * 32;
                live[kb] = __ballot(o1 || o2) != 0;
            }
            if (!live[0] && !live[1]) {
                if (spread)
#pragma unroll
                    for (int i = 0; i < NL; i++) ld_next(i);
                return;
            }
        }

        // S^T = K Q^T: rows = keys (A from LDS), columns = this wave's queries;
        // masked scores become -inf; each chain starts from an inline zero
        // accumulator (no vector instructions to clear it)
        f32x16 sacc[2];
        // (with_loads: the first evaluation of the tile, which also issues
        // the next tile's loads; the rare-case recompute does not)
        auto scores = [&](bool with_loads) {
            auto qk_step = [&](int kb, int ks) {
                const int r = kb * 32 + kr_row;
                const int c = (2 * ks + hh) ^ kswz(r);
                const bf16x8 af =
                    __builtin_bit_cast(bf16x8, *(const u32x4 *)(ksm + r * ROWB + c * 16));
                sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                    af, qf[ks], ks == 0 ? f32x16{} : sacc[kb], 0, 0, 0);
            };
            if (live[0] && live[1]) {
                // all K fragments of key block 0 first, then its MFMAs while the
                // fragments of block 1 stream in behind them
                bf16x8 kf[KS];
#pragma unroll
                for (int ks = 0; ks < KS; ks++) {
                    const int c = (2 * ks + hh) ^ kswz(kr_row);
                    kf[ks] = __builtin_bit_cast(bf16x8, ld16(ksm + kr_row * ROWB + c * 16));
                }
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int ks = 0; ks < KS; ks++) {
                    sacc[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                        kf[ks], qf[ks], ks == 0 ? f32x16{} : sacc[0], 0, 0, 0);
                    const int r = 32 + kr_row;
                    const int c = (2 * ks + hh) ^ kswz(r);
                    kf[ks] = __builtin_bit_cast(bf16x8, ld16(ksm + r * ROWB + c * 16));
                    if (spread && with_loads) ld_after(ks);
                }
                if (spread && with_loads)  // MFMA, K read, its share of the loads
#pragma unroll
                    for (int ks = 0; ks < KS; ks++) {
                        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
                        if (ld_count(ks) > 0) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
                    }
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int ks = 0; ks < KS; ks++) {
                    sacc[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                        kf[ks], qf[ks], ks == 0 ? f32x16{} : sacc[1], 0, 0, 0);
                    if (spread && with_loads) ld_after(KS + ks);
                }
                if (spread && with_loads)
#pragma unroll
                    for (int ks = 0; ks < KS; ks++) {
                        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                        if (ld_count(KS + ks) > 0)
                            __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
                    }
            } else if (live[0]) {
                // one half skipped: its scores only need to be finite (they are
                // masked, the tile being partial)
                if (spread && with_loads)
#pragma unroll
                    for (int i = 0; i < NL; i++) ld_next(i);
#pragma unroll
                for (int ks = 0; ks < KS; ks++) qk_step(0, ks);
                sacc[1] = f32x16{};
            } else {
                if (spread && with_loads)
#pragma unroll
                    for (int i = 0; i < NL; i++) ld_next(i);
#pragma unroll
                for (int ks = 0; ks < KS; ks++) qk_step(1, ks);
                sacc[0] = f32x16{};
            }
            if (partial) {
                // key k is visible iff (unsigned)(k - a) <= b - a; an empty interval
                // gets an offset that no tile key reaches.  Lane key of
                // sacc[kb][4i+j] is kb*32 + 8i + 4hh + j.
                const bool x1 = b1 < a1, x2 = !two || b2 < a2;
                const int L1 = x1 ? -(1 << 20) : a1 - 4 * hh, L2 = x2 ? -(1 << 20) : a2 - 4 * hh;
                const uint32_t n1 = x1 ? 0u : (uint32_t)(b1 - a1);
                const uint32_t n2 = x2 ? 0u : (uint32_t)(b2 - a2);
#pragma unroll
                for (int kb = 0; kb < 2; kb++) {
                    // a 32-key half that every row of the wave sees whole
                    // needs no mask (in a partial tile most halves are whole
                    // or dead for a given wave; only the diagonal ones mix)
                    const bool whole = (a1 <= kb * 32 && b1 >= kb * 32 + 31) ||
                                       (two && a2 <= kb * 32 && b2 >= kb * 32 + 31);
                    if (__ballot(!whole) == 0) continue;
#pragma unroll
                    for (int i = 0; i < 4; i++)
#pragma unroll
                        for (int j = 0; j < 4; j++) {
                            const int c = kb * 32 + 8 * i + j;
                            const bool vis =
                                ((uint32_t)(c - L1) <= n1) | ((uint32_t)(c - L2) <= n2);
                            sacc[kb][4 * i + j] = vis ? sacc[kb][4 * i + j] : -INFINITY;
                        }
                }
            }
        };
        // P = exp2(S*c2 - m_ref) rounded to bf16, packed as the PV B operands
        // (pk[kk] for 16-key step kk), and this tile's row sum of P
        bf16x8 pk[4];
        auto probs = [&]() -> float {
            // one partial sum per 16-key step: four short dependency chains
            // instead of one of 16, so that the row sum (and the rare-case
            // check that waits for it) is ready sooner
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
        __builtin_amdgcn_s_setprio(2);
        scores(true);
        __builtin_amdgcn_s_setprio(0);
        float psum = probs();
        const bool lane_vis = !partial || (b1 >= a1) || (two && b2 >= a2);
        const bool rare = psum > P_HI || (guess && lane_vis && psum < P_LO);
        if (__ballot(rare) != 0) {
            // take the real max of this tile's scores and move the reference
            scores(false);
            float mloc = -INFINITY;
#pragma unroll
            for (int kb = 0; kb < 2; kb++)
#pragma unroll
                for (int e2 = 0; e2 < 16; e2++) mloc = fmaxf(mloc, sacc[kb][e2]);
            mloc = half_swap_max(mloc) * c2;
            if (mloc != -INFINITY && (guess || mloc > m_ref)) {
                // A guessed reference may move down.  The new one is kept at
                // or above log2 of the mass already summed (l_run <= 2^32 in
                // guess mode), so l_run and O shrink or grow to at most 1x and
                // never overflow; with nothing summed yet there is nothing to
                // scale (O = l = 0, and exp2 of a large gap would be inf).
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

        __builtin_amdgcn_s_setprio(2);
        // O^T += V^T P^T in 16-key steps kk; the MFMA k index hh*8 + 4r + t of
        // both operands stands for tile key 16kk + 8r + 4hh + t.  Per live
        // 32-key half, every V^T fragment is read before the first of its
        // MFMAs (the scheduling barrier keeps the compiler from moving each
        // read next to its MFMA, where every MFMA of the first key step
        // waited out a full LDS latency).
        auto vread = [&](int kk, int db, int r) __attribute__((always_inline)) {
            const int row = kk * 16 + 8 * r + tr_row;
            const int col = db * 32 + tr_col;
            const int c = (col >> 3) ^ vswz(row);
            const char *p = vsm + row * ROWB + c * 16 + (col & 7) * 2;
            return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)p);
        };
#pragma unroll
        for (int kb = 0; kb < 2; kb++) {
            if (!live[kb]) continue;
            i16x4 vr[2][DB][2];
#pragma unroll
            for (int s2 = 0; s2 < 2; s2++)
#pragma unroll
                for (int db = 0; db < DB; db++)
#pragma unroll
                    for (int r = 0; r < 2; r++) vr[s2][db][r] = vread(2 * kb + s2, db, r);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int s2 = 0; s2 < 2; s2++)
#pragma unroll
                for (int db = 0; db < DB; db++) {
                    const u32x2 lo = __builtin_bit_cast(u32x2, vr[s2][db][0]);
                    const u32x2 hi = __builtin_bit_cast(u32x2, vr[s2][db][1]);
                    const u32x4 vv = {lo[0], lo[1], hi[0], hi[1]};
                    oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                        __builtin_bit_cast(bf16x8, vv), pk[2 * kb + s2], oacc[db], 0, 0, 0);
                }
        }
        __builtin_amdgcn_s_setprio(0);
    };
    {
        const int first = (e1 > e0) ? __builtin_amdgcn_readfirstlane(v_col) * sub : -1;
        if (first != pred) {
            if (pred >= 0) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            if (first >= 0) issue(first, stage0);
        }
    }
    auto meta = [&](int &kt, int &cls, int &kt1) {
        kt = __builtin_amdgcn_readfirstlane(v_col);
        cls = __builtin_amdgcn_readfirstlane(v_cls);
        kt1 = __builtin_amdgcn_readfirstlane(v_col1);
    };
    if (SUB == 1) {
        for (int e = e0; e < e1; e += 2) {
            int kt, cls, kt1;
            meta(kt, cls, kt1);
            tile(e, kt, cls, e + 1 < e1 ? kt1 : -1, true, stage0, stage1);
            if (e + 1 < e1) {
                meta(kt, cls, kt1);
                tile(e + 1, kt, cls, e + 2 < e1 ? kt1 : -1, true, stage1, stage0);
            }
        }
    } else {
        // a 128-key entry: its two halves go through the two stages in order
        for (int e = e0; e < e1; e++) {
            int kt, cls, kt1;
            meta(kt, cls, kt1);
            tile(e, 2 * kt, cls, 2 * kt + 1, false, stage0, stage1);
            tile(e, 2 * kt + 1, cls, e + 1 < e1 ? 2 * kt1 : -1, true, stage1, stage0);
        }
    }

    // the plain forward's last tile loaded zeros into the free stage
    if (MODE == 0 && (SUB == 1 || !SK)) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

    // ---- epilogue: O = O / l; rows without any visible key (padding) get 0.
    // The row log-sum-exp (natural log) of the scaled scores is
    // (m_ref + log2 l) * ln 2, since l = sum exp2(s*c2 - m_ref).
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

template <int MODE, int D, int NW, int SUB>
hipError_t launch_one(const AttnArgs &a, hipStream_t s) {
    const long nqt = (a.nq + 32 * NW - 1) / (32 * NW);
    const long total = nqt * a.H * a.B;
    if (total > 0x7fffffffL) return hipErrorInvalidConfiguration;
    const dim3 grid((unsigned)total), block(NW * 64);
    if constexpr (MODE == 1)
        hipLaunchKernelGGL((tile_kernel<MODE, D, NW, false, SUB, true>), grid, block, 0, s, a);
    else if (a.cu && a.n_sink > 0)
        hipLaunchKernelGGL((tile_kernel<MODE, D, NW, true, SUB, true>), grid, block, 0, s, a);
    else if (a.cu)
        hipLaunchKernelGGL((tile_kernel<MODE, D, NW, true, SUB, false>), grid, block, 0, s, a);
    else if (a.n_sink > 0)
        hipLaunchKernelGGL((tile_kernel<MODE, D, NW, false, SUB, true>), grid, block, 0, s, a);
    else
        hipLaunchKernelGGL((tile_kernel<MODE, D, NW, false, SUB, false>), grid, block, 0, s, a);
    return hipGetLastError();
}

template <int MODE, int D, int NW>
hipError_t launch_sub(const AttnArgs &a, hipStream_t s) {
    return a.tile_k == 2 * BN ? launch_one<MODE, D, NW, 2>(a, s) : launch_one<MODE, D, NW, 1>(a, s);
}

template <int MODE>
hipError_t launch_mode(const AttnArgs &a, hipStream_t s) {
    if (a.d == 128) {
        if (a.tile_q == 128) return launch_sub<MODE, 128, 4>(a, s);
        return launch_sub<MODE, 128, 2>(a, s);
    }
    if (a.tile_q == 128) return launch_sub<MODE, 64, 4>(a, s);
    return launch_sub<MODE, 64, 2>(a, s);
}

}  // namespace

hipError_t launch_tile_bf16(const AttnArgs &a, hipStream_t s) {
    return a.mode == 0 ? launch_mode<0>(a, s) : launch_mode<1>(a, s);
}

}  // namespace swa
