// swa_f32.hip -- fp32 path of causal sliding-window attention (any head dim
// that is a multiple of 4 up to 128, any tile sizes).  One thread per query
// row with an fp32 online softmax; key tiles come from the block metadata as
// on the bf16 path ("Weight sparsity vs attention sparsity" §04), so skipped
// tiles are never read.  Visibility: the query at logical position t reads
// keys at t-W+1 .. t, softmax over exactly those ("Weight sparsity vs
// attention sparsity" §03; "LLMs from scratch" ch.10 §10.1).
#include <hip/hip_runtime.h>
#include <math.h>

#include "ring_state.h"
#include "swa_internal.h"

namespace swa {
namespace {

// One query row: fold key (pos, krow, vrow) into the running state.  The
// methods are inlined at every call site: called out of line (the chunk and
// decode kernels call add from two places), the state went through scratch.
template <int DMAX>
struct RowState {
    float q[DMAX], o[DMAX];
    float m, l;
    __device__ __forceinline__ void init(const float *qrow, int d) {
#pragma unroll
        for (int c = 0; c < DMAX; c++) {
            q[c] = (c < d) ? qrow[c] : 0.f;
            o[c] = 0.f;
        }
        m = -INFINITY;
        l = 0.f;
    }
    __device__ __forceinline__ void add(const float *krow, const float *vrow, int d, float scale) {
        float s = 0.f;
#pragma unroll
        for (int c = 0; c < DMAX; c++)
            if (c < d) s = fmaf(q[c], krow[c], s);
        s *= scale;
        const float m2 = fmaxf(m, s);
        const float corr = expf(m - m2);  // m = -inf on the first key: 0
        const float p = expf(s - m2);
        l = l * corr + p;
#pragma unroll
        for (int c = 0; c < DMAX; c++)
            if (c < d) o[c] = fmaf(p, vrow[c], o[c] * corr);
        m = m2;
    }
    __device__ __forceinline__ float lse() const { return (l > 0.f) ? m + logf(l) : -INFINITY; }
    __device__ __forceinline__ void store(float *orow, int d) const {
        const float inv = (l > 0.f) ? 1.f / l : 0.f;
#pragma unroll
        for (int c = 0; c < DMAX; c++)
            if (c < d) orow[c] = o[c] * inv;
    }
};

// grid (nqt, H, B), 64 threads; rows of the query tile strided over threads.
template <int MODE, int DMAX>
__global__ __launch_bounds__(64) void tile_f32_kernel(AttnArgs a) {
    const int qt = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int d = a.d, nq = a.nq, W = a.W;
    const int g = h / (a.H / a.Hkv);
    const int nqt = (nq + a.tile_q - 1) / a.tile_q;
    // chunk key axis: [NS sink slots (with sinks) | W ring slots | nq new rows]
    const int NS =
        (MODE == 1 && a.n_sink > 0) ? (a.n_sink + a.tile_k - 1) / a.tile_k * a.tile_k : 0;
    const int nk = (MODE == 1 ? NS + W : 0) + nq;
    // packed batch: sequence b owns tokens cu[b] .. cu[b+1]-1 (token-major)
    const bool pk = MODE == 0 && a.cu;
    const int cub = pk ? a.cu[b] : 0;
    const int nrows = pk ? a.cu[b + 1] - cub : nq;
    const int qlen = pk ? nrows : ((MODE == 0) ? (a.q_len ? a.q_len[b] : nq) : nq);
    const int rs = (MODE == 1) ? a.ring_start[b] : 0;
    const int cl = (MODE == 1) ? a.cache_len[b] : 0;
    const int np = (MODE == 1) ? a.next_pos[b] : 0;
    // a chunk over an unusable ring state sees no key
    const bool st_ok = MODE == 0 || ring_state_ok(rs, cl, np, W, nq);
    const size_t kvh = (size_t)b * a.Hkv + g;
    // linear key row t: kvh row t, or token cub + t in the packed layout
    const size_t krs = pk ? (size_t)a.Hkv * d : (size_t)d;
    const float *klin = (const float *)a.k + (pk ? ((size_t)cub * a.Hkv + g) * d : kvh * nq * d);
    const float *vlin = (const float *)a.v + (pk ? ((size_t)cub * a.Hkv + g) * d : kvh * nq * d);
    const float *kring = (MODE == 1) ? (const float *)a.kc + kvh * W * d : nullptr;
    const float *vring = (MODE == 1) ? (const float *)a.vc + kvh * W * d : nullptr;
    const float *ksink = NS ? (const float *)a.sk + kvh * a.n_sink * d : nullptr;
    const float *vsink = NS ? (const float *)a.sv + kvh * a.n_sink * d : nullptr;
    const int e0 = a.row_ptr[b * nqt + qt], e1 = a.row_ptr[b * nqt + qt + 1];
    const int i_end = min(nrows, (qt + 1) * a.tile_q);

    for (int i = qt * a.tile_q + threadIdx.x; i < i_end; i += 64) {
        const size_t ridx = pk ? (size_t)(cub + i) * a.H + h : ((size_t)b * a.H + h) * nq + i;
        const float *qrow = (const float *)a.q + ridx * d;
        float *orow = (float *)a.o + ridx * d;
        RowState<DMAX> st;
        st.init(qrow, d);
        const int qpos = ((MODE == 1) ? np : 0) + i;
        if (i < qlen && st_ok) {
            for (int e = e0; e < e1; e++) {
                const int kt = a.col[e];
                const int j1 = min(nk, (kt + 1) * a.tile_k);
                for (int j = kt * a.tile_k; j < j1; j++) {
                    int pos;
                    bool ok;
                    const float *kr, *vr;
                    if (MODE == 1 && j < NS) {
                        // sink slot j holds position j; the chunk's other keys
                        // below n_sink are skipped, so each position counts once
                        if (j < a.n_sink && j <= qpos)
                            st.add(ksink + (size_t)j * d, vsink + (size_t)j * d, d, a.scale);
                        continue;
                    }
                    const int jr = j - NS;
                    if (MODE == 1 && jr < W) {
                        int r = jr - rs;
                        r += (r < 0) ? W : 0;
                        ok = r < cl;
                        pos = np - cl + r;
                        kr = kring + (size_t)jr * d;
                        vr = vring + (size_t)jr * d;
                    } else {
                        const int t = jr - (MODE == 1 ? W : 0);
                        pos = ((MODE == 1) ? np : 0) + t;
                        ok = (MODE == 1) ? true : (t < qlen);
                        kr = klin + (size_t)t * krs;
                        vr = vlin + (size_t)t * krs;
                    }
                    const bool sinkvis = MODE == 0 && pos < a.n_sink;
                    if (MODE == 1 && pos < a.n_sink) ok = false;  // taken from the sink slots
                    if (ok && pos <= qpos && (pos >= qpos - W + 1 || sinkvis))
                        st.add(kr, vr, d, a.scale);
                }
            }
        }
        st.store(orow, d);
        if (MODE == 0 && a.lse) a.lse[ridx] = st.lse();
    }
}

// Decode, after the new row has been written: the query at logical position
// next_pos attends over the valid slots of the ring as it is after the
// append.  grid (B, H), 64 threads each folding a strided subset of slots,
// then a merge of the 64 partial states through LDS.
template <int DMAX>
__global__ __launch_bounds__(64) void decode_f32_kernel(DecodeArgs a) {
    __shared__ float sm[64], sl[64];
    __shared__ float so[64][DMAX];
    const int b = blockIdx.x, h = blockIdx.y;
    const int d = a.d, W = a.W;
    const int g = h / (a.H / a.Hkv);
    const int rs = a.ring_start[b], cl = a.cache_len[b], np = a.next_pos[b];
    const bool st_ok = ring_state_ok(rs, cl, np, W, 1);  // else: no append, no key
    const bool full = cl == W;
    const int rs2 = full ? (rs + 1) % W : rs;
    const int cl2 = full ? W : cl + 1;
    const int qpos = np;  // position of the new token
    const float *kring = (const float *)a.kc + ((size_t)b * a.Hkv + g) * W * d;
    const float *vring = (const float *)a.vc + ((size_t)b * a.Hkv + g) * W * d;
    RowState<DMAX> st;
    st.init((const float *)a.q + ((size_t)b * a.H + h) * d, d);
    for (int s = threadIdx.x; s < W; s += 64) {
        int r = s - rs2;
        r += (r < 0) ? W : 0;
        const int pos = np + 1 - cl2 + r;
        if (st_ok && r < cl2 && pos <= qpos && pos >= qpos - W + 1)
            st.add(kring + (size_t)s * d, vring + (size_t)s * d, d, a.scale);
    }
    // attention sinks ("Sparse attention taxonomy" §3.2): positions below
    // n_sink that the ring no longer holds come from the sink cache; a token
    // appended at a sink position is copied there (that slot is not read in
    // this step, since the ring still holds it)
    if (a.n_sink > 0) {
        const int nsink = st_ok ? min(a.n_sink, np + 1 - cl2) : 0;
        const float *ks = (const float *)a.sk + ((size_t)b * a.Hkv + g) * a.n_sink * d;
        const float *vs = (const float *)a.sv + ((size_t)b * a.Hkv + g) * a.n_sink * d;
        for (int p = threadIdx.x; p < nsink; p += 64)
            st.add(ks + (size_t)p * d, vs + (size_t)p * d, d, a.scale);
        if (st_ok && np < a.n_sink && h % (a.H / a.Hkv) == 0) {
            const float *kn = (const float *)a.k_new + ((size_t)b * a.Hkv + g) * d;
            const float *vn = (const float *)a.v_new + ((size_t)b * a.Hkv + g) * d;
            float *kd = (float *)a.sk + (((size_t)b * a.Hkv + g) * a.n_sink + np) * d;
            float *vd = (float *)a.sv + (((size_t)b * a.Hkv + g) * a.n_sink + np) * d;
            for (int c = threadIdx.x; c < d; c += 64) {
                kd[c] = kn[c];
                vd[c] = vn[c];
            }
        }
    }
    const int t = threadIdx.x;
    sm[t] = st.m;
    sl[t] = st.l;
#pragma unroll
    for (int c = 0; c < DMAX; c++) so[t][c] = st.o[c];
    __syncthreads();
    if (t == 0) {
        float M = -INFINITY;
        for (int u = 0; u < 64; u++) M = fmaxf(M, sm[u]);
        float L = 0.f;
        float acc[DMAX];
#pragma unroll
        for (int c = 0; c < DMAX; c++) acc[c] = 0.f;
        for (int u = 0; u < 64; u++) {
            const float w = (sm[u] == -INFINITY) ? 0.f : expf(sm[u] - M);
            L += w * sl[u];
#pragma unroll
            for (int c = 0; c < DMAX; c++) acc[c] += w * so[u][c];
        }
        float *orow = (float *)a.o + ((size_t)b * a.H + h) * d;
        const float inv = (L > 0.f) ? 1.f / L : 0.f;
#pragma unroll
        for (int c = 0; c < DMAX; c++)
            if (c < d) orow[c] = acc[c] * inv;
    }
}

template <int MODE, int DMAX>
hipError_t launch_tile_dm(const AttnArgs &a, hipStream_t s) {
    const int nqt = (a.nq + a.tile_q - 1) / a.tile_q;
    hipLaunchKernelGGL((tile_f32_kernel<MODE, DMAX>), dim3(nqt, a.H, a.B), dim3(64), 0, s, a);
    return hipGetLastError();
}

template <int MODE>
hipError_t launch_tile_mode(const AttnArgs &a, hipStream_t s) {
    if (a.d <= 16) return launch_tile_dm<MODE, 16>(a, s);
    if (a.d <= 32) return launch_tile_dm<MODE, 32>(a, s);
    if (a.d <= 64) return launch_tile_dm<MODE, 64>(a, s);
    return launch_tile_dm<MODE, 128>(a, s);
}

template <int DMAX>
hipError_t launch_decode_dm(const DecodeArgs &a, hipStream_t s) {
    hipLaunchKernelGGL((decode_f32_kernel<DMAX>), dim3(a.B, a.H), dim3(64), 0, s, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_tile_f32(const AttnArgs &a, hipStream_t s) {
    return a.mode == 0 ? launch_tile_mode<0>(a, s) : launch_tile_mode<1>(a, s);
}

// Append (ring write), attend, then advance the ring state.
hipError_t launch_decode_f32(const DecodeArgs &a, hipStream_t s) {
    CommitArgs c = {};
    c.B = a.B;
    c.Hkv = a.Hkv;
    c.Tq = 1;
    c.d = a.d;
    c.W = a.W;
    c.elem_bytes = 4;
    c.k_new = a.k_new;
    c.v_new = a.v_new;
    c.kc = a.kc;
    c.vc = a.vc;
    c.ring_start = a.ring_start;
    c.cache_len = a.cache_len;
    c.next_pos = a.next_pos;
    hipError_t e = launch_ring_write(c, s);
    if (e != hipSuccess) return e;
    if (a.d <= 16)
        e = launch_decode_dm<16>(a, s);
    else if (a.d <= 32)
        e = launch_decode_dm<32>(a, s);
    else if (a.d <= 64)
        e = launch_decode_dm<64>(a, s);
    else
        e = launch_decode_dm<128>(a, s);
    if (e != hipSuccess) return e;
    return launch_ring_state(c, s);
}

}  // namespace swa
