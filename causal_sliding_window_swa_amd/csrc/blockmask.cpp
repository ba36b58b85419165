// blockmask.cpp -- host-side block metadata for the tile kernels.
//
// "Weight sparsity vs attention sparsity" (AI-infra KB), §04: a device works
// in whole tiles, so the set of visible (query, key) pairs is summarised per
// (query tile, key tile) as skip / full / partial, and the kernel only visits
// live tiles and masks per element only in partial ones.  §07 of that page
// notes that building the metadata costs time too: this builder works on
// runs of consecutive logical positions, so a tile costs O(rows x runs)
// instead of O(rows x keys), and tiles whose position range cannot meet the
// query window are rejected in O(1).
#include <limits.h>
#include <string.h>

#include <algorithm>

#include "../../include/swa.h"
#include "swa_internal.h"

namespace {

// Keys at tile offsets [j0, j0+len) hold consecutive logical positions
// plo, plo+1, ... and are all valid.  `sink`: the run lies in the sink
// segment of a ring key axis.
struct Run {
    int64_t plo;
    int len;
    bool sink;
};

// Positions of run r inside [lo, hi].
inline int64_t count_in(const Run &r, int64_t lo, int64_t hi) {
    lo = std::max(r.plo, lo);
    hi = std::min(r.plo + r.len - 1, hi);
    return hi >= lo ? hi - lo + 1 : 0;
}

// Visible keys of a run for a query at logical position t: positions in
// [t-W+1, t] [M003 §03], plus the sinks [0, min(S-1, t)] ("Sparse attention
// taxonomy" §3.2), each position counted once.  On a segmented axis (ring
// with sinks) the sink segment supplies every position below S (visible to
// any later query) and the other keys count only at positions >= S.
inline int64_t overlap(int64_t t, int64_t W, int64_t S, bool seg, const Run &r) {
    if (r.sink) return count_in(r, 0, t);
    if (seg) return count_in(r, std::max(t - W + 1, S), t);
    int64_t n = count_in(r, t - W + 1, t);
    if (S > 0) n += count_in(r, 0, std::min(S - 1, t)) - count_in(r, t - W + 1, std::min(S - 1, t));
    return n;
}

struct KeyAxis {
    int NS, S;  // sink segment length (S rounded up to the key tile) and sinks
    int W_ring, nk_lin;
    int64_t k_start;
    int k_len;
    int rs, cl;
    int64_t np;

    // Runs of valid keys with consecutive positions inside [j0, j1).
    int runs(int j0, int j1, Run *out) const {
        int n = 0;
        // sink segment: slot s stands for position s, valid below S
        const int z1 = std::min(std::min(j1, NS), S);
        if (j0 < z1) out[n++] = Run{j0, z1 - j0, true};
        j0 = std::max(j0, NS) - NS;
        j1 = std::max(j1, NS) - NS;
        // ring part: slot s holds position np - cl + ((s - rs) mod W_ring) when
        // that offset is below cl; offsets grow by one per slot except where
        // they wrap at s == rs.
        const int a0 = j0, a1 = std::min(j1, W_ring);
        if (a0 < a1) {
            int cuts[3] = {a0, a1, a1};
            int nc = 2;
            if (rs > a0 && rs < a1) {
                cuts[1] = rs;
                cuts[2] = a1;
                nc = 3;
            }
            for (int c = 0; c + 1 < nc; c++) {
                const int sa = cuts[c], sb = cuts[c + 1];
                const int ra = ((sa - rs) % W_ring + W_ring) % W_ring;
                const int len = std::min(sb - sa, cl - ra);
                if (len > 0) out[n++] = Run{np - cl + ra, len, false};
            }
        }
        // linear part: key W_ring + t sits at k_start + t, valid below k_len
        const int b0 = std::max(j0, W_ring) - W_ring, b1 = std::min(j1 - W_ring, k_len);
        if (b1 > b0) out[n++] = Run{k_start + b0, b1 - b0, false};
        return n;
    }
};

}  // namespace

extern "C" int swa_blockmask_size(int B, int nq, int nk, int tile_q, int tile_k,
                                  size_t *cls_elems, size_t *max_nnz) {
    swa::clear_error();
    if (B < 1 || nq < 0 || nk < 0 || tile_q < 1 || tile_k < 1)
        return swa::fail(SWA_EINVAL, "blockmask_size: need B>=1, nq>=0, nk>=0, tiles>=1");
    if (!cls_elems || !max_nnz) return swa::fail(SWA_EINVAL, "blockmask_size: NULL output");
    const size_t nqt = (size_t)(nq + tile_q - 1) / tile_q;
    const size_t nkt = (size_t)(nk + tile_k - 1) / tile_k;
    *cls_elems = (size_t)B * nqt * nkt;
    *max_nnz = (size_t)B * nqt * nkt;
    return SWA_OK;
}

extern "C" int swa_blockmask_build(int B, int nq, int nk_lin, int W, int n_sink, int tile_q,
                                   int tile_k,
                                   const int32_t *q_start, const int32_t *k_start,
                                   const int32_t *q_len, const int32_t *k_len, int W_ring,
                                   const int32_t *ring_start, const int32_t *cache_len,
                                   const int32_t *next_pos, uint8_t *cls, int32_t *row_ptr,
                                   int32_t *col, uint8_t *col_cls, swa_mask_stats *stats) {
    swa::clear_error();
    if (W < 1) return swa::fail(SWA_EINVAL, "blockmask_build: window W=%d must be >= 1", W);
    if (B < 1 || nq < 0 || nk_lin < 0 || tile_q < 1 || tile_k < 1 || W_ring < 0)
        return swa::fail(SWA_EINVAL, "blockmask_build: bad sizes (B=%d nq=%d nk_lin=%d "
                         "tile_q=%d tile_k=%d W_ring=%d)", B, nq, nk_lin, tile_q, tile_k, W_ring);
    if (!cls || !row_ptr || !col || !col_cls)
        return swa::fail(SWA_EINVAL, "blockmask_build: NULL output array");
    if (n_sink < 0) return swa::fail(SWA_EINVAL, "blockmask_build: n_sink=%d < 0", n_sink);
    if (W_ring > 0) {
        if (W_ring % tile_k != 0)
            return swa::fail(SWA_EINVAL, "blockmask_build: ring size %d not a multiple of "
                             "tile_k %d", W_ring, tile_k);
        if (!ring_start || !cache_len || !next_pos)
            return swa::fail(SWA_EINVAL, "blockmask_build: ring state arrays required");
    }
    // a ring axis with sinks starts with a sink segment of whole key tiles
    const bool seg = W_ring > 0 && n_sink > 0;
    const int64_t NS = seg ? ((int64_t)n_sink + tile_k - 1) / tile_k * tile_k : 0;
    if (NS + W_ring + nk_lin > INT_MAX)
        return swa::fail(SWA_EINVAL, "blockmask_build: key axis too long");
    const int nk = (int)(NS + W_ring + nk_lin);
    const int nqt = (nq + tile_q - 1) / tile_q;
    const int nkt = (nk + tile_k - 1) / tile_k;

    // validate every batch entry before writing anything
    for (int b = 0; b < B; b++) {
        const int64_t qs = q_start ? q_start[b] : 0, ks = k_start ? k_start[b] : 0;
        const int ql = q_len ? q_len[b] : nq, kl = k_len ? k_len[b] : nk_lin;
        if (qs < 0 || ks < 0 || ql < 0 || ql > nq || kl < 0 || kl > nk_lin)
            return swa::fail(SWA_EINVAL, "blockmask_build: batch %d: bad start/length "
                             "(q_start=%lld k_start=%lld q_len=%d k_len=%d)", b,
                             (long long)qs, (long long)ks, ql, kl);
        if (qs + nq > (int64_t)INT32_MAX - W || ks + nk_lin > (int64_t)INT32_MAX - W)
            return swa::fail(SWA_EINVAL, "blockmask_build: batch %d: positions overflow "
                             "int32", b);
        if (W_ring > 0) {
            const int64_t rs = ring_start[b], cl = cache_len[b], np = next_pos[b];
            if (rs < 0 || rs >= W_ring || cl < 0 || cl > W_ring || np < cl ||
                np > (int64_t)INT32_MAX - W)
                return swa::fail(SWA_EINVAL, "blockmask_build: batch %d: bad ring state "
                                 "(start=%lld len=%lld next_pos=%lld, W=%d)", b,
                                 (long long)rs, (long long)cl, (long long)np, W_ring);
        }
    }

    swa_mask_stats st;
    memset(&st, 0, sizeof(st));
    int64_t nnz = 0;
    row_ptr[0] = 0;
    Run runs[4];
    for (int b = 0; b < B; b++) {
        KeyAxis ax;
        ax.NS = (int)NS;
        ax.S = n_sink;
        ax.W_ring = W_ring;
        ax.nk_lin = nk_lin;
        ax.k_start = k_start ? k_start[b] : 0;
        ax.k_len = k_len ? k_len[b] : nk_lin;
        ax.rs = W_ring > 0 ? ring_start[b] : 0;
        ax.cl = W_ring > 0 ? cache_len[b] : 0;
        ax.np = W_ring > 0 ? next_pos[b] : 0;
        const int64_t qs = q_start ? q_start[b] : 0;
        const int ql = q_len ? q_len[b] : nq;

        // distinct keys visible to some valid query: a key at position P is
        // touched iff some valid query position lies in [P, P+W-1], or, for a
        // sink, at or after P
        if (ql > 0) {
            const int nr = ax.runs(0, nk, runs);
            const int64_t last = qs + ql - 1;
            for (int r = 0; r < nr; r++) {
                if (runs[r].sink) {
                    st.keys_touched += count_in(runs[r], 0, last);
                    continue;
                }
                if (seg) {
                    st.keys_touched += count_in(runs[r], std::max<int64_t>(qs - W + 1, n_sink), last);
                    continue;
                }
                st.keys_touched += count_in(runs[r], qs - W + 1, last);
                if (n_sink > 0)
                    st.keys_touched += count_in(runs[r], 0, std::min<int64_t>(n_sink - 1, last)) -
                                       count_in(runs[r], qs - W + 1,
                                                std::min<int64_t>(n_sink - 1, last));
            }
        }
        for (int qt = 0; qt < nqt; qt++) {
            const int i0 = qt * tile_q, i1 = std::min(nq, i0 + tile_q);
            const int iv1 = std::min(i1, ql);  // valid rows are [i0, iv1)
            uint8_t *crow = cls + ((size_t)b * nqt + qt) * nkt;
            for (int kt = 0; kt < nkt; kt++) {
                const int j0 = kt * tile_k, j1 = std::min(nk, j0 + tile_k);
                const int64_t area = (int64_t)(i1 - i0) * (j1 - j0);
                int64_t count = 0;
                if (iv1 > i0) {
                    const int nr = ax.runs(j0, j1, runs);
                    int64_t pmin = INT64_MAX, pmax = INT64_MIN;
                    for (int r = 0; r < nr; r++) {
                        pmin = std::min(pmin, runs[r].plo);
                        pmax = std::max(pmax, runs[r].plo + runs[r].len - 1);
                    }
                    const int64_t tmin = qs + i0, tmax = qs + iv1 - 1;
                    const bool near = pmax >= tmin - W + 1 || pmin < n_sink;
                    if (nr > 0 && near && pmin <= tmax) {
                        for (int i = i0; i < iv1; i++)
                            for (int r = 0; r < nr; r++)
                                count += overlap(qs + i, W, n_sink, seg, runs[r]);
                    }
                }
                const uint8_t c = count == 0 ? SWA_BLOCK_SKIP
                                             : (count == area ? SWA_BLOCK_FULL : SWA_BLOCK_PARTIAL);
                crow[kt] = c;
                st.valid_pairs += count;
                if (c != SWA_BLOCK_SKIP) {
                    col[nnz] = kt;
                    col_cls[nnz] = c;
                    nnz++;
                    st.covered_coords += area;
                    st.n_live++;
                    if (c == SWA_BLOCK_FULL)
                        st.n_full++;
                    else
                        st.n_partial++;
                }
            }
            if (nnz > INT32_MAX) return swa::fail(SWA_EINVAL, "blockmask_build: too many blocks");
            row_ptr[(size_t)b * nqt + qt + 1] = (int32_t)nnz;
        }
    }
    if (stats) *stats = st;
    return SWA_OK;
}
