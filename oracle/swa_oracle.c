/*
 * swa_oracle.c -- plain fp64 CPU oracle for causal sliding-window attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the CPU
 * baseline leg of the benchmark may load this library.  It shares no code,
 * header, table or helper with the GPU library: it is written straight from
 * the pages' statement of the method and is deliberately slow and literal.
 *
 * Sources (cited by page title and section):
 *   [M003]  "Weight sparsity vs attention sparsity" (AI-infra knowledge base,
 *           xuujii.github.io/ai-infra-kb/details/M003.html)
 *   [Ch10]  "Chapter 10: local and sparse attention, SWA and DSA"
 *           (LLMs-from-scratch book, book.ozine.me)
 *   [Blog]  "Dense attention vs sliding-window sparse attention"
 *           (maplevalley.com.cn/news/3171860)
 *
 * Conventions (readings where the pages leave a step open are marked READING):
 *   - W counts the current token: query at logical position t may read keys at
 *     logical positions max(0, t-W+1) .. t  [M003 §03], [Ch10 §10.1].
 *   - scores s_j = scale * <q, k_j>; softmax is normalised over exactly the
 *     allowed keys and the output is the weighted sum of their V rows
 *     [M003 §03].  Keys are visited in ascending logical position.
 *   - READING: a query with no allowed key (only padded rows) outputs 0; the
 *     pages warn that such a row would otherwise give NaN [Ch10 §10.3].
 *   - READING: grouped KV heads are contiguous groups, kv head = h / (H/Hkv).
 *   - Tensors are row-major [B][heads][rows][d] with d fastest.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

/* The visibility rule of [M003 §03]: key j is visible from query i iff
 * j <= i and j >= i-W+1.  Written on logical positions so that ring slots
 * (whose physical index is not their position, [M003 §06]) use it unchanged.
 * [Ch10 §10.1] states the same rule as: forbidden iff (i-j) < 0 or (i-j) >= W. */
static int allowed(int64_t qpos, int64_t kpos, int64_t W)
{
    return kpos <= qpos && kpos >= qpos - W + 1;
}

/* Window plus attention sinks ("Sparse attention taxonomy" §3.2, the
 * StreamingLLM rule): the first S tokens stay visible to every later query
 * besides the last W.  READING: sinks are causal (a sink at position p is
 * seen by queries at p or later) and a key in both sets counts once.  S = 0
 * is the plain window. */
static int visible(int64_t qpos, int64_t kpos, int64_t W, int64_t S)
{
    return allowed(qpos, kpos, W) || (kpos < S && kpos <= qpos);
}

/* Attention of one query row over a list of candidate keys given in ascending
 * logical position.  Only keys passing allowed() take part; softmax is
 * normalised over exactly those [M003 §03].  Two passes: the maximum score
 * first, then exp(s - max), so that exp never overflows (the result is the
 * same softmax).  scratch must hold nk doubles. */
static void attend_row(int d, int64_t W, int64_t S, double scale,
                       const double *q, int64_t qpos,
                       int nk, const double *const *krow, const double *const *vrow,
                       const int64_t *kpos, double *scratch, double *out)
{
    int c, j, any = 0;
    double m = -INFINITY, l = 0.0;

    for (c = 0; c < d; c++)
        out[c] = 0.0;

    /* s_j = scale * sum_c q_c k_jc for every allowed key */
    for (j = 0; j < nk; j++) {
        double s = 0.0;
        if (!visible(qpos, kpos[j], W, S))
            continue;
        for (c = 0; c < d; c++)
            s += q[c] * krow[j][c];
        s *= scale;
        scratch[j] = s;
        if (!any || s > m)
            m = s;
        any = 1;
    }
    if (!any)
        return; /* READING: empty allowed set -> output 0 */

    /* e_j = exp(s_j - m); l = sum e_j; o = sum e_j v_j / l */
    for (j = 0; j < nk; j++) {
        double e;
        if (!visible(qpos, kpos[j], W, S))
            continue;
        e = exp(scratch[j] - m);
        l += e;
        for (c = 0; c < d; c++)
            out[c] += e * vrow[j][c];
    }
    for (c = 0; c < d; c++)
        out[c] /= l;
}

/* ------------------------------------------------------------------------ */
/* Full-sequence forward.  Query row i and key row j sit at logical positions
 * i and j.  q_len[b] (NULL = N) is the valid length of sequence b: rows and
 * keys at or past it are padding.  Padded rows are written as 0 (READING).
 * q: [B][H][N][d], k, v: [B][Hkv][N][d], o: [B][H][N][d]. */
void orc_fwd_sink(int B, int H, int Hkv, int N, int d, int W, int S,
                  const double *q, const double *k, const double *v,
                  const int32_t *q_len, double scale, double *o)
{
    int64_t b, h;
    const int G = H / Hkv;

    for (b = 0; b < B; b++) {
        const int len = q_len ? q_len[b] : N;
        for (h = 0; h < H; h++) {
            const int64_t g = h / G; /* READING: contiguous head groups */
            const double *kb = k + ((b * Hkv + g) * (int64_t)N) * d;
            const double *vb = v + ((b * Hkv + g) * (int64_t)N) * d;
            int64_t i;
#pragma omp parallel for schedule(dynamic, 16)
            for (i = 0; i < N; i++) {
                const double *qi = q + ((b * H + h) * (int64_t)N + i) * d;
                double *oi = o + ((b * H + h) * (int64_t)N + i) * d;
                int c, j;
                const double **kr;
                const double **vr;
                int64_t *kp;
                double *sc;
                if (i >= len) { /* padded row */
                    for (c = 0; c < d; c++)
                        oi[c] = 0.0;
                    continue;
                }
                /* candidate keys: every valid key of the sequence, in order */
                kr = malloc(sizeof(*kr) * (size_t)len);
                vr = malloc(sizeof(*vr) * (size_t)len);
                kp = malloc(sizeof(*kp) * (size_t)len);
                sc = malloc(sizeof(*sc) * (size_t)len);
                for (j = 0; j < len; j++) {
                    kr[j] = kb + (int64_t)j * d;
                    vr[j] = vb + (int64_t)j * d;
                    kp[j] = j;
                }
                attend_row(d, W, S, scale, qi, i, len, kr, vr, kp, sc, oi);
                free(kr); free(vr); free(kp); free(sc);
            }
        }
    }
}

void orc_fwd(int B, int H, int Hkv, int N, int d, int W,
             const double *q, const double *k, const double *v,
             const int32_t *q_len, double scale, double *o)
{
    orc_fwd_sink(B, H, Hkv, N, d, W, 0, q, k, v, q_len, scale, o);
}

/* The same forward, for a list of selected rows only (for large inputs).
 * Row r is (rb[r], rh[r], ri[r]); its output goes to o_rows + r*d. */
void orc_fwd_rows_sink(int B, int H, int Hkv, int N, int d, int W, int S,
                  const double *q, const double *k, const double *v,
                  const int32_t *q_len, double scale,
                  int nrows, const int32_t *rb, const int32_t *rh, const int32_t *ri,
                  double *o_rows)
{
    int r;
    const int G = H / Hkv;
    (void)B;
#pragma omp parallel for schedule(dynamic, 1)
    for (r = 0; r < nrows; r++) {
        const int64_t b = rb[r], h = rh[r], i = ri[r];
        const int64_t g = h / G;
        const int len = q_len ? q_len[b] : N;
        const double *qi = q + ((b * H + h) * (int64_t)N + i) * d;
        const double *kb = k + ((b * Hkv + g) * (int64_t)N) * d;
        const double *vb = v + ((b * Hkv + g) * (int64_t)N) * d;
        double *oi = o_rows + (int64_t)r * d;
        int c, j;
        const double **kr;
        const double **vr;
        int64_t *kp;
        double *sc;
        if (i >= len) {
            for (c = 0; c < d; c++)
                oi[c] = 0.0;
            continue;
        }
        kr = malloc(sizeof(*kr) * (size_t)len);
        vr = malloc(sizeof(*vr) * (size_t)len);
        kp = malloc(sizeof(*kp) * (size_t)len);
        sc = malloc(sizeof(*sc) * (size_t)len);
        for (j = 0; j < len; j++) {
            kr[j] = kb + (int64_t)j * d;
            vr[j] = vb + (int64_t)j * d;
            kp[j] = j;
        }
        attend_row(d, W, S, scale, qi, i, len, kr, vr, kp, sc, oi);
        free(kr); free(vr); free(kp); free(sc);
    }
}

void orc_fwd_rows(int B, int H, int Hkv, int N, int d, int W,
                  const double *q, const double *k, const double *v,
                  const int32_t *q_len, double scale,
                  int nrows, const int32_t *rb, const int32_t *rh, const int32_t *ri,
                  double *o_rows)
{
    orc_fwd_rows_sink(B, H, Hkv, N, d, W, 0, q, k, v, q_len, scale, nrows, rb, rh, ri, o_rows);
}

/* ------------------------------------------------------------------------ */
/* Ring-buffer cache [Blog §3.2]: a [heads][W][d] buffer per request plus a
 * start index and a fill count.  While the fill count is below W a new row
 * goes to the next free slot; once full it overwrites the slot at the start
 * index, which then advances by one modulo W.  The free slot is taken as
 * (start + len) mod W, which is the page's "slot len" when start is 0
 * (READING).  next_pos counts logical positions appended so far, so the row
 * in logical order r (0 = oldest) sits in slot (start + r) mod W at logical
 * position next_pos - len + r: slots keep their original positions after
 * being overwritten [M003 §06], [Ch10 §10.2]. */
static void ring_append_one(int Hkv, int W, int d, double *kc, double *vc,
                            int32_t *start, int32_t *len, int32_t *next_pos,
                            const double *k_row_heads, const double *v_row_heads,
                            int64_t head_stride)
{
    int slot, g;
    if (*len < W) {
        slot = (*start + *len) % W;
        *len += 1;
    } else {
        slot = *start;
        *start = (*start + 1) % W;
    }
    for (g = 0; g < Hkv; g++) {
        memcpy(kc + ((int64_t)g * W + slot) * d, k_row_heads + g * head_stride,
               sizeof(double) * (size_t)d);
        memcpy(vc + ((int64_t)g * W + slot) * d, v_row_heads + g * head_stride,
               sizeof(double) * (size_t)d);
    }
    *next_pos += 1;
}

/* Chunked prefill of Tq new tokens against the ring [Ch10 §10.2]:
 * the old cache (old_len = cache_len rows, in logical order) is joined with
 * the new rows; key positions start at next_pos - old_len, queries start at
 * next_pos.  Every query attends over that union (which is why the step
 * needs up to W+Tq-1 keys although only W stay cached).  Afterwards the new
 * rows are appended to the ring one by one, so the ring keeps the last W.
 * With S > 0 sink tokens ("Sparse attention taxonomy" §3.2) the sink cache
 * sink_k, sink_v [B][Hkv][S][d] holds the rows of positions 0 .. S-1
 * (READING, as in decode): the queries also attend over the sink positions
 * that neither the ring nor the chunk holds (each position once), and new
 * tokens at positions below S are copied into the sink cache at commit.
 * q: [B][H][Tq][d]; k_new, v_new: [B][Hkv][Tq][d];
 * k_cache, v_cache: [B][Hkv][W][d] (in/out); ring state arrays [B] (in/out);
 * o: [B][H][Tq][d]. */
void orc_chunk_sink(int B, int H, int Hkv, int Tq, int d, int W, int S,
                    const double *q, const double *k_new, const double *v_new,
                    double *k_cache, double *v_cache, double *sink_k, double *sink_v,
                    int32_t *ring_start, int32_t *cache_len, int32_t *next_pos,
                    double scale, double *o)
{
    int b;
    const int G = H / Hkv;
    for (b = 0; b < B; b++) {
        const int old_len = cache_len[b];
        const int64_t p0 = next_pos[b];
        const int64_t oldest = p0 - old_len; /* oldest position the ring holds */
        const int nsink = (int)(S < oldest ? S : (oldest > 0 ? oldest : 0));
        const int nk = nsink + old_len + Tq;
        int h, t, g;
        for (h = 0; h < H; h++) {
            const int64_t gg = h / G;
            const double *kc = k_cache + ((int64_t)b * Hkv + gg) * (int64_t)W * d;
            const double *vc = v_cache + ((int64_t)b * Hkv + gg) * (int64_t)W * d;
            const double *kn = k_new + ((int64_t)b * Hkv + gg) * (int64_t)Tq * d;
            const double *vn = v_new + ((int64_t)b * Hkv + gg) * (int64_t)Tq * d;
            const double **kr = malloc(sizeof(*kr) * (size_t)nk);
            const double **vr = malloc(sizeof(*vr) * (size_t)nk);
            int64_t *kp = malloc(sizeof(*kp) * (size_t)nk);
            int r;
            /* sink positions held by neither the ring nor the chunk */
            for (r = 0; r < nsink; r++) {
                kr[r] = sink_k + (((int64_t)b * Hkv + gg) * S + r) * d;
                vr[r] = sink_v + (((int64_t)b * Hkv + gg) * S + r) * d;
                kp[r] = r;
            }
            /* combined keys: old cache in logical order, then the new rows */
            for (r = 0; r < old_len; r++) {
                const int slot = (ring_start[b] + r) % W;
                kr[nsink + r] = kc + (int64_t)slot * d;
                vr[nsink + r] = vc + (int64_t)slot * d;
                kp[nsink + r] = p0 - old_len + r; /* k_start_pos_abs = ptr - old_len */
            }
            for (t = 0; t < Tq; t++) {
                kr[nsink + old_len + t] = kn + (int64_t)t * d;
                vr[nsink + old_len + t] = vn + (int64_t)t * d;
                kp[nsink + old_len + t] = p0 + t;
            }
#pragma omp parallel for schedule(dynamic, 4)
            for (t = 0; t < Tq; t++) {
                double *sc = malloc(sizeof(*sc) * (size_t)nk);
                attend_row(d, W, S, scale,
                           q + (((int64_t)b * H + h) * Tq + t) * d, p0 + t,
                           nk, kr, vr, kp, sc,
                           o + (((int64_t)b * H + h) * Tq + t) * d);
                free(sc);
            }
            free(kr); free(vr); free(kp);
        }
        /* commit only after every query of the chunk has read the old ring */
        for (t = 0; t < Tq; t++) {
            if (p0 + t < S) {
                for (g = 0; g < Hkv; g++) {
                    const int64_t slot = ((int64_t)b * Hkv + g) * S + p0 + t;
                    memcpy(sink_k + slot * d, k_new + (((int64_t)b * Hkv + g) * Tq + t) * d,
                           sizeof(double) * (size_t)d);
                    memcpy(sink_v + slot * d, v_new + (((int64_t)b * Hkv + g) * Tq + t) * d,
                           sizeof(double) * (size_t)d);
                }
            }
            ring_append_one(Hkv, W, d,
                            k_cache + (int64_t)b * Hkv * W * d,
                            v_cache + (int64_t)b * Hkv * W * d,
                            &ring_start[b], &cache_len[b], &next_pos[b],
                            k_new + ((int64_t)b * Hkv * Tq + t) * d,
                            v_new + ((int64_t)b * Hkv * Tq + t) * d,
                            (int64_t)Tq * d);
        }
    }
}

void orc_chunk(int B, int H, int Hkv, int Tq, int d, int W,
               const double *q, const double *k_new, const double *v_new,
               double *k_cache, double *v_cache,
               int32_t *ring_start, int32_t *cache_len, int32_t *next_pos,
               double scale, double *o)
{
    orc_chunk_sink(B, H, Hkv, Tq, d, W, 0, q, k_new, v_new, k_cache, v_cache, NULL, NULL,
                   ring_start, cache_len, next_pos, scale, o);
}

/* One decode step: the new token's K/V row is appended to the ring first
 * (READING: append, then attend, so the ring holds exactly the W positions
 * the new query may see), then the query at the new token's position attends
 * over the ring's valid slots taken in logical order.
 * With S > 0 sink tokens ("Sparse attention taxonomy" §3.2: the first tokens
 * are kept besides the last W) the first S positions also live in a sink
 * cache sink_k, sink_v [B][Hkv][S][d]: a token appended at position p < S is
 * copied there as well, and the query also attends over the sink positions
 * that the ring no longer holds (each position counted once; READING).
 * q: [B][H][d]; k_new, v_new: [B][Hkv][d]; cache and state as orc_chunk. */
void orc_decode_sink(int B, int H, int Hkv, int d, int W, int S,
                     const double *q, const double *k_new, const double *v_new,
                     double *k_cache, double *v_cache, double *sink_k, double *sink_v,
                     int32_t *ring_start, int32_t *cache_len, int32_t *next_pos,
                     double scale, double *o)
{
    int b;
    const int G = H / Hkv;
    for (b = 0; b < B; b++) {
        int64_t qpos, oldest;
        int h, len, nsink, g;
        if (S > 0 && next_pos[b] < S) {
            for (g = 0; g < Hkv; g++) {
                const int64_t slot = ((int64_t)b * Hkv + g) * S + next_pos[b];
                memcpy(sink_k + slot * d, k_new + ((int64_t)b * Hkv + g) * d,
                       sizeof(double) * (size_t)d);
                memcpy(sink_v + slot * d, v_new + ((int64_t)b * Hkv + g) * d,
                       sizeof(double) * (size_t)d);
            }
        }
        ring_append_one(Hkv, W, d,
                        k_cache + (int64_t)b * Hkv * W * d,
                        v_cache + (int64_t)b * Hkv * W * d,
                        &ring_start[b], &cache_len[b], &next_pos[b],
                        k_new + (int64_t)b * Hkv * d, v_new + (int64_t)b * Hkv * d,
                        (int64_t)d);
        qpos = (int64_t)next_pos[b] - 1;
        len = cache_len[b];
        oldest = (int64_t)next_pos[b] - len; /* oldest position still in the ring */
        nsink = (int)(S < oldest ? S : oldest);
        if (nsink < 0)
            nsink = 0;
#pragma omp parallel for schedule(static)
        for (h = 0; h < H; h++) {
            const int64_t gg = h / G;
            const double *kc = k_cache + ((int64_t)b * Hkv + gg) * (int64_t)W * d;
            const double *vc = v_cache + ((int64_t)b * Hkv + gg) * (int64_t)W * d;
            const int n = nsink + len;
            const double **kr = malloc(sizeof(*kr) * (size_t)(n > 0 ? n : 1));
            const double **vr = malloc(sizeof(*vr) * (size_t)(n > 0 ? n : 1));
            int64_t *kp = malloc(sizeof(*kp) * (size_t)(n > 0 ? n : 1));
            double *sc = malloc(sizeof(*sc) * (size_t)(n > 0 ? n : 1));
            int r;
            /* sink positions the ring has dropped, then the ring in logical order */
            for (r = 0; r < nsink; r++) {
                kr[r] = sink_k + (((int64_t)b * Hkv + gg) * S + r) * d;
                vr[r] = sink_v + (((int64_t)b * Hkv + gg) * S + r) * d;
                kp[r] = r;
            }
            for (r = 0; r < len; r++) {
                const int slot = (ring_start[b] + r) % W;
                kr[nsink + r] = kc + (int64_t)slot * d;
                vr[nsink + r] = vc + (int64_t)slot * d;
                kp[nsink + r] = (int64_t)next_pos[b] - len + r;
            }
            attend_row(d, W, S, scale, q + ((int64_t)b * H + h) * d, qpos,
                       n, kr, vr, kp, sc, o + ((int64_t)b * H + h) * d);
            free(kr); free(vr); free(kp); free(sc);
        }
    }
}

void orc_decode(int B, int H, int Hkv, int d, int W,
                const double *q, const double *k_new, const double *v_new,
                double *k_cache, double *v_cache,
                int32_t *ring_start, int32_t *cache_len, int32_t *next_pos,
                double scale, double *o)
{
    orc_decode_sink(B, H, Hkv, d, W, 0, q, k_new, v_new, k_cache, v_cache, NULL, NULL,
                    ring_start, cache_len, next_pos, scale, o);
}

/* ------------------------------------------------------------------------ */
/* Block metadata by brute force [M003 §04]: every (query tile, key tile)
 * pair is classified by counting the visible pairs among its coordinates:
 * none -> skip (0), all in-range coordinates -> full (1), else partial (2).
 * READING: tiles cut by the array edge count only their in-range area.
 *
 * Key axis: if W_ring > 0, keys 0..W_ring-1 are ring slots (positions from
 * the ring state as in ring_append_one's comment; unfilled slots are
 * invalid), followed by nk_lin linear keys.  Linear key t of batch b sits at
 * k_start[b] + t and is valid iff t < k_len[b]; query i sits at q_start[b]+i
 * and is valid iff i < q_len[b].  NULL position arrays mean 0, NULL length
 * arrays mean "all valid".
 * With a ring and S > 0 sinks (the chunk with sinks) the axis starts with a
 * sink segment of NS = S rounded up to tile_k slots: slot s stands for
 * position s (valid iff s < S) and is visible to every query at or after s;
 * positions below S are then taken from that segment only, so ring and
 * linear keys are visible by the window rule and only at positions >= S
 * (READING: each position counted once, as the method's definition asks).
 *
 * Outputs: cls[b][qt][kt]; CSR over rows b*nqt+qt in ascending key tile
 * (row_ptr, col, col_cls); stats[6] = valid pairs, covered coordinates
 * (in-range area of live blocks), distinct keys touched, live, full, partial
 * blocks, each summed over b.  Returns the number of live blocks. */
int64_t orc_blockmask_sink(int B, int nq, int nk_lin, int W, int S, int tile_q, int tile_k,
                           const int32_t *q_start, const int32_t *k_start,
                           const int32_t *q_len, const int32_t *k_len,
                           int W_ring, const int32_t *ring_start,
                           const int32_t *cache_len, const int32_t *next_pos,
                           uint8_t *cls, int32_t *row_ptr, int32_t *col,
                           uint8_t *col_cls, int64_t *stats)
{
    const int seg = W_ring > 0 && S > 0;
    const int NS = seg ? (S + tile_k - 1) / tile_k * tile_k : 0;
    const int nk = NS + W_ring + nk_lin;
    const int nqt = (nq + tile_q - 1) / tile_q;
    const int nkt = (nk + tile_k - 1) / tile_k;
    int64_t nnz = 0;
    int b, s;
    int64_t *qpos = malloc(sizeof(int64_t) * (size_t)(nq > 0 ? nq : 1));
    int64_t *kpos = malloc(sizeof(int64_t) * (size_t)(nk > 0 ? nk : 1));
    char *qok = malloc((size_t)(nq > 0 ? nq : 1));
    char *kok = malloc((size_t)(nk > 0 ? nk : 1));
    char *ksink = malloc((size_t)(nk > 0 ? nk : 1));
    char *touched = malloc((size_t)(nk > 0 ? nk : 1));
    int64_t *counts = malloc(sizeof(int64_t) * (size_t)(nqt > 0 && nkt > 0 ? nqt * nkt : 1));

    for (s = 0; s < 6; s++)
        stats[s] = 0;
    row_ptr[0] = 0;

    for (b = 0; b < B; b++) {
        int i, j, qt, kt;
        for (i = 0; i < nq; i++) {
            qpos[i] = (q_start ? q_start[b] : 0) + (int64_t)i;
            qok[i] = q_len ? (i < q_len[b]) : 1;
        }
        for (j = 0; j < nk; j++)
            ksink[j] = 0;
        for (j = 0; j < NS; j++) {
            kpos[j] = j;
            kok[j] = j < S;
            ksink[j] = 1;
        }
        for (j = 0; j < W_ring; j++)
            kok[NS + j] = 0;
        if (W_ring > 0) {
            int r;
            for (r = 0; r < cache_len[b]; r++) {
                const int slot = (ring_start[b] + r) % W_ring;
                kpos[NS + slot] = (int64_t)next_pos[b] - cache_len[b] + r;
                kok[NS + slot] = 1;
            }
        }
        for (j = 0; j < nk_lin; j++) {
            kpos[NS + W_ring + j] = (k_start ? k_start[b] : 0) + (int64_t)j;
            kok[NS + W_ring + j] = k_len ? (j < k_len[b]) : 1;
        }
        /* visible-pair count of every tile pair, by brute force over its
         * coordinates (tiles are independent: counted in parallel) */
#pragma omp parallel for collapse(2) schedule(dynamic, 4)
        for (qt = 0; qt < nqt; qt++) {
            for (kt = 0; kt < nkt; kt++) {
                const int i0 = qt * tile_q;
                const int i1 = (i0 + tile_q < nq) ? i0 + tile_q : nq;
                const int j0 = kt * tile_k;
                const int j1 = (j0 + tile_k < nk) ? j0 + tile_k : nk;
                int64_t count = 0;
                int ii, jj;
                for (ii = i0; ii < i1; ii++)
                    for (jj = j0; jj < j1; jj++)
                        if (qok[ii] && kok[jj] &&
                            (!seg ? visible(qpos[ii], kpos[jj], W, S)
                                  : ksink[jj] ? kpos[jj] <= qpos[ii]
                                              : visible(qpos[ii], kpos[jj], W, 0) && kpos[jj] >= S))
                            count++;
                counts[(int64_t)qt * nkt + kt] = count;
            }
        }
        /* a key is touched if some valid query sees it */
#pragma omp parallel for schedule(dynamic, 64)
        for (j = 0; j < nk; j++) {
            int ii;
            touched[j] = 0;
            for (ii = 0; ii < nq && kok[j]; ii++)
                if (qok[ii] &&
                    (!seg ? visible(qpos[ii], kpos[j], W, S)
                          : ksink[j] ? kpos[j] <= qpos[ii]
                                     : visible(qpos[ii], kpos[j], W, 0) && kpos[j] >= S)) {
                    touched[j] = 1;
                    break;
                }
        }

        for (qt = 0; qt < nqt; qt++) {
            const int i0 = qt * tile_q;
            const int i1 = (i0 + tile_q < nq) ? i0 + tile_q : nq;
            for (kt = 0; kt < nkt; kt++) {
                const int j0 = kt * tile_k;
                const int j1 = (j0 + tile_k < nk) ? j0 + tile_k : nk;
                const int64_t area = (int64_t)(i1 - i0) * (j1 - j0);
                const int64_t count = counts[(int64_t)qt * nkt + kt];
                uint8_t c;
                c = (count == 0) ? 0 : (count == area ? 1 : 2);
                cls[((int64_t)b * nqt + qt) * nkt + kt] = c;
                stats[0] += count;
                if (c != 0) {
                    col[nnz] = kt;
                    col_cls[nnz] = c;
                    nnz++;
                    stats[1] += area;
                    stats[3] += 1;
                    stats[c == 1 ? 4 : 5] += 1;
                }
            }
            row_ptr[(int64_t)b * nqt + qt + 1] = (int32_t)nnz;
        }
        for (j = 0; j < nk; j++)
            stats[2] += touched[j];
    }
    free(qpos); free(kpos); free(qok); free(kok); free(ksink); free(touched); free(counts);
    return nnz;
}

int64_t orc_blockmask(int B, int nq, int nk_lin, int W, int tile_q, int tile_k,
                      const int32_t *q_start, const int32_t *k_start,
                      const int32_t *q_len, const int32_t *k_len,
                      int W_ring, const int32_t *ring_start,
                      const int32_t *cache_len, const int32_t *next_pos,
                      uint8_t *cls, int32_t *row_ptr, int32_t *col,
                      uint8_t *col_cls, int64_t *stats)
{
    return orc_blockmask_sink(B, nq, nk_lin, W, 0, tile_q, tile_k, q_start, k_start, q_len,
                              k_len, W_ring, ring_start, cache_len, next_pos, cls, row_ptr,
                              col, col_cls, stats);
}

/* Threads the OpenMP runtime will use (for reporting). */
int orc_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Sets the thread count of later calls (timing at one thread); n < 1 is 1. */
void orc_set_num_threads(int n)
{
#ifdef _OPENMP
    omp_set_num_threads(n < 1 ? 1 : n);
#else
    (void)n;
#endif
}

/* ------------------------------------------------------------------------ */
/* Gradients of the full-sequence forward, for a scalar loss whose gradient
 * with respect to the output o is dout.  [M003 §07] asks that the Q/K/V
 * gradients of the masked attention be checked by finite differences; this is
 * the plain chain rule through s_ij = scale <q_i, k_j>, the softmax over the
 * allowed keys and o_i = sum_j P_ij v_j:
 *   dv_j  = sum_i P_ij dout_i
 *   dP_ij = <dout_i, v_j>
 *   D_i   = sum_j P_ij dP_ij              (softmax Jacobian: dS = P (dP - D))
 *   dS_ij = P_ij (dP_ij - D_i)
 *   dq_i  = scale sum_j dS_ij k_j
 *   dk_j  = scale sum_i dS_ij q_i
 * with the sums over allowed (i, j) only.  READING: padded rows and keys (at or
 * past q_len) get zero gradients, like their zero outputs.  Grouped heads: the
 * key and value gradients of kv head g sum over its G query heads.
 * The row values (log-sum-exp, D) are computed per row from its scores. */

/* Log-sum-exp of row i's allowed scores and D_i = sum_j P_ij <dout_i, v_j>.
 * Returns 0 (and leaves the outputs untouched) when the row sees no key. */
static int row_stats(int d, int W, int S, int len, double scale, const double *qi, int64_t i,
                     const double *kb, const double *vb, const double *doi,
                     double *lse, double *D)
{
    int64_t j;
    int c, any = 0;
    double m = -INFINITY, l = 0.0, dd = 0.0;
    for (j = 0; j < len; j++) {
        double s = 0.0;
        if (!visible(i, j, W, S))
            continue;
        for (c = 0; c < d; c++)
            s += qi[c] * kb[j * d + c];
        s *= scale;
        if (!any || s > m)
            m = s;
        any = 1;
    }
    if (!any || i >= len)
        return 0;
    for (j = 0; j < len; j++) {
        double s = 0.0;
        if (!visible(i, j, W, S))
            continue;
        for (c = 0; c < d; c++)
            s += qi[c] * kb[j * d + c];
        l += exp(s * scale - m);
    }
    *lse = m + log(l);
    for (j = 0; j < len; j++) {
        double s = 0.0, p, dp = 0.0;
        if (!visible(i, j, W, S))
            continue;
        for (c = 0; c < d; c++)
            s += qi[c] * kb[j * d + c];
        p = exp(s * scale - *lse);
        for (c = 0; c < d; c++)
            dp += doi[c] * vb[j * d + c];
        dd += p * dp;
    }
    *D = dd;
    return 1;
}

/* dq_i = scale sum_j P_ij (dP_ij - D_i) k_j over row i's allowed keys. */
static void row_dq(int d, int W, int S, int len, double scale, const double *qi, int64_t i,
                   const double *kb, const double *vb, const double *doi, double lse,
                   double D, double *dqi)
{
    int64_t j;
    int c;
    for (c = 0; c < d; c++)
        dqi[c] = 0.0;
    for (j = 0; j < len; j++) {
        double s = 0.0, p, dp = 0.0, ds;
        if (!visible(i, j, W, S))
            continue;
        for (c = 0; c < d; c++)
            s += qi[c] * kb[j * d + c];
        p = exp(s * scale - lse);
        for (c = 0; c < d; c++)
            dp += doi[c] * vb[j * d + c];
        ds = p * (dp - D);
        for (c = 0; c < d; c++)
            dqi[c] += scale * ds * kb[j * d + c];
    }
}

/* dk_j, dv_j of key j of kv head g of sequence b: sums over the rows of every
 * query head of the group that see key j.  lse/D: per-row values ([B][H][N]),
 * valid where ok[] is set. */
static void key_grad(int H, int G, int N, int d, int W, int S, int len, double scale, int64_t b,
                     int64_t g, int64_t j, const double *q, const double *kb,
                     const double *vb, const double *dout, const double *lse,
                     const double *Dv, const unsigned char *ok, double *dkj, double *dvj)
{
    int64_t h, i;
    int c;
    for (c = 0; c < d; c++) {
        dkj[c] = 0.0;
        dvj[c] = 0.0;
    }
    if (j >= len)
        return;
    for (h = g * G; h < (g + 1) * G; h++) {
        for (i = 0; i < len; i++) {
            const int64_t row = (b * H + h) * (int64_t)N + i;
            const double *qi = q + row * d;
            const double *doi = dout + row * d;
            double s = 0.0, p, dp = 0.0, ds;
            if (!visible(i, j, W, S) || !ok[row])
                continue;
            for (c = 0; c < d; c++)
                s += qi[c] * kb[j * d + c];
            p = exp(s * scale - lse[row]);
            for (c = 0; c < d; c++)
                dp += doi[c] * vb[j * d + c];
            ds = p * (dp - Dv[row]);
            for (c = 0; c < d; c++) {
                dvj[c] += p * doi[c];
                dkj[c] += scale * ds * qi[c];
            }
        }
    }
}

/* Full backward.  q, dout, dq: [B][H][N][d]; k, v, dk, dv: [B][Hkv][N][d];
 * lse_out (may be NULL): [B][H][N] natural-log log-sum-exp of each row's
 * allowed scores, -inf for rows that see no key. */
void orc_bwd_sink(int B, int H, int Hkv, int N, int d, int W, int S, const double *q,
                  const double *k, const double *v, const double *dout, const int32_t *q_len,
                  double scale, double *dq, double *dk, double *dv, double *lse_out)
{
    const int G = H / Hkv;
    const int64_t rows = (int64_t)B * H * N;
    double *lse = malloc(sizeof(double) * (size_t)rows);
    double *Dv = malloc(sizeof(double) * (size_t)rows);
    unsigned char *ok = malloc((size_t)rows);
    int64_t r, key;

#pragma omp parallel for schedule(dynamic, 16)
    for (r = 0; r < rows; r++) {
        const int64_t b = r / ((int64_t)H * N), h = (r / N) % H, i = r % N;
        const int len = q_len ? q_len[b] : N;
        const int64_t g = h / G;
        const double *kb = k + ((b * Hkv + g) * (int64_t)N) * d;
        const double *vb = v + ((b * Hkv + g) * (int64_t)N) * d;
        int c;
        ok[r] = (unsigned char)row_stats(d, W, S, len, scale, q + r * d, i, kb, vb,
                                         dout + r * d, &lse[r], &Dv[r]);
        if (ok[r])
            row_dq(d, W, S, len, scale, q + r * d, i, kb, vb, dout + r * d, lse[r], Dv[r],
                   dq + r * d);
        else
            for (c = 0; c < d; c++)
                dq[r * d + c] = 0.0;
        if (lse_out)
            lse_out[r] = ok[r] ? lse[r] : -INFINITY;
    }
#pragma omp parallel for schedule(dynamic, 16)
    for (key = 0; key < (int64_t)B * Hkv * N; key++) {
        const int64_t b = key / ((int64_t)Hkv * N), g = (key / N) % Hkv, j = key % N;
        const int len = q_len ? q_len[b] : N;
        const double *kb = k + ((b * Hkv + g) * (int64_t)N) * d;
        const double *vb = v + ((b * Hkv + g) * (int64_t)N) * d;
        key_grad(H, G, N, d, W, S, len, scale, b, g, j, q, kb, vb, dout, lse, Dv, ok,
                 dk + key * d, dv + key * d);
    }
    free(lse); free(Dv); free(ok);
}

void orc_bwd(int B, int H, int Hkv, int N, int d, int W, const double *q, const double *k,
             const double *v, const double *dout, const int32_t *q_len, double scale,
             double *dq, double *dk, double *dv, double *lse_out)
{
    orc_bwd_sink(B, H, Hkv, N, d, W, 0, q, k, v, dout, q_len, scale, dq, dk, dv, lse_out);
}

/* The same gradients for selected entries only (large inputs): dq of rows
 * (qb, qh, qi)[r] and dk, dv of keys (kb_, kg, kj)[r].  Row values are
 * computed for exactly the rows each selection needs. */
void orc_bwd_sel_sink(int B, int H, int Hkv, int N, int d, int W, int S, const double *q,
                      const double *k, const double *v, const double *dout,
                      const int32_t *q_len, double scale, int nq_sel, const int32_t *qb,
                      const int32_t *qh, const int32_t *qi, double *dq_rows, int nk_sel,
                      const int32_t *kb_, const int32_t *kg, const int32_t *kj,
                      double *dk_rows, double *dv_rows)
{
    const int G = H / Hkv;
    int r;
    (void)B;
#pragma omp parallel for schedule(dynamic, 1)
    for (r = 0; r < nq_sel; r++) {
        const int64_t b = qb[r], h = qh[r], i = qi[r], g = h / G;
        const int len = q_len ? q_len[b] : N;
        const int64_t row = (b * H + h) * (int64_t)N + i;
        const double *kb = k + ((b * Hkv + g) * (int64_t)N) * d;
        const double *vb = v + ((b * Hkv + g) * (int64_t)N) * d;
        double lse, D;
        int c;
        if (row_stats(d, W, S, len, scale, q + row * d, i, kb, vb, dout + row * d, &lse, &D))
            row_dq(d, W, S, len, scale, q + row * d, i, kb, vb, dout + row * d, lse, D,
                   dq_rows + (int64_t)r * d);
        else
            for (c = 0; c < d; c++)
                dq_rows[(int64_t)r * d + c] = 0.0;
    }
    for (r = 0; r < nk_sel; r++) {
        const int64_t b = kb_[r], g = kg[r], j = kj[r];
        const int len = q_len ? q_len[b] : N;
        const double *kb = k + ((b * Hkv + g) * (int64_t)N) * d;
        const double *vb = v + ((b * Hkv + g) * (int64_t)N) * d;
        /* row values of every row that sees key j */
        double *lse = calloc((size_t)H * N, sizeof(double));
        double *Dv = calloc((size_t)H * N, sizeof(double));
        unsigned char *ok = calloc((size_t)H * N, 1);
        int64_t h;
        for (h = g * G; h < (g + 1) * G; h++) {
            int64_t i;
            /* rows that can see key j: j .. j+W-1, or every later row for a sink */
            const int64_t iend = (j < S || j + W >= N) ? N : j + W;
#pragma omp parallel for schedule(dynamic, 4)
            for (i = j; i < iend; i++) {
                const int64_t row = (b * H + h) * (int64_t)N + i;
                ok[h * N + i] = (unsigned char)row_stats(d, W, S, len, scale, q + row * d, i,
                                                         kb, vb, dout + row * d,
                                                         &lse[h * N + i], &Dv[h * N + i]);
            }
        }
        /* key_grad indexes row values as [b][h][i]; view this sequence's slice */
        key_grad(H, G, N, d, W, S, len, scale, 0, g, j, q + b * (int64_t)H * N * d, kb, vb,
                 dout + b * (int64_t)H * N * d, lse, Dv, ok, dk_rows + (int64_t)r * d,
                 dv_rows + (int64_t)r * d);
        free(lse); free(Dv); free(ok);
    }
}

void orc_bwd_sel(int B, int H, int Hkv, int N, int d, int W, const double *q,
                 const double *k, const double *v, const double *dout, const int32_t *q_len,
                 double scale, int nq_sel, const int32_t *qb, const int32_t *qh,
                 const int32_t *qi, double *dq_rows, int nk_sel, const int32_t *kb_,
                 const int32_t *kg, const int32_t *kj, double *dk_rows, double *dv_rows)
{
    orc_bwd_sel_sink(B, H, Hkv, N, d, W, 0, q, k, v, dout, q_len, scale, nq_sel, qb, qh, qi,
                     dq_rows, nk_sel, kb_, kg, kj, dk_rows, dv_rows);
}

/* ------------------------------------------------------------------------ */
/* Packed variable-length batch ("Dense vs sliding-window sparse attention"
 * §3.3 calls the varlen kernel with cu_seqlens; §5.2: in a batch the window
 * is per sequence, and a wrong split lets windows leak across sequences).
 * Sequence b owns tokens cu[b] .. cu[b+1]-1 of the packed axis; its token i
 * sits at logical position i and sees only its own sequence's keys, under
 * the same rule as orc_fwd_sink.  Layout is token-major:
 * q, o [total][H][d]; k, v [total][Hkv][d]. */
void orc_fwd_varlen(int B, int H, int Hkv, const int32_t *cu, int d, int W, int S,
                    const double *q, const double *k, const double *v, double scale,
                    double *o)
{
    const int G = H / Hkv;
    int b;
    for (b = 0; b < B; b++) {
        const int64_t t0 = cu[b];
        const int len = cu[b + 1] - cu[b];
        int h;
        for (h = 0; h < H; h++) {
            const int64_t g = h / G;
            int64_t i;
#pragma omp parallel for schedule(dynamic, 8)
            for (i = 0; i < len; i++) {
                const double **kr = malloc(sizeof(*kr) * (size_t)(len > 0 ? len : 1));
                const double **vr = malloc(sizeof(*vr) * (size_t)(len > 0 ? len : 1));
                int64_t *kp = malloc(sizeof(*kp) * (size_t)(len > 0 ? len : 1));
                double *sc = malloc(sizeof(*sc) * (size_t)(len > 0 ? len : 1));
                int j;
                for (j = 0; j < len; j++) {
                    kr[j] = k + ((t0 + j) * Hkv + g) * d;
                    vr[j] = v + ((t0 + j) * Hkv + g) * d;
                    kp[j] = j;
                }
                attend_row(d, W, S, scale, q + ((t0 + i) * H + h) * d, i, len, kr, vr, kp, sc,
                           o + ((t0 + i) * H + h) * d);
                free(kr); free(vr); free(kp); free(sc);
            }
        }
    }
}

/* ---------------------------------------------------------------------------
 * Persistent KV-cache size over a stack of layers [Ch10 §10.2].
 *
 * A windowed layer keeps at most its last W positions of K and V, so after T
 * tokens it holds min(T, W) rows per KV head; a full-history (global) layer
 * holds all T.  With L_s windowed and L_f global layers the pages estimate
 *     2 * B * G * d * s * [ L_s * min(T, W) + L_f * T ]      bytes
 * (G KV heads, s bytes per element, the 2 for K and V).  The counts must be
 * whole layers: the pages warn that a ratio such as 5:1 is not itself a
 * layer count.
 * READING (the pages only say the ratio is resolved into whole layers, and
 * that a stride option picks the windowed layers): the ratio a:b is a
 * repeating period of a windowed layers followed by b global ones, from
 * layer 0 upward; a stack of L layers takes the first L layers of that
 * pattern.
 * READING: a window of -1 marks a global layer, as a (-1, -1) window means
 * dense attention in [Blog §3.3].
 * --------------------------------------------------------------------------- */

/* Layer l of the repeating a:b pattern is windowed (1) or global (0). */
void orc_layer_plan(int L, int a, int b, uint8_t *is_local, int *L_s, int *L_f)
{
    int l, ns = 0, nf = 0;
    for (l = 0; l < L; l++) {
        const int local = (l % (a + b)) < a;
        is_local[l] = (uint8_t)local;
        if (local) ns++; else nf++;
    }
    *L_s = ns;
    *L_f = nf;
}

/* The pages' estimate with one window W for every windowed layer. */
int64_t orc_cache_bytes(int64_t B, int64_t G, int64_t d, int64_t s, int64_t T, int64_t W,
                        int64_t L_s, int64_t L_f)
{
    const int64_t kept = T < W ? T : W;
    return 2 * B * G * d * s * (L_s * kept + L_f * T);
}

/* The same count layer by layer, each layer with its own window W_layer[l]
 * (-1 = global), as in the per-layer window tip of [Blog §3.1]. */
int64_t orc_cache_bytes_layers(int64_t B, int64_t G, int64_t d, int64_t s, int64_t T, int L,
                               const int32_t *W_layer)
{
    int64_t total = 0;
    int l;
    for (l = 0; l < L; l++) {
        const int64_t w = W_layer[l];
        const int64_t kept = (w < 0 || T < w) ? T : w;
        total += 2 * B * G * d * s * kept;
    }
    return total;
}
