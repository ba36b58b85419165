// cache_plan.cpp -- host-side KV-cache sizing for stacks of windowed and
// global layers ("LLMs from scratch, chapter 10: SWA and DSA", §10.2; the
// per-layer window tip of "Dense attention vs sliding-window sparse
// attention", §3.1).  Pure integer arithmetic, no device work.
#include <stdint.h>

#include "../../include/swa.h"
#include "swa_internal.h"

using swa::fail;

// Layers repeat a period of n_local windowed layers followed by n_global
// global ones, starting at layer 0; a stack of L layers takes the first L.
extern "C" int swa_layer_plan(int L, int n_local, int n_global, int W, int32_t *W_layer,
                              int32_t *L_s, int32_t *L_f) {
    swa::clear_error();
    if (L < 0) return fail(SWA_EINVAL, "swa_layer_plan: L=%d must be >= 0", L);
    if (n_local < 0 || n_global < 0 || n_local > INT32_MAX - n_global || n_local + n_global < 1)
        return fail(SWA_EINVAL, "swa_layer_plan: ratio %d:%d needs non-negative parts, not both 0",
                    n_local, n_global);
    if (W < 1) return fail(SWA_EINVAL, "swa_layer_plan: window W=%d must be >= 1", W);
    if (!L_s || !L_f || (L > 0 && !W_layer))
        return fail(SWA_EINVAL, "swa_layer_plan: NULL output");
    const int period = n_local + n_global;
    // whole periods first, then the windowed head of the last partial period
    const int64_t full = L / period, rest = L % period;
    const int64_t ns = full * n_local + (rest < n_local ? rest : n_local);
    int phase = 0;
    for (int l = 0; l < L; l++) {
        W_layer[l] = phase < n_local ? W : -1;
        if (++phase == period) phase = 0;
    }
    *L_s = (int32_t)ns;
    *L_f = (int32_t)(L - ns);
    return SWA_OK;
}

extern "C" int swa_cache_bytes(int B, int G, int d, int elem_bytes, int64_t T, int L,
                               const int32_t *W_layer, int64_t *bytes) {
    swa::clear_error();
    if (B < 1 || G < 1 || d < 1 || elem_bytes < 1)
        return fail(SWA_EINVAL, "swa_cache_bytes: B=%d G=%d d=%d elem_bytes=%d must be >= 1", B,
                    G, d, elem_bytes);
    if (T < 0) return fail(SWA_EINVAL, "swa_cache_bytes: T=%lld must be >= 0", (long long)T);
    if (L < 0) return fail(SWA_EINVAL, "swa_cache_bytes: L=%d must be >= 0", L);
    if (!bytes || (L > 0 && !W_layer)) return fail(SWA_EINVAL, "swa_cache_bytes: NULL pointer");
    // rows of K (and as many of V) kept per KV head, summed over layers
    int64_t rows = 0;
    for (int l = 0; l < L; l++) {
        const int32_t w = W_layer[l];
        if (w < 1 && w != -1)
            return fail(SWA_EINVAL, "swa_cache_bytes: W_layer[%d]=%d (need >= 1, or -1 = global)",
                        l, w);
        const int64_t kept = (w == -1 || T < w) ? T : (int64_t)w;
        if (__builtin_add_overflow(rows, kept, &rows))
            return fail(SWA_EINVAL, "swa_cache_bytes: row count overflows int64");
    }
    int64_t per_row = 2;  // K and V
    if (__builtin_mul_overflow(per_row, (int64_t)B, &per_row) ||
        __builtin_mul_overflow(per_row, (int64_t)G, &per_row) ||
        __builtin_mul_overflow(per_row, (int64_t)d, &per_row) ||
        __builtin_mul_overflow(per_row, (int64_t)elem_bytes, &per_row) ||
        __builtin_mul_overflow(per_row, rows, bytes))
        return fail(SWA_EINVAL, "swa_cache_bytes: byte count overflows int64");
    return SWA_OK;
}
