"""Planted mistakes in the oracle must be caught by its pins (CPU only).

Each case copies ``oracle/swa_oracle.c`` to a temporary directory, replaces one
fragment with a plausible bug (an off-by-one window, a dropped term, a wrong
index or operand, a ring bookkeeping slip), compiles it with gcc and runs the
pins against it: at least one pin must fail.  Mutations are chosen so that the
mutant never reads outside its arrays.
"""
import os

import pytest

import oracle
from pins import PINS

MUTANTS = {
    # the window boundary read as (t - j) > W, the slip the SWA chapter warns of
    "window_off_by_one": ("kpos >= qpos - W + 1;", "kpos >= qpos - W;"),
    "no_causal_bound": ("return kpos <= qpos && kpos >= qpos - W + 1;",
                        "return kpos >= qpos - W + 1;"),
    "no_max_subtraction": ("e = exp(scratch[j] - m);", "e = exp(scratch[j]);"),
    "scale_dropped": ("s *= scale;", "s *= 1.0;"),
    "gqa_interleaved": ("h / G", "h % Hkv"),
    "k_used_for_v": ("out[c] += e * vrow[j][c];", "out[c] += e * krow[j][c];"),
    "no_normalisation": ("out[c] /= l;", "out[c] /= 1.0;"),
    "chunk_key_position_shift": ("kp[nsink + r] = p0 - old_len + r;",
                                 "kp[nsink + r] = p0 - old_len + r + 1;"),
    "chunk_query_position_shift": ("p0 + t,\n", "p0 + t + 1,\n"),
    "ring_fill_ignores_start": ("slot = (*start + *len) % W;", "slot = *len % W;"),
    "ring_start_not_advanced": ("*start = (*start + 1) % W;", "*start = *start % W;"),
    "decode_query_position": ("qpos = (int64_t)next_pos[b] - 1;",
                              "qpos = (int64_t)next_pos[b];"),
    "decode_key_position_shift": ("kp[nsink + r] = (int64_t)next_pos[b] - len + r;",
                                  "kp[nsink + r] = (int64_t)next_pos[b] - len + r - 1;"),
    "padding_row_kept": ("if (i >= len) { /* padded row */", "if (i > len) {"),
    "full_threshold": ("(count == area ? 1 : 2)", "(count * 2 >= area ? 1 : 2)"),
    "edge_area_not_clipped": ("const int64_t area = (int64_t)(i1 - i0) * (j1 - j0);",
                              "const int64_t area = (int64_t)tile_q * tile_k;"),
    "ring_slot_position_shift": ("kpos[NS + slot] = (int64_t)next_pos[b] - cache_len[b] + r;",
                                 "kpos[NS + slot] = (int64_t)next_pos[b] - cache_len[b] + r + 1;"),
    "bwd_row_D_dropped": ("ds = p * (dp - D);", "ds = p * dp;"),
    "bwd_key_D_dropped": ("ds = p * (dp - Dv[row]);", "ds = p * dp;"),
    "bwd_dk_scale_dropped": ("dkj[c] += scale * ds * qi[c];", "dkj[c] += ds * qi[c];"),
    "bwd_dv_uses_ds": ("dvj[c] += p * doi[c];", "dvj[c] += ds * doi[c];"),
    "bwd_dq_uses_v": ("dqi[c] += scale * ds * kb[j * d + c];",
                      "dqi[c] += scale * ds * vb[j * d + c];"),
    "bwd_lse_no_log": ("*lse = m + log(l);", "*lse = m + l;"),
    "bwd_group_first_head_only": ("for (h = g * G; h < (g + 1) * G; h++) {",
                                  "for (h = g * G; h < g * G + 1; h++) {"),
    "sink_bound_off_by_one": ("(kpos < S && kpos <= qpos)", "(kpos <= S && kpos <= qpos)"),
    "sink_not_causal": ("(kpos < S && kpos <= qpos)", "(kpos < S)"),
    "sink_decode_double_count": ("nsink = (int)(S < oldest ? S : oldest);", "nsink = S;"),
    "chunk_sink_cache_not_written": ("            if (p0 + t < S) {", "            if (p0 + t < 0) {"),
    "chunk_sink_double_count": ("const int nsink = (int)(S < oldest ? S : (oldest > 0 ? oldest : 0));",
                                "const int nsink = S;"),
    "ring_sink_counted_twice": (": visible(qpos[ii], kpos[jj], W, 0) && kpos[jj] >= S))",
                                ": visible(qpos[ii], kpos[jj], W, 0) && kpos[jj] >= 0))"),
    "sink_segment_ignores_causality": ("? kpos[jj] <= qpos[ii]", "? kpos[jj] >= 0"),
    "sink_cache_not_written": ("if (S > 0 && next_pos[b] < S) {", "if (S > 0 && next_pos[b] < 0) {"),
    "varlen_key_from_previous_sequence": ("kr[j] = k + ((t0 + j) * Hkv + g) * d;",
                                          "kr[j] = k + ((t0 + j - (j == 0 && t0 > 0)) * Hkv + g) * d;"),
    "varlen_query_position_global": ("attend_row(d, W, S, scale, q + ((t0 + i) * H + h) * d, i, len,",
                                     "attend_row(d, W, S, scale, q + ((t0 + i) * H + h) * d, t0 + i, len,"),
    "cache_kv_factor_dropped": ("return 2 * B * G * d * s * (L_s * kept + L_f * T);",
                                "return B * G * d * s * (L_s * kept + L_f * T);"),
    "cache_window_not_clipped": ("const int64_t kept = T < W ? T : W;",
                                 "const int64_t kept = W;"),
    "cache_layers_global_ignored": ("const int64_t kept = (w < 0 || T < w) ? T : w;",
                                    "const int64_t kept = (T < w) ? T : (w < 0 ? 0 : w);"),
    "layer_plan_global_first": ("const int local = (l % (a + b)) < a;",
                                "const int local = (l % (a + b)) >= b;"),
    "layer_plan_fractional_count": ("if (local) ns++; else nf++;",
                                    "if (local) ns++; else nf++;\n        if (l == L - 1) "
                                    "ns = L * a / (a + b), nf = L - ns;"),
    # the selected-row forward: the KV group and the valid length of its row
    "rows_group_interleaved": ("const int64_t g = h / G;\n        const int len = q_len ? q_len[b] : N;",
                               "const int64_t g = h % Hkv;\n        const int len = q_len ? q_len[b] : N;"),
    "rows_length_of_first_sequence": ("const int64_t g = h / G;\n        const int len = q_len ? q_len[b] : N;",
                                      "const int64_t g = h / G;\n        const int len = q_len ? q_len[0] : N;"),
    "csr_row_ptr_shift": ("row_ptr[(int64_t)b * nqt + qt + 1] = (int32_t)nnz;",
                          "row_ptr[(int64_t)b * nqt + qt + 1] = (int32_t)(nnz - (nnz > 0));"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path):
    old, new = MUTANTS[name]
    with open(oracle.SRC) as f:
        src = f.read()
    assert old in src, "mutation anchor missing: %r" % old
    mutated = src.replace(old, new)
    path = os.path.join(str(tmp_path), "mutant.c")
    with open(path, "w") as f:
        f.write(mutated)
    lib = oracle.build(force=True, src=path, out=os.path.join(str(tmp_path), "mutant.so"))
    O = oracle.Oracle(lib)
    caught = []
    for pin in PINS:
        try:
            pin(O)
        except AssertionError:
            caught.append(pin.__name__)
            break
    assert caught, "no pin caught the planted mistake %s" % name
