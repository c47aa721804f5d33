"""The pins are strong enough: every plausible slip planted in a copy of the oracle fails one.

Each mutant is a one-place textual change to oracle/oracle.c, compiled on the
CPU into a temporary library; the pin suite from oracle_pins.py is run against
it and at least one pin must fail.  Nothing here touches a GPU.
"""
import json
import os
import subprocess
import sys

import pytest

import oracle
from oracle_pins import ALL_PINS

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle", "oracle.c")

# (id, exact text in oracle.c, replacement) -- each a mistake one could plausibly make.
MUTANTS = [
    ("no_max_subtraction", "scores[j] = exp(scores[j] - mu);", "scores[j] = exp(scores[j]);"),
    ("min_instead_of_max", "if (scores[j] > mu) mu = scores[j];", "if (scores[j] < mu) mu = scores[j];"),
    ("sign_flip_exp", "scores[j] = exp(scores[j] - mu);", "scores[j] = exp(mu - scores[j]);"),
    ("dropped_scale", "scores[j] = scale * dot;", "scores[j] = dot;"),
    ("dropped_normalisation", "out[l] = acc / z;", "out[l] = acc;"),
    ("v_index_ignores_column", "vbase[j * vstride + l]", "vbase[j * vstride]"),
    ("k_used_as_q", "const float *qi = q + (b * S + i) * row + h * d;",
     "const float *qi = k + (b * S + i) * row + h * d;"),
    ("causal_excludes_diagonal", "int64_t n = causal ? i + 1 : S;", "int64_t n = causal ? i : S;"),
    ("causal_sees_next", "int64_t n = causal ? i + 1 : S;", "int64_t n = causal ? (i + 2 < S ? i + 2 : S) : S;"),
    ("head_offset_dropped_in_q", "const float *qi = q + (b * S + i) * row + h * d;",
     "const float *qi = q + (b * S + i) * row;"),
    ("token_stride_is_d", "attend_row(qi, k + b * S * row + h * d, row, v + b * S * row + h * d,\n                       row,",
     "attend_row(qi, k + b * S * row + h * d, d, v + b * S * row + h * d,\n                       d,"),
    ("gqa_modulo_map", "int64_t kh = h / group;", "int64_t kh = h % Hkv;"),
    ("decode_reads_max_len", "lens[mm], d, (double)scale, scores, out + mm * H * d + h * d);",
     "max_len, d, (double)scale, scores, out + mm * H * d + h * d);"),
    ("decode_one_short", "lens[mm], d, (double)scale, scores, out + mm * H * d + h * d);",
     "lens[mm] > 0 ? lens[mm] - 1 : 0, d, (double)scale, scores, out + mm * H * d + h * d);"),
    ("scatter_ignores_cache_len", "cache_lens[m] + r) * d;", "r) * d;"),
    ("scatter_rows_reversed", "cache_lens[m] + r) * d;", "cache_lens[m] + (n_new - 1 - r)) * d;"),
    ("scatter_head_major_swap", "int64_t dst = ((m * Hkv + kh) * max_len", "int64_t dst = ((kh * M + m) * max_len"),
    ("scatter_src_heads_major", "int64_t src = (m * n_new + r) * Hkv * d + kh * d;",
     "int64_t src = (m * Hkv + kh) * n_new * d + r * d;"),
    ("scatter_v_from_k", "memcpy(&bits, &v_new[src + l], 4);", "memcpy(&bits, &k_new[src + l], 4);"),
    ("empty_sequence_not_zero", "for (l = 0; l < d; ++l) out[l] = 0.0;", "for (l = 0; l < d; ++l) out[l] = 1.0;"),
    ("rows_entry_ignores_causal", "row, causal ? i + 1 : S, d,", "row, S, d,"),
    ("cached_offset_dropped", "vals, d, P + r + 1, d,", "vals, d, r + 1, d,"),
    ("cached_reads_cache_row_P", "                if (j < P) {", "                if (j <= P) {"),
    ("cached_new_rows_shifted", "int64_t c = (mm * n_new + (j - P)) * Hkv * d",
     "int64_t c = (mm * n_new + (j - P + 1 < n_new ? j - P + 1 : j - P)) * Hkv * d"),
    ("cached_rows_offset_dropped", "        n = P + r + 1; /* keys visible to this query */",
     "        n = r + 1; /* keys visible to this query */"),
    ("cached_modulo_head_map", "kh = h / (H / Hkv), r, j, l;", "kh = h % Hkv, r, j, l;"),
    ("slot_copy_one_block", "            int64_t s = (kh * src_max_len + r) * d;\n            int64_t t = ((slot * Hkv + kh) * max_len + r) * d;",
     "            int64_t s = (kh * seq_len + r) * d;\n            int64_t t = (slot * Hkv * max_len + kh * seq_len + r) * d;"),
    ("slot_copy_stride_uses_src_len", "int64_t t = ((slot * Hkv + kh) * max_len + r) * d;",
     "int64_t t = ((slot * Hkv + kh) * src_max_len + r) * d;"),
    ("slot_copy_one_row_short", "        for (r = 0; r < seq_len; ++r) {\n            int64_t s",
     "        for (r = 0; r + 1 < seq_len; ++r) {\n            int64_t s"),
    ("slot_copy_v_from_k", "memcpy(&bits, &src_v[s + l], 4);", "memcpy(&bits, &src_k[s + l], 4);"),
    ("round16_truncates", "r = nearbyint(x / q) * q;", "r = trunc(x / q) * q;"),
    ("round16_ties_away", "r = nearbyint(x / q) * q;", "r = round(x / q) * q;"),
    ("round16_bf16_seven_bits", "p = 8; emin = -126;", "p = 7; emin = -126;"),
    ("round16_no_subnormal_floor", "    if (e < emin) e = emin;\n", ""),
    ("round16_no_overflow", "if (fabs(r) > maxv) return copysign(INFINITY, x);", "(void)maxv;"),
    ("lowp_v_not_rounded", "oracle_round16(v, rv, n, fmt) == 0)\n        rc = oracle_prefill(rq, rk, rv,",
     "oracle_round16(v, rv, n, fmt) == 0)\n        rc = oracle_prefill(rq, rk, v,"),
    ("rope_sign_flip", "z = z * turn;", "z = z * conj(turn);"),
    ("rope_sin_cos_swapped", "double complex turn = cexp(I * a);", "double complex turn = sin(a) + I * cos(a);"),
    ("rope_exponent_uses_head_dim", "-2.0 * (double)k / (double)rotary_ndims", "-2.0 * (double)k / (double)d"),
    ("rope_exponent_off_by_one", "-2.0 * (double)k / (double)rotary_ndims", "-2.0 * (double)(k + 1) / (double)rotary_ndims"),
    ("rope_adjacent_pairs", "double complex z = (double)src[k] + I * (double)src[k + half];",
     "double complex z = (double)src[2 * k] + I * (double)src[2 * k + 1];"),
    ("rope_real_imag_swapped", "dst[k] = creal(z);\n                dst[k + half] = cimag(z);",
     "dst[k] = cimag(z);\n                dst[k + half] = creal(z);"),
    ("rope_row_index_as_position", "double a = (double)pos[t] * pow(", "double a = (double)t * pow("),
    ("rope_tail_zeroed", "for (l = rotary_ndims; l < d; ++l) dst[l] = (double)src[l];",
     "for (l = rotary_ndims; l < d; ++l) dst[l] = 0.0;"),
    ("cached_rope_drops_cache_offset", "pos[m * n_new + r] = cache_lens[m] + (int32_t)r;",
     "pos[m * n_new + r] = (int32_t)r;"),
    ("cached_rope_queries_unrotated", "rc = oracle_prefill_cached(qf, kf, v_new,", "rc = oracle_prefill_cached(q, kf, v_new,"),
    ("cached_rope_keys_unrotated", "rc = oracle_prefill_cached(qf, kf, v_new,", "rc = oracle_prefill_cached(qf, k_new, v_new,"),
    ("cached_rope_query_heads_as_kv_heads", "oracle_rope(q, pos, qr, M * n_new, H, d,", "oracle_rope(q, pos, qr, M * n_new * (H / Hkv), Hkv, d,"),
]


_RUNNER = """
import json, sys
sys.path[:0] = [{root!r}, {tests!r}]
import oracle
from oracle_pins import ALL_PINS
orc = oracle.Oracle(oracle.load({lib!r}))
failed = []
for name, pin in ALL_PINS:
    try:
        pin(orc)
    except (AssertionError, ValueError, FloatingPointError):
        failed.append(name)
print(json.dumps(failed))
"""


def _failing_pins(lib_path):
    """Run every pin against one mutant in a fresh process (a mutant may corrupt memory)."""
    tests = os.path.dirname(os.path.abspath(__file__))
    code = _RUNNER.format(root=os.path.dirname(tests), tests=tests, lib=lib_path)
    res = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=300)
    assert res.returncode == 0, f"pin run crashed: {res.stderr[-2000:]}"
    return json.loads(res.stdout.strip().splitlines()[-1])


@pytest.mark.parametrize("mid,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(mid, old, new, tmp_path):
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation site for {mid} must be unique in oracle.c"
    mutated = tmp_path / f"oracle_{mid}.c"
    mutated.write_text(src.replace(old, new))
    lib = tmp_path / f"liboracle_{mid}.so"
    oracle.build(str(mutated), str(lib))
    failed = _failing_pins(str(lib))
    assert failed, f"mutant {mid} passed every pin"
