"""Plant plausible mistakes in a copy of the oracle (on the CPU) and check
that the pin suite rejects every one of them.

Each mutant is the oracle's C source with one textual change, compiled with
the same flags into a temporary library; the pin tests then run against it in
a child process and must fail.
"""
import os
import subprocess
import sys
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "attn_oracle.c")

MUTANTS = {
    "head_map_modulo": ("const int r = h / g;", "const int r = h % c->Hkv;"),
    "causal_not_end_aligned": ("int64_t p = (int64_t)i + kv_length(c, b) - q_length(c, b);",
                               "int64_t p = (int64_t)i;"),
    "causal_off_by_one": ("if (c->causal && j > p)", "if (c->causal && j >= p)"),
    "mask_ignored": ("if (c->mask && c->mask[(int64_t)b * c->Skv + j] == 0)", "if (0)"),
    "default_scale_wrong": ("return (double)(float)(1.0 / sqrt((double)D));",
                            "return 1.0 / (double)D;"),
    "lse_base_two": ("*lse_out = m + log(l);", "*lse_out = m + log2(l);"),
    "lse_shift_dropped": ("*lse_out = m + log(l);", "*lse_out = log(l);"),
    "empty_row_nan": ("o_row[d] = 0.0;", "o_row[d] = NAN;"),
    "page_offset_unscaled": ("row = phys_page * c->page_size + in_page;",
                             "row = phys_page + in_page;"),
    "scores_read_v": ("kv_value(c, 0, k_off + d);", "kv_value(c, 1, k_off + d);"),
    "fp16_exponent_bias": ("mag = ldexp((double)(1024 + frac), e - 25);",
                           "mag = ldexp((double)(1024 + frac), e - 24);"),
    "bf16_low_bit": ("uint32_t u = (uint32_t)bits << 16;",
                     "uint32_t u = ((uint32_t)bits << 16) | 1u;"),
    "score_sign": ("s[j] = c->alpha * dot;", "s[j] = -c->alpha * dot;"),
    "dot_drops_last_term": ("for (int d = 0; d < D; ++d)\n            dot +=",
                            "for (int d = 0; d < D - 1; ++d)\n            dot +="),
    "window_left_off_by_one": ("j < p - c->window_left", "j <= p - c->window_left"),
    "window_right_off_by_one": ("j > p + c->window_right", "j >= p + c->window_right"),
    "window_left_ignored": ("if (c->window_left != -1 && j < p - c->window_left)", "if (0)"),
    "window_sides_swapped": ("j < p - c->window_left", "j < p - c->window_right"),
    "window_not_at_query_position": ("j > p + c->window_right", "j > i + c->window_right"),
    "softcap_ignored": ("if (c->softcap > 0.0) /*", "if (0) /*"),
    "softcap_outer_factor_dropped": ("s[j] = c->softcap * tanh(s[j] / c->softcap);",
                                     "s[j] = tanh(s[j] / c->softcap);"),
    "softcap_before_scale": ("s[j] = c->softcap * tanh(s[j] / c->softcap);",
                             "s[j] = c->alpha * c->softcap * tanh(dot / c->softcap);"),
    "sink_scaled": ("const double sink = c->sinks ? (double)c->sinks[h] : -INFINITY;",
                    "const double sink = c->sinks ? c->alpha * (double)c->sinks[h] : -INFINITY;"),
    "sink_capped": ("const double sink = c->sinks ? (double)c->sinks[h] : -INFINITY;",
                    "const double sink = c->sinks ? (c->softcap > 0.0 ? c->softcap * tanh(c->sinks[h] / c->softcap) : c->sinks[h]) : -INFINITY;"),
    "sink_left_out_of_denominator": ("l += exp(sink - m);", "l += 0.0;"),
    "empty_row_lse_ignores_sink": ("*lse_out = n_visible == 0 ? sink : INFINITY;",
                                   "*lse_out = n_visible == 0 ? -INFINITY : INFINITY;"),
    "varlen_position_uses_request_0": ("int64_t p = (int64_t)i + kv_length(c, b) - q_length(c, b);",
                                       "int64_t p = (int64_t)i + kv_length(c, b) - q_length(c, 0);"),
    "varlen_keys_at_query_offsets": ("row = (int64_t)c->cu_kv[b] + j;", "row = (int64_t)c->cu_q[b] + j;"),
    "varlen_lse_batched_layout": ("lse[(int64_t)h * c->total_q + q_row(c, b, i)] = lse_rows[t++];",
                                  "lse[q_row(c, b, i) * c->Hq + h] = lse_rows[t++];"),
    "e4m3_ties_to_odd": ("(err == best_err && (c & 1) == 0)", "(err == best_err && (c & 1) == 1)"),
    "e4m3_overflow_to_nan": ("    if (a >= 448.0)\n        return sign | 0x7e;", "    if (a > 448.0)\n        return sign | 0x7f;"),
    "e4m3_subnormal_step": ("mag = ldexp((double)f, -9);", "mag = ldexp((double)f, -10);"),
    "fp8_scale_multiplies": ("float kq = (float)decode(k, src, dtype) / k_scale;",
                             "float kq = (float)decode(k, src, dtype) * k_scale;"),
    "fp8_read_scales_swapped": ("* (which ? c->v_scale : c->k_scale);",
                                "* (which ? c->k_scale : c->v_scale);"),
    "fp8_read_scale_dropped": ("* (which ? c->v_scale : c->k_scale);", "* 1.0;"),
    "fp8_read_as_16bit": ("    if (c->cache_fp8)\n        return e4m3_value(",
                          "    if (0)\n        return e4m3_value("),
    "fp8_append_writes_v_with_k_scale": ("(int64_t)num_pages * page_size, cache_fp8, k_scale, v_scale,",
                                         "(int64_t)num_pages * page_size, cache_fp8, k_scale, k_scale,"),
    "write_skips_slot_zero": ("        if (slot[n] < 0)\n            continue;", "        if (slot[n] <= 0)\n            continue;"),
    "append_position_off_by_one": ("int64_t pos = (int64_t)cache_seqlens[b] + (i - cu_q[b]);",
                                   "int64_t pos = (int64_t)cache_seqlens[b] + (i - cu_q[b]) + 1;"),
    "append_lengths_not_grown": ("lens[b] = cache_seqlens[b] + (cu_q[b + 1] - cu_q[b]);", "lens[b] = cache_seqlens[b];"),
    "bwd_D_ignores_o": ("Di += decode(dout, qo + d, dtype) * o[qo + d];", "Di += 0.0 * o[qo + d];"),
    "bwd_dq_unscaled": ("dq[qo + d] += alpha * ds * decode(k, ko + d, dtype);",
                        "dq[qo + d] += ds * decode(k, ko + d, dtype);"),
    "bwd_dv_uses_dS": ("dv[ko + d] += p * decode(dout, qo + d, dtype);",
                       "dv[ko + d] += ds * decode(dout, qo + d, dtype);"),
    "bwd_dk_reads_k": ("dk[ko + d] += alpha * ds * decode(q, qo + d, dtype);",
                       "dk[ko + d] += alpha * ds * decode(k, ko + d, dtype);"),
    "bwd_lse_unshifted": ("const double p = exp(alpha * s - l_i);", "const double p = exp(alpha * s);"),
    "bwd_dp_uses_k": ("dp += decode(dout, qo + d, dtype) * decode(v, ko + d, dtype);",
                      "dp += decode(dout, qo + d, dtype) * decode(k, ko + d, dtype);"),
    "value_sum_skips_first_key": ("for (int64_t j = 0; j < n; ++j) {\n            if (!visible(c, b, i, j))\n                continue;\n            acc +=",
                                  "for (int64_t j = 1; j < n; ++j) {\n            if (!visible(c, b, i, j))\n                continue;\n            acc +="),
}

PIN_FILES = ["test_oracle_pins.py", "test_oracle_pins_window_softcap.py",
             "test_oracle_pins_varlen_sinks.py", "test_oracle_pins_kv_write.py",
             "test_oracle_pins_bwd.py", "test_oracle_pins_fp8_cache.py"]

PLUGIN = "import os, oracle\noracle._LIB = os.environ['ORACLE_MUTANT_LIB']\n"


@pytest.fixture(scope="module")
def workdir():
    with tempfile.TemporaryDirectory() as d:
        with open(os.path.join(d, "oracle_mutant_plugin.py"), "w") as f:
            f.write(PLUGIN)
        yield d


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_reject_planted_mistake(name, workdir):
    before, after = MUTANTS[name]
    with open(SRC) as f:
        src = f.read()
    assert before in src, f"mutation site for {name} no longer exists in the oracle"
    csrc = os.path.join(workdir, f"{name}.c")
    lib = os.path.join(workdir, f"{name}.so")
    with open(csrc, "w") as f:
        f.write(src.replace(before, after, 1))
    subprocess.run(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp",
                    "-ffp-contract=off", csrc, "-o", lib, "-lm"], check=True)
    env = dict(os.environ, ORACLE_MUTANT_LIB=lib,
               PYTHONPATH=os.pathsep.join([workdir, ROOT]), OMP_NUM_THREADS="2")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        "-p", "oracle_mutant_plugin",
                        *[os.path.join(ROOT, "tests", f) for f in PIN_FILES]],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode == 1, f"mutant {name} survived the pins:\n{r.stdout[-2000:]}"
