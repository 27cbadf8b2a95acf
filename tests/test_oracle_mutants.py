"""The oracle's pins must be able to fail (CPU only).

Each case plants one plausible mistake into a copy of oracle/oracle.c, builds
it into a temporary library and runs the pin suite against it through the
ORACLE_LIB override; the suite has to fail for every mutant.  Nothing here
touches the GPU or the library under test.
"""
import concurrent.futures as cf
import os
import subprocess
import sys
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "oracle.c")

MUTANTS = {
    "dropped_scale": ("w[t] = scale * dot;", "w[t] = dot;"),
    "rope_sign": ("out[row + 2 * i] = x0 * c - x1 * sn;", "out[row + 2 * i] = x0 * c + x1 * sn;"),
    "rope_freq_sign": ("pow(theta, -2.0 * i / D)", "pow(theta, 2.0 * i / D)"),
    "rope_half_split": ("double x1 = load(x, row + 2 * i + 1, dt);",
                        "double x1 = load(x, row + i + D / 2, dt);"),
    "rope_ignores_offset": ("double p = (double)(off + s);", "double p = (double)(s);"),
    "prefill_modulo_groups": ("int j = h / G;\n                size_t q_base",
                              "int j = h % Hkv;\n                size_t q_base"),
    "causal_off_by_one": ("i + 1, D,", "i, D,"),
    "value_from_keys": ("o[d] += w[t] * load(v,", "o[d] += w[t] * load(k,"),
    "decode_modulo_groups": ("int j = h / G;\n                int n",
                             "int j = h % Hkv;\n                int n"),
    "decode_length_short": ("int n = seqlens[b];", "int n = seqlens[b] > 0 ? seqlens[b] - 1 : 0;"),
    "bf16_truncates": ("double r = rint(ldexp(x, -k));", "double r = trunc(ldexp(x, -k));"),
    "f32_truncates": ("out[i] = (float)in[i]; /* C conversion",
                      "{ float f = (float)in[i]; if (fabs((double)f) > fabs(in[i])) "
                      "f = nextafterf(f, 0.0f); out[i] = f; } /* C conversion"),
    "f32_flushes_subnormals": ("out[i] = (float)in[i]; /* C conversion",
                               "out[i] = fabs(in[i]) < 0x1p-126 ? (float)copysign(0.0, in[i]) "
                               ": (float)in[i]; /* C conversion"),
    "missing_normalisation": ("o[d] /= l;", "o[d] /= 1.0;"),
    "paged_ignores_table": ("size_t pg = (size_t)block_table[(size_t)b * max_pages + t / page_size];",
                            "size_t pg = (size_t)b * max_pages + t / page_size;"),
    "paged_row_in_page": ("(size_t)(t % page_size)) * D;", "(size_t)(t / page_size)) * D;"),
    "paged_head_major_pages": ("((pg * Hkv + j) * page_size", "((j * num_pages + pg) * page_size"),
    "window_off_by_one": ("? len - window : 0;\n                double *o",
                          "? len - window + 1 : 0;\n                double *o"),
    "paged_normalisation": ("o[d] = o[d] / l;", "o[d] = o[d];"),
    "lse_without_log": ("const double lse = top + log(z);", "const double lse = top;"),
    "backward_drops_delta": ("delta += exp(sc[t] - lse) * dp;", "delta += 0.0 * dp;"),
    "dq_missing_scale": ("g[d] += scale * ds * load(k,", "g[d] += ds * load(k,"),
    "dq_from_values": ("g[d] += scale * ds * load(k,", "g[d] += scale * ds * load(v,"),
    "dq_sees_one_key_less": ("for (int t = 0; t <= i; ++t) {\n                    double s = 0.0",
                             "for (int t = 0; t < i; ++t) {\n                    double s = 0.0"),
    "dk_missing_scale": ("gk[d] += scale * ds *", "gk[d] += ds *"),
    "dv_weighted_by_ds": ("gv[d] += p * load(dout,", "gv[d] += ds * load(dout,"),
    "dkv_first_head_only": ("for (int h = j * G; h < (j + 1) * G; ++h)",
                            "for (int h = j * G; h < j * G + 1; ++h)"),
    "dkv_skips_own_query": ("for (int i = t; i < S; ++i)", "for (int i = t + 1; i < S; ++i)"),
    "rope_transpose_is_the_rotation": ("out[at + 2 * j] = g0 * ca + g1 * sa;",
                                       "out[at + 2 * j] = g0 * ca - g1 * sa;"),
    "rope_transpose_ignores_offset": ("(double)(base + t) * pow", "(double)(t) * pow"),
    "cca_conv_taps_reversed": ("acc += load(cw, ((size_t)h * W + i) * D + c, dt) *",
                               "acc += load(cw, ((size_t)h * W + (W - 1 - i)) * D + c, dt) *"),
    "cca_conv_wraps_around": ("if (src < 0)\n                                continue;",
                              "if (src < 0)\n                                src += S;"),
    "cca_conv_looks_ahead": ("int src = t - i;", "int src = t + i < S ? t + i : -1;"),
    "cca_mix_transposed": ("load(mw, ((size_t)h * D + c) * D + c2, dt)",
                           "load(mw, ((size_t)h * D + c2) * D + c, dt)"),
    "cca_mean_without_half": ("mean[(size_t)j * D + c] = 0.5 * (qsum / G + kv);",
                              "mean[(size_t)j * D + c] = (qsum / G + kv);"),
    "cca_mean_of_sum_not_average": ("0.5 * (qsum / G + kv)", "0.5 * (qsum + kv)"),
    "cca_mean_modulo_groups": ("mean + (size_t)(isq ? h / G : h) * D",
                               "mean + (size_t)(isq ? h % Hkv : h) * D"),
    "cca_mean_dropped_from_keys": ("out[c] = acc + mrow[c];", "out[c] = acc + (isq ? mrow[c] : 0.0);"),
    "cca_shift_wrong_half": ("if (c < D / 2)\n                            val = load(v, at, dt);",
                             "if (c >= D / 2)\n                            val = load(v, at, dt);"),
    "cca_shift_from_next_token": ("val = t > 0 ? load(v, at - (size_t)D, dt) : 0.0;",
                                  "val = t + 1 < S ? load(v, at + (size_t)D, dt) : 0.0;"),
    "cca_rope_misses_keys": ("oracle_rope(k_out, tmp, OR_F64, B, Hkv, S, D, pos_offset, theta);",
                             "memcpy(k_out, tmp, sizeof(double) * (size_t)B * Hkv * S * D);"),
    "cca_bwd_mix_not_transposed": ("g += load(mw, ((size_t)h * D + c2) * D + c, dt) *",
                                   "g += load(mw, ((size_t)h * D + c) * D + c2, dt) *"),
    "cca_bwd_conv_not_reversed": ("acc += tap * ds[(size_t)(t + i) * D + c];",
                                  "acc += tap * (t - i >= 0 ? ds[(size_t)(t - i) * D + c] : 0.0);"),
    "cca_bwd_mean_weight_without_group": ("const double mean_w = isq ? 0.5 / G : 0.5;",
                                          "const double mean_w = 0.5;"),
    "cca_bwd_shift_from_previous_token": ("dv[at] = t + 1 < S ? load(gv, at + (size_t)D, dt) : 0.0;",
                                          "dv[at] = t > 0 ? load(gv, at - (size_t)D, dt) : 0.0;"),
    "cca_bwd_no_rope_transpose": ("if (theta > 0.0) {\n        oracle_rope_transpose(aq",
                                  "if (0) {\n        oracle_rope_transpose(aq"),
    "cca_bwd_dmix_transposed": ("dmix[(size_t)c * D + c2] += av *", "dmix[(size_t)c2 * D + c] += av *"),
    "cca_bwd_dconv_unshifted": ("ds[(size_t)t * D + c] * load(x, (row0 + t - i) * D + c, dt);",
                                "ds[(size_t)t * D + c] * load(x, (row0 + t) * D + c, dt);"),
}


def _run_mutant(name, tmp):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation site for {name} not unique"
    mpath = os.path.join(tmp, f"{name}.c")
    open(mpath, "w").write(src.replace(old, new))
    lib = os.path.join(tmp, f"lib{name}.so")
    subprocess.run(["gcc", "-O2", "-ffp-contract=off", "-fopenmp", "-shared", "-fPIC",
                    mpath, "-o", lib, "-lm"], check=True)
    env = dict(os.environ, ORACLE_LIB=lib, OMP_NUM_THREADS="1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_pins.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    return r.returncode


def test_every_planted_mistake_fails_a_pin():
    with tempfile.TemporaryDirectory() as tmp:
        with cf.ThreadPoolExecutor(max_workers=min(6, os.cpu_count() or 1)) as ex:
            codes = dict(zip(MUTANTS, ex.map(lambda n: _run_mutant(n, tmp), MUTANTS)))
    survivors = [n for n, rc in codes.items() if rc == 0]
    assert not survivors, f"mutants not caught by the pins: {survivors}"
    # rc 1 = tests failed; anything else would mean the run itself broke
    assert all(rc == 1 for rc in codes.values()), codes
