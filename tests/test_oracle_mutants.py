"""Planted mistakes in the oracle must be caught by its pins (CPU only).

Each case copies oracle/ttref.c, applies one plausible slip (a dropped scale, a flipped
sign, a wrong KV-head index, a transposed layout, values read from K, a dropped block key,
>= instead of >, a wrong tie rule, a missing fallback, a cache update at the wrong rows,
without the length bump or with an off-by-one fit test, an LM head read transposed, from
the wrong sequence, short of its last feature or with a flipped product; a Mamba-2 scan with a
flipped decay, no softplus, no skip term, a wrong head-to-group map, an unseeded state, the
update reading C, the readout before the update or the decay applied to the new input; an
adaLN without the mean, without the 1 +, with shift and scale or gate slots mixed up, without
the layer's offsets or with eps outside the root), builds that copy into a temporary library
and runs both pin suites against it in a child process. The suites must fail.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "ttref.c")

MUTANTS = {
    "no_scale": ("s[j] = dot * inv_sqrt_d;", "s[j] = dot;"),
    "exp_sign": ("s[j] = exp(s[j] - mx);", "s[j] = exp(mx - s[j]);"),
    "kv_head_modulo": ("const int g = h / G;", "const int g = h % Hkv;"),
    "blk_layout_transposed": ("koff = (((size_t)b * S + (j - nctx)) * Hkv + g) * D;",
                              "koff = ((size_t)b * S + (j - nctx) + (size_t)g * S) * D;"),
    "values_from_keys": ("vbase = v_ctx;", "vbase = k_ctx;"),
    "drop_last_block_key": ("const int n = nctx + S;", "const int n = nctx + S - 1;"),
    "threshold_ge": ("committed[r] = (uint8_t)(conf > gamma);", "committed[r] = (uint8_t)(conf >= gamma);"),
    "argmax_tie_highest": ("if (x > m) {", "if (x >= m) {"),
    "fallback_tie_highest": ("if (conf > best_conf) {", "if (conf >= best_conf) {"),
    "no_fallback": ("if (any_masked && !any_committed)", "if (0)"),
    "z_sign": ("z += exp(ttref_load(logits, off + v, dtype) - m);",
               "z += exp(m - ttref_load(logits, off + v, dtype));"),
    "lmhead_weight_transposed": ("ttref_load(weight, woff + k, TTREF_BF16);",
                                 "ttref_load(weight, (size_t)k * V + v, TTREF_BF16);"),
    "lmhead_hidden_ignores_sequence": ("const size_t hoff = r * (size_t)K;",
                                       "const size_t hoff = (size_t)i * K;"),
    "lmhead_drops_last_feature": ("for (int k = 0; k < K; ++k)\n                    dot +=",
                                  "for (int k = 0; k < K - 1; ++k)\n                    dot +="),
    "lmhead_product_sign": ("dot += ttref_load(hidden, hoff + k, TTREF_BF16) *",
                            "dot -= ttref_load(hidden, hoff + k, TTREF_BF16) *"),
    "append_ignores_length": ("const size_t dst = ((size_t)b * Lmax + n + i) * row;",
                              "const size_t dst = ((size_t)b * Lmax + i) * row;"),
    "append_no_bump": ("ctx_len[b] = n + S;", "ctx_len[b] = n;"),
    "append_fit_off_by_one": ("(long long)n + S > Lmax", "(long long)n + S >= Lmax"),
    "append_values_from_keys": ("memcpy((char *)v_ctx + dst, (const char *)v_new + src, row);",
                                "memcpy((char *)v_ctx + dst, (const char *)k_new + src, row);"),
    # the denoiser's Mamba-2 scan from the seeded state
    "mamba_decay_sign": ("const double A = -exp((double)A_log[h]);", "const double A = exp((double)A_log[h]);"),
    "mamba_no_softplus": ("const double delta = ttref_softplus(", "const double delta = ("),
    "mamba_no_skip": ("y[xoff + p] = acc + (double)Dskip[h] * xp;", "y[xoff + p] = acc;"),
    "mamba_group_modulo": ("const int g = h / hpg;", "const int g = h % G;"),
    "mamba_unseeded": ("st[k] = (double)h0[soff + k];", "st[k] = 0.0;"),
    "mamba_update_reads_c": ("*s = a * *s + delta * xp * ttref_load(Bm, boff + n, dtype);",
                             "*s = a * *s + delta * xp * ttref_load(Cm, boff + n, dtype);"),
    "mamba_readout_before_update": (
        "*s = a * *s + delta * xp * ttref_load(Bm, boff + n, dtype);\n"
        "                        acc += *s * ttref_load(Cm, boff + n, dtype);",
        "acc += *s * ttref_load(Cm, boff + n, dtype);\n"
        "                        *s = a * *s + delta * xp * ttref_load(Bm, boff + n, dtype);"),
    "mamba_decay_on_input": ("*s = a * *s + delta * xp * ttref_load(Bm, boff + n, dtype);",
                             "*s = a * (*s + delta * xp * ttref_load(Bm, boff + n, dtype));"),
    # adaLN-single modulation and gated residual
    "adaln_no_mean": ("const double e = ttref_load(x, off + k, dtype) - mean;",
                      "const double e = ttref_load(x, off + k, dtype);"),
    "adaln_no_one_plus": ("y[off + k] = u * (1.0 + scale) + shift;", "y[off + k] = u * scale + shift;"),
    "adaln_shift_from_scale_slot": ("const double shift = (double)tm[k] + (double)table[k];",
                                    "const double shift = (double)tm[d + k] + (double)table[d + k];"),
    "adaln_no_layer_table": ("const double scale = (double)tm[d + k] + (double)table[d + k];",
                             "const double scale = (double)tm[d + k];"),
    "adaln_eps_outside_root": ("const double rstd = 1.0 / sqrt(var + eps);",
                               "const double rstd = 1.0 / (sqrt(var) + eps);"),
    "adaln_gate_slot": ("const double gate = (double)tm[2 * d + k] + (double)table[2 * d + k];",
                        "const double gate = (double)tm[d + k] + (double)table[d + k];"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_mistake(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation anchor for {name} not found exactly once"
    msrc = tmp_path / "ttref_mutant.c"
    msrc.write_text(src.replace(old, new))
    lib = tmp_path / "libttref_mutant.so"
    subprocess.run(["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-fopenmp", "-w", str(msrc), "-o",
                    str(lib), "-lm"], check=True)
    env = dict(os.environ, TTREF_LIB=str(lib), OMP_NUM_THREADS="2")
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_pins.py"),
                        os.path.join(ROOT, "tests", "test_oracle_pins_f4.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode != 0, f"mutant {name} passed every pin:\n{r.stdout[-2000:]}"
    assert "failed" in r.stdout, r.stdout[-2000:] + r.stderr[-2000:]
