"""The oracle's pins must catch plausible mistakes.

Each case plants one mistake in a copy of oracle.c (on the CPU), builds it,
runs the pin suite against that build in a subprocess and expects a failure.
"""
import os
import subprocess
import sys
import tempfile

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRC = os.path.join(ROOT, "oracle", "oracle.c")

MUTANTS = {
    "rope_sign": ("u[2 * i] = a * c - b * s;", "u[2 * i] = a * c + b * s;"),
    "rope_freq": ("pow(theta, -2.0 * (double)i / (double)hd)", "pow(theta, -1.0 * (double)i / (double)hd)"),
    "norm_gain_dropped": ("y[i] = (double)g[i] * x[i] * r;", "y[i] = x[i] * r;"),
    "norm_no_mean": ("sqrt(ss / (double)D + eps)", "sqrt(ss + eps)"),
    "attn_scale": ("s[t] = acc / sqrt((double)hd);", "s[t] = acc;"),
    "attn_positions": ("orc_attend(hd, L + 1,", "orc_attend(hd, L,"),
    "gqa_map": ("const int64_t hk = (s * Hq_s + h) / G;", "const int64_t hk = (s * Hq_s + h) % Hkv;"),
    "q8_half_even": ("float r = roundf(xb[i] / scale);", "float r = rintf(xb[i] / scale);"),
    "q8_scale_255": ("float scale = amax / 127.0f;", "float scale = amax / 128.0f;"),
    "merge_no_residual": ("double acc = residual[i];", "double acc = 0.0;"),
    "wo_column_offset": ("Hq * hd, s * Hq_s * hd, att", "Hq * hd, 0, att"),
    "swiglu_swapped": ("a[f] = orc_silu(g1) * g3;", "a[f] = orc_silu(g3) * g1;"),
    "append_slot": ("* C + L) * hd;", "* C + L - 1) * hd;"),
    "w2_column_offset": ("w->w2, c->w_dtype, F, s * Fs,", "w->w2, c->w_dtype, F, 0,"),
    "ffn2d_gate_in_swapped": ("hgt[f] = orc_silu(g) * u;", "hgt[f] = orc_silu(u) * g;"),
    "logits_row_offset": ("(const char *)Wcls + s * Vs * D * esz", "(const char *)Wcls"),
    "logits_no_final_norm": ("orc_rmsnorm(D, x + b * D, g, eps, xn);",
                             "memcpy(xn, x + b * D, sizeof(double) * (size_t)D);"),
    "batch_attn_kv_map": ("const int64_t base = (b * Hkv + h / G) * C * hd;",
                          "const int64_t base = (b * Hkv + h % Hkv) * C * hd;"),
    "batch_attn_positions": ("const int64_t n_pos = L + 1;", "const int64_t n_pos = L;"),
    "a2a_source_row": ("src[((int64_t)i * B + r * nb + b) * C + c]", "src[((int64_t)i * B + b) * C + c]"),
    "merge_logits_order": ("out[b * T * Vs + i * Vs + j]", "out[b * T * Vs + (T - 1 - i) * Vs + j]"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_mistake(name):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation anchor for {name} not unique/found"
    with tempfile.TemporaryDirectory() as td:
        c = os.path.join(td, "oracle_mut.c")
        so = os.path.join(td, "liboracle_mut.so")
        open(c, "w").write(src.replace(old, new))
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math",
                               "-fPIC", "-shared", "-o", so, c, "-lm"])
        env = dict(os.environ, TP_ORACLE_LIB=so)
        r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                            os.path.join(HERE, "test_oracle_pins.py")],
                           cwd=ROOT, env=env, capture_output=True, text=True, timeout=300)
        assert r.returncode != 0, f"pins did not catch mutant {name}:\n{r.stdout[-2000:]}"
