"""Plant plausible mistakes in a copy of the oracle's C source, on the CPU,
and check that the pin tests catch every one of them."""
import os
import subprocess
import sys
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "moe_oracle.c")

MUTATIONS = {
    "swapped_nibbles": ("(c & 1) ? (byte >> 4) : (byte & 15)", "(c & 1) ? (byte & 15) : (byte >> 4)"),
    "e2m1_bias": ("ldexp(1.0 + 0.5 * m, e - 1)", "ldexp(1.0 + 0.5 * m, e)"),
    "e4m3_bias": ("ldexp(1.0 + m / 8.0, e - 7)", "ldexp(1.0 + m / 8.0, e - 8)"),
    "scale_block_index": ("s[srow + c / 16]", "s[srow + c / 32]"),
    "ties_to_higher_index": ("(x->idx < y->idx) ? -1 : (x->idx > y->idx)", "(x->idx > y->idx) ? -1 : (x->idx < y->idx)"),
    "shared_dropped": ("for (n = 0; n < H; ++n) yr[n] += o[n];", "for (n = 0; n < H; ++n) yr[n] += 0.0 * o[n];"),
    "routed_scale_dropped": ("yr[n] = rs * acc[n];", "yr[n] = acc[n];"),
    "silu_sign": ("return g / (1.0 + exp(-g));", "return g / (1.0 + exp(g));"),
    "softmax_unnormalised": ("for (j = 0; j < k; ++j) w[(size_t)r * k + j] /= sum;\n        } else",
                             "for (j = 0; j < k; ++j) w[(size_t)r * k + j] /= 1.0;\n        } else"),
    "rms_missing_mean": ("inv = 1.0 / sqrt(ss / H + eps);", "inv = 1.0 / sqrt(ss + eps);"),
    "bias_in_weights": ("double v = 1.0 / (1.0 + exp(-(double)l[ids[(size_t)r * k + j]]));",
                        "double v = 1.0 / (1.0 + exp(-(double)l[ids[(size_t)r * k + j]])) + bias[ids[(size_t)r * k + j]];"),
    "dedup_slot_order": ("asg[pos] = s;\n                inv[s] = pos;", "asg[pos] = n - 1 - s;\n                inv[n - 1 - s] = pos;"),
    "gamma_inside_norm": ("for (n = 0; n < H; ++n) ss += yr[n] * yr[n];",
                          "for (n = 0; n < H; ++n) ss += yr[n] * yr[n] * (gamma ? orc_bf16(gamma[n]) * orc_bf16(gamma[n]) : 1.0);"),
    "gamma_reversed": ("if (gamma) v *= orc_bf16(gamma[n]);", "if (gamma) v *= orc_bf16(gamma[H - 1 - n]);"),
    "residual_dropped": ("yr[n] += orc_bf16(residual[(size_t)r * H + n]);", "yr[n] += 0.0 * orc_bf16(residual[(size_t)r * H + n]);"),
    "argmax_ties_to_higher": ("if (l[v] > l[best]) best = v;", "if (l[v] >= l[best]) best = v;"),
    "bonus_token_row": ("emitted[a] = target[a];", "emitted[a] = target[a > 0 ? a - 1 : 0];"),
    "tie_rule_sign": ("l[d] >= l[target[a]] - tie_tol", "l[d] >= l[target[a]] + tie_tol"),
    "lm_head_transposed": ("acc += xr[h] * orc_bf16(wv[h]);", "acc += xr[h] * orc_bf16(w[((size_t)h * V + v) % ((size_t)V * H)]);"),
    "router_transposed": ("orc_bf16(wr[(size_t)e * H + h])", "orc_bf16(wr[(size_t)h * E % (E * H) + e])"),
    "down_transposed": ("orc_nvfp4_weight(dq, ds, dts, H, I, e, n, i)", "orc_nvfp4_weight(dq, ds, dts, H, I, e, (n + 1) % H, i)"),
    "dense_silu_on_up": ("            hbuf[i] = silu(g) * v;", "            hbuf[i] = g * silu(v);"),
    "dense_down_transposed": ("acc += hbuf[i] * orc_bf16(wd[(size_t)n * I + i]);",
                              "acc += hbuf[i] * orc_bf16(wd[((size_t)i * H + n) % ((size_t)H * I)]);"),
    "dense_residual_dropped": ("if (residual) acc += orc_bf16(residual[(size_t)t * H + n]);",
                               "if (residual) acc += 0.0 * orc_bf16(residual[(size_t)t * H + n]);"),
    "dense_gate_from_up": ("g += xd[c] * orc_bf16(wg[(size_t)i * H + c]);", "g += xd[c] * orc_bf16(wu[(size_t)i * H + c]);"),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_pins_catch_planted_mistake(name, tmp_path):
    old, new = MUTATIONS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, "mutation anchor must be unique: %s" % name
    mut = tmp_path / "mut.c"
    mut.write_text(src.replace(old, new))
    so = tmp_path / "libmut.so"
    subprocess.check_call(["gcc", "-O2", "-std=c99", "-fPIC", "-shared", str(mut), "-o", str(so), "-lm"])
    env = dict(os.environ, SBV_ORACLE_LIB=str(so))
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_pins.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode != 0, "pins did not catch mutation %s:\n%s" % (name, r.stdout[-2000:])
