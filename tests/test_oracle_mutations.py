"""Strength of the oracle's pins: plant plausible mistakes in a copy of the
oracle's C source, rebuild it in a temporary folder and check that the pin
suite (tests/test_oracle_pins.py) fails for every one of them.

CPU only.  The mistakes are planted in the oracle, never in the HIP path.
"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

# (name, original text, planted mistake)
MUTATIONS = [
    ("rotation_sign_first_slot", "y[offset + 2 * i] = x0 * c - x1 * s;",
     "y[offset + 2 * i] = x0 * c + x1 * s;"),
    ("rotation_sign_second_slot", "y[offset + 2 * i + 1] = x0 * s + x1 * c;",
     "y[offset + 2 * i + 1] = -x0 * s + x1 * c;"),
    ("frequency_exponent", "pow(theta, -2.0 * (double)i / (double)da)",
     "pow(theta, -1.0 * (double)i / (double)da)"),
    ("axis_split_order", "int64_t width[3] = {d / 4, 3 * d / 8, 3 * d / 8};",
     "int64_t width[3] = {3 * d / 8, 3 * d / 8, d / 4};"),
    ("h_w_positions_swapped", "pos[1] = (n / Ws) % Hs;\n  pos[2] = n % Ws;",
     "pos[2] = (n / Ws) % Hs;\n  pos[1] = n % Ws;"),
    ("eps_dropped", "den += eps;", "den += 0.0;"),
    ("eps_as_clamp", "den += eps;", "den = den > eps ? den : eps;"),
    ("state_transposed", "num += rotq[p] * Sh[p * d + e];", "num += rotq[p] * Sh[e * d + p];"),
    ("denominator_rotated", "for (int64_t p = 0; p < d; ++p) den += phiq[p] * zh[p];",
     "for (int64_t p = 0; p < d; ++p) den += rotq[p] * zh[p];"),
    ("normaliser_rotated", "zacc[p] += phik[p];", "zacc[p] += rotk[p];"),
    ("relu_dropped_on_q", "phiq[p] = x > 0.0 ? x : 0.0;", "phiq[p] = x;"),
    ("relu_dropped_on_k", "phik[p] = x > 0.0 ? x : 0.0; /* phi = ReLU */", "phik[p] = x;"),
    ("gate_sign", "exp(-(double)gn[e])", "exp((double)gn[e])"),
    ("gate_index", "exp(-(double)gn[e])", "exp(-(double)gn[(e + 1) % d])"),
    ("numerator_unrotated_q", "num += rotq[p] * Sh[p * d + e];", "num += phiq[p] * Sh[p * d + e];"),
    ("block_state_never_written", "if ((n + 1) % tokens_per_block == 0) {",
     "if ((n + 1) % tokens_per_block == 0 && n + 1 == N) {"),
    ("block_index_shifted", "int64_t blk = n / tokens_per_block;\n        int64_t pos[3];",
     "int64_t blk = (n / tokens_per_block + 1) % nb;\n        int64_t pos[3];"),
    ("value_dropped_last_feature", "vrow[p] = (double)vn[p];",
     "vrow[p] = (p + 1 < d) ? (double)vn[p] : 0.0;"),
    ("block_step_cache_ignored", "for (int64_t i = 0; i < B * H * d * d; ++i) S[i] += S_cache[i];",
     "for (int64_t i = 0; i < B * H * d * d; ++i) S[i] += 0.0 * S_cache[i];"),
    ("block_step_normaliser_cache_ignored", "for (int64_t i = 0; i < B * H * d; ++i) z[i] += z_cache[i];",
     "for (int64_t i = 0; i < B * H * d; ++i) z[i] += 0.0 * z_cache[i];"),
    ("write_gate_on_normaliser", "for (int64_t p = 0; p < d; ++p) rotk[p] *= bt;",
     "for (int64_t p = 0; p < d; ++p) { rotk[p] *= bt; phik[p] *= bt; }"),
    ("rmsnorm_mean_over_d_minus_1", "const double inv_rms = 1.0 / sqrt(ss / (double)d + rms_eps);",
     "const double inv_rms = 1.0 / sqrt(ss / (double)(d - 1) + rms_eps);"),
    ("rmsnorm_weight_index", "on[e] = on[e] * inv_rms * (double)w[e];",
     "on[e] = on[e] * inv_rms * (double)w[(e + 1) % d];"),
    ("backward_prefix_not_suffix", "for (int64_t blk = nb - 2; blk >= 0; --blk) {\n          for (int64_t i = 0; i < dd; ++i) dS[blk * dd + i] += dS[(blk + 1) * dd + i];",
     "for (int64_t blk = nb - 2; blk >= 0; --blk) {\n          for (int64_t i = 0; i < dd; ++i) dS[(blk + 1) * dd + i] += dS[blk * dd + i];"),
    ("backward_dden_sign", "const double dden = -dyy / den;", "const double dden = dyy / den;"),
    ("backward_forward_rotation", "ora_rope(t1, t2, d, neg, theta); /* back through the rotation */",
     "ora_rope(t1, t2, d, pos, theta); /* back through the rotation */"),
    ("backward_relu_mask_dropped_on_k", "dk[row + p] = (double)k[row + p] > 0.0 ? t2[p] + Gz[p] : 0.0;",
     "dk[row + p] = t2[p] + Gz[p];"),
    ("token_causal_normaliser_rotated", "z[p] += phik[p];", "z[p] += rotk[p];"),
    ("token_causal_state_transposed", "num += rotq[p] * S[p * d + e];",
     "num += rotq[p] * S[e * d + p];"),
    ("token_causal_relu_dropped_on_k",
     "phik[p] = x > 0.0 ? x : 0.0;\n  }\n  ora_rope(phik, rotk, d, pos, theta);",
     "phik[p] = x;\n  }\n  ora_rope(phik, rotk, d, pos, theta);"),
    ("token_causal_gate_sign", "out[row + e] = num / den / (1.0 + exp(-(double)g[row + e]));",
     "out[row + e] = num / den / (1.0 + exp((double)g[row + e]));"),
    ("token_causal_strict_no_diagonal",
     "causal_add(k, v, row, d, pos, theta, tmp, tmp + d, S, z);\n"
     "          causal_read(q, g, row, d, pos, theta, eps, tmp + 2 * d, tmp + 3 * d, S, z, out);",
     "causal_read(q, g, row, d, pos, theta, eps, tmp + 2 * d, tmp + 3 * d, S, z, out);\n"
     "          causal_add(k, v, row, d, pos, theta, tmp, tmp + d, S, z);"),
    ("block_step_offset_ignored", "const int64_t pos0[3] = {t_offset, 0, 0};",
     "const int64_t pos0[3] = {0, 0, 0};"),
]


def _run_pins_against(src_text, workdir):
    for sub in ("oracle", "tests", "relu_linear_attention_amd"):
        shutil.copytree(os.path.join(ROOT, sub), os.path.join(workdir, sub),
                        ignore=shutil.ignore_patterns("*.so", "__pycache__", "*.tmp"))
    shutil.copy(os.path.join(ROOT, "pytest.ini"), workdir)
    with open(os.path.join(workdir, "oracle", "oracle.c"), "w") as f:
        f.write(src_text)
    return subprocess.run(
        [sys.executable, "-m", "pytest", "tests/test_oracle_pins.py", "-q", "-x",
         "-p", "no:cacheprovider"], cwd=workdir, capture_output=True, text=True, timeout=300)


@pytest.mark.parametrize("name,original,mistake", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_pins_catch_planted_mistake(name, original, mistake, tmp_path):
    with open(os.path.join(ROOT, "oracle", "oracle.c")) as f:
        src = f.read()
    assert src.count(original) >= 1, f"mutation anchor for {name} not found"
    r = _run_pins_against(src.replace(original, mistake), str(tmp_path))
    assert r.returncode != 0, f"planted mistake {name} went unnoticed:\n{r.stdout[-2000:]}"
