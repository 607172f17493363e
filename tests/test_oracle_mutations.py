"""The oracle's pins must catch plausible mistakes: each case below plants one error in a
copy of the oracle source (on the CPU only), builds it, and runs the pin suite against it; the
suite must fail.  The unmodified source must pass (checked by the pin suite itself).  C mutants
change adamw4_oracle.c; the PY_MUTANTS change the oracle's Python wrapper (its per-tensor state
handling), run from a copy of the oracle package placed first on the import path."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "adamw4_oracle.c")

MUTANTS = {
    "no_bias_correction_v": ("s.rs2 = (float)(1.0 / sqrt(bc2));", "s.rs2 = 1.0f;"),
    "no_bias_correction_m": ("s.step_size = (float)((double)hp->lr / bc1);",
                             "s.step_size = hp->lr;"),
    "decay_sign": ("s.decay = (float)(1.0 - (double)hp->lr * (double)hp->weight_decay);",
                   "s.decay = (float)(1.0 + (double)hp->lr * (double)hp->weight_decay);"),
    "v_uses_g_not_g2": ("float gg = g * g;", "float gg = g;"),
    "m_beta_swapped": ("float m1 = hp->beta1 * m;", "float m1 = s->omb1 * m;"),
    "eps_dropped": ("den = den + hp->eps;", "den = den + 0.0f;"),
    "weights_after_quant": ("orc_elem r = adamw_elem(w[i], widen_grad(g, g_bf16, i), m, v, hp, &s);\n                w[i] = r.w;",
                            "orc_elem r = adamw_elem(w[i], widen_grad(g, g_bf16, i), m, v, hp, &s);\n                w[i] = r.w + 0.5f * (r.m - m) * s.step_size;"),
    "zip_sqrt_swapped": ("float n2 = sb + sa;", "float n2 = sb + sy;"),
    "zip_choice_inverted": ("codes[j] = (uint8_t)(u < p ? k : k + 1);\n    }\n}\n\n/* v block under ZE-EDEN",
                            "codes[j] = (uint8_t)(u < p ? k + 1 : k);\n    }\n}\n\n/* v block under ZE-EDEN"),
    "zip_state_space_p": ("float p = orc_zip_p(y, lo, hi, c, eps);\n        float u = orc_uniform(seed, t, pos, 0, i0 + j);",
                          "float p = (hi - y) / (hi - lo);\n        float u = orc_uniform(seed, t, pos, 0, i0 + j);"),
    "m_sr_p_inverted": ("float p = (hi - y) / (hi - lo);\n        float u = orc_uniform(seed, t, pos, 1, i0 + j);",
                        "float p = (y - lo) / (hi - lo);\n        float u = orc_uniform(seed, t, pos, 1, i0 + j);"),
    "rtn_ties_high": ("if (y > mid) ++code;", "if (y >= mid) ++code;"),
    "nibble_order": ("bytes[q] = (uint8_t)(lo | (hi << 4));", "bytes[q] = (uint8_t)(hi | (lo << 4));"),
    "eden_gamma_inverted": ("float gamma = nrm / fmaxf(dot, 1e-12f);", "float gamma = dot / fmaxf(nrm, 1e-12f);"),
    "eden_no_rescale": ("*scale = gamma * s;", "*scale = s;"),
    "philox_key_bump": ("k1 += 0xBB67AE85u;", "k1 += 0x9E3779B9u;"),
    "rng_stream_ignored": ("(uint32_t)(j >> 32) | ((uint32_t)stream << 31)", "(uint32_t)(j >> 32)"),
    "prev_mode_ignored": ("const float* Vin = uses_v1(hp->prev_mode < 0 ? hp->mode : hp->prev_mode) ? V1 : V0;",
                          "const float* Vin = uses_v1(hp->mode) ? V1 : V0;"),
    "v0_codebook_k16": ("out[k] = (float)((double)k / 15.0);", "out[k] = (float)((double)k / 16.0);"),
    "nf4_delta": ("const double delta = 1.0 - 0.5 * (1.0 / 30.0 + 1.0 / 32.0);",
                  "const double delta = 0.9677083;"),
    "absmax_not_abs": ("for (int j = 0; j < ORC_BLOCK; ++j) s = fmaxf(s, fabsf(x[j]));",
                       "for (int j = 0; j < ORC_BLOCK; ++j) s = fmaxf(s, x[j]);"),
    "ssr_p_inverted": ("float p = (hi - y) / (hi - lo);\n        float u = orc_uniform(seed, t, pos, 0, i0 + j);",
                       "float p = (y - lo) / (hi - lo);\n        float u = orc_uniform(seed, t, pos, 0, i0 + j);"),
    "prtn_state_space": ("float p = orc_zip_p(y, lo, hi, c, eps);\n        if (dbg && j < nvalid) { dbg[j].u_v = 0.5f;",
                         "float p = (hi - y) / (hi - lo);\n        if (dbg && j < nvalid) { dbg[j].u_v = 0.5f;"),
    "prtn_threshold": ("codes[j] = (uint8_t)(p >= 0.5f ? k : k + 1);",
                       "codes[j] = (uint8_t)(p >= 0.25f ? k : k + 1);"),
    "fp32m_m_not_updated": ("                m32[i] = e.m;\n", "                m32[i] = m32[i];\n"),
    "bf16_truncates": ("out[i] = (uint16_t)((u + 0x7FFFu + keep_lsb) >> 16);",
                       "out[i] = (uint16_t)(u >> 16);"),
    "bf16_ties_away": ("out[i] = (uint16_t)((u + 0x7FFFu + keep_lsb) >> 16);",
                       "out[i] = (uint16_t)((u + 0x8000u) >> 16);"),
    "baseline_keeps_zero": ("case ORC_V_ZE_RTN: encode_v_rtn_block(vw, V1, cv, vscale); break;",
                            "case ORC_V_ZE_RTN: encode_v_rtn_block(vw, V0, cv, vscale); break;"),
    "baseline_rescales": ("case ORC_V_ZE_RTN: encode_v_rtn_block(vw, V1, cv, vscale); break;",
                          "case ORC_V_ZE_RTN: encode_v_eden_block(vw, V1, cv, vscale); break;"),
    "baseline_decodes_v0": ("static int uses_v1(int mode) { return mode == ORC_ZE_EDEN || mode == ORC_V_ZE_RTN; }",
                            "static int uses_v1(int mode) { return mode == ORC_ZE_EDEN; }"),
    # the initial-state encoder
    "init_eden_no_gamma": ("        if (mode == ORC_ZE_EDEN) encode_v_eden_block(vw, V1, cv, &vscale[b]);",
                           "        if (0) encode_v_eden_block(vw, V1, cv, &vscale[b]);"),
    "init_eden_on_v0": ("        if (mode == ORC_ZE_EDEN) encode_v_eden_block(vw, V1, cv, &vscale[b]);",
                        "        if (mode == ORC_ZE_EDEN) encode_v_eden_block(vw, V0, cv, &vscale[b]);"),
    "init_baseline_on_v0": ("        else encode_v_rtn_block(vw, uses_v1(mode) ? V1 : V0, cv, &vscale[b]);",
                            "        else encode_v_rtn_block(vw, V0, cv, &vscale[b]);"),
    "v_beta_swapped": ("float v1 = hp->beta2 * v;", "float v1 = s->omb2 * v;"),
    "zip_h_without_bias_correction": (
        "                               uint8_t* codes, float* scale, orc_dbg* dbg) {\n    float s = 0.0f;\n"
        "    for (int j = 0; j < ORC_BLOCK; ++j) s = fmaxf(s, x[j]);\n    *scale = s;\n    float c = sqrtf(s) * rs2;",
        "                               uint8_t* codes, float* scale, orc_dbg* dbg) {\n    float s = 0.0f;\n"
        "    for (int j = 0; j < ORC_BLOCK; ++j) s = fmaxf(s, x[j]);\n    *scale = s;\n    float c = sqrtf(s);"),
    "prtn_h_without_bias_correction": (
        "                                float eps, uint8_t* codes, float* scale, orc_dbg* dbg) {\n    float s = 0.0f;\n"
        "    for (int j = 0; j < ORC_BLOCK; ++j) s = fmaxf(s, x[j]);\n    *scale = s;\n    float c = sqrtf(s) * rs2;",
        "                                float eps, uint8_t* codes, float* scale, orc_dbg* dbg) {\n    float s = 0.0f;\n"
        "    for (int j = 0; j < ORC_BLOCK; ++j) s = fmaxf(s, x[j]);\n    *scale = s;\n    float c = sqrtf(s);"),
    "zip_eps_only_in_denominator": ("    n3 = n3 + eps;", "    n3 = n3 + 0.0f;"),
    "init_m_stochastic": ("        encode_m_block(mw, nvalid, 0, NF4, 0, 0, 0, 0, cm, &mscale[b], NULL);",
                          "        encode_m_block(mw, nvalid, 1, NF4, 0, 0, 0, 0, cm, &mscale[b], NULL);"),
}

PY_MUTANTS = {
    "fallback_boundary_4095": ("MIN_QUANT = 4096", "MIN_QUANT = 4095"),
    "fallback_boundary_4097": ("MIN_QUANT = 4096", "MIN_QUANT = 4097"),
    "norm_layers_quantized": ("    return numel >= MIN_QUANT and not norm", "    return numel >= MIN_QUANT"),
    "init_fp32m_drops_m0": ("        m = np.zeros(n, np.float32) if m0 is None else np.asarray(m0, np.float32).copy()\n"
                            "        return State(True, None, full.vcodes",
                            "        m = np.zeros(n, np.float32)\n"
                            "        return State(True, None, full.vcodes"),
    "init_fp32m_ignores_v0": ("        full = init_state(n, norm, mode, None, v0)",
                              "        full = init_state(n, norm, mode, None, None)"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation anchor for {name} not unique/present"
    mut = tmp_path / "mut.c"
    mut.write_text(src.replace(old, new))
    lib = tmp_path / "libmut.so"
    subprocess.run(["gcc", "-std=c11", "-O2", "-ffp-contract=off", "-fopenmp", "-fPIC", "-shared",
                    "-o", str(lib), str(mut), "-lm"], check=True, capture_output=True)
    env = dict(os.environ, ADAMW4_ORACLE_LIB=str(lib))
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_pins.py")],
                       env=env, capture_output=True, text=True, cwd=ROOT)
    assert r.returncode != 0, f"pin suite passed with mutant {name}:\n{r.stdout[-2000:]}"


@pytest.mark.parametrize("name", sorted(PY_MUTANTS))
def test_pins_catch_wrapper_mutant(name, tmp_path):
    old, new = PY_MUTANTS[name]
    pkg = tmp_path / "oracle"
    pkg.mkdir()
    src = open(os.path.join(ROOT, "oracle", "__init__.py")).read()
    assert src.count(old) == 1, f"mutation anchor for {name} not unique/present"
    (pkg / "__init__.py").write_text(src.replace(old, new))
    (pkg / "adamw4_oracle.c").write_text(open(SRC).read())
    env = dict(os.environ, ADAMW4_ORACLE_PKG=str(tmp_path))
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_pins.py")],
                       env=env, capture_output=True, text=True, cwd=ROOT)
    assert r.returncode != 0, f"pin suite passed with mutant {name}:\n{r.stdout[-2000:]}"
