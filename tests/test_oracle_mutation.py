"""Plant mistakes in copies of oracle.c (on the CPU) and require that the pins catch each.

A pin that cannot tell a plausible mistake from the right answer pins nothing;
this is the check that the pins in tests/pins.py have teeth. Every planted
snippet must occur exactly once in oracle.c, so this test fails loudly if the
oracle source drifts away from the mutation list.
"""
import os

import pytest

import pins

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "oracle.c")

MUTANTS = {
    "nibble_order": ("return (k & 1) ? (byte >> 4) : (byte & 15u);",
                     "return (k & 1) ? (byte & 15u) : (byte >> 4);"),
    "scale_index": ("scales[(size_t)n * (K / 16) + k / 16]", "scales[(size_t)n * (K / 16) + (k + 1) / 16 % (K / 16)]"),
    "e4m3_bias": ("ldexp(1.0 + (double)m / 8.0, (int)e - 7)", "ldexp(1.0 + (double)m / 8.0, (int)e - 8)"),
    "e4m3_subnormal": ("ldexp((double)m, -9)", "ldexp((double)m, -10)"),
    "e2m1_table": ("{0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0}", "{0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 5.0}"),
    "tie_to_higher_id": ("(best < 0 || l[e] > l[best])", "(best < 0 || l[e] >= l[best])"),
    "sigmoid_sign": ("v[j] = 1.0 / (1.0 + exp(-lj));", "v[j] = 1.0 / (1.0 + exp(lj));"),
    "perm_tokens_descending": ("for (int e = 0; e < E; ++e)\n    for (int t = 0; t < T; ++t)",
                               "for (int e = 0; e < E; ++e)\n    for (int t = T - 1; t >= 0; --t)"),
    "gate_up_swapped": ("gi += proj_weight(P, 0, g, 2 * I, H, i, k) * x[k];",
                        "gi += proj_weight(P, 0, g, 2 * I, H, I + i, k) * x[k];"),
    "e8m0_bias_128": ("return ldexp(1.0, (int)byte - 127);", "return ldexp(1.0, (int)byte - 128);"),
    "mx_block_16": ("orc_e8m0(scales[(size_t)n * (K / 32) + k / 32])",
                    "orc_e8m0(scales[(size_t)n * (K / 32) + k / 16 % (K / 32)])"),
    "mx_expert_stride_nvfp4": ("const int bs = P->mx ? 32 : 16;", "const int bs = 16;"),
    "silu_dropped": ("h[i] = gi / (1.0 + exp(-gi)) * ui;", "h[i] = gi * ui;"),
    "combine_unweighted": ("o[n] += w[(size_t)t * k + j] * y[n];", "o[n] += y[n] / k;"),
    "shared_weight_half": ("      for (int n = 0; n < H; ++n) o[n] += y[n];",
                           "      for (int n = 0; n < H; ++n) o[n] += 0.5 * y[n];"),
    "gs_divisor": ("gs_out[g] = A / 2688.0f;", "gs_out[g] = A / 2687.0f;"),
    "block_scale_factor": ("float six_gs = 6.0f * gs;", "float six_gs = 4.0f * gs;"),
    "quant_sign_lost": ("uint32_t code = signbit(v) ? 8u : 0u;", "uint32_t code = 0u;"),
    "score_sqrt_dropped": ("return sqrt(fmax(l, 0.0) + log1p(exp(-fabs(l))));", "return fmax(l, 0.0) + log1p(exp(-fabs(l)));"),
    "bias_in_weights": ("sum += s[best];", "sum += key[best];\n      s[best] = key[best];"),
    "bias_not_added": ("if (bias) key[e] = key[e] + bias[e];", "if (bias) key[e] = key[e];"),
    "group_score_max_only": ("gscore[q] = b < 0 ? key[a] : key[a] + key[b];", "gscore[q] = key[a];"),
    "group_tie_to_higher_id": ("if (!gkeep[q] && (best < 0 || gscore[q] > gscore[best])) best = q;",
                               "if (!gkeep[q] && (best < 0 || gscore[q] >= gscore[best])) best = q;"),
    "routed_scaling_dropped": ("w[(size_t)t * k + j] = (renorm ? sj / sum : sj) * scaling;",
                               "w[(size_t)t * k + j] = (renorm ? sj / sum : sj);"),
    "gate_clamped_both_sides": ("      gi = fmin(gi, limit);", "      gi = fmin(fmax(gi, -limit), limit);"),
    "up_clamped_above_only": ("      ui = fmin(fmax(ui, -limit), limit);", "      ui = fmin(ui, limit);"),
    "clamp_on_shared": ("      orc_expert_ffn_q(shared, s, H, I, x + (size_t)i * H, y, 0, 0.0, hq);",
                        "      orc_expert_ffn_q(shared, s, H, I, x + (size_t)i * H, y, clamp, limit, hq);"),
    "hq_skipped": ("  } else if (hq) {", "  } else if (0) {"),
    "mx8_exponent_off_by_one": ("        X = E - 1 - 8;", "        X = E - 1 - 7;"),
    "mx8_amax_half_block": ("      for (int j = 0; j < 32; ++j)\n        if (fabsf(xr[b * 32 + j]) > A)",
                            "      for (int j = 0; j < 16; ++j)\n        if (fabsf(xr[b * 32 + j]) > A)"),
    "mx8_sign_lost": ("const uint32_t sign = signbit(v) ? 0x80u : 0u;", "const uint32_t sign = 0u;"),
    "mx8_h_as_nvfp4": ("  } else if (hq == 2) {   /* MXFP8 h (W4A8 profile) */",
                       "  } else if (0) {   /* MXFP8 h (W4A8 profile) */"),
    "fp8_divisor": ("const float s = A / 448.0f;", "const float s = A / 447.0f;"),
    "fp8_amax_skips_last": ("    for (int k = 0; k < K; ++k)\n      if (fabsf(xr[k]) > A) A = fabsf(xr[k]);",
                            "    for (int k = 0; k + 1 < K; ++k)\n      if (fabsf(xr[k]) > A) A = fabsf(xr[k]);"),
    "fp8_sign_lost": ("const uint32_t sign = signbit(xr[k]) ? 0x80u : 0u;", "const uint32_t sign = 0u;"),
    "fp8_decode_scale_dropped": ("orc_e4m3fn(codes[(size_t)r * K + k]) * (double)scale[r];",
                                 "orc_e4m3fn(codes[(size_t)r * K + k]);"),
    "fp8_h_skipped": ("  if (hq == 3) {", "  if (0) {"),
    "hq_not_on_shared": ("      orc_expert_ffn_q(shared, s, H, I, x + (size_t)i * H, y, 0, 0.0, hq);",
                         "      orc_expert_ffn_q(shared, s, H, I, x + (size_t)i * H, y, 0, 0.0, 0);"),
    "hq_decode_gs_halved": ("    orc_quantize(h32, 1, I, 1, hp, hs, &hg);",
                        "    orc_quantize(h32, 1, I, 1, hp, hs, &hg);\n    hg = hg * 0.5f;"),
    "e4m3_ties_odd": ("if (d < bestd || (d == bestd && (c & 1u) == 0 && (best & 1u) == 1)) {\n      best = c;\n      bestd = d;\n    }\n  }\n  return (uint8_t)best;\n}\n\n/* Nearest E2M1",
                      "if (d < bestd || (d == bestd && (c & 1u) == 1)) {\n      best = c;\n      bestd = d;\n    }\n  }\n  return (uint8_t)best;\n}\n\n/* Nearest E2M1"),
}


@pytest.fixture(scope="module")
def source():
    with open(SRC) as f:
        return f.read()


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, source, tmp_path):
    import oracle
    import oracle.build
    old, new = MUTANTS[name]
    assert source.count(old) == 1, f"mutation site for {name} not found exactly once"
    src = tmp_path / "oracle_mut.c"
    src.write_text(source.replace(old, new))
    lib = oracle.build.build(str(src), str(tmp_path / "liboracle_mut.so"))
    mutant = oracle.Oracle(lib)
    failed = []
    for pin in pins.ALL_PINS:
        try:
            pin(mutant)
        except AssertionError:
            failed.append(pin.__name__)
    assert failed, f"no pin catches the planted mistake {name}"
