"""Plant plausible mistakes in a copy of the oracle and check the pins catch each.

A pin set that still passes on a broken oracle would not be a pin. Each
mutation below edits one line of a private copy of ``oracle/oracle.c``
(the committed file is never touched), builds it with gcc, swaps it in
for the real library, and runs the pins; at least one must fail.
"""
import os
import shutil
import subprocess

import pytest

import oracle
import test_oracle as pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "oracle.c")

MUTATIONS = {
    "bias dropped": ("return sc * (double)qo_code(bits, wq + n * words, k) + bi;",
                     "return sc * (double)qo_code(bits, wq + n * words, k) + 0.0 * bi;"),
    "nibble order reversed": ("int shift = bits * (int)(k % per_word);",
                              "int shift = bits * (int)(per_word - 1 - k % per_word);"),
    "scale and bias swapped": ("double sc = qo_f16_to_f64(s[n * groups + g]);",
                               "double sc = qo_f16_to_f64(b[n * groups + g]) + 0.0 * qo_f16_to_f64(s[0]);"),
    "wrong group": ("int64_t g = k / 64;", "int64_t g = (k / 64 + 1) % groups;"),
    "fp16 exponent bias": ("v = ldexp((double)(1024 + m), e - 25);",
                           "v = ldexp((double)(1024 + m), e - 24);"),
    "bf16 exponent bias": ("v = ldexp((double)(128 + m), e - 134);",
                           "v = ldexp((double)(128 + m), e - 133);"),
    "activation reversed": ("double prod = weight(bits, wq, s, b, K, n, k) * x[k];",
                            "double prod = weight(bits, wq, s, b, K, n, k) * x[K - 1 - k];"),
    "ties to higher index": ("if (best < 0 || l[e] > l[best]) best = e;",
                             "if (best < 0 || l[e] >= l[best]) best = e;"),
    "no renormalization": ("p[t * k + j] = prob[idx[t * k + j]] / kept;",
                           "p[t * k + j] = prob[idx[t * k + j]] / (0.0 * kept + 1.0);"),
    "gelu sign": ("return 0.5 * u * (1.0 + erf(u / sqrt(2.0)));",
                  "return 0.5 * u * (1.0 - erf(u / sqrt(2.0)));"),
    "gate and up swapped": ("h[i] = qo_gelu(z[i], act) * z[I + i];",
                            "h[i] = qo_gelu(z[I + i], act) * z[i];"),
    "routing weight ignored": ("yt[n] += pj * o[n];", "yt[n] += o[n] + 0.0 * pj;"),
    "mirai zero point ignored": ("return sc * (double)(q - z);", "return sc * (double)(q - 0 * z);"),
    "mirai zero point of the wrong group": ("int z = qo_code(4, zp + n * zwords, grp);",
                                            "int z = qo_code(4, zp + n * zwords, (grp + 1) % groups);"),
    "mirai zero point added": ("return sc * (double)(q - z);", "return sc * (double)(q + z);"),
    "mirai scale read as fp16": ("double sc = qo_bf16_to_f64(s[n * groups + grp]);",
                                 "double sc = qo_f16_to_f64(s[n * groups + grp]);"),
    "mirai wrong scale group": ("const int64_t grp = k / 64;", "const int64_t grp = (k / 64 + 1) % groups;"),
    "mirai-l codes unsigned": ("int q = u >= 128 ? u - 256 : u;", "int q = u;"),
    "mirai-l sign threshold": ("int q = u >= 128 ? u - 256 : u;", "int q = u > 128 ? u - 256 : u;"),
    "hadamard sign rule": ("acc += (__builtin_popcount((unsigned)(i & j)) & 1) ? -v[j] : v[j];",
                           "acc += (__builtin_popcount((unsigned)(i | j)) & 1) ? -v[j] : v[j];"),
    "hadamard not normalized": ("out[32 * blk + i] = c * acc;", "out[32 * blk + i] = acc + 0.0 * c;"),
    "hadamard signs ignored": ("int neg = signs ? (int)((signs[blk] >> j) & 1u) : 0;", "int neg = 0;"),
    "hadamard signs on outputs": ("int neg = signs ? (int)((signs[blk] >> j) & 1u) : 0;",
                                  "int neg = signs ? (int)((signs[blk] >> (31 - j)) & 1u) : 0;"),
    "rmsnorm eps outside": ("const double r = 1.0 / sqrt(ss / (double)K + eps);",
                            "const double r = 1.0 / (sqrt(ss / (double)K) + eps);"),
    "rmsnorm mean over K-1": ("const double r = 1.0 / sqrt(ss / (double)K + eps);",
                              "const double r = 1.0 / sqrt(ss / (double)(K - 1) + eps);"),
    "rmsnorm gamma ignored": ("out[k] = x[k] * r * (gamma ? gamma[k] : 1.0);", "out[k] = x[k] * r;"),
    "attention head group": ("const int64_t hk = h / grp;", "const int64_t hk = h % Hkv;"),
    "attention slot shifted": ("int64_t qo_attn_slot(int64_t pos, int64_t window) { return window > 0 ? pos % window : pos; }",
                               "int64_t qo_attn_slot(int64_t pos, int64_t window) { return window > 0 ? (pos + 1) % window : pos; }"),
    "attention window short": ("const int64_t n = window > 0 ? (pos + 1 < window ? pos + 1 : window) : pos + 1;",
                               "const int64_t n = window > 0 ? (pos + 1 < window ? pos + 1 : window - 1) : pos + 1;"),
    "attention scale dropped": ("sc[j] = scale * acc;", "sc[j] = acc + 0.0 * scale;"),
    "attention unnormalized": ("acc += sc[j] / z * vj[d];", "acc += sc[j] * vj[d] + 0.0 * z;"),
    "attention no max shift": ("sc[j] = exp(sc[j] - smax);", "sc[j] = exp(sc[j]) + 0.0 * smax;"),
    "int8 activation codes truncated": ("q[m * K + k] = amax > 0.0f ? (int8_t)rintf(v / sc) : (int8_t)0;",
                                        "q[m * K + k] = amax > 0.0f ? (int8_t)truncf(v / sc) : (int8_t)0;"),
    "int8 activation scale over 128": ("const float sc = amax / 127.0f;", "const float sc = amax / 128.0f;"),
    "int8 activation scale dropped": ("scale[m] = sc;", "scale[m] = 1.0f + 0.0f * sc;"),
    "int8 activation max over half the row": ("const float v = fabsf((float)qo_f16_to_f64(xr[k]));",
                                              "const float v = fabsf((float)qo_f16_to_f64(xr[k / 2]));"),
    "shared expert halved": ("yt[n] += o[n];\n            if (at) at[n] += oa[n];\n        }\n    }",
                             "yt[n] += 0.5 * o[n];\n            if (at) at[n] += oa[n];\n        }\n    }"),
}

PIN_CALLS = [
    (pins.test_f16_decode_exhaustive, {}),
    (pins.test_bf16_decode_exhaustive, {}),
    (pins.test_code_unpack_matches_divmod, {"bits": 4}),
    (pins.test_code_unpack_matches_divmod, {"bits": 8}),
    (pins.test_code_order_lsb_first, {}),
    (pins.test_gemv_matches_bruteforce, {"bits": 4, "N": 17, "K": 256, "T": 3}),
    (pins.test_gemv_matches_bruteforce, {"bits": 8, "N": 5, "K": 192, "T": 8}),
    (pins.test_gemv_grouped_closed_form, {"bits": 4}),
    (pins.test_zero_codes_give_bias_term, {"bits": 4}),
    (pins.test_one_hot_activation_is_exact_weight, {"bits": 4}),
    (pins.test_chunk_is_rowwise_gemv_on_bf16, {}),
    (pins.test_topk_matches_stable_sort, {}),
    (pins.test_topk_renormalized_softmax_identity, {}),
    (pins.test_gelu_textbook_values_and_identities, {}),
    (pins.test_moe_block_matches_bruteforce, {"act": 0}),
    (pins.test_moe_identical_experts_do_not_depend_on_routing, {}),
    (pins.test_mirai_gemv_matches_bruteforce, {"fmt": "M", "N": 5, "K": 704, "T": 3}),
    (pins.test_mirai_gemv_matches_bruteforce, {"fmt": "L", "N": 4, "K": 1024, "T": 8}),
    (pins.test_mirai_m_explicit_decode, {}),
    (pins.test_mirai_l_explicit_decode, {}),
    (pins.test_mirai_m_equals_affine_with_bias_minus_s_z, {}),
    (pins.test_mirai_l_equals_affine8_with_offset_codes, {}),
    (pins.test_mirai_code_equal_to_zero_point_gives_zero, {}),
    (pins.test_rht_columns_are_scipy_hadamard, {}),
    (pins.test_rht_with_signs_matches_explicit_rotation, {}),
    (pins.test_rht_is_orthogonal_and_self_inverse_without_signs, {}),
    (pins.test_rmsnorm_closed_forms, {}),
    (pins.test_mirai_gemv_with_rotation_prologue_matches_bruteforce, {"fmt": "M"}),
    (pins.test_attn_matches_bruteforce, {"Hq": 6, "Hkv": 3, "D": 32, "cap": 16, "window": 16, "pos": 37}),
    (pins.test_attn_matches_bruteforce, {"Hq": 4, "Hkv": 2, "D": 64, "cap": 40, "window": 0, "pos": 17}),
    (pins.test_attn_first_token_returns_its_value, {}),
    (pins.test_attn_equal_keys_give_the_mean_value, {}),
    (pins.test_attn_circular_equals_linear_over_the_window, {}),
    (pins.test_attn_large_scores_are_stable, {}),
    (pins.test_attn_slot_rule, {}),
    (pins.test_int8_activations_on_the_exact_grid_reduce_to_the_gemm, {}),
    (pins.test_int8_activation_ties_go_to_even, {}),
    (pins.test_int8_activation_bounds_and_extremes, {}),
    (pins.test_int8_activation_zero_row_and_row_independence, {}),
    (pins.test_int8_activations_match_the_second_route, {}),
]


def _build_mutant(tmp_path, old, new):
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation anchor not unique or missing: {old!r}"
    mdir = tmp_path / "m"
    mdir.mkdir()
    shutil.copy(os.path.join(os.path.dirname(SRC), "oracle.h"), mdir / "oracle.h")
    (mdir / "oracle.c").write_text(src.replace(old, new))
    lib = str(mdir / "liboracle_mut.so")
    subprocess.run(["gcc", "-std=gnu11", "-O1", "-fopenmp", "-fPIC", "-shared", "-o", lib,
                    str(mdir / "oracle.c"), "-lm"], check=True)
    return lib


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_pins_catch_planted_mistake(name, tmp_path):
    old, new = MUTATIONS[name]
    lib = _build_mutant(tmp_path, old, new)
    saved_lib, saved_path = oracle._lib, oracle._LIB_PATH
    failed = []
    try:
        oracle._lib = None
        oracle._LIB_PATH = lib
        oracle._load()
        for fn, kw in PIN_CALLS:
            try:
                fn(**kw)
            except AssertionError:
                failed.append(fn.__name__)
    finally:
        oracle._lib, oracle._LIB_PATH = saved_lib, saved_path
    assert failed, f"no pin caught the planted mistake '{name}'"
