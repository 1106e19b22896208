"""The pins reject planted mistakes.

Each case copies vq_oracle.c, plants one plausible mistake (a dropped or
sign-flipped term, a wrong index, a swapped operand, a changed rounding or
order), builds the mutant with gcc on the CPU and checks that at least one of
the oracle pins in test_oracle.py fails against it.
"""
import os
import subprocess
import tempfile

import pytest

import oracle
from tests import test_oracle as pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "vq_oracle.c")

MUTANTS = {
    "q4k min term sign": ("float t3 = t1 - t2;", "float t3 = t1 + t2;",
                          ["test_oracle_gemm_vs_fp64_definition"]),
    "q4k bsum pairing": ("((int32_t)bs[2 * j] + (int32_t)bs[2 * j + 1])",
                         "((int32_t)bs[j] + (int32_t)bs[j + 1])",
                         ["test_oracle_gemm_vs_fp64_definition", "test_closed_forms"]),
    "q4k nibble order": ("f->q[64 * c + l] = qs[32 * c + l] & 15;\n            f->q[64 * c + 32 + l] = qs[32 * c + l] >> 4;",
                         "f->q[64 * c + l] = qs[32 * c + l] >> 4;\n            f->q[64 * c + 32 + l] = qs[32 * c + l] & 15;",
                         ["test_q4k_layout_golden", "test_layout_decoders_agree_on_random_bytes"]),
    "q4k min bits": ("f->m[j] = (s[j] >> 6) | (hi4 << 2);", "f->m[j] = (s[j] >> 6) | (hi4 << 4);",
                     ["test_q4k_layout_golden"]),
    "q6k zero point": ("I += (f->q[16 * j + i] - 32) * (int32_t)a[16 * j + i];",
                       "I += (f->q[16 * j + i] - 31) * (int32_t)a[16 * j + i];",
                       ["test_oracle_gemm_vs_fp64_definition"]),
    "q6k scale index": ("S += f->sc[j] * I;\n    }\n    float t1 = f->d * (float)S;\n    return da * t1;",
                        "S += f->sc[15 - j] * I;\n    }\n    float t1 = f->d * (float)S;\n    return da * t1;",
                        ["test_oracle_gemm_vs_fp64_definition"]),
    "q8_0 scale operand": ("float s = dw * da;", "float s = dw * dw;",
                           ["test_oracle_gemm_vs_fp64_definition"]),
    "q8k last occurrence": ("if (ax > amax) { amax = ax; mx = x[i]; }",
                            "if (ax >= amax) { amax = ax; mx = x[i]; }",
                            ["test_q8k_golden"]),
    "q8k ties away": ("float r = rintf(v);", "float r = roundf(v);", ["test_q8k_golden"]),
    "q8k stored d": ("*d = 1.0f / iscale;", "*d = mx / -127.0f;", ["test_q8k_golden", "test_q8k_invariants"]),
    "q8_1 ties even": ("float r = roundf(x[i] / d);", "float r = rintf(x[i] / d);", ["test_q8_1_golden"]),
    "q8_1 sum order": ("for (int o = 16; o >= 1; o >>= 1) {", "for (int o = 1; o <= 16; o <<= 1) {",
                       ["test_q8_1_golden"]),
    "route unstable": ("for (int64_t p = 0; p < T * top_k; ++p) list[pos[ids[p]]++] = (int32_t)p;",
                       "for (int64_t p = T * top_k - 1; p >= 0; --p) list[pos[ids[p]]++] = (int32_t)p;",
                       ["test_route_golden_and_library_sort"]),
    "expert sum fma": ("acc = acc + p;", "acc = fmaf(w[t * top_k + s], Y[(t * top_k + s) * N + n], acc); (void)p;",
                       ["test_weighted_sum_golden"]),
    "rmsnorm sum not mean": ("sqrt(ss / (double)K + eps)", "sqrt(ss + eps)", ["test_rmsnorm_pins"]),
    "rmsnorm eps outside root": ("sqrt(ss / (double)K + eps)", "(sqrt(ss / (double)K) + eps)",
                                 ["test_rmsnorm_pins"]),
    "rmsnorm gamma reversed": ("* r * (double)gamma[i];", "* r * (double)gamma[K - 1 - i];",
                               ["test_rmsnorm_pins"]),
    "silu sigmoid sign": ("g / (1.0 + exp(-g))", "g / (1.0 + exp(g))", ["test_silu_mul_pins"]),
    "silu drops up": ("* (double)U[m * ldx + i];", "* 1.0;", ["test_silu_mul_pins"]),
    "q5k fifth bit index": ("f->q[e] |= ((qh[e % 32] >> (e / 32)) & 1) << 4;",
                            "f->q[e] |= ((qh[e % 32] >> (e % 8)) & 1) << 4;",
                            ["test_q5k_layout_golden", "test_layout_decoders_agree_on_random_bytes"]),
    "q5k quant levels": ("fit_min_blocks(w, 31, &f, &d16, &dmin16);", "fit_min_blocks(w, 15, &f, &d16, &dmin16);",
                         ["test_weight_encoder_roundtrip_bounds"]),
    "q5k read as q4k": ("q5k_unpack(wrow + b * Q5K_BYTES, &f);", "q4k_unpack(wrow + b * Q5K_BYTES, &f);",
                        ["test_oracle_gemm_vs_fp64_definition"]),
    "f16 ties up": ("if (rem > 0x1000u || (rem == 0x1000u && (h & 1u))) h += 1u;",
                    "if (rem >= 0x1000u) h += 1u;", ["test_f16_encode_matches_numpy_rne"]),
}


def _call(name):
    fn = getattr(pins, name)
    import inspect
    params = inspect.signature(fn).parameters
    if "wtype" in params:
        for w in (oracle.Q4_K, oracle.Q6_K, oracle.Q8_0, oracle.Q5_K):
            fn(w)
    else:
        fn()


@pytest.mark.parametrize("label", sorted(MUTANTS))
def test_pins_reject_mutant(label):
    old_text, new_text, tests = MUTANTS[label]
    src = open(SRC).read()
    assert src.count(old_text) == 1, "mutation anchor not found exactly once: " + label
    with tempfile.TemporaryDirectory() as td:
        c = os.path.join(td, "mut.c")
        so = os.path.join(td, "libmut.so")
        open(c, "w").write(src.replace(old_text, new_text))
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fopenmp", "-fPIC",
                               "-shared", "-o", so, c, "-lm"])
        old = oracle._swap_library(so)
        try:
            failed = False
            for name in tests:
                try:
                    _call(name)
                except AssertionError:
                    failed = True
            assert failed, "no pin caught the planted mistake: " + label
        finally:
            oracle._swap_library(old)
