"""Plants plausible mistakes in a copy of the oracle (on the CPU) and checks
that at least one pin fails for each: the pins are only worth something if a
dropped term, a wrong sign, index or bias, or a swapped field trips them."""
import os
import subprocess

import pytest

import oracle
from tests import test_oracle_audit as audit
from tests import test_oracle_codecs as codecs
from tests import test_oracle_gemm as gemm
from tests import test_oracle_int8 as int8
from tests import test_oracle_prune as prune
from tests import test_oracle_quant as quant
from tests import test_oracle_quant_i8 as quant_i8

SRC = os.path.join(os.path.dirname(oracle.__file__), "sp24_oracle.c")

# (name, original text, mutated text)
MUTANTS = [
    ("ties-to-higher-index", "(key[j] == key[i] && j < i)", "(key[j] == key[i] && j > i)"),
    ("nibble-fields-swapped", "(uint32_t)p0 | ((uint32_t)p1 << 2)", "(uint32_t)p1 | ((uint32_t)p0 << 2)"),
    ("sign-not-stripped", "(bits & 0x7fff)", "(bits & 0xffff)"),
    ("meta-word-overlap", "nibble << (4 * (g % 8))", "nibble << (4 * (g % 4))"),
    ("kept-order-reversed", "memcpy(vrow + (2 * g) * eb, row + (4 * g + p0) * eb, eb);",
     "memcpy(vrow + (2 * g) * eb, row + (4 * g + p1) * eb, eb);"),
    ("dropped-fill-nonzero", "memset(row, 0, (size_t)K * eb);", "memset(row, 1, (size_t)K * eb);"),
    ("f16-bias-off-by-one", "ldexp((double)(1024 + f), e - 25)", "ldexp((double)(1024 + f), e - 24)"),
    ("e4m3-subnormal-scale", "ldexp((double)f, -9)", "ldexp((double)f, -10)"),
    ("e4m3-nan-missing", "if ((b & 0x7f) == 0x7f)", "if ((b & 0xff) == 0xff)"),
    ("encode-truncates", "double q = rint(ldexp(a, man_bits - e));", "double q = floor(ldexp(a, man_bits - e));"),
    ("weight-scale-dropped", "acc *= (double)scale_w[n];", "acc *= 1.0;"),
    ("k-index-reversed", "acc += x[k] * wrow[k];", "acc += x[k] * wrow[K - 1 - k];"),
    ("last-term-dropped", "for (int64_t k = 0; k < K; ++k)\n                    acc", "for (int64_t k = 0; k < K - 1; ++k)\n                    acc"),
    ("e4m3-no-saturation", "if (a >= 448.0)\n        return s | 0x7e;", "if (a >= 480.0)\n        return s | 0x7e;"),
    ("quant-scale-off", "amax / 448.0f", "amax / 447.0f"),
    ("quant-scale-fp64", "float t = v / sc;", "double t = (double)v / (double)sc;"),
    ("quant-absmax-signed", "float a = fabsf(v);", "float a = v;"),
    ("audit-coverage-drops-compress", "sparse_time += t_sparse[i] + t_compress[i];", "sparse_time += t_sparse[i];"),
    ("audit-fallback-skips-ineligible", "n_dense += 1;", "n_dense += eligible[i] ? 1 : 0;"),
    ("audit-selection-over-candidates", "(double)n_sparse / (double)n_eligible", "(double)n_sparse / (double)candidate"),
    ("audit-ignores-eligibility", "if (eligible[i] && sparse[i]) {", "if (sparse[i]) {"),
    ("int8-magnitude-from-bits", "    if (dt == OR_I8) {\n        int v", "    if (0) {\n        int v"),
    ("int8-decoded-unsigned", "return (double)((const int8_t *)base)[i];", "return (double)((const uint8_t *)base)[i];"),
    ("i8-scale-off", "amax / 127.0f", "amax / 128.0f"),
    ("i8-zero-row-scale", "amax / 127.0f : 1.0f", "amax / 127.0f : 0.0f"),
    ("i8-ties-away", "float r = nearbyintf(t);", "float r = roundf(t);"),
    ("i8-negative-saturation", "if (r < -127.0f)\n        r = -127.0f;", "if (r < -128.0f)\n        r = -128.0f;"),
    ("i8-nan-to-max", "if (isnan(t))\n        return 0;", "if (isnan(t))\n        return 127;"),
    ("i8-code-decided-in-fp64", "oracle_encode_i8((float)decode_elem(dt, row, k) / sc)",
     "oracle_encode_i8((float)rint(decode_elem(dt, row, k) / (double)sc))"),
    ("i8-nan-counts-in-max", "            if (a > amax)\n                amax = a;\n        }\n        float sc = amax > 0.0f ? amax / 127.0f",
     "            if (!(a <= amax))\n                amax = a;\n        }\n        float sc = amax > 0.0f ? amax / 127.0f"),
]

PINS = [
    codecs.test_decode_every_f16_pattern,
    codecs.test_decode_every_e4m3_pattern,
    codecs.test_encode_decode_roundtrip,
    codecs.test_encode_f16_rne_matches_torch,
    lambda: prune.test_worked_example(oracle.F16, __import__("torch").float16),
    lambda: prune.test_select_pair_exhaustive(4),
    lambda: prune.test_compress_matches_fp64_brute_force(oracle.BF16),
    lambda: prune.test_format_invariants(oracle.F16, 100),
    prune.test_compress_matches_topk_recipe_on_tie_free_data,
    lambda: gemm.test_sparse_w_matches_float64_matmul(oracle.E4M3),
    lambda: gemm.test_exact_integer_product(oracle.BF16),
    gemm.test_one_hot_rows_read_back_decompressed_weights,
    quant.test_encode_e4m3_saturates_and_keeps_nan,
    lambda: quant.test_quantize_exact_round_trip(oracle.BF16),
    lambda: quant.test_quantize_row_maximum_and_error_bound(oracle.BF16),
    quant.test_quantize_decides_codes_in_fp32,
    audit.test_page_example_counts_and_selection_ratio,
    audit.test_coverage_worked_by_hand,
    audit.test_invariants,
    audit.test_extremes,
    int8.test_decode_every_int8_pattern,
    int8.test_prune_matches_brute_force_and_orders_minus_128_first,
    int8.test_int8_gemm_is_exact_integer_arithmetic,
    quant_i8.test_encode_i8_hand_picked,
    lambda: quant_i8.test_quantize_i8_exact_multiples(oracle.BF16),
    lambda: quant_i8.test_quantize_i8_maximum_bound_symmetry_monotone(oracle.F16),
    quant_i8.test_quantize_i8_zero_row_nan_and_inf,
    quant_i8.test_quantize_i8_decides_codes_in_fp32,
    lambda: quant_i8.test_quantize_i8_matches_torch_fp32(oracle.BF16),
]


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_planted_mistake(tmp_path, name, old, new):
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation anchor for {name} not found exactly once"
    mutant = tmp_path / "mutant.c"
    mutant.write_text(src.replace(old, new))
    lib = tmp_path / "libmutant.so"
    subprocess.run(["gcc", "-std=c11", "-O1", "-fopenmp", "-fPIC", "-shared", str(mutant),
                    "-o", str(lib), "-lm"], check=True)
    caught = []
    with oracle.use_library(str(lib)):
        for pin in PINS:
            try:
                pin()
            except (AssertionError, ValueError):
                caught.append(getattr(pin, "__name__", "pin"))
                break
    assert caught, f"no pin caught the planted mistake '{name}'"
