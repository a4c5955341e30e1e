"""Each plausible mistake planted in a copy of oracle.c must trip a pin.

The copies are compiled on the CPU into a temporary directory; the real oracle
is never modified.  A mutant that passes every pin would mean the pins cannot
tell that mistake from the correct oracle.
"""
import os

import pytest

import oracle
import oracle_pins

MUTANTS = {
    "nibble_order_swapped": ("if (k % 2 == 0)\n        return byte & 0x0F;",
                             "if (k % 2 == 1)\n        return byte & 0x0F;"),
    "row_stride_in_codes": ("Wpacked[n * (K / 2) + k / 2]", "Wpacked[n * K / 4 + k / 2]"),
    "block_index_by_byte": ("return n * (K / bs) + k / bs;", "return n * (K / bs) + (k / 2) / bs;"),
    "block_index_transposed": ("return n * (K / bs) + k / bs;", "return n + (k / bs) * (K / bs);"),
    "absmax_dropped": ("volatile float w = codebook[code] * scale;",
                       "volatile float w = codebook[code] + 0.0f * scale;"),
    "code_off_by_one": ("volatile float w = codebook[code] * scale;",
                        "volatile float w = codebook[(code + 1) & 15] * scale;"),
    "product_at_bf16_precision": ("volatile float w = codebook[code] * scale;",
                                  "union { float f; uint32_t u; } cvt = { codebook[code] * scale };\n"
                                  "    cvt.u &= 0xFFFF0000u;\n    volatile float w = cvt.f;"),
    "bf16_truncates": ("if (lower > 0x8000 || (lower == 0x8000 && (upper & 1) != 0))",
                       "if (0)"),
    "bf16_ties_away": ("if (lower > 0x8000 || (lower == 0x8000 && (upper & 1) != 0))",
                       "if (lower >= 0x8000)"),
    "bf16_nan_to_inf": ("return (uint16_t)((u >> 16) | 0x0040);", "return (uint16_t)(u >> 16);"),
    "q4_sum_in_float": ("double sum = 0.0, sum_abs = 0.0;\n            for (int64_t k = 0; k < K; k++) {\n                double a = bf16_to_double(A[m * K + k]);\n                double w = (double)oracle_w32",
                        "float sum = 0.0, sum_abs = 0.0;\n            for (int64_t k = 0; k < K; k++) {\n                double a = bf16_to_double(A[m * K + k]);\n                double w = (double)oracle_w32"),
    "q4_a_transposed": ("double a = bf16_to_double(A[m * K + k]);\n                double w = (double)oracle_w32",
                        "double a = bf16_to_double(A[k * M + m]);\n                double w = (double)oracle_w32"),
    "q4_skips_last_k": ("double w = (double)oracle_w32(Wpacked, absmax, codebook, K, bs, n, k);\n                double p = a * w;",
                        "double w = (double)oracle_w32(Wpacked, absmax, codebook, K, bs, n, k);\n                double p = (k == K - 1) ? 0.0 : a * w;"),
    "bias_dropped": ("sum += b;", "sum += 0.0 * b;"),
    "bf16_w_transposed": ("bf16_to_double(W[n * K + k])", "bf16_to_double(W[k * N + n])"),
    "f16_subnormal_scale": ("v = ldexp((double)f, -24);", "v = ldexp((double)f, -25);"),
    "f16_exponent_bias": ("v = ldexp(1.0 + f / 1024.0, e - 15);", "v = ldexp(1.0 + f / 1024.0, e - 16);"),
    "f16_truncates": ("if (rem > half || (rem == half && (q & 1)))\n        q += 1;", "if (0)\n        q += 1;"),
    "f16_ties_away": ("if (rem > half || (rem == half && (q & 1)))\n        q += 1;",
                      "if (rem >= half)\n        q += 1;"),
    "f16_no_binade_carry": ("if (q == 2048) { /* carried into the next binade */",
                            "if (q == 4096) { /* carried into the next binade */"),
    "f16_no_overflow": ("if (e16 >= 31)\n            return (uint16_t)(sign | 0x7C00);", "if (0)\n            return 0;"),
    "ex_fp16_read_as_bf16": ("return dtype == 2 ? oracle_f16_to_double(b) : bf16_to_double(b);",
                             "return bf16_to_double(b);"),
    "ex_bias_dropped": ("double b = elem(bias, n, bias_dtype);\n                sum += b;",
                        "double b = elem(bias, n, bias_dtype);\n                sum += 0.0 * b;"),
    "ex_a_transposed": ("double a = elem(A, m * K + k, a_dtype);", "double a = elem(A, k * M + m, a_dtype);"),
    "quantize_ties_up": ("if (mid[i] * scale < w)", "if (mid[i] * scale <= w)"),
    "quantize_signed_max": ("double w = fabs(elem(W, n * K + k, w_dtype));", "double w = elem(W, n * K + k, w_dtype);"),
    "quantize_mid_is_entry": ("mid[i] = ((double)codebook[i] + (double)codebook[i + 1]) / 2.0;",
                              "mid[i] = (double)codebook[i];"),
    "quantize_block_shift": ("for (int64_t k = b * bs; k < (b + 1) * bs; k++) {\n                double w = fabs",
                             "for (int64_t k = b * bs + 1; k < (b + 1) * bs && k < K; k++) {\n                double w = fabs"),
    "w16_not_rounded": ("double p = a * bf16_to_double(w16);",
                        "double p = a * (double)oracle_w32(Wpacked, absmax, codebook, K, bs, n, k) + 0.0 * w16;"),
    "tile_lanes_transposed": ("int64_t piece = r + 16 * (2 * (a % 2) + a / 2);",
                              "int64_t piece = 4 * r + (2 * (a % 2) + a / 2);"),
    "tile_quarters_in_row_order": ("int64_t piece = r + 16 * (2 * (a % 2) + a / 2);",
                                   "int64_t piece = r + 16 * a;"),
    "tile_halves_swapped": ("return (t * segs + s) * 1024 + piece * 16 + half * 8 + q % 8;",
                            "return (t * segs + s) * 1024 + piece * 16 + (1 - half) * 8 + q % 8;"),
    "tile_segment_of_128_bytes": ("int64_t s = j / 64, q = j % 64;", "int64_t s = j / 128, q = j % 128;"),
    "bf16_tile_lanes_transposed": ("int64_t piece = r + 16 * (q / 8);", "int64_t piece = 4 * r + q / 8;"),
    "bf16_tile_step_of_64": ("int64_t s = k / 32, q = k % 32;", "int64_t s = k / 64, q = k % 64;"),
    "bf16_repack_reads_columns": ("out[oracle_bf16_tile_index(N, K, n, k)] = W[n * K + k];",
                                  "out[oracle_bf16_tile_index(N, K, n, k)] = W[k * N + n];"),
}


@pytest.fixture(scope="module")
def source():
    with open(oracle.SOURCE) as f:
        return f.read()


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name, source, tmp_path):
    old, new = MUTANTS[name]
    assert source.count(old) >= 1, "mutation anchor not found: " + name
    src = tmp_path / "mutant.c"
    src.write_text(source.replace(old, new, 1))
    lib = oracle.compile_c(str(src), str(tmp_path / "libmutant.so"))
    orc = oracle.Oracle(lib)
    caught = []
    for pin in oracle_pins.ALL_PINS:
        try:
            pin(orc)
        except (AssertionError, ValueError, IndexError):
            caught.append(pin.__name__)
    assert caught, "no pin notices the planted mistake " + name
