"""GPU parity of the fused pass over 17..32 token rows.

bf16 activations with 17..32 rows run as one matrix-core pass holding two
blocks of 16 token rows that share each decoded weight unit; matrices of more
than 8 tiles per CU run that pass as two 16-row launches instead.  Each output
is computed by the same MFMA sequence and summation order as in a 16-row
pass, so the two-block result must equal the two 16-row passes bit for bit,
and it must meet the elementwise tolerance against the fp64 oracle.  Shapes
with 8 tiles per chunk (more than 2048 weight rows per CU) take the tiled
kernel at 17..32 rows instead; they are checked against the oracle.
"""
import numpy as np
import pytest

import bit_dequant_skinny_amd as q4
import oracle
import synth
from gpu_util import (assert_within_tolerance, bf16_host, codebook_16bit, hilo_products,
                      q4_to_dev, q4_weights, sample_cols, to_dev, torch)

pytestmark = pytest.mark.gpu


def _sync():
    torch().cuda.synchronize()


@pytest.mark.parametrize("M", [17, 20, 31, 32])
@pytest.mark.parametrize("N,K,bs", [(37, 640, 64), (300, 1024, 64), (5000, 256, 128),
                                    (129, 2048, 256)])
def test_two_block_pass_parity(M, N, K, bs):
    p = synth.q4_problem(M, N, K, bs, config=61, shape=N % 7)
    A, Wp, am, cb = q4_to_dev(p)
    C = q4.q4_gemm_skinny(A, Wp, am, cb, bs, path="fused")
    _sync()
    Cr, S = oracle.q4_gemm(p["A"], p["Wpacked"], p["absmax"], p["codebook"], M, N, K, bs)
    assert_within_tolerance(bf16_host(C), Cr, S, "two-block M=%d N=%d K=%d" % (M, N, K))


@pytest.mark.parametrize("M", [18, 32])
@pytest.mark.parametrize("N,K", [(300, 1024), (28672, 256)])
def test_two_block_pass_equals_16_row_passes(M, N, K):
    """Rows 0..15 and 16..M-1 computed in one pass equal two separate calls."""
    bs = 64
    p = synth.q4_problem(M, N, K, bs, config=62, shape=N % 5)
    A, Wp, am, cb = q4_to_dev(p)
    C = bf16_host(q4.q4_gemm_skinny(A, Wp, am, cb, bs, path="fused"))
    C0 = bf16_host(q4.q4_gemm_skinny(A[:16].contiguous(), Wp, am, cb, bs, path="fused"))
    C1 = bf16_host(q4.q4_gemm_skinny(A[16:].contiguous(), Wp, am, cb, bs, path="fused"))
    _sync()
    assert np.array_equal(C, np.concatenate([C0, C1], axis=0))


@pytest.mark.parametrize("M", [17, 32])
def test_eight_tile_shapes_take_the_tiled_kernel(M):
    N, K, bs = 40000, 128, 64
    p = synth.q4_problem(M, N, K, bs, config=64)
    A, Wp, am, cb = q4_to_dev(p)
    C = q4.q4_gemm_skinny(A, Wp, am, cb, bs, path="fused")
    _sync()
    cols = sample_cols(N, 512, 65 + M)
    Cr, S = oracle.q4_gemm(p["A"], p["Wpacked"], p["absmax"], p["codebook"], M, N, K, bs,
                           cols=cols)
    assert_within_tolerance(bf16_host(C)[:, cols], Cr, S, "8-tile shape M=%d" % M)


@pytest.mark.parametrize("cbname", ["int4", "random16", "nf4style"])
def test_two_block_one_hot_rows_return_dequantized_rows(cbname):
    """Row m = e_j gives the dequantized weight w(n, j) bit for bit when every
    codebook entry has at most 16 significant bits (the kernel's bf16 hi + lo
    pair is then the entry itself).  With the 24-bit NF4-style table the
    kernel gives fl32(absmax (hi + lo)) rounded to bf16, which may be the
    neighbouring bf16 value where the fp32 product lies within 2^-16 of a
    rounding midpoint: there either value is accepted."""
    N, K, bs = 300, 1024, 64
    cb = {"int4": q4.q4_codebook_preset("int4"), "random16": codebook_16bit(63),
          "nf4style": synth.nf4_style_codebook()}[cbname]
    p = synth.q4_problem(1, N, K, bs, config=63, codebook=cb)
    js = [0, 1, 7, 31, 32, 63, 64, 100, 127, 128, 255, 256, 511, 512, 700, 767,
          768, 800, 900, 1000, 1010, 1015, 1020, 1021, 1022, 1023, 2, 3, 4, 5, 6, 8]
    A = np.zeros((len(js), K), np.uint16)
    for m, j in enumerate(js):
        A[m, j] = 0x3F80
    _, Wp, am, cbd = q4_to_dev(p)
    C = bf16_host(q4.q4_gemm_skinny(to_dev(A, "bf16"), Wp, am, cbd, bs, path="fused"))
    _sync()
    w16 = oracle.dequant_bf16(p["Wpacked"], p["absmax"], p["codebook"], N, K, bs)[:, js].T
    if cbname != "nf4style":
        assert np.array_equal(C, w16)
        return
    codes = oracle.unpack(p["Wpacked"], N, K)[:, js].T
    scales = p["absmax"].reshape(N, K // bs)[:, np.array(js) // bs].T
    alt = hilo_products(p["codebook"])(codes, scales)
    same = w16 == alt
    assert np.array_equal(C[same], w16[same])
    assert np.all((C[~same] == w16[~same]) | (C[~same] == alt[~same]))


@pytest.mark.parametrize("M", [24, 32])
def test_two_block_ffn_sampled(M):
    """The 28672 x 8192 FFN (7 tiles per CU) at 24 and 32 token rows."""
    N, K, bs = 28672, 8192, 64
    Wp, am, cb = q4_weights(N, K, bs, 1, 0)
    A = synth.activations_bf16(M, K, synth.seed(1, 0, 10 * M + 1))
    C = q4.q4_gemm_skinny(to_dev(A, "bf16"), to_dev(Wp, "u8"), to_dev(am, "f32"),
                          to_dev(cb, "f32"), bs)
    _sync()
    cols = sample_cols(N, 256, 13 * M)
    Cr, S = oracle.q4_gemm(A, Wp, am, cb, M, N, K, bs, cols=cols)
    assert_within_tolerance(bf16_host(C)[:, cols], Cr, S, "FFN M=%d" % M)
