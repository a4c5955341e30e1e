"""GPU parity at the full sizes of the five decode workloads.

The oracle computes a sample of output columns one by one (both ends and the
last ragged tile always included); the GPU computes the whole output through
the same entry points and launch configuration the benchmark times.

Workloads (seeded synthetic stand-ins for the pages' model layers):
  C1 fused 4-bit GEMV, M=1, K=4096, N=4096 (whole output compared)
  C2 fused 4-bit, M=1,2,4,8, K=8192, N=28672
  C3 fused 4-bit decode layers, M=1,4,8,16, (K,N) in (5120,8192) (5120,5120)
     (17408,5120) (8192,8192); the split path too at M=16
  C4 bf16 skinny, M=1..5, K=2560, N in {96, 2048, 16384, 31040}, with and
     without bias
  C5 K=2560, N=248320: fused 4-bit at M=1,8 and bf16 skinny at M=1..5
Beyond the decode sizes, the dispatcher's routes at these shapes: the tiled
fused kernel in both work layouts (M = 64 .. 384) and dequantize + tiled GEMM
above the shape's crossover (M = 400 on the decode layers).
"""
import numpy as np
import pytest

import bit_dequant_skinny_amd as q4
import oracle
import synth
from gpu_util import (assert_within_tolerance, bf16_host, bf16_weights, q4_weights,
                      sample_cols, to_dev, torch)

pytestmark = pytest.mark.gpu

BS = 64


def _q4_case(M, N, K, config, shape, path="auto", ncols=384, full=False):
    Wp, am, cb = q4_weights(N, K, BS, config, shape)
    A = synth.activations_bf16(M, K, synth.seed(config, shape, 10 * M + 1))
    dA, dW, dam, dcb = to_dev(A, "bf16"), to_dev(Wp, "u8"), to_dev(am, "f32"), to_dev(cb, "f32")
    C = q4.q4_gemm_skinny(dA, dW, dam, dcb, BS, path=path)
    torch().cuda.synchronize()
    got = bf16_host(C)
    del dA, dW, dam, dcb, C
    cols = None if full else sample_cols(N, ncols, 7 * N + M)
    Cr, S = oracle.q4_gemm(A, Wp, am, cb, M, N, K, BS, cols=cols)
    sel = got if full else got[:, cols]
    return assert_within_tolerance(sel, Cr, S, "q4 %s M=%d N=%d K=%d" % (path, M, N, K))


def test_c1_gemv_full_output():
    _q4_case(1, 4096, 4096, config=0, shape=0, full=True)


@pytest.mark.parametrize("M", [1, 2, 4, 8])
def test_c2_ffn_up(M):
    _q4_case(M, 28672, 8192, config=1, shape=0)


C3 = [(5120, 8192), (5120, 5120), (17408, 5120), (8192, 8192)]


@pytest.mark.parametrize("M", [1, 4, 8, 16])
@pytest.mark.parametrize("shape", range(len(C3)))
def test_c3_decode_layers(shape, M):
    K, N = C3[shape]
    _q4_case(M, N, K, config=2, shape=shape)


@pytest.mark.parametrize("M", [64, 200, 400])
@pytest.mark.parametrize("shape", range(len(C3)))
def test_c3_beyond_16_rows(shape, M):
    K, N = C3[shape]
    _q4_case(M, N, K, config=2, shape=shape, ncols=256)


@pytest.mark.parametrize("M", [100, 384])
def test_c2_ffn_beyond_16_rows(M):
    _q4_case(M, 28672, 8192, config=1, shape=0, ncols=256)


@pytest.mark.parametrize("shape", range(len(C3)))
def test_c3_split_path(shape):
    K, N = C3[shape]
    _q4_case(16, N, K, config=2, shape=shape, path="split")


def _bf16_case(M, N, K, with_bias, config, shape, ncols=384):
    W, bias = bf16_weights(N, K, config, shape)
    b = bias if with_bias else None
    A = synth.activations_bf16(M, K, synth.seed(config, shape, 10 * M + 1))
    dW = to_dev(W, "bf16")
    C = q4.bf16_gemm_skinny(to_dev(A, "bf16"), dW, None if b is None else to_dev(b, "bf16"))
    torch().cuda.synchronize()
    got = bf16_host(C)
    del dW, C
    cols = sample_cols(N, ncols, 11 * N + M)
    Cr, S = oracle.bf16_gemm(A, W, b, M, N, K, cols=cols)
    return assert_within_tolerance(got[:, cols], Cr, S, "bf16 M=%d N=%d" % (M, N))


C4_N = [96, 2048, 16384, 31040]


@pytest.mark.parametrize("with_bias", [False, True])
@pytest.mark.parametrize("M", [1, 2, 3, 4, 5])
@pytest.mark.parametrize("shape", range(len(C4_N)))
def test_c4_bf16_skinny(shape, M, with_bias):
    _bf16_case(M, C4_N[shape], 2560, with_bias, config=3, shape=shape)


@pytest.mark.parametrize("M", [1, 8, 64])
def test_c5_lm_head_q4(M):
    _q4_case(M, 248320, 2560, config=4, shape=0)


@pytest.mark.parametrize("M", [1, 2, 3, 4, 5])
def test_c5_lm_head_bf16(M):
    _bf16_case(M, 248320, 2560, with_bias=(M % 2 == 1), config=4, shape=1)
