"""GPU parity of the split path at larger M, where its GEMM is the tiled kernel
(128 x 128 tiles through LDS): dequantize to bf16, then GEMM.

Random data meet the tolerance against the fp64 oracle; one-hot rows must
return the bf16-dequantized weights exactly; fp16 activations run as two bf16
planes whose partials are summed; ragged M, N and K (K % 64 == 32) exercise
the zero-filled tile edges.
"""
import numpy as np
import pytest

import bit_dequant_skinny_amd as q4
import oracle
import synth
from gpu_util import (assert_within_tolerance, bf16_host, host_f64, q4_to_dev, to_dev,
                      to_dev_dtype, torch)

pytestmark = pytest.mark.gpu


def _sync():
    torch().cuda.synchronize()


@pytest.mark.parametrize("M", [17, 64, 129, 300])
@pytest.mark.parametrize("N,K,bs", [(300, 1056, 32), (128, 512, 64), (517, 2048, 128)])
def test_split_tiled_parity(M, N, K, bs):
    p = synth.q4_problem(M, N, K, bs, config=73, shape=N % 5)
    A, Wp, am, cb = q4_to_dev(p)
    C = q4.q4_gemm_skinny(A, Wp, am, cb, bs, path="split")
    _sync()
    Cr, S = oracle.q4_gemm(p["A"], p["Wpacked"], p["absmax"], p["codebook"], M, N, K, bs)
    assert_within_tolerance(bf16_host(C), Cr, S, "split tiled M=%d N=%d K=%d" % (M, N, K))


def test_split_tiled_one_hot_rows_return_dequantized_rows():
    N, K, bs = 200, 1024, 64
    p = synth.q4_problem(1, N, K, bs, config=74)
    js = list(range(0, K, 7))[:150]
    A = np.zeros((len(js), K), np.uint16)
    for m, j in enumerate(js):
        A[m, j] = 0x3F80
    _, Wp, am, cb = q4_to_dev(p)
    C = q4.q4_gemm_skinny(to_dev(A, "bf16"), Wp, am, cb, bs, path="split")
    _sync()
    w16 = oracle.dequant_bf16(p["Wpacked"], p["absmax"], p["codebook"], N, K, bs)
    assert np.array_equal(bf16_host(C), w16[:, js].T)


@pytest.mark.parametrize("adt", ["bf16", "fp16"])
@pytest.mark.parametrize("cdt", ["bf16", "fp32"])
def test_split_tiled_dtypes_and_bias(adt, cdt):
    t = torch()
    M, N, K, bs = 150, 333, 1024, 64
    p = synth.q4_problem(M, N, K, bs, config=75, codebook=synth.random_codebook(83))
    A_h = synth.activations(M, K, 84, adt)
    b_h = synth.bias(N, 85, cdt)
    _, Wp, am, cb = q4_to_dev(p)
    C = q4.q4_gemm_skinny(to_dev_dtype(A_h, adt), Wp, am, cb, bs, path="split",
                          bias=to_dev_dtype(b_h, cdt),
                          out_dtype=t.bfloat16 if cdt == "bf16" else t.float32)
    _sync()
    Cr, S = oracle.q4_gemm_ex(A_h, adt, p["Wpacked"], p["absmax"], p["codebook"], M, N, K, bs,
                              bias=b_h, bias_dtype=cdt)
    assert_within_tolerance(None, Cr, S, "split %s->%s" % (adt, cdt), out=cdt, values=host_f64(C))


def test_split_tiled_scaling_by_two_is_exact():
    M, N, K, bs = 100, 140, 768, 64
    p = synth.q4_problem(M, N, K, bs, config=76)
    A, Wp, am, cb = q4_to_dev(p)
    C1 = q4.q4_gemm_skinny(A, Wp, am, cb, bs, path="split")
    C2 = q4.q4_gemm_skinny(A * 2, Wp, am, cb, bs, path="split")
    _sync()
    assert torch().equal(C2, C1 * 2)
