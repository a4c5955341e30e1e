"""GPU parity of the fused bias epilogue and the other element types of the
4-bit path (q4_gemm_skinny_ex) and of the fp16 dequantize, against the CPU
oracle.

Per the maintainer's comment on the bitsandbytes pull request "[ROCm] Optimize
kgemm_4bit_inference_naive ..." (fused bias epilogue; fp32/fp16/bf16 variants,
all accumulating in fp32).  Acceptance is elementwise
|C_gpu - C_ref| <= 2 u_out |C_ref| + 1e-3 * (sum |a*w| + |bias|), u_out the unit
roundoff of the output type (plus half the fp16 subnormal quantum for fp16
outputs); the fp16 dequantize must match the oracle bit for bit.
"""
import numpy as np
import pytest

import bit_dequant_skinny_amd as q4
import oracle
import synth
from gpu_util import assert_within_tolerance, host_f64, q4_to_dev, to_dev, to_dev_dtype, torch

pytestmark = pytest.mark.gpu

TDT = {"bf16": "bfloat16", "fp16": "float16", "fp32": "float32"}


def _tdtype(name):
    return getattr(torch(), TDT[name])


def _run(M, N, K, bs, adt, cdt, with_bias, path, config=60, cbseed=78):
    p = synth.q4_problem(M, N, K, bs, config=config, shape=N % 7,
                         codebook=synth.random_codebook(cbseed))
    A_h = synth.activations(M, K, synth.seed(config, N % 7, 10 * M + 1), adt)
    b_h = synth.bias(N, synth.seed(config, N % 7, 3), cdt) if with_bias else None
    _, Wp, am, cb = q4_to_dev(p)
    A = to_dev_dtype(A_h, adt)
    b = None if b_h is None else to_dev_dtype(b_h, cdt)
    C = q4.q4_gemm_skinny(A, Wp, am, cb, bs, path=path, bias=b, out_dtype=_tdtype(cdt))
    torch().cuda.synchronize()
    assert C.dtype == _tdtype(cdt)
    Cr, S = oracle.q4_gemm_ex(A_h, adt, p["Wpacked"], p["absmax"], p["codebook"], M, N, K, bs,
                              bias=b_h, bias_dtype=cdt)
    return C, Cr, S


@pytest.mark.parametrize("adt", ["bf16", "fp16", "fp32"])
@pytest.mark.parametrize("cdt", ["bf16", "fp16", "fp32"])
@pytest.mark.parametrize("with_bias", [False, True])
@pytest.mark.parametrize("M", [1, 3, 16])
def test_fused_dtypes_bias(adt, cdt, with_bias, M):
    N, K, bs = 37, 640, 64
    C, Cr, S = _run(M, N, K, bs, adt, cdt, with_bias, "fused")
    assert_within_tolerance(None, Cr, S, "fused %s->%s bias=%s M=%d" % (adt, cdt, with_bias, M),
                            out=cdt, values=host_f64(C))


@pytest.mark.parametrize("adt", ["bf16", "fp16", "fp32"])
@pytest.mark.parametrize("N,K,bs", [(100, 2048, 32), (70, 2560, 128), (9, 4096, 256)])
def test_fused_dtypes_blocksizes(adt, N, K, bs):
    C, Cr, S = _run(5, N, K, bs, adt, "fp32", True, "fused", config=61)
    assert_within_tolerance(None, Cr, S, "fused %s bs=%d" % (adt, bs), out="fp32",
                            values=host_f64(C))


@pytest.mark.parametrize("adt", ["bf16", "fp16"])
@pytest.mark.parametrize("cdt", ["bf16", "fp32"])
@pytest.mark.parametrize("M", [2, 17, 40])
def test_split_dtypes_bias(adt, cdt, M):
    # the split path rounds the weights to bf16 first; on these N(0,1) x
    # N(0,0.02) draws that stays far inside 1e-3 * S
    N, K, bs = 37, 640, 64
    C, Cr, S = _run(M, N, K, bs, adt, cdt, True, "split", config=62)
    assert_within_tolerance(None, Cr, S, "split %s->%s M=%d" % (adt, cdt, M), out=cdt,
                            values=host_f64(C))


def test_auto_path_above_fused_range_with_fp16():
    C, Cr, S = _run(20, 33, 512, 64, "fp16", "fp16", True, "auto", config=63)
    assert_within_tolerance(None, Cr, S, "auto fp16 M=20", out="fp16", values=host_f64(C))


def test_fp32_activations_reject_split():
    t = torch()
    p = synth.q4_problem(2, 16, 128, 64, config=64)
    _, Wp, am, cb = q4_to_dev(p)
    A = to_dev(synth.activations(2, 128, 5, "fp32"), "f32")
    with pytest.raises(q4.Q4Error) as e:
        q4.q4_gemm_skinny(A, Wp, am, cb, 64, path="split")
    assert e.value.status == q4.Q4_ERR_UNSUPPORTED
    A20 = to_dev(synth.activations(20, 128, 6, "fp32"), "f32")
    old = q4.q4_get_crossover_m()
    try:
        q4.q4_set_crossover_m(16)   # M = 20 now routes to split, which fp32 cannot take
        with pytest.raises(q4.Q4Error) as e:
            q4.q4_gemm_skinny(A20, Wp, am, cb, 64)
    finally:
        q4.q4_set_crossover_m(old)
    assert e.value.status == q4.Q4_ERR_UNSUPPORTED
    C = q4.q4_gemm_skinny(A20, Wp, am, cb, 64, path="fused")   # in two passes
    t.cuda.synchronize()
    assert C.shape == (20, 16)


def test_fused_bias_alone_and_determinism():
    """A = 0 gives the bias rounded once; two runs are bitwise equal."""
    t = torch()
    M, N, K, bs = 4, 50, 256, 64
    p = synth.q4_problem(M, N, K, bs, config=65)
    _, Wp, am, cb = q4_to_dev(p)
    b_h = synth.bias(N, 9, "fp32")
    b = to_dev(b_h, "f32")
    A = t.zeros((M, K), dtype=t.float16, device=Wp.device)
    C = q4.q4_gemm_skinny(A, Wp, am, cb, bs, bias=b, out_dtype=t.float32)
    t.cuda.synchronize()
    assert np.array_equal(C.cpu().numpy(), np.broadcast_to(b_h, (M, N)))
    A = to_dev_dtype(synth.activations(M, K, 10, "fp16"), "fp16")
    C1 = q4.q4_gemm_skinny(A, Wp, am, cb, bs, bias=b, out_dtype=t.float32)
    C2 = q4.q4_gemm_skinny(A, Wp, am, cb, bs, bias=b, out_dtype=t.float32)
    t.cuda.synchronize()
    assert t.equal(C1, C2)


@pytest.mark.parametrize("N,K,bs", [(3, 64, 64), (17, 640, 64), (5, 256, 128), (33, 96, 32)])
def test_dequant_f16_bit_exact(N, K, bs):
    t = torch()
    p = synth.q4_problem(1, N, K, bs, config=66, shape=N, codebook=synth.random_codebook(79))
    _, Wp, am, cb = q4_to_dev(p)
    w = q4.q4_dequant(Wp, am, cb, bs, out_dtype=t.float16)
    t.cuda.synchronize()
    ref = oracle.dequant_f16(p["Wpacked"], p["absmax"], p["codebook"], N, K, bs)
    assert np.array_equal(w.cpu().view(t.int16).numpy().view(np.uint16), ref)


def test_dequant_f16_overflow_and_subnormals():
    """Scales that push products past 65504 and below 2^-14."""
    t = torch()
    N, K, bs = 2, 256, 64
    codes = synth.rng(12).integers(0, 16, size=(N, K), dtype=np.uint8)
    am = np.array([[7.0e4, 1.0e5, 3.0e-6, 6.0e-8], [1.0, 65504.0, 2.0 ** -20, 0.0]],
                  dtype=np.float32)
    cb = synth.random_codebook(80)
    Wp = synth.pack_nibbles(codes)
    w = q4.q4_dequant(to_dev(Wp, "u8"), to_dev(am, "f32"), to_dev(cb, "f32"), bs,
                      out_dtype=t.float16)
    t.cuda.synchronize()
    ref = oracle.dequant_f16(Wp, am, cb, N, K, bs)
    assert np.array_equal(w.cpu().view(t.int16).numpy().view(np.uint16), ref)


@pytest.mark.parametrize("M", [1, 8, 11])
def test_fp32_activations_wide_exponent_range(M):
    """fp32 activations with full 24-bit significands over 2^-60 .. 2^60 take
    the matrix-core route as three exact bf16 planes."""
    N, K, bs = 70, 512, 64
    p = synth.q4_problem(M, N, K, bs, config=67, codebook=synth.random_codebook(81))
    g = synth.rng(82)
    mant = 1.0 + g.integers(0, 1 << 23, size=(M, K)) / float(1 << 23)
    A_h = (np.where(g.random((M, K)) < 0.5, -1.0, 1.0) * mant *
           np.exp2(g.integers(-60, 61, size=(M, K)))).astype(np.float32)
    _, Wp, am, cb = q4_to_dev(p)
    C = q4.q4_gemm_skinny(to_dev(A_h, "f32"), Wp, am, cb, bs, out_dtype=torch().float32)
    torch().cuda.synchronize()
    Cr, S = oracle.q4_gemm_ex(A_h, "fp32", p["Wpacked"], p["absmax"], p["codebook"], M, N, K, bs)
    assert_within_tolerance(None, Cr, S, "fp32 wide range", out="fp32", values=host_f64(C))


def test_fp32_activations_near_the_largest_float():
    """Activations a few ulps below FLT_MAX split without overflow."""
    M, N, K, bs = 2, 40, 128, 64
    p = synth.q4_problem(M, N, K, bs, config=68)
    A_h = np.zeros((M, K), np.float32)
    big = np.finfo(np.float32).max
    A_h[0, 3] = big
    A_h[0, 77] = -np.nextafter(big, 0, dtype=np.float32)
    A_h[1, 10] = np.float32(3.3961e38)
    A_h[1, 100] = np.float32(1.5)
    _, Wp, am, cb = q4_to_dev(p)
    C = q4.q4_gemm_skinny(to_dev(A_h, "f32"), Wp, am, cb, bs, out_dtype=torch().float32)
    torch().cuda.synchronize()
    Cr, S = oracle.q4_gemm_ex(A_h, "fp32", p["Wpacked"], p["absmax"], p["codebook"], M, N, K, bs)
    got = host_f64(C)
    assert np.all(np.isfinite(got))
    assert_within_tolerance(None, Cr, S, "fp32 near max", out="fp32", values=got)
