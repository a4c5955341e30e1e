"""The allocation-free entry point q4_gemm_skinny_ex_noalloc, called through
the C ABI, against q4_gemm_skinny_ex on the same inputs.

Both run the same kernels; only where the scratch lives differs (a fixed
device array against the per-stream workspace), so the outputs must be equal
bit for bit.  Each case runs two calls in a row, the second on a smaller
input, because every call shares the device's array.  A request above the
array's size is refused before anything is launched, and a first call can be
captured into a HIP graph (it allocates nothing).
"""
import ctypes

import numpy as np
import pytest

import bit_dequant_skinny_amd as q4
import oracle
import synth
from gpu_util import assert_within_tolerance, host_f64, q4_to_dev, to_dev_dtype, torch

pytestmark = pytest.mark.gpu

DT = {"bf16": q4.Q4_DTYPE_BF16, "fp16": q4.Q4_DTYPE_FP16, "fp32": q4.Q4_DTYPE_FP32}
PATH = {"auto": 0, "fused": 1, "split": 2}


def _tdt(name):
    t = torch()
    return {"bf16": t.bfloat16, "fp16": t.float16, "fp32": t.float32}[name]


def _call(fn, A, adt, Wp, am, cb, bias, M, N, K, bs, C, cdt, path, stream=None):
    t = torch()
    s = t.cuda.current_stream().cuda_stream if stream is None else stream
    return fn(A.data_ptr(), DT[adt], Wp.data_ptr(), am.data_ptr(), cb.data_ptr(),
              None if bias is None else bias.data_ptr(), M, N, K, bs, C.data_ptr(), DT[cdt],
              ctypes.c_void_p(s), PATH[path])


def _case(M, N, K, bs, adt, cdt, path, with_bias, config):
    t = torch()
    p = synth.q4_problem(M, N, K, bs, config=config)
    _, Wp, am, cb = q4_to_dev(p)
    A_h = synth.activations(M, K, config + 1, adt)
    A = to_dev_dtype(A_h, adt)
    b_h = synth.bias(N, config + 2, cdt) if with_bias else None
    bias = to_dev_dtype(b_h, cdt) if with_bias else None
    C_ref = t.full((M, N), 7.0, dtype=_tdt(cdt), device=A.device)
    C_new = t.full((M, N), 7.0, dtype=_tdt(cdt), device=A.device)
    L = q4.lib()
    assert _call(L.q4_gemm_skinny_ex, A, adt, Wp, am, cb, bias, M, N, K, bs, C_ref, cdt,
                 path) == q4.Q4_OK, L.q4_last_error()
    st = _call(L.q4_gemm_skinny_ex_noalloc, A, adt, Wp, am, cb, bias, M, N, K, bs, C_new, cdt,
               path)
    assert st == q4.Q4_OK, L.q4_last_error()
    t.cuda.synchronize()
    return p, A_h, b_h, C_ref, C_new


# (M, N, K, adt, cdt, path, bias): the fp16 / fp32 activation planes, the
# split path's dequantized weights, the tiled kernel's fp32 K parts, a call
# that needs no scratch at all, and the skinny kernel's K parts.
CASES = [
    ((8, 600, 2048, "fp32", "fp32", "auto", True), (3, 200, 1024, "fp32", "fp32", "auto", True)),
    ((5, 512, 1536, "fp16", "bf16", "auto", True), (2, 96, 512, "fp16", "fp16", "auto", False)),
    ((16, 1024, 2048, "bf16", "bf16", "split", False), (4, 256, 1024, "bf16", "bf16", "split", False)),
    ((200, 256, 4096, "bf16", "bf16", "fused", True), (70, 128, 2048, "bf16", "bf16", "fused", True)),
    ((4, 1024, 4096, "bf16", "bf16", "fused", False), (1, 512, 1024, "bf16", "bf16", "fused", False)),
    # the skinny kernel's K parts: their fp32 sums in the array (also for a
    # pass of two token blocks, then a one-block call)
    ((4, 1536, 16384, "bf16", "bf16", "fused", True), (1, 1536, 16448, "bf16", "fp32", "fused", False)),
    ((24, 1536, 16384, "bf16", "bf16", "fused", True), (3, 1536, 16384, "bf16", "bf16", "fused", True)),
]


@pytest.mark.parametrize("first,second", CASES)
def test_noalloc_equals_workspace_entry_point(first, second):
    t = torch()
    for n, (M, N, K, adt, cdt, path, with_bias) in enumerate((first, second)):
        p, A_h, b_h, C_ref, C_new = _case(M, N, K, 64, adt, cdt, path, with_bias, 300 + 10 * n)
        assert t.equal(C_ref, C_new), "noalloc differs from q4_gemm_skinny_ex (%s)" % str(
            (M, N, K, adt, cdt, path))
        if path == "split":
            Cr, S = oracle.q4_gemm_w16(A_h, p["Wpacked"], p["absmax"], p["codebook"], M, N, K, 64)
            assert_within_tolerance(None, Cr, S, "noalloc split", out=cdt, values=host_f64(C_new))
        else:
            Cr, S = oracle.q4_gemm_ex(A_h, adt, p["Wpacked"], p["absmax"], p["codebook"], M, N, K,
                                      64, bias=b_h, bias_dtype=cdt)
            assert_within_tolerance(None, Cr, S, "noalloc", out=cdt, values=host_f64(C_new))


def test_noalloc_refuses_requests_above_its_array():
    """The split path of an 8192 x 8192 weight needs 128 MiB of bf16 weights:
    above the fixed array, so the call is refused and writes nothing."""
    t = torch()
    M, N, K, bs = 2, 8192, 8192, 64
    assert N * K * 2 > q4.Q4_NOALLOC_SCRATCH_BYTES
    Wp = t.zeros((N, K // 2), dtype=t.uint8, device="cuda:0")
    am = t.ones((N, K // bs), dtype=t.float32, device="cuda:0")
    cb = t.zeros(16, dtype=t.float32, device="cuda:0")
    A = t.zeros((M, K), dtype=t.bfloat16, device="cuda:0")
    C = t.full((M, N), 3.0, dtype=t.bfloat16, device="cuda:0")
    L = q4.lib()
    st = _call(L.q4_gemm_skinny_ex_noalloc, A, "bf16", Wp, am, cb, None, M, N, K, bs, C, "bf16",
               "split")
    assert st == q4.Q4_ERR_UNSUPPORTED
    assert b"scratch" in L.q4_last_error()
    t.cuda.synchronize()
    assert bool((C == 3.0).all())


def test_noalloc_first_call_can_be_captured():
    """A call that needs scratch captured into a HIP graph on a fresh stream
    (no earlier call on it): the capture succeeds and every replay equals the
    eager result."""
    t = torch()
    M, N, K, bs = 6, 384, 2048, 64
    p = synth.q4_problem(M, N, K, bs, config=330)
    _, Wp, am, cb = q4_to_dev(p)
    A = to_dev_dtype(synth.activations(M, K, 331, "fp32"), "fp32")
    C_eager = t.empty((M, N), dtype=t.float32, device="cuda:0")
    C_graph = t.zeros((M, N), dtype=t.float32, device="cuda:0")
    L = q4.lib()
    assert _call(L.q4_gemm_skinny_ex_noalloc, A, "fp32", Wp, am, cb, None, M, N, K, bs, C_eager,
                 "fp32", "auto") == q4.Q4_OK
    t.cuda.synchronize()
    side = t.cuda.Stream()
    g = t.cuda.CUDAGraph()
    with t.cuda.graph(g, stream=side):
        st = _call(L.q4_gemm_skinny_ex_noalloc, A, "fp32", Wp, am, cb, None, M, N, K, bs,
                   C_graph, "fp32", "auto", stream=side.cuda_stream)
    assert st == q4.Q4_OK, L.q4_last_error()
    for _ in range(3):
        C_graph.zero_()
        t.cuda.synchronize()
        g.replay()
        t.cuda.synchronize()
        assert t.equal(C_graph, C_eager)
