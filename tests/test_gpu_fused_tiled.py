"""GPU parity of the fused path above 32 token rows, where it takes the tiled
matrix-core kernel (tiles of 64 tokens x 64 features, each decoded weight
serving every token of the tile; K split over workgroups when the tiles
cannot fill the CUs).

Random data must meet the elementwise tolerance against the fp64 oracle for
ragged M, N and K (K % 128 == 64 leaves half a segment), every blocksize the
kernel takes (64, 128, 256), the K-split partial sums, every activation and
output type with a bias, and the 28672 x 8192 FFN at full size on sampled
columns.  Structured checks: 2A gives 2C bit for bit, repeated calls are
bitwise equal, zero and extreme block scales, and one-hot rows return the
dequantized weights.  The kernel has two work layouts (waves splitting K over
64-feature tiles, or splitting 256-feature tiles by N with the activations
staged through LDS), chosen per shape; child processes force each layout on
every case, and lower the tiled threshold to 0 to run the 32-row tiles on
1..32 rows.
"""
import os
import subprocess
import sys

import numpy as np
import pytest

import bit_dequant_skinny_amd as q4
import oracle
import synth
from gpu_util import (assert_within_tolerance, bf16_host, hilo_products, host_f64, q4_to_dev,
                      q4_weights, sample_cols, to_dev, to_dev_dtype, torch)

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _sync():
    torch().cuda.synchronize()


@pytest.mark.parametrize("M", [33, 64, 100, 129])
@pytest.mark.parametrize("N,K,bs", [(300, 1088, 64), (64, 4096, 128), (517, 2048, 256),
                                    (1000, 640, 64)])
def test_fused_tiled_parity(M, N, K, bs):
    p = synth.q4_problem(M, N, K, bs, config=80, shape=N % 7,
                         codebook=synth.random_codebook(86))
    A, Wp, am, cb = q4_to_dev(p)
    C = q4.q4_gemm_skinny(A, Wp, am, cb, bs, path="fused")
    _sync()
    Cr, S = oracle.q4_gemm(p["A"], p["Wpacked"], p["absmax"], p["codebook"], M, N, K, bs)
    assert_within_tolerance(bf16_host(C), Cr, S, "tiled M=%d N=%d K=%d bs=%d" % (M, N, K, bs))


@pytest.mark.parametrize("M", [40, 300])
def test_fused_tiled_scaling_and_determinism(M):
    N, K, bs = 140, 1536, 64
    p = synth.q4_problem(M, N, K, bs, config=81)
    A, Wp, am, cb = q4_to_dev(p)
    C1 = q4.q4_gemm_skinny(A, Wp, am, cb, bs, path="fused")
    C1b = q4.q4_gemm_skinny(A, Wp, am, cb, bs, path="fused")
    C2 = q4.q4_gemm_skinny(A * 2, Wp, am, cb, bs, path="fused")
    _sync()
    assert torch().equal(C1, C1b)
    assert torch().equal(C2, C1 * 2)


def test_fused_tiled_one_hot_rows_return_dequantized_rows():
    """Row m = e_j gives C[m, n] = the dequantized weight w(n, j).  The tiled
    kernel holds each codebook value as hi + lo (within 2^-16 relative), so
    where the fp32 product cb * absmax lies that close to a bf16 rounding
    midpoint the result may be the neighbouring bf16 value; everywhere else it
    must be the oracle's dequantized bf16 weight exactly."""
    N, K, bs = 200, 1024, 64
    p = synth.q4_problem(1, N, K, bs, config=82)
    js = list(range(0, K, 11))[:90]
    A = np.zeros((len(js), K), np.uint16)
    for m, j in enumerate(js):
        A[m, j] = 0x3F80
    _, Wp, am, cb = q4_to_dev(p)
    C = bf16_host(q4.q4_gemm_skinny(to_dev(A, "bf16"), Wp, am, cb, bs, path="fused"))
    _sync()
    w16 = oracle.dequant_bf16(p["Wpacked"], p["absmax"], p["codebook"], N, K, bs)[:, js].T
    hilo = hilo_products(p["codebook"])
    codes = oracle.unpack(p["Wpacked"], N, K)[:, js].T
    scales = p["absmax"].reshape(N, K // bs)[:, np.array(js) // bs].T
    alt = hilo(codes, scales)
    same = w16 == alt
    assert np.array_equal(C[same], w16[same])
    assert np.all((C[~same] == w16[~same]) | (C[~same] == alt[~same]))
    assert same.mean() > 0.99


@pytest.mark.parametrize("adt", ["bf16", "fp16", "fp32"])
@pytest.mark.parametrize("cdt", ["bf16", "fp16", "fp32"])
def test_fused_tiled_dtypes_and_bias(adt, cdt):
    t = torch()
    M, N, K, bs = 48, 333, 1024, 64
    p = synth.q4_problem(M, N, K, bs, config=83, codebook=synth.random_codebook(87))
    A_h = synth.activations(M, K, 88, adt)
    b_h = synth.bias(N, 89, cdt)
    _, Wp, am, cb = q4_to_dev(p)
    C = q4.q4_gemm_skinny(to_dev_dtype(A_h, adt), Wp, am, cb, bs, path="fused",
                          bias=to_dev_dtype(b_h, cdt),
                          out_dtype={"bf16": t.bfloat16, "fp16": t.float16,
                                     "fp32": t.float32}[cdt])
    _sync()
    Cr, S = oracle.q4_gemm_ex(A_h, adt, p["Wpacked"], p["absmax"], p["codebook"], M, N, K, bs,
                              bias=b_h, bias_dtype=cdt)
    assert_within_tolerance(None, Cr, S, "tiled %s->%s" % (adt, cdt), out=cdt,
                            values=host_f64(C))


def test_fused_tiled_special_block_scales():
    """Blocks scaled by zero, by subnormals and by large finite values."""
    M, N, K, bs = 70, 96, 1024, 64
    p = synth.q4_problem(M, N, K, bs, config=84)
    am = p["absmax"].copy().reshape(N, K // bs)
    am[3, :] = 0.0
    am[10, 2] = np.float32(1e-40)
    am[11, 5] = np.float32(3e-39)
    am[20, 7] = np.float32(1e30)
    am[:, 9] = 0.0
    A, Wp, _, cb = q4_to_dev(p)
    C = q4.q4_gemm_skinny(A, Wp, to_dev(am, "f32"), cb, bs, path="fused",
                          out_dtype=torch().float32)
    _sync()
    Cr, S = oracle.q4_gemm(p["A"], p["Wpacked"], am, p["codebook"], M, N, K, bs)
    got = host_f64(C)
    assert np.all(got[:, 3] == 0.0)
    assert_within_tolerance(None, Cr, S, "special scales", out="fp32", values=got)


@pytest.mark.parametrize("M", [64, 256])
def test_fused_tiled_ffn_sampled(M):
    """The 28672 x 8192 FFN at 64 and 256 token rows, sampled columns."""
    N, K, bs = 28672, 8192, 64
    Wp, am, cb = q4_weights(N, K, bs, 1, 0)
    A = synth.activations_bf16(M, K, synth.seed(1, 0, 10 * M + 1))
    C = q4.q4_gemm_skinny(to_dev(A, "bf16"), to_dev(Wp, "u8"), to_dev(am, "f32"),
                          to_dev(cb, "f32"), bs, path="fused")
    _sync()
    cols = sample_cols(N, 192, 17 * M)
    Cr, S = oracle.q4_gemm(A, Wp, am, cb, M, N, K, bs, cols=cols)
    assert_within_tolerance(bf16_host(C)[:, cols], Cr, S, "FFN tiled M=%d" % M)


CHILD = r'''
import sys
import numpy as np
import torch
import bit_dequant_skinny_amd as q4
import oracle, synth
sys.path.insert(0, "tests")
from gpu_util import (assert_within_tolerance, bf16_host, host_f64, q4_to_dev, to_dev,
                      to_dev_dtype)

which = sys.argv[1]
sync = torch.cuda.synchronize
if which == "few_rows":
    cases = [(M, N, K, bs) for M in (1, 5, 16, 17, 32)
             for (N, K, bs) in ((300, 1088, 64), (70, 2048, 128), (600, 512, 64))]
else:
    cases = [(M, N, K, bs) for M in (33, 64, 100, 129)
             for (N, K, bs) in ((300, 1088, 64), (64, 4096, 128), (517, 2048, 256),
                                (1000, 640, 64), (2100, 1024, 64))]
for (M, N, K, bs) in cases:
    p = synth.q4_problem(M, N, K, bs, config=85, shape=N % 7, codebook=synth.random_codebook(90))
    A, Wp, am, cb = q4_to_dev(p)
    C = q4.q4_gemm_skinny(A, Wp, am, cb, bs, path="fused")
    C2 = q4.q4_gemm_skinny(A * 2, Wp, am, cb, bs, path="fused")
    sync()
    Cr, S = oracle.q4_gemm(p["A"], p["Wpacked"], p["absmax"], p["codebook"], M, N, K, bs)
    assert_within_tolerance(bf16_host(C), Cr, S, "%s M=%d N=%d K=%d" % (which, M, N, K))
    assert torch.equal(C2, C * 2), "2A != 2C"
    print("ok", M, N, K, flush=True)
if which != "few_rows":
    M, N, K, bs = 48, 333, 1024, 64
    p = synth.q4_problem(M, N, K, bs, config=83, codebook=synth.random_codebook(87))
    _, Wp, am, cb = q4_to_dev(p)
    for adt in ("bf16", "fp16", "fp32"):
        for cdt, tdt in (("bf16", torch.bfloat16), ("fp32", torch.float32)):
            A_h = synth.activations(M, K, 88, adt)
            b_h = synth.bias(N, 89, cdt)
            C = q4.q4_gemm_skinny(to_dev_dtype(A_h, adt), Wp, am, cb, bs, path="fused",
                                  bias=to_dev_dtype(b_h, cdt), out_dtype=tdt)
            sync()
            Cr, S = oracle.q4_gemm_ex(A_h, adt, p["Wpacked"], p["absmax"], p["codebook"], M, N,
                                      K, bs, bias=b_h, bias_dtype=cdt)
            assert_within_tolerance(None, Cr, S, "%s %s->%s" % (which, adt, cdt), out=cdt,
                                    values=host_f64(C))
            print("ok", adt, cdt, flush=True)
print("done", flush=True)
'''


def _child(which, env_extra):
    env = dict(os.environ)
    env.update(env_extra)
    env["PYTHONPATH"] = ROOT + os.pathsep + env.get("PYTHONPATH", "")
    r = subprocess.run([sys.executable, "-c", CHILD, which], cwd=ROOT, env=env,
                       capture_output=True, text=True, timeout=280)
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-4000:]
    assert "done" in r.stdout
    return r.stdout


@pytest.mark.parametrize("layout", ["0", "1"])
def test_fused_tiled_each_layout(layout):
    """Every case with the layout forced: 20 shapes and 6 type pairs."""
    out = _child("layouts", {"Q4_FUSED_TILED_LAYOUT": layout})
    assert out.count("ok ") == 20 + 6


@pytest.mark.parametrize("layout", ["0", "1"])
def test_fused_tiled_32_row_tiles_on_few_rows(layout):
    out = _child("few_rows", {"Q4_FUSED_TILED_MIN_M": "0", "Q4_FUSED_TILED_LAYOUT": layout})
    assert out.count("ok ") == 15


def test_fused_tiled_n_split_layout_at_scale():
    """A shape the dispatcher gives the N-split layout (many 256-feature
    tiles): 100 rows over 9984 features, K = 1088 (ragged), sampled columns."""
    M, N, K, bs = 100, 9984, 1088, 64
    p = synth.q4_problem(M, N, K, bs, config=86)
    A, Wp, am, cb = q4_to_dev(p)
    C = q4.q4_gemm_skinny(A, Wp, am, cb, bs, path="fused")
    _sync()
    cols = sample_cols(N, 600, 91)
    Cr, S = oracle.q4_gemm(p["A"], p["Wpacked"], p["absmax"], p["codebook"], M, N, K, bs,
                           cols=cols)
    assert_within_tolerance(bf16_host(C)[:, cols], Cr, S, "N-split at scale")
