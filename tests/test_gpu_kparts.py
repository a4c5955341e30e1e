"""K split over workgroups in the fused skinny kernel (q4_skinny_kparts).

When the 16-row tiles of a weight leave compute units idle (N = 5120 on 256
CUs) and the split saves enough of each workgroup's walk, the kernel cuts K
into parts computed by different workgroups; a second kernel adds the parts'
fp32 sums in part order, adds the bias and rounds once.

CPU: the plan the library picks for the decode shapes (it assumes 256 CUs
when no GPU is visible, the count of MI355X).
GPU: results meet the oracle's tolerance with both weight layouts, every
blocksize, ragged K, a bias and fp16 / fp32 outputs; repeated calls are
bitwise identical in each layout (the two layouts walk K in different
orders, so they agree to the oracle's tolerance); graph
replays equal the eager result.
"""
import numpy as np
import pytest

import bit_dequant_skinny_amd as q4
import oracle
import synth

CB = synth.random_codebook(77)


@pytest.mark.parametrize("M,N,K,parts", [
    (1, 5120, 17408, 3), (16, 5120, 17408, 3), (1, 5120, 5120, 1), (8, 5120, 5120, 1),
    (1, 28672, 8192, 1), (1, 8192, 5120, 1), (1, 8192, 8192, 1), (1, 4096, 4096, 1),
    (1, 248320, 2560, 1), (17, 5120, 17408, 3), (32, 5120, 17408, 3), (33, 5120, 17408, 1),
    (24, 248320, 2560, 1), (17, 1536, 16384, 8), (32, 768, 32768, 5), (20, 1544, 16384, 2),
    (1, 1536, 16384, 8), (1, 1536, 16448, 5), (1, 768, 32768, 5), (0, 5120, 17408, 1),
    (1, 0, 17408, 1),
])
def test_kparts_plan(M, N, K, parts):
    assert q4.q4_skinny_kparts(M, N, K) == parts


def _gpu():
    import gpu_util
    return gpu_util


def _problem(M, N, K, bs, config):
    g = _gpu()
    p = synth.q4_problem(M, N, K, bs, config=config, shape=N % 5, codebook=CB)
    return p, g.q4_to_dev(p)


@pytest.mark.gpu
@pytest.mark.parametrize("layout", ["rows", "tiles"])
@pytest.mark.parametrize("M,N,K,bs", [
    (1, 1536, 16384, 64), (4, 1536, 16384, 64), (16, 768, 32768, 64), (1, 1536, 16448, 64),
    (3, 1536, 16512, 128), (2, 1536, 16384, 256), (5, 768, 32768, 64), (2, 1544, 16384, 64),
    (17, 1536, 16384, 64), (32, 768, 32768, 64), (20, 1544, 16384, 64), (32, 1536, 16448, 64),
    (24, 1536, 16512, 128),
])
def test_kparts_parity(M, N, K, bs, layout):
    g = _gpu()
    assert q4.q4_skinny_kparts(M, N, K) > 1
    if layout == "tiles" and (K % 128 or N % 16):
        pytest.skip("the tile layout needs K % 128 == 0 and N % 16 == 0")
    p, (A, Wp, am, cb) = _problem(M, N, K, bs, 700 + M)
    W = q4.q4_repack_tiles(Wp) if layout == "tiles" else Wp
    C = q4.q4_gemm_skinny(A, W, am, cb, bs, path="fused", layout=layout)
    g.torch().cuda.synchronize()
    Cr, S = oracle.q4_gemm(p["A"], p["Wpacked"], p["absmax"], p["codebook"], M, N, K, bs)
    g.assert_within_tolerance(g.bf16_host(C), Cr, S, "kparts M=%d N=%d K=%d" % (M, N, K))


@pytest.mark.gpu
@pytest.mark.parametrize("cdt", ["bf16", "fp16", "fp32"])
@pytest.mark.parametrize("M", [3, 24])
def test_kparts_bias_and_output_types(cdt, M):
    g = _gpu()
    t = g.torch()
    N, K, bs = 1536, 16384, 64
    assert q4.q4_skinny_kparts(M, N, K) > 1
    p, (A, Wp, am, cb) = _problem(M, N, K, bs, 710)
    b_h = synth.bias(N, 711, cdt)
    bias = g.to_dev_dtype(b_h, cdt)
    odt = {"bf16": t.bfloat16, "fp16": t.float16, "fp32": t.float32}[cdt]
    C = q4.q4_gemm_skinny(A, Wp, am, cb, bs, path="fused", bias=bias, out_dtype=odt)
    t.cuda.synchronize()
    Cr, S = oracle.q4_gemm_ex(p["A"], "bf16", p["Wpacked"], p["absmax"], p["codebook"], M, N, K,
                              bs, bias=b_h, bias_dtype=cdt)
    g.assert_within_tolerance(None, Cr, S, "kparts bias %s M=%d" % (cdt, M), out=cdt,
                              values=g.host_f64(C))


@pytest.mark.gpu
def test_kparts_special_scales():
    """Zero, subnormal and huge block scales, and a zero block at every part
    boundary of one row, through the K parts."""
    g = _gpu()
    M, N, K, bs = 2, 1536, 16448, 64
    assert q4.q4_skinny_kparts(M, N, K) == 5
    p, _ = _problem(M, N, K, bs, 720)
    am = p["absmax"].copy()
    rng = np.random.default_rng(721)
    specials = np.array([0.0, 1e-40, 3e-39, 1e30, 2.0 ** -126], dtype=np.float32)
    idx = rng.integers(0, am.size, size=400)
    am.flat[idx] = specials[rng.integers(0, len(specials), size=idx.size)]
    am[7, ::16] = 0.0  # parts are multiples of 8 segments: 16 blocks of 64
    A, Wp, dam, cb = g.to_dev(p["A"], "bf16"), g.to_dev(p["Wpacked"], "u8"), g.to_dev(am, "f32"), \
        g.to_dev(p["codebook"], "f32")
    C = q4.q4_gemm_skinny(A, Wp, dam, cb, bs, path="fused")
    g.torch().cuda.synchronize()
    Cr, S = oracle.q4_gemm(p["A"], p["Wpacked"], am, p["codebook"], M, N, K, bs)
    g.assert_within_tolerance(g.bf16_host(C), Cr, S, "kparts special scales")


@pytest.mark.gpu
@pytest.mark.parametrize("M,N,K", [(1, 5120, 17408), (16, 5120, 17408), (17, 5120, 17408),
                                   (32, 5120, 17408)])
def test_kparts_deterministic_and_layouts_agree(M, N, K):
    g = _gpu()
    t = g.torch()
    bs = 64
    assert q4.q4_skinny_kparts(M, N, K) > 1
    A = g.to_dev(synth.activations_bf16(M, K, 731), "bf16")
    Wp_h, am_h, cb_h = g.q4_weights(N, K, bs, 73, 1)
    Wp, am, cb = g.to_dev(Wp_h, "u8"), g.to_dev(am_h, "f32"), g.to_dev(cb_h, "f32")
    Wt = q4.q4_repack_tiles(Wp)
    rows = [q4.q4_gemm_skinny(A, Wp, am, cb, bs, path="fused") for _ in range(3)]
    tiles = [q4.q4_gemm_skinny(A, Wt, am, cb, bs, path="fused", layout="tiles") for _ in range(3)]
    t.cuda.synchronize()
    for runs in (rows, tiles):
        for r in runs[1:]:
            assert t.equal(r, runs[0])
    cols = g.sample_cols(N, 256, 733)
    Cr, S = oracle.q4_gemm(synth.activations_bf16(M, K, 731), Wp_h, am_h, cb_h, M, N, K, bs,
                           cols=cols)
    for name, runs in (("rows", rows), ("tiles", tiles)):
        g.assert_within_tolerance(g.bf16_host(runs[0])[:, cols], Cr, S, "kparts full size " + name)


@pytest.mark.gpu
@pytest.mark.parametrize("M", [20, 32])
def test_kparts_two_token_blocks_equal_16_row_passes(M):
    """With K parts, rows 0..15 and 16..M-1 in one two-block pass equal two
    separate calls bit for bit (same plan, same MFMA sequence per output, the
    parts added in the same order)."""
    g = _gpu()
    N, K, bs = 5120, 17408, 64
    assert q4.q4_skinny_kparts(M, N, K) == q4.q4_skinny_kparts(16, N, K) > 1
    A = g.to_dev(synth.activations_bf16(M, K, 751), "bf16")
    Wp_h, am_h, cb_h = g.q4_weights(N, K, bs, 75, 1)
    Wp, am, cb = g.to_dev(Wp_h, "u8"), g.to_dev(am_h, "f32"), g.to_dev(cb_h, "f32")
    C = g.bf16_host(q4.q4_gemm_skinny(A, Wp, am, cb, bs, path="fused"))
    C0 = g.bf16_host(q4.q4_gemm_skinny(A[:16].contiguous(), Wp, am, cb, bs, path="fused"))
    C1 = g.bf16_host(q4.q4_gemm_skinny(A[16:].contiguous(), Wp, am, cb, bs, path="fused"))
    g.torch().cuda.synchronize()
    assert np.array_equal(C, np.concatenate([C0, C1], axis=0))


@pytest.mark.gpu
def test_kparts_graph_replays():
    """Three K-split calls captured into one graph (each a split kernel and
    the sum of its parts), replayed several times with eager calls between
    the replays: every replay equals the eager result."""
    g = _gpu()
    t = g.torch()
    bs = 64
    shapes = [(1, 1536, 16384), (4, 1536, 16448), (2, 768, 32768)]
    probs = [_problem(M, N, K, bs, 740 + i) for i, (M, N, K) in enumerate(shapes)]
    side = t.cuda.Stream()
    eager, outs = [], []
    with t.cuda.stream(side):
        for (M, N, K), (p, (A, Wp, am, cb)) in zip(shapes, probs):
            eager.append(q4.q4_gemm_skinny(A, Wp, am, cb, bs, path="fused"))
            outs.append(t.zeros((M, N), dtype=t.bfloat16, device=A.device))
    t.cuda.synchronize()
    graph = t.cuda.CUDAGraph()
    with t.cuda.graph(graph, stream=side):
        for (M, N, K), (p, (A, Wp, am, cb)), o in zip(shapes, probs, outs):
            q4.q4_gemm_skinny(A, Wp, am, cb, bs, path="fused", out=o)
    for rep in range(4):
        for o in outs:
            o.zero_()
        t.cuda.synchronize()
        graph.replay()
        t.cuda.synchronize()
        for o, e in zip(outs, eager):
            assert t.equal(o, e), "replay %d differs" % rep
        # eager work on the default stream between replays
        p, (A, Wp, am, cb) = probs[rep % 3]
        q4.q4_gemm_skinny(A, Wp, am, cb, bs, path="fused")
        t.cuda.synchronize()
