"""The tile layout of unquantized bf16 weights (bf16_repack_tiles,
bf16_gemm_skinny_tiles).

CPU: the oracle's layout (O13) is pinned by indices worked by hand
(tests/golden/bf16_tile_layout.txt), by being a bijection onto [0, N*K), by
each tile occupying its own contiguous 16*K elements and each unit holding
exactly the 16 rows x 32 k of its step, and by each 16-byte piece holding 8
consecutive k of one row (the row of the lane that loads it).  The
entry points reject shapes the layout cannot hold before touching the GPU
runtime.

GPU: the repack kernel equals the oracle element for element; the GEMM over
tiles equals the GEMM over row-major weights bit for bit and meets the
oracle's tolerance, at small and ragged shapes (K split over waves), at the
decode shapes and at the 248320-row projection.
"""
import os

import numpy as np
import pytest

import bit_dequant_skinny_amd as q4
import oracle
import synth

HERE = os.path.dirname(os.path.abspath(__file__))
FAKE = 0x10000
INV, UNS, OK = q4.Q4_ERR_INVALID_ARGUMENT, q4.Q4_ERR_UNSUPPORTED, q4.Q4_OK


def _golden():
    rows = []
    for line in open(os.path.join(HERE, "golden", "bf16_tile_layout.txt")):
        line = line.strip()
        if line and not line.startswith("#"):
            rows.append(tuple(int(v) for v in line.split()))
    return rows


def test_bf16_tile_index_matches_worked_values():
    rows = _golden()
    assert len(rows) >= 8
    for n, k, idx in rows:
        assert oracle.bf16_tile_index(32, 64, n, k) == idx, (n, k)


@pytest.mark.parametrize("N,K", [(16, 32), (48, 96), (32, 256)])
def test_bf16_tile_layout_is_a_bijection_of_whole_tiles_and_units(N, K):
    idx = np.array([[oracle.bf16_tile_index(N, K, n, k) for k in range(K)] for n in range(N)])
    assert sorted(idx.ravel().tolist()) == list(range(N * K))
    for t in range(N // 16):  # tile t is the contiguous run [16*K*t, 16*K*(t+1))
        blk = idx[16 * t:16 * t + 16]
        assert blk.min() == 16 * K * t and blk.max() == 16 * K * (t + 1) - 1
        for s in range(K // 32):  # one 512-element unit per (tile, step)
            u = blk[:, 32 * s:32 * s + 32]
            assert u.min() % 512 == 0 and u.max() == u.min() + 511
            # 8 consecutive k of a row stay consecutive (one 16-byte piece)
            assert np.all(np.diff(u.reshape(16, 4, 8), axis=2) == 1)
            # piece p of the unit is row p % 16: lanes of one k group are rows 0..15
            assert np.array_equal(u[:, 0] - u.min(), 8 * np.arange(16))


@pytest.mark.parametrize("N,K", [(16, 32), (32, 96), (48, 64)])
def test_bf16_pieces_are_8_consecutive_k_of_one_row(N, K):
    # a lane's 16 bytes are 8 consecutive k of one row, and piece p of a unit
    # belongs to row p % 16 of the tile, k = 8 (p / 16) .. +7 of the step
    idx = np.array([[oracle.bf16_tile_index(N, K, n, k) for k in range(K)] for n in range(N)])
    assert np.all(np.diff(idx.reshape(N, K // 8, 8), axis=2) == 1)
    piece = (idx % 512) // 8
    for n in range(N):
        for k in range(0, K, 8):
            assert piece[n, k] % 16 == n % 16 and piece[n, k] // 16 == (k % 32) // 8


def test_bf16_repack_moves_elements_not_values():
    N, K = 32, 128
    rng = np.random.default_rng(7)
    W = rng.integers(0, 1 << 16, size=(N, K), dtype=np.uint16)
    T = oracle.bf16_repack_tiles(W, N, K).ravel()
    back = np.empty_like(W)
    for n in range(N):
        for k in range(K):
            back[n, k] = T[oracle.bf16_tile_index(N, K, n, k)]
    assert np.array_equal(back, W)
    # piece 17 of unit (0, 0) is row 1, k 8..15 (lane 17 of a 16-row tile)
    assert np.array_equal(T[17 * 8:18 * 8], W[1, 8:16])


@pytest.mark.parametrize("args,expect", [
    ((FAKE, FAKE + 0x100000, 20, 64), INV), ((FAKE, FAKE + 0x100000, 16, 48), INV),
    ((FAKE, FAKE + 0x100000, -16, 64), INV), ((FAKE, FAKE + 0x100000, 16, 0), INV),
    ((None, FAKE, 16, 64), INV), ((FAKE, None, 16, 64), INV),
    ((FAKE + 8, FAKE + 0x100000, 16, 64), INV), ((FAKE, FAKE + 0x100008, 16, 64), INV),
    ((FAKE, FAKE + 1024, 16, 64), INV), ((FAKE, FAKE, 0, 64), OK),
    ((FAKE, FAKE + 0x100000, 65536, 16384), UNS),
])
def test_bf16_repack_validation(args, expect):
    W, T, N, K = args
    assert q4.lib().bf16_repack_tiles(W, T, N, K, None) == expect
    assert (q4.lib().q4_last_error().decode() == "") == (expect == OK)


@pytest.mark.parametrize("kw,expect", [
    (dict(N=20), INV), (dict(K=48), INV), (dict(K=12), INV), (dict(M=6), UNS),
    (dict(M=-1), INV), (dict(A=None), INV), (dict(C=None), INV), (dict(M=0), OK),
    (dict(N=0), OK), (dict(N=20, M=0), INV), (dict(N=65536, K=16384), UNS),
    (dict(W=FAKE + 8), INV),
])
def test_bf16_gemm_tiles_validation(kw, expect):
    p = dict(A=FAKE, W=FAKE, bias=None, M=1, N=16, K=64, C=FAKE)
    p.update(kw)
    st = q4.lib().bf16_gemm_skinny_tiles(p["A"], p["W"], p["bias"], p["M"], p["N"], p["K"],
                                         p["C"], None)
    assert st == expect


# ---------------------------------------------------------------- GPU parity

def _gpu():
    import gpu_util
    return gpu_util


@pytest.mark.gpu
@pytest.mark.parametrize("N,K", [(16, 32), (48, 96), (2048, 2560), (31040, 2560)])
def test_gpu_bf16_repack_matches_oracle(N, K):
    g = _gpu()
    rng = np.random.default_rng(N + 3 * K)
    W = rng.integers(0, 1 << 16, size=(N, K), dtype=np.uint16)
    T = q4.bf16_repack_tiles(g.to_dev(W, "bf16"))
    g.torch().cuda.synchronize()
    got = g.bf16_host(T)
    if N * K <= 2048 * 2560:
        assert np.array_equal(got, oracle.bf16_repack_tiles(W, N, K))
    else:  # every element of sampled rows, at its oracle index
        flat = got.ravel()
        for n in [0, 15, 16, 4097, N - 1]:
            idx = [oracle.bf16_tile_index(N, K, n, k) for k in range(K)]
            assert np.array_equal(flat[idx], W[n]), n


def _tiles_case(M, N, K, with_bias, config, shape, ncols=None):
    g = _gpu()
    p = synth.bf16_problem(M, N, K, with_bias, config=config, shape=shape)
    A, W = g.to_dev(p["A"], "bf16"), g.to_dev(p["W"], "bf16")
    b = g.to_dev(p["bias"], "bf16") if with_bias else None
    Wt = q4.bf16_repack_tiles(W)
    C_rows = q4.bf16_gemm_skinny(A, W, b)
    C_tiles = q4.bf16_gemm_skinny(A, Wt, b, layout="tiles")
    g.torch().cuda.synchronize()
    rows, tiles = g.bf16_host(C_rows), g.bf16_host(C_tiles)
    assert np.array_equal(rows, tiles), "tile layout differs from row-major (M=%d N=%d K=%d)" % (M, N, K)
    cols = None if ncols is None else g.sample_cols(N, ncols, 13 * N + M)
    Cr, S = oracle.bf16_gemm(p["A"], p["W"], p["bias"], M, N, K, cols=cols)
    got = tiles if cols is None else tiles[:, cols]
    g.assert_within_tolerance(got, Cr, S, "bf16 tiles M=%d N=%d K=%d" % (M, N, K))


@pytest.mark.gpu
@pytest.mark.parametrize("M", [1, 2, 3, 4, 5])
@pytest.mark.parametrize("N,K", [(16, 32), (48, 96), (96, 2560), (160, 1056), (2048, 2560)])
@pytest.mark.parametrize("with_bias", [False, True])
def test_gpu_bf16_tiles_parity(M, N, K, with_bias):
    _tiles_case(M, N, K, with_bias, config=61, shape=N % 3)


@pytest.mark.gpu
@pytest.mark.parametrize("M", [1, 5])
@pytest.mark.parametrize("N", [16384, 31040, 248320])
def test_gpu_bf16_tiles_full_size(M, N):
    _tiles_case(M, N, 2560, with_bias=(M == 5), config=62, shape=0, ncols=256)


@pytest.mark.gpu
def test_gpu_bf16_tiles_reject_wider_slabs_and_bad_shapes():
    g = _gpu()
    t = g.torch()
    d = g.dev()
    A = t.zeros((6, 64), dtype=t.bfloat16, device=d)
    W = t.zeros((32, 64), dtype=t.bfloat16, device=d)
    with pytest.raises(q4.Q4Error) as e:
        q4.bf16_gemm_skinny(A, W, layout="tiles")
    assert e.value.status == q4.Q4_ERR_UNSUPPORTED
    with pytest.raises(q4.Q4Error) as e:
        q4.bf16_gemm_skinny(A[:1], W[:20], layout="tiles")
    assert e.value.status == q4.Q4_ERR_INVALID_ARGUMENT
    # no sticky error left behind
    C = q4.bf16_gemm_skinny(A[:5], q4.bf16_repack_tiles(W), layout="tiles")
    t.cuda.synchronize()
    assert C.shape == (5, 32) and not C.float().abs().sum().item()
