"""The tile layout of the packed weights (q4_repack_tiles, q4_gemm_skinny_tiles,
q4_dequant_tiles).

CPU: the oracle's layout is pinned by offsets worked by hand
(tests/golden/tile_layout.txt), by being a bijection onto [0, N*K/2), by each
tile occupying its own contiguous 16*K/2 bytes, by each 1 KiB unit holding
exactly the 16 rows x 64 bytes of its segment, and by each 16-byte piece
holding 8 bytes of each 64-wide half of one row's segment.  The entry points reject
shapes the layout cannot hold before touching the GPU runtime.

GPU: the repack kernel equals the oracle byte for byte; GEMMs over tiles and
over the row-major weights they were made from both meet the oracle's
tolerance on every path (skinny kernel, two token blocks, tiled kernel,
planes for fp16/fp32 activations, split path), and equal each other bit for
bit wherever the kernels sum in the same order over both layouts (the tiled
kernel above 32 rows, the split path); the skinny kernel walks K in a
rotated order over rows only, so up to 32 rows the two layouts may differ by
rounding.  Dequantizing tiles equals the oracle's dequantize bit for bit.
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
    for line in open(os.path.join(HERE, "golden", "tile_layout.txt")):
        line = line.strip()
        if line and not line.startswith("#"):
            rows.append(tuple(int(v) for v in line.split()))
    return rows


def test_tile_offsets_match_worked_values():
    rows = _golden()
    assert len(rows) >= 8
    for n, j, off in rows:
        assert oracle.tile_offset(32, 256, n, j) == off, (n, j)


@pytest.mark.parametrize("N,K", [(16, 128), (48, 384), (32, 1024)])
def test_tile_layout_is_a_bijection_of_whole_tiles_and_units(N, K):
    rb = K // 2
    offs = np.array([[oracle.tile_offset(N, K, n, j) for j in range(rb)] for n in range(N)])
    assert sorted(offs.ravel().tolist()) == list(range(N * rb))
    for t in range(N // 16):  # tile t is the contiguous run [t*16*rb, (t+1)*16*rb)
        blk = offs[16 * t:16 * t + 16]
        assert blk.min() == 16 * t * rb and blk.max() == 16 * (t + 1) * rb - 1
        for s in range(K // 128):  # one 1 KiB unit per (tile, segment)
            u = blk[:, 64 * s:64 * s + 64]
            assert u.min() % 1024 == 0 and u.max() == u.min() + 1023
            # 8 consecutive bytes of a row stay consecutive (half a piece),
            # and a piece holds bytes c*8.. of the segment's first 32 bytes
            # then (c+4)*8.. of its second 32 (one 16-byte piece per lane,
            # each half from its own 64-wide block of k)
            q = u.reshape(16, 8, 8)
            assert np.all(np.diff(q, axis=2) == 1)
            assert np.all(q[:, 4:, 0] == q[:, :4, 0] + 8)
            assert np.all(q[:, :4, 0] % 16 == 0)


def test_repack_moves_bytes_not_values():
    N, K = 32, 512
    rng = np.random.default_rng(5)
    W = rng.integers(0, 256, size=(N, K // 2), dtype=np.uint8)
    T = oracle.repack_tiles(W, N, K).ravel()
    back = np.empty_like(W)
    for n in range(N):
        for j in range(K // 2):
            back[n, j] = T[oracle.tile_offset(N, K, n, j)]
    assert np.array_equal(back, W)
    assert np.array_equal(np.sort(T), np.sort(W.ravel()))
    # piece 17 of unit (0, 0) (lane 17 of a 16-row tile) is row 1, bytes
    # 16..23 and 48..55: quarter 2 of each 64-wide half of the segment
    assert np.array_equal(T[17 * 16:17 * 16 + 8], W[1, 16:24])
    assert np.array_equal(T[17 * 16 + 8:18 * 16], W[1, 48:56])


@pytest.mark.parametrize("args,expect", [
    ((FAKE, FAKE + 0x100000, 20, 128), INV), ((FAKE, FAKE + 0x100000, 16, 192), INV),
    ((FAKE, FAKE + 0x100000, -16, 128), INV), ((FAKE, FAKE + 0x100000, 16, 0), INV),
    ((None, FAKE, 16, 128), INV), ((FAKE, None, 16, 128), INV),
    ((FAKE + 8, FAKE + 0x100000, 16, 128), INV), ((FAKE, FAKE + 0x100008, 16, 128), INV),
    ((FAKE, FAKE + 512, 16, 128), INV), ((FAKE, FAKE, 0, 128), OK),
    ((FAKE, FAKE + 0x100000, 65536, 131072), UNS),
])
def test_repack_validation(args, expect):
    W, T, N, K = args
    assert q4.lib().q4_repack_tiles(W, T, N, K, None) == expect
    assert (q4.lib().q4_last_error().decode() == "") == (expect == OK)


@pytest.mark.parametrize("kw,expect", [
    (dict(N=20), INV), (dict(K=192, bs=64), INV), (dict(bs=32), UNS), (dict(M=-1), INV),
    (dict(A=None), INV), (dict(path=5), INV), (dict(M=0), OK), (dict(N=0), OK),
    (dict(N=20, M=0), INV),
])
def test_gemm_tiles_validation(kw, expect):
    p = dict(A=FAKE, adt=0, W=FAKE, am=FAKE, cb=FAKE, bias=None, M=1, N=16, K=128, bs=64,
             C=FAKE, cdt=0, path=0)
    p.update(kw)
    st = q4.lib().q4_gemm_skinny_tiles(p["A"], p["adt"], p["W"], p["am"], p["cb"], p["bias"],
                                       p["M"], p["N"], p["K"], p["bs"], p["C"], p["cdt"], None,
                                       p["path"])
    assert st == expect


@pytest.mark.parametrize("kw,expect", [
    (dict(N=24), INV), (dict(K=64, bs=64), INV), (dict(bs=32), UNS), (dict(out=None), INV),
    (dict(N=0), OK),
])
def test_dequant_tiles_validation(kw, expect):
    p = dict(W=FAKE, am=FAKE, cb=FAKE, N=16, K=128, bs=64, out=FAKE, dtype=0)
    p.update(kw)
    assert q4.lib().q4_dequant_tiles(p["W"], p["am"], p["cb"], p["N"], p["K"], p["bs"],
                                     p["out"], p["dtype"], None) == expect


# ---------------------------------------------------------------- GPU parity

def _gpu():
    from gpu_util import (assert_within_tolerance, bf16_host, q4_to_dev, to_dev, to_dev_dtype,
                          host_f64, torch)
    return assert_within_tolerance, bf16_host, q4_to_dev, to_dev, to_dev_dtype, host_f64, torch


@pytest.mark.gpu
@pytest.mark.parametrize("N,K", [(16, 128), (48, 1152), (4096, 4096), (28672, 8192)])
def test_gpu_repack_matches_oracle(N, K):
    _, _, _, to_dev, _, _, torch = _gpu()
    rng = np.random.default_rng(N + K)
    W = rng.integers(0, 256, size=(N, K // 2), dtype=np.uint8)
    T = q4.q4_repack_tiles(to_dev(W, "u8"))
    torch().cuda.synchronize()
    if N * K <= 4096 * 4096:
        assert np.array_equal(T.cpu().numpy(), oracle.repack_tiles(W, N, K))
    else:  # every byte of sampled rows, at its oracle offset
        flat = T.cpu().numpy().ravel()
        for n in [0, 15, 16, 4097, N - 1]:
            offs = [oracle.tile_offset(N, K, n, j) for j in range(K // 2)]
            assert np.array_equal(flat[offs], W[n]), n


def _tiles_case(M, N, K, bs, config, adt="bf16", cdt="bf16", bias=False, path="auto",
                cols=None):
    """Runs the GEMM over row-major weights and over their tiles and checks
    both against the oracle (on the sampled columns cols, or all of them).
    Where both layouts sum in the same order (above the skinny kernel's 32
    rows, or the split path) the two must also be equal bit for bit."""
    tol, bf16_host, q4_to_dev, to_dev, to_dev_dtype, host_f64, torch = _gpu()
    p = synth.q4_problem(M, N, K, bs, config=config)
    A, Wp, am, cb = q4_to_dev(p)
    T = q4.q4_repack_tiles(Wp)
    tdt = {"bf16": torch().bfloat16, "fp16": torch().float16, "fp32": torch().float32}
    if adt != "bf16":
        A = A.to(tdt[adt])
    b = None
    if bias:
        b = (torch().randn(N, generator=torch().Generator().manual_seed(config)) * 0.5).to(
            tdt[cdt]).to(A.device)
    kw = dict(path=path, bias=b, out_dtype=tdt[cdt])
    C_rows = q4.q4_gemm_skinny(A, Wp, am, cb, bs, **kw)
    C_tiles = q4.q4_gemm_skinny(A, T, am, cb, bs, layout="tiles", **kw)
    torch().cuda.synchronize()

    def host_bits(x):  # the oracle's input format: bit patterns, or fp32 values
        x = x.cpu()
        return x.numpy() if x.dtype == torch().float32 else x.view(torch().int16).numpy().view(
            np.uint16)
    A_h = host_bits(A)
    b_h = None if b is None else host_bits(b)
    Cr, S = oracle.q4_gemm_ex(A_h, adt, p["Wpacked"], p["absmax"], p["codebook"], M, N, K, bs,
                              bias=b_h, bias_dtype=cdt, cols=cols)
    sel = slice(None) if cols is None else cols
    for name, C in (("rows", C_rows), ("tiles", C_tiles)):
        tol(None, Cr, S, "%s M=%d N=%d K=%d %s->%s" % (name, M, N, K, adt, cdt), out=cdt,
            values=host_f64(C)[:, sel])
    if path == "split" or M > 32:
        assert torch().equal(C_rows.view(torch().int16) if cdt != "fp32" else C_rows,
                             C_tiles.view(torch().int16) if cdt != "fp32" else C_tiles), \
            "tiles differ from rows at M=%d N=%d K=%d" % (M, N, K)
    return p, C_tiles


@pytest.mark.gpu
@pytest.mark.parametrize("M", [1, 2, 4, 8, 16, 17, 32, 33, 64, 129])
@pytest.mark.parametrize("N,K,bs", [(512, 1024, 64), (1040, 2304, 128), (4096, 4096, 64),
                                    (96, 768, 256)])
def test_gpu_gemm_tiles_equal_rows_and_oracle(M, N, K, bs):
    _tiles_case(M, N, K, bs, config=90 + M)


@pytest.mark.gpu
@pytest.mark.parametrize("M,path", [(300, "auto"), (40, "split"), (8, "split")])
def test_gpu_gemm_tiles_split_path(M, path):
    N, K, bs = 1024, 1536, 64
    tol, bf16_host = _gpu()[:2]
    p, C = _tiles_case(M, N, K, bs, config=97, path=path)
    Cr, S = oracle.q4_gemm_w16(p["A"], p["Wpacked"], p["absmax"], p["codebook"], M, N, K, bs)
    tol(bf16_host(C), Cr, S, "tiles split M=%d" % M)


@pytest.mark.gpu
@pytest.mark.parametrize("adt,cdt,M", [("fp16", "fp32", 4), ("fp32", "bf16", 20),
                                       ("fp16", "fp16", 70), ("bf16", "fp32", 100)])
def test_gpu_gemm_tiles_dtypes_and_bias(adt, cdt, M):
    _tiles_case(M, 768, 2048, 64, config=98, adt=adt, cdt=cdt, bias=True)


@pytest.mark.gpu
@pytest.mark.parametrize("bs,dt", [(64, "bf16"), (128, "fp32"), (256, "fp16")])
def test_gpu_dequant_tiles_bit_exact(bs, dt):
    _, _, q4_to_dev, _, _, _, torch = _gpu()
    N, K = 272, 1280
    p = synth.q4_problem(1, N, K, bs, config=99)
    _, Wp, am, cb = q4_to_dev(p)
    tdt = {"bf16": torch().bfloat16, "fp16": torch().float16, "fp32": torch().float32}[dt]
    T = q4.q4_repack_tiles(Wp)
    D_rows = q4.q4_dequant(Wp, am, cb, bs, out_dtype=tdt)
    D_tiles = q4.q4_dequant(T, am, cb, bs, out_dtype=tdt, layout="tiles")
    torch().cuda.synchronize()
    ref = {"bf16": oracle.dequant_bf16, "fp16": oracle.dequant_f16,
           "fp32": oracle.dequant_f32}[dt](p["Wpacked"], p["absmax"], p["codebook"], N, K, bs)
    got = D_tiles.cpu()
    got = got.numpy() if dt == "fp32" else got.view(torch().int16).numpy().view(np.uint16)
    assert np.array_equal(got.view(np.uint32 if dt == "fp32" else np.uint16),
                          np.asarray(ref).view(np.uint32 if dt == "fp32" else np.uint16))
    assert torch().equal(D_rows.view(torch().int16) if dt != "fp32" else D_rows,
                         D_tiles.view(torch().int16) if dt != "fp32" else D_tiles)


@pytest.mark.gpu
@pytest.mark.parametrize("M", [1, 2, 4, 8, 64])
def test_gpu_gemm_tiles_ffn_full_size_equal_rows(M):
    """The 28672 x 8192 FFN over tiles, in the instantiations the benchmark
    times (M = 1, 2, 4, 8): within tolerance of the oracle on sampled columns,
    as is the row-major call (equal to it bit for bit at M = 64)."""
    from gpu_util import sample_cols
    _tiles_case(M, 28672, 8192, 64, config=2, cols=sample_cols(28672, 96, 31 * M))
