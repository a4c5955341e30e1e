"""Seeded synthetic inputs shared by the tests, the benchmark and the smoke check.

This module makes inputs only.  It holds none of the computation under test: it
never decodes codes, never multiplies a codebook entry by a scale and never
forms a dot product.  Rounding fp32 samples to bf16 goes through torch's own
cast (round-to-nearest-even), not through code written here.

Input recipe (shapes and distributions follow the decode workloads of the
bitsandbytes 4-bit kernel pull request, the RDNA GPTQ tuning pull request and
the aiter gfx950 tuned-GEMM pull request; the pages measure on real model
weights, which these seeded draws stand in for):
  * A     : N(0, 1) in fp32, rounded to bf16, shape [M, K].
  * W     : N(0, 0.02) in fp32 (0.02 is the standard deviation), shape [N, K].
  * 4-bit : per block of ``bs`` weights along K, absmax = max |w|;
            x = w / absmax in fp64; code = nearest codebook entry, ties to the
            lower index, decided with the fp64 midpoints of neighbouring
            sorted entries; a block of zeros stores absmax 0 and the code of
            the 0.0 entry.  Codes are packed two per byte, low nibble = even k.
  * bf16 W: N(0, 0.02) in fp32 rounded to bf16.
  * bias  : N(0, 1) in fp32 rounded to bf16, shape [N].
  * other element types: the same N(0, 1) draws kept in fp32, or rounded to
    IEEE binary16 by numpy's cast (round-to-nearest-even).
Seeds: ``seed(config, shape, tensor)`` = 1000*config + 100*shape + tensor, with
tensor 2 for W, 3 for the bias and 10*M + 1 for A, so an M sweep reuses one W.
"""
from __future__ import annotations

import os
import statistics
from concurrent.futures import ThreadPoolExecutor

import numpy as np

__all__ = [
    "seed", "rng", "nf4_style_codebook", "random_codebook", "activations_bf16",
    "weights_f32", "quantize_blockwise", "pack_nibbles", "bf16_from_f32",
    "bf16_weights", "bias_bf16", "q4_problem", "bf16_problem", "activations", "bias",
]


def seed(config: int, shape: int, tensor: int) -> int:
    return 1000 * config + 100 * shape + tensor


def rng(s: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(s))


def bf16_from_f32(x: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) of fp32 values, via torch's RNE cast."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()


def nf4_style_codebook(p_max: float = 0.97) -> np.ndarray:
    """A sorted 16-entry fp32 table in [-1, 1] holding -1, 0 and 1.

    Own rule (the pages name NF4 but print no values): 8 positive entries at
    the standard-normal quantiles of probabilities 0.5 + (i/8)(p_max - 0.5),
    i = 1..8, 7 negative entries at 0.5 - (i/7)(p_max - 0.5), i = 1..7, each
    side divided by its largest magnitude so its extreme is exactly +-1, plus
    an exact 0.  Computed in fp64, rounded to fp32.
    """
    nd = statistics.NormalDist()
    pos = [nd.inv_cdf(0.5 + (i / 8.0) * (p_max - 0.5)) for i in range(1, 9)]
    neg = [nd.inv_cdf(0.5 - (i / 7.0) * (p_max - 0.5)) for i in range(1, 8)]
    pos = [v / pos[-1] for v in pos]
    neg = [v / -neg[-1] for v in neg]
    vals = sorted(neg + [0.0] + pos)
    cb = np.array(vals, dtype=np.float64).astype(np.float32)
    assert cb[0] == -1.0 and cb[-1] == 1.0 and 0.0 in cb
    assert np.all(np.diff(cb) > 0)
    return cb


def random_codebook(s: int) -> np.ndarray:
    """Sorted distinct fp32 values in [-1, 1] holding -1, 0 and 1 (asymmetric)."""
    g = rng(s)
    while True:
        inner = g.uniform(-1.0, 1.0, size=13).astype(np.float32)
        vals = np.unique(np.concatenate([inner, np.array([-1.0, 0.0, 1.0], np.float32)]))
        if vals.size == 16:
            return vals.astype(np.float32)


def activations_bf16(M: int, K: int, s: int) -> np.ndarray:
    """[M, K] bf16 bit patterns of N(0, 1) draws."""
    return bf16_from_f32(rng(s).standard_normal((M, K), dtype=np.float32))


def weights_f32(N: int, K: int, s: int, std: float = 0.02) -> np.ndarray:
    g = rng(s)
    return (g.standard_normal((N, K), dtype=np.float32) * np.float32(std)).astype(np.float32)


def quantize_blockwise(W: np.ndarray, codebook: np.ndarray, bs: int, rows_per_chunk: int = 1024):
    """Blockwise absmax quantization to the nearest codebook entry.

    Returns (codes uint8 [N, K], absmax float32 [N, K // bs]).
    """
    W = np.ascontiguousarray(W, dtype=np.float32)
    N, K = W.shape
    if K % bs:
        raise ValueError("K must be a multiple of the blocksize")
    cb = np.asarray(codebook, dtype=np.float32)
    if not np.all(np.diff(cb) > 0):
        raise ValueError("codebook must be sorted and distinct")
    cb64 = cb.astype(np.float64)
    mids = (cb64[:-1] + cb64[1:]) * 0.5
    zero_code = int(np.nonzero(cb == 0.0)[0][0]) if np.any(cb == 0.0) else int(np.argmin(np.abs(cb64)))
    nb = K // bs
    codes = np.empty((N, K), dtype=np.uint8)
    absmax = np.empty((N, nb), dtype=np.float32)

    def work(r0):
        r1 = min(N, r0 + rows_per_chunk)
        blk = W[r0:r1].reshape(r1 - r0, nb, bs)
        am = np.abs(blk).max(axis=2)
        absmax[r0:r1] = am
        am64 = am.astype(np.float64)
        safe = np.where(am64 > 0, am64, 1.0)
        x = blk.astype(np.float64) / safe[:, :, None]
        c = np.searchsorted(mids, x, side="left").astype(np.uint8)
        c[am64 == 0] = zero_code
        codes[r0:r1] = c.reshape(r1 - r0, K)

    # Row chunks are independent and numpy releases the GIL inside them.
    starts = range(0, N, rows_per_chunk)
    if N > rows_per_chunk:
        with ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as pool:
            list(pool.map(work, starts))
    else:
        for r0 in starts:
            work(r0)
    return codes, absmax


def pack_nibbles(codes: np.ndarray) -> np.ndarray:
    """[N, K] codes (0..15) -> [N, K/2] bytes, even k in the low nibble."""
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    if codes.shape[-1] % 2:
        raise ValueError("K must be even")
    if codes.size and codes.max() > 15:
        raise ValueError("codes must be 4-bit")
    lo = codes[..., 0::2]
    hi = codes[..., 1::2]
    return (lo | (hi << 4)).astype(np.uint8)


def bf16_weights(N: int, K: int, s: int, std: float = 0.02) -> np.ndarray:
    return bf16_from_f32(weights_f32(N, K, s, std))


def bias_bf16(N: int, s: int) -> np.ndarray:
    return bf16_from_f32(rng(s).standard_normal(N, dtype=np.float32))


def q4_problem(M: int, N: int, K: int, bs: int = 64, config: int = 0, shape: int = 0,
               codebook: np.ndarray | None = None) -> dict:
    """One seeded 4-bit problem: A, packed W, absmax, codebook (numpy arrays)."""
    cb = nf4_style_codebook() if codebook is None else np.asarray(codebook, np.float32)
    W = weights_f32(N, K, seed(config, shape, 2))
    codes, absmax = quantize_blockwise(W, cb, bs)
    del W
    return {
        "A": activations_bf16(M, K, seed(config, shape, 10 * M + 1)),
        "Wpacked": pack_nibbles(codes),
        "absmax": absmax,
        "codebook": cb,
        "M": M, "N": N, "K": K, "bs": bs,
    }


def bf16_problem(M: int, N: int, K: int, with_bias: bool, config: int = 0, shape: int = 0) -> dict:
    return {
        "A": activations_bf16(M, K, seed(config, shape, 10 * M + 1)),
        "W": bf16_weights(N, K, seed(config, shape, 2)),
        "bias": bias_bf16(N, seed(config, shape, 3)) if with_bias else None,
        "M": M, "N": N, "K": K,
    }


def _cast(x: np.ndarray, dtype: str) -> np.ndarray:
    """fp32 draws as bf16 / fp16 bit patterns (uint16) or fp32 values."""
    if dtype == "fp32":
        return np.ascontiguousarray(x, dtype=np.float32)
    if dtype == "fp16":
        return np.ascontiguousarray(x.astype(np.float16).view(np.uint16))
    if dtype == "bf16":
        return bf16_from_f32(x)
    raise ValueError("dtype must be bf16, fp16 or fp32")


def activations(M: int, K: int, s: int, dtype: str = "bf16") -> np.ndarray:
    """[M, K] N(0, 1) draws in dtype ("bf16" and "fp16" as uint16 bit patterns)."""
    return _cast(rng(s).standard_normal((M, K), dtype=np.float32), dtype)


def bias(N: int, s: int, dtype: str = "bf16") -> np.ndarray:
    """[N] N(0, 1) draws in dtype."""
    return _cast(rng(s).standard_normal(N, dtype=np.float32), dtype)
