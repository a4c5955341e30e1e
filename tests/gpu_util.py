"""Helpers for the GPU tests: moving seeded numpy inputs to the device, the
elementwise acceptance rule, and cached full-size problems."""
from __future__ import annotations

import functools

import numpy as np

import synth

# |C_gpu - C_ref| <= 2^-7 |C_ref| + 1e-3 * sum_k |a_k w_k|: 2^-7 is twice the bf16
# output rounding, 1e-3 * S covers fp32 accumulation (chains up to ~4096 terms)
# and, on the split path, the bf16 rounding of the weights on random data.
REL = 2.0 ** -7
ABS_S = 1e-3


def torch():
    import torch as t
    return t


def dev():
    t = torch()
    assert t.cuda.is_available(), "GPU tests need an MI355X; none is visible"
    return t.device("cuda:0")


def to_dev(arr: np.ndarray, kind: str):
    t = torch()
    if kind == "bf16":
        x = t.from_numpy(np.ascontiguousarray(arr, np.uint16).view(np.int16)).view(t.bfloat16)
    elif kind == "u8":
        x = t.from_numpy(np.ascontiguousarray(arr, np.uint8))
    elif kind == "f32":
        x = t.from_numpy(np.ascontiguousarray(arr, np.float32))
    else:
        raise ValueError(kind)
    return x.to(dev())


def q4_to_dev(p: dict):
    return (to_dev(p["A"], "bf16"), to_dev(p["Wpacked"], "u8"), to_dev(p["absmax"], "f32"),
            to_dev(p["codebook"], "f32"))


def bf16_host(x) -> np.ndarray:
    """bf16 device tensor -> uint16 bit patterns on the host."""
    t = torch()
    return x.contiguous().view(t.int16).cpu().numpy().view(np.uint16)


def as_f64(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


# Twice the unit roundoff of each output type (2^-7 for bf16 as above); an
# fp16 output also carries an absolute half-quantum below 2^-14.
REL_OUT = {"bf16": 2.0 ** -7, "fp16": 2.0 ** -10, "fp32": 2.0 ** -23}
ABS_OUT = {"bf16": 0.0, "fp16": 2.0 ** -25, "fp32": 0.0}


def host_f64(x) -> np.ndarray:
    """Device tensor of bf16 / fp16 / fp32 -> fp64 values on the host."""
    t = torch()
    if x.dtype == t.bfloat16:
        return as_f64(bf16_host(x))
    return x.float().cpu().numpy().astype(np.float64)


def to_dev_dtype(arr: np.ndarray, dtype: str):
    """Seeded input in dtype ("bf16"/"fp16" bit patterns or fp32 values) -> device."""
    t = torch()
    if dtype == "fp32":
        return to_dev(arr, "f32")
    x = t.from_numpy(np.ascontiguousarray(arr, np.uint16).view(np.int16))
    return x.view(t.bfloat16 if dtype == "bf16" else t.float16).to(dev())


def assert_within_tolerance(C_gpu_bits, C_ref, S, what="", out="bf16", values=None):
    """Elementwise |C_gpu - C_ref| <= 2 u_out |C_ref| + 1e-3 S (+ the fp16
    subnormal half-quantum).  C_gpu is bf16 bit patterns, or fp64 values."""
    got = as_f64(C_gpu_bits) if values is None else values
    assert got.shape == C_ref.shape, (got.shape, C_ref.shape)
    bound = REL_OUT[out] * np.abs(C_ref) + ABS_S * S + ABS_OUT[out]
    err = np.abs(got - C_ref)
    bad = ~(err <= bound)
    if bad.any():
        idx = np.argwhere(bad)[:5]
        ratio = float(np.max(np.where(bound > 0, err / np.maximum(bound, 1e-300), np.inf)))
        raise AssertionError("%s: %d of %d outside tolerance (worst err/bound %.3g); first %s: "
                             "got %s ref %s S %s" % (
                                 what, int(bad.sum()), bad.size, ratio, idx.tolist(),
                                 got[tuple(idx.T)].tolist(), C_ref[tuple(idx.T)].tolist(),
                                 S[tuple(idx.T)].tolist()))
    return float(np.max(err / np.maximum(bound, 1e-300))) if err.size else 0.0


def sample_cols(N: int, count: int, seed: int) -> np.ndarray:
    """Sorted sample of output columns that always includes both ends and the
    last 16-wide tile."""
    g = synth.rng(seed)
    pick = g.choice(N, size=min(count, N), replace=False)
    ends = np.array([0, 1, N - 1] + list(range(max(0, N - 17), N)), dtype=np.int64)
    return np.unique(np.concatenate([pick.astype(np.int64), ends]))


@functools.lru_cache(maxsize=4)
def q4_weights(N: int, K: int, bs: int, config: int, shape: int):
    """Seeded packed weights for a full-size 4-bit workload (cached)."""
    p = synth.q4_problem(1, N, K, bs, config=config, shape=shape)
    return p["Wpacked"], p["absmax"], p["codebook"]


@functools.lru_cache(maxsize=2)
def bf16_weights(N: int, K: int, config: int, shape: int):
    return (synth.bf16_weights(N, K, synth.seed(config, shape, 2)),
            synth.bias_bf16(N, synth.seed(config, shape, 3)))


def _rne_bf16(x) -> np.ndarray:
    u = np.asarray(x, np.float32).view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint32)


def _widen_bf16(b) -> np.ndarray:
    return (np.asarray(b).astype(np.uint32) << 16).view(np.float32)


def hilo_codebook(cb) -> np.ndarray:
    """The codebook as the matrix-core kernels hold it: bf16 hi = RNE(cb) plus
    bf16 lo = RNE(cb - hi), summed in fp32 (hi + lo is exact in fp32).  It
    equals cb exactly when cb has at most 16 significant bits, and is within
    2^-16 relative otherwise."""
    cb = np.asarray(cb, np.float32)
    hi = _widen_bf16(_rne_bf16(cb))
    lo = _widen_bf16(_rne_bf16((cb - hi).astype(np.float32)))
    return (hi + lo).astype(np.float32)


def hilo_products(cb):
    """The bf16 bits a one-hot activation row yields through the matrix-core
    kernels: fl32(absmax * (hi + lo)) rounded once to bf16."""
    v = hilo_codebook(cb)
    return lambda code, am: _rne_bf16(v[code] * np.asarray(am, np.float32)).astype(np.uint16)


def codebook_16bit(seed: int) -> np.ndarray:
    """A sorted random codebook in [-1, 1] holding -1, 0 and 1 whose entries
    have at most 16 significant bits (the low 8 bits of each fp32 significand
    cleared), so the matrix-core kernels' hi + lo pair holds it exactly."""
    while True:
        cb = synth.random_codebook(seed)
        cb16 = (cb.view(np.uint32) & np.uint32(0xFFFFFF00)).view(np.float32)
        if len(np.unique(cb16)) == 16:
            assert np.array_equal(hilo_codebook(cb16), cb16)
            return cb16
        seed += 1000
