"""GPU parity of the blockwise 4-bit quantizer (q4_quantize) against the CPU
oracle: absmax and every code bit for bit.

The quantizer's rule (this library's reading; the pages describe blockwise
absmax quantization to a 16-entry NF4/FP4 table, blocksize 64 by default, in
the maintainer's comment on the bitsandbytes pull request "[ROCm] Optimize
kgemm_4bit_inference_naive ..."): absmax = max |w| over the block; code = the
entry nearest to the exact ratio w / absmax, ties to the lower entry; a block
of zeros takes the entry nearest 0.
"""
import numpy as np
import pytest

import bit_dequant_skinny_amd as q4
import oracle
import synth
from gpu_util import to_dev, to_dev_dtype, torch

pytestmark = pytest.mark.gpu

CODEBOOKS = {"nf4style": q4.q4_codebook_preset("nf4_style"), "int4": q4.q4_codebook_preset("int4"),
             "random": synth.random_codebook(81)}


def _weights(N, K, dt, s):
    # weights of std 0.02 in the requested element type
    w = synth.weights_f32(N, K, s)
    if dt == "fp32":
        return w
    if dt == "fp16":
        return w.astype(np.float16).view(np.uint16)
    return synth.bf16_from_f32(w)


def _quantize_gpu(W_h, dt, cb, bs):
    t = torch()
    Wp, am = q4.q4_quantize(to_dev_dtype(W_h, dt), cb, bs)
    t.cuda.synchronize()
    return Wp.cpu().numpy(), am.cpu().numpy()


def _check(W_h, dt, cb, bs):
    N, K = W_h.shape
    Wp, am = _quantize_gpu(W_h, dt, cb, bs)
    codes, am_ref = oracle.quantize(W_h, dt, cb, N, K, bs)
    assert np.array_equal(am.view(np.uint32), am_ref.view(np.uint32))
    got = oracle.unpack(Wp, N, K)
    if not np.array_equal(got, codes):
        bad = np.argwhere(got != codes)[:5]
        raise AssertionError("codes differ at %s: got %s want %s" % (
            bad.tolist(), got[tuple(bad.T)].tolist(), codes[tuple(bad.T)].tolist()))


@pytest.mark.parametrize("dt", ["bf16", "fp16", "fp32"])
@pytest.mark.parametrize("bs", [32, 64, 128, 256])
@pytest.mark.parametrize("cbname", sorted(CODEBOOKS))
def test_quantize_bit_exact(dt, bs, cbname):
    N, K = 37, 1536
    _check(_weights(N, K, dt, 400 + bs), dt, CODEBOOKS[cbname], bs)


def test_quantize_ragged_word_count():
    # N*K/8 words not a multiple of the 64-word wave step
    _check(_weights(3, 96, "fp32", 5), "fp32", CODEBOOKS["nf4style"], 32)
    _check(_weights(1, 64, "bf16", 6), "bf16", CODEBOOKS["random"], 64)


def test_quantize_special_values():
    """Zero blocks, negative zeros, subnormal and huge weights, exact midpoint ties."""
    cb = CODEBOOKS["int4"]
    K, bs = 512, 64
    rows = []
    rows.append(np.zeros(K, np.float32))                        # all zero
    r = np.zeros(K, np.float32); r[::2] = -0.0; r[5] = -0.0     # negative zeros
    rows.append(r)
    rows.append(np.full(K, 1e-45, np.float32) * (np.arange(K) % 7 - 3))   # subnormals
    rows.append(np.linspace(-3e38, 3e38, K).astype(np.float32))          # huge
    mids = [((i - 8) / 8 + (i - 7) / 8) / 2 for i in range(15)]
    r = np.zeros(K, np.float32)
    r[0] = 1.0                                                  # block absmax 1: ratio = weight
    for i, m in enumerate(mids):
        r[1 + 3 * i] = m
        r[2 + 3 * i] = np.nextafter(np.float32(m), np.float32(2))
        r[3 + 3 * i] = np.nextafter(np.float32(m), np.float32(-2))
    r[64:128] = -r[0:64]                                        # and the mirror block
    rows.append(r)
    W = np.stack(rows).astype(np.float32)
    _check(W, "fp32", cb, bs)
    _check(W, "fp32", CODEBOOKS["nf4style"], bs)


def test_quantize_dequant_round_trip():
    t = torch()
    N, K, bs = 64, 2048, 64
    cb = CODEBOOKS["random"]
    g = synth.rng(82)
    codes = g.integers(0, 16, size=(N, K), dtype=np.uint8)
    codes[:, ::bs] = int(np.nonzero(cb == 1.0)[0][0])   # every block reaches its scale
    am = g.uniform(0.01, 0.1, size=(N, K // bs)).astype(np.float32)
    Wp = synth.pack_nibbles(codes)
    w = q4.q4_dequant(to_dev(Wp, "u8"), to_dev(am, "f32"), to_dev(cb, "f32"), bs,
                      out_dtype=t.float32)
    Wp2, am2 = q4.q4_quantize(w, cb, bs)
    t.cuda.synchronize()
    assert np.array_equal(am2.cpu().numpy(), am)
    assert np.array_equal(Wp2.cpu().numpy(), Wp)


def test_quantize_full_size_rows():
    """The 28672 x 8192 FFN shape: sampled rows checked against the oracle."""
    t = torch()
    N, K, bs = 28672, 8192, 64
    cb = CODEBOOKS["nf4style"]
    W = synth.weights_f32(N, K, 83)
    Wp, am = q4.q4_quantize(to_dev(W, "f32"), cb, bs)
    t.cuda.synchronize()
    rows = np.unique(np.concatenate([synth.rng(84).choice(N, 48, replace=False), [0, N - 1]]))
    codes, am_ref = oracle.quantize(W[rows], "fp32", cb, rows.size, K, bs)
    assert np.array_equal(am.cpu().numpy()[rows], am_ref)
    assert np.array_equal(oracle.unpack(Wp.cpu().numpy()[rows], rows.size, K), codes)
