"""The seeded input generator: codebooks, quantizer, packing, determinism."""
import numpy as np

import synth
from conftest import golden_lines


def test_codebooks_meet_the_workload_constraints():
    for cb in (synth.nf4_style_codebook(), synth.random_codebook(1), synth.random_codebook(2)):
        assert cb.dtype == np.float32 and cb.shape == (16,)
        assert np.all(np.diff(cb) > 0)
        assert cb[0] == -1.0 and cb[-1] == 1.0 and np.any(cb == 0.0)
        assert np.all(np.abs(cb) <= 1.0)


def test_pack_matches_nibble_golden():
    for line in golden_lines("nibble_order.txt"):
        b, lo, hi = line.split()
        assert synth.pack_nibbles(np.array([[int(lo), int(hi)]]))[0, 0] == int(b, 16)


def test_quantizer_is_nearest_entry_ties_low():
    g = synth.rng(5)
    cb = synth.random_codebook(6)
    W = g.standard_normal((64, 256)).astype(np.float32)
    codes, absmax = synth.quantize_blockwise(W, cb, 64)
    x = W.reshape(64, 4, 64).astype(np.float64) / absmax.astype(np.float64)[:, :, None]
    dist = np.abs(x[..., None] - cb.astype(np.float64))
    brute = np.argmin(dist, axis=-1)  # argmin returns the lowest index on a tie
    assert np.array_equal(codes.reshape(64, 4, 64), brute)
    assert np.array_equal(absmax, np.abs(W).reshape(64, 4, 64).max(axis=2))


def test_quantizer_reproduces_codes_of_dequantized_blocks():
    g = synth.rng(7)
    cb = synth.nf4_style_codebook()
    N, K, bs = 8, 256, 64
    codes = g.integers(0, 16, size=(N, K), dtype=np.uint8)
    codes[:, ::bs] = 15  # every block holds the +1 entry, so its absmax is the scale
    am = g.uniform(0.01, 0.1, size=(N, K // bs)).astype(np.float32)
    W = cb[codes] * np.repeat(am, bs, axis=1)
    c2, am2 = synth.quantize_blockwise(W, cb, bs)
    assert np.array_equal(am2, am)
    assert np.array_equal(c2, codes)


def test_zero_block_stores_zero_scale_and_zero_code():
    cb = synth.nf4_style_codebook()
    W = np.zeros((2, 128), np.float32)
    W[1, 64:] = 0.5
    codes, absmax = synth.quantize_blockwise(W, cb, 64)
    zero = int(np.nonzero(cb == 0)[0][0])
    assert absmax[0, 0] == 0 and absmax[0, 1] == 0 and absmax[1, 0] == 0
    assert np.all(codes[0] == zero) and np.all(codes[1, :64] == zero)
    assert np.all(codes[1, 64:] == 15) and absmax[1, 1] == np.float32(0.5)


def test_generators_are_seeded():
    a = synth.q4_problem(2, 16, 128, 64, config=1, shape=2)
    b = synth.q4_problem(2, 16, 128, 64, config=1, shape=2)
    c = synth.q4_problem(2, 16, 128, 64, config=1, shape=3)
    for key in ("A", "Wpacked", "absmax", "codebook"):
        assert np.array_equal(a[key], b[key])
    assert not np.array_equal(a["Wpacked"], c["Wpacked"])
    # the weights do not depend on M
    d = synth.q4_problem(4, 16, 128, 64, config=1, shape=2)
    assert np.array_equal(a["Wpacked"], d["Wpacked"]) and not np.array_equal(a["A"], d["A"][:2])


def test_distributions():
    A = synth.activations_bf16(4, 8192, 3)
    a = (A.astype(np.uint32) << 16).view(np.float32)
    assert abs(a.mean()) < 0.03 and abs(a.std() - 1.0) < 0.03
    W = synth.weights_f32(64, 1024, 4)
    assert abs(W.std() - 0.02) < 0.001
