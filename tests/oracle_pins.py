"""Pins that tie the CPU oracle to something other than itself.

Each ``pin_*`` function takes a loaded oracle (``oracle.Oracle``) and raises
AssertionError when the oracle disagrees with:
  * hand-worked fixtures under tests/golden (nibble order, a dequantize + GEMM
    example, bf16 rounding cases),
  * the definition of correct rounding checked with exact rationals,
  * torch's bf16 cast and numpy's fp16 cast and widening (library routines)
    on random and structured bit patterns,
  * exact rational brute force on tiny GEMMs (error within the fp64
    recursive-summation bound),
  * invariants: one-hot rows return a dequantized weight exactly, scaling A by
    a power of two scales C exactly, additivity over disjoint supports,
    dequantize-then-GEMM equals the fused oracle bit for bit, the split-path
    diagnostic equals the bf16 GEMM on bf16-dequantized weights.

The same functions run against deliberately broken copies of oracle.c in
test_oracle_mutants.py, which checks that every planted mistake trips a pin.
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np

import synth
from conftest import golden_lines

ONE_BF16 = 0x3F80


def _f32(x) -> np.float32:
    return np.float32(x)


def _frac(x) -> Fraction:
    return Fraction(float(x))


def _bf16_val(bits) -> float:
    return float(np.array([int(bits) << 16], dtype=np.uint32).view(np.float32)[0])


def _golden_worked():
    g = {"packed": {}, "absmax": {}, "w": {}}
    for line in golden_lines("dequant_worked.txt"):
        tok = line.split()
        key = tok[0]
        if key in ("N", "K", "bs"):
            g[key] = int(tok[1])
        elif key == "codebook":
            g[key] = np.array([float(t) for t in tok[1:]], dtype=np.float32)
        elif key == "packed":
            g["packed"][int(tok[1])] = [int(t, 16) for t in tok[2:]]
        elif key in ("absmax", "w"):
            g[key][int(tok[1])] = [float(t) for t in tok[2:]]
        elif key in ("a", "C", "S"):
            g[key] = [float(t) for t in tok[1:]]
    N = g["N"]
    g["Wpacked"] = np.array([g["packed"][n] for n in range(N)], dtype=np.uint8)
    g["absmax_arr"] = np.array([g["absmax"][n] for n in range(N)], dtype=np.float32)
    g["w_arr"] = np.array([g["w"][n] for n in range(N)], dtype=np.float32)
    return g


# --------------------------------------------------------------------------- O1
def pin_nibble_order_golden(orc):
    for line in golden_lines("nibble_order.txt"):
        b, lo, hi = line.split()
        byte = np.array([[int(b, 16)]], dtype=np.uint8)
        assert orc.code(byte, 2, 0, 0) == int(lo), line
        assert orc.code(byte, 2, 0, 1) == int(hi), line
        assert list(orc.unpack(byte, 1, 2)[0]) == [int(lo), int(hi)], line


def pin_pack_unpack_roundtrip(orc):
    g = synth.rng(11)
    for N, K in [(1, 2), (3, 64), (5, 130), (7, 256)]:
        codes = g.integers(0, 16, size=(N, K), dtype=np.uint8)
        assert np.array_equal(orc.unpack(synth.pack_nibbles(codes), N, K), codes)


# --------------------------------------------------------------------------- O2
def pin_block_index_flat(orc):
    # Blocks run along K inside a row; with K % bs == 0 this equals blocking
    # the flattened row-major matrix.
    for N, K, bs in [(3, 64, 64), (4, 128, 32), (2, 512, 128), (3, 256, 256)]:
        for n in range(N):
            for k in range(0, K, 7):
                assert orc.block_index(K, bs, n, k) == (n * K + k) // bs


# ------------------------------------------------------------------------ O3/O4
def pin_dequant_worked_golden(orc):
    g = _golden_worked()
    N, K, bs = g["N"], g["K"], g["bs"]
    w = orc.dequant_f32(g["Wpacked"], g["absmax_arr"], g["codebook"], N, K, bs)
    assert np.array_equal(w, g["w_arr"]), (w, g["w_arr"])
    w16 = orc.dequant_bf16(g["Wpacked"], g["absmax_arr"], g["codebook"], N, K, bs)
    # every worked value is bf16-exact, so bf16 holds the top half of its fp32 pattern
    assert np.array_equal(w16, (g["w_arr"].view(np.uint32) >> 16).astype(np.uint16))


def pin_gemm_worked_golden(orc):
    g = _golden_worked()
    N, K, bs = g["N"], g["K"], g["bs"]
    a = synth.bf16_from_f32(np.array([g["a"]], dtype=np.float32))
    C, S = orc.q4_gemm(a, g["Wpacked"], g["absmax_arr"], g["codebook"], 1, N, K, bs)
    assert list(C[0]) == g["C"], C
    assert list(S[0]) == g["S"], S


def _check_correctly_rounded(r: np.float32, exact: Fraction):
    """r is the binary32 value nearest to exact, ties to an even significand."""
    assert np.isfinite(r)
    d = abs(_frac(r) - exact)
    for nb in (np.nextafter(r, np.float32(-np.inf)), np.nextafter(r, np.float32(np.inf))):
        if not np.isfinite(nb):
            continue
        dn = abs(_frac(nb) - exact)
        assert d <= dn, (r, nb, exact)
        if d == dn:  # a tie: the chosen neighbour has an even significand
            assert int(np.array([r], np.float32).view(np.uint32)[0]) % 2 == 0


def pin_w32_correct_rounding(orc):
    g = synth.rng(21)
    for cb in (synth.nf4_style_codebook(), synth.random_codebook(3)):
        scales = [1.0, 0.5, 3.0, 0.0625, 1e-3, 7.3e-2, 1.17549435e-38, 1e-39, 3e-44,
                  2.0 ** 100, 1.5e-38]
        scales += list(g.uniform(1e-3, 0.2, size=20)) + list(g.uniform(1e-40, 1e-37, size=8))
        am = np.array(scales, dtype=np.float32)
        nb = am.size
        K = 64 * nb
        # row 0 walks through all 16 codes in every block
        codes = np.tile(np.arange(16, dtype=np.uint8), K // 16)[None, :]
        Wp = synth.pack_nibbles(codes)
        w = orc.dequant_f32(Wp, am[None, :], cb, 1, K, 64)[0]
        for k in range(K):
            exact = _frac(cb[codes[0, k]]) * _frac(am[k // 64])
            _check_correctly_rounded(w[k], exact)
        # the table's exact entries reproduce the scale exactly
        for b in range(nb):
            base = 64 * b
            assert w[base + int(np.nonzero(cb == 1.0)[0][0])] == am[b]
            assert w[base + int(np.nonzero(cb == -1.0)[0][0])] == -am[b]
            assert w[base + int(np.nonzero(cb == 0.0)[0][0])] == 0.0


def pin_bf16_rounding_golden(orc):
    for line in golden_lines("bf16_rounding.txt"):
        src, dst = line.split()[:2]
        x = np.array([int(src, 16)], dtype=np.uint32).view(np.float32)
        got = int(orc.f32_to_bf16(x)[0])
        assert got == int(dst, 16), (line, hex(got))


def pin_bf16_rounding_vs_torch(orc):
    import torch
    g = synth.rng(31)
    bits = g.integers(0, 2 ** 32, size=1 << 20, dtype=np.uint64).astype(np.uint32)
    # add every upper half with the tie and near-tie lower halves
    up = np.arange(1 << 16, dtype=np.uint32) << 16
    bits = np.concatenate([bits, up | 0x8000, up | 0x7FFF, up | 0x8001, up])
    x = bits.view(np.float32)
    x = x[~np.isnan(x)]
    got = orc.f32_to_bf16(x)
    ref = torch.from_numpy(x.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got, ref)


# --------------------------------------------------------------------------- O5
def _exact_q4(a_bits, codes, absmax, cb, bs):
    """Exact rationals: sum a * fl32(cb * absmax) and sum |a * w|."""
    M, K = a_bits.shape
    N = codes.shape[0]
    C = [[Fraction(0)] * N for _ in range(M)]
    S = [[Fraction(0)] * N for _ in range(M)]
    wf = [[Fraction(float(np.float32(float(_frac(cb[codes[n, k]]) * _frac(absmax[n, k // bs])))))
           for k in range(K)] for n in range(N)]
    for m in range(M):
        af = [_frac(_bf16_val(a_bits[m, k])) for k in range(K)]
        for n in range(N):
            s = sum((af[k] * wf[n][k] for k in range(K)), Fraction(0))
            t = sum((abs(af[k] * wf[n][k]) for k in range(K)), Fraction(0))
            C[m][n], S[m][n] = s, t
    return C, S


def _fp64_sum_bound(K: int) -> float:
    u = 2.0 ** -53
    return (K - 1) * u / (1 - (K - 1) * u)


def pin_q4_gemm_bruteforce(orc):
    g = synth.rng(41)
    for (M, N, K, bs), cb in [((1, 3, 64, 64), synth.nf4_style_codebook()),
                              ((3, 4, 128, 64), synth.random_codebook(7)),
                              ((2, 2, 128, 32), synth.random_codebook(8)),
                              ((2, 3, 256, 128), synth.nf4_style_codebook())]:
        codes = g.integers(0, 16, size=(N, K), dtype=np.uint8)
        absmax = g.uniform(0.01, 0.1, size=(N, K // bs)).astype(np.float32)
        A = synth.activations_bf16(M, K, int(g.integers(1 << 30)))
        Wp = synth.pack_nibbles(codes)
        C, S = orc.q4_gemm(A, Wp, absmax, cb, M, N, K, bs)
        Ce, Se = _exact_q4(A, codes, absmax, cb, bs)
        for m in range(M):
            for n in range(N):
                err = abs(_frac(C[m, n]) - Ce[m][n])
                assert err <= Fraction(_fp64_sum_bound(K)) * Se[m][n], (m, n, float(err))
                assert abs(_frac(S[m, n]) - Se[m][n]) <= Fraction(_fp64_sum_bound(K)) * Se[m][n]


def pin_q4_one_hot_rows(orc):
    g = synth.rng(51)
    N, K, bs = 5, 256, 64
    cb = synth.random_codebook(9)
    codes = g.integers(0, 16, size=(N, K), dtype=np.uint8)
    absmax = g.uniform(0.01, 0.1, size=(N, K // bs)).astype(np.float32)
    Wp = synth.pack_nibbles(codes)
    js = [0, 1, 63, 64, 65, 128, 201, 255]
    A = np.zeros((len(js), K), dtype=np.uint16)
    for m, j in enumerate(js):
        A[m, j] = ONE_BF16
    C, S = orc.q4_gemm(A, Wp, absmax, cb, len(js), N, K, bs)
    w = orc.dequant_f32(Wp, absmax, cb, N, K, bs)
    for m, j in enumerate(js):
        for n in range(N):
            exact = np.float32(float(_frac(cb[codes[n, j]]) * _frac(absmax[n, j // bs])))
            assert C[m, n] == float(exact) == float(w[n, j]), (m, n)
            assert S[m, n] == abs(float(exact))


def pin_q4_homogeneity(orc):
    g = synth.rng(61)
    M, N, K, bs = 2, 4, 192, 64
    p = synth.q4_problem(M, N, K, bs, config=90)
    C1, S1 = orc.q4_gemm(p["A"], p["Wpacked"], p["absmax"], p["codebook"], M, N, K, bs)
    for e in (1, 3, -2):
        A2 = synth.bf16_from_f32(np.vectorize(_bf16_val)(p["A"]).astype(np.float32) * np.float32(2.0 ** e))
        C2, S2 = orc.q4_gemm(A2, p["Wpacked"], p["absmax"], p["codebook"], M, N, K, bs)
        assert np.array_equal(C2, C1 * 2.0 ** e)
        assert np.array_equal(S2, S1 * 2.0 ** e)
    del g


def pin_q4_additivity(orc):
    M, N, K, bs = 2, 4, 256, 64
    p = synth.q4_problem(M, N, K, bs, config=91, codebook=synth.random_codebook(4))
    A = p["A"]
    A1 = A.copy()
    A1[:, 1::2] = 0
    A2 = A.copy()
    A2[:, 0::2] = 0
    args = (p["Wpacked"], p["absmax"], p["codebook"], M, N, K, bs)
    C, S = orc.q4_gemm(A, *args)
    C1, _ = orc.q4_gemm(A1, *args)
    C2, _ = orc.q4_gemm(A2, *args)
    assert np.all(np.abs(C - (C1 + C2)) <= 3 * _fp64_sum_bound(K) * S)
    # and the halves really are different from the whole
    assert not np.array_equal(C1, C)


def pin_fused_equals_dequant_then_gemm(orc):
    for M, N, K, bs in [(1, 6, 128, 64), (4, 5, 320, 64), (3, 3, 256, 32)]:
        p = synth.q4_problem(M, N, K, bs, config=92)
        C, _ = orc.q4_gemm(p["A"], p["Wpacked"], p["absmax"], p["codebook"], M, N, K, bs)
        W = orc.dequant_f32(p["Wpacked"], p["absmax"], p["codebook"], N, K, bs)
        C8 = orc.gemm_f32w(p["A"], W, M, N, K)
        assert np.array_equal(C, C8)


def pin_column_subset(orc):
    M, N, K, bs = 3, 9, 128, 64
    p = synth.q4_problem(M, N, K, bs, config=93)
    args = (p["A"], p["Wpacked"], p["absmax"], p["codebook"], M, N, K, bs)
    C, S = orc.q4_gemm(*args)
    cols = [8, 0, 3, 3]
    Cs, Ss = orc.q4_gemm(*args, cols=cols)
    assert np.array_equal(Cs, C[:, cols]) and np.array_equal(Ss, S[:, cols])


# ------------------------------------------------------------------------ O6/O7
def _exact_bf16(A, W, bias):
    M, K = A.shape
    N = W.shape[0]
    C = [[Fraction(0)] * N for _ in range(M)]
    S = [[Fraction(0)] * N for _ in range(M)]
    for m in range(M):
        for n in range(N):
            terms = [_frac(_bf16_val(A[m, k])) * _frac(_bf16_val(W[n, k])) for k in range(K)]
            if bias is not None:
                terms.append(_frac(_bf16_val(bias[n])))
            C[m][n] = sum(terms, Fraction(0))
            S[m][n] = sum((abs(t) for t in terms), Fraction(0))
    return C, S


def pin_bf16_gemm_bruteforce(orc):
    for M, N, K, with_bias in [(1, 3, 64, True), (5, 4, 40, True), (3, 2, 96, False)]:
        p = synth.bf16_problem(M, N, K, with_bias, config=94)
        C, S = orc.bf16_gemm(p["A"], p["W"], p["bias"], M, N, K)
        Ce, Se = _exact_bf16(p["A"], p["W"], p["bias"])
        bound = Fraction(_fp64_sum_bound(K + 1))
        for m in range(M):
            for n in range(N):
                assert abs(_frac(C[m, n]) - Ce[m][n]) <= bound * Se[m][n], (m, n)
                assert abs(_frac(S[m, n]) - Se[m][n]) <= bound * Se[m][n]


def pin_bf16_gemm_structure(orc):
    M, N, K = 3, 6, 64
    p = synth.bf16_problem(M, N, K, True, config=95)
    # one-hot rows return W[:, j] plus the bias, exactly (two terms, one rounding)
    A = np.zeros((M, K), dtype=np.uint16)
    js = [0, 17, 63]
    for m, j in enumerate(js):
        A[m, j] = ONE_BF16
    C, _ = orc.bf16_gemm(A, p["W"], None, M, N, K)
    for m, j in enumerate(js):
        for n in range(N):
            assert C[m, n] == _bf16_val(p["W"][n, j])
    # A = 0 returns the bias alone
    C0, S0 = orc.bf16_gemm(np.zeros((M, K), np.uint16), p["W"], p["bias"], M, N, K)
    for n in range(N):
        assert np.all(C0[:, n] == _bf16_val(p["bias"][n]))
        assert np.all(S0[:, n] == abs(_bf16_val(p["bias"][n])))


def pin_split_diagnostic(orc):
    M, N, K, bs = 3, 5, 256, 64
    p = synth.q4_problem(M, N, K, bs, config=96)
    C7, S7 = orc.q4_gemm_w16(p["A"], p["Wpacked"], p["absmax"], p["codebook"], M, N, K, bs)
    W16 = orc.dequant_bf16(p["Wpacked"], p["absmax"], p["codebook"], N, K, bs)
    C6, S6 = orc.bf16_gemm(p["A"], W16, None, M, N, K)
    assert np.array_equal(C7, C6) and np.array_equal(S7, S6)


# --------------------------------------------------------------------------- O9
def _f16_val(bits) -> float:
    return float(np.array([int(bits)], dtype=np.uint16).view(np.float16)[0])


def pin_f16_decode_exhaustive(orc):
    bits = np.arange(1 << 16, dtype=np.uint16)
    got = orc.f16_to_double(bits)
    ref = bits.view(np.float16).astype(np.float64)  # numpy's exact widening
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))


def pin_f16_rounding_golden(orc):
    for line in golden_lines("f16_rounding.txt"):
        src, dst = line.split()[:2]
        x = np.array([int(src, 16)], dtype=np.uint32).view(np.float32)
        got = int(orc.f32_to_f16(x)[0])
        assert got == int(dst, 16), (line, hex(got))


def pin_f16_rounding_vs_numpy(orc):
    g = synth.rng(32)
    bits = g.integers(0, 2 ** 32, size=1 << 19, dtype=np.uint64).astype(np.uint32)
    # every fp32 exponent that lands in or near the fp16 range, with the tie,
    # near-tie and carry-out low bits of the 13 dropped bits
    exps = np.arange(95, 145, dtype=np.uint32) << 23
    mants = np.array([0, 0x1000, 0xFFF, 0x1001, 0x3000, 0x7FF000, 0x7FFFFF, 0x7FE000, 0x2000],
                     dtype=np.uint32)
    edge = (exps[:, None] | mants[None, :]).ravel()
    bits = np.concatenate([bits, edge, edge | 0x80000000])
    x = bits.view(np.float32)
    x = x[~np.isnan(x)]
    with np.errstate(over="ignore"):
        ref = x.astype(np.float16).view(np.uint16)
    assert np.array_equal(orc.f32_to_f16(x), ref)


def pin_dequant_f16_is_rounded_product(orc):
    N, K, bs = 4, 128, 64
    p = synth.q4_problem(1, N, K, bs, config=97, codebook=synth.random_codebook(5))
    w = orc.dequant_f32(p["Wpacked"], p["absmax"], p["codebook"], N, K, bs)
    h = orc.dequant_f16(p["Wpacked"], p["absmax"], p["codebook"], N, K, bs)
    assert np.array_equal(h, w.astype(np.float16).view(np.uint16))


# -------------------------------------------------------------------------- O10
def _act_val(x, dtype) -> float:
    if dtype == "fp32":
        return float(x)
    return _f16_val(x) if dtype == "fp16" else _bf16_val(x)


def pin_q4_gemm_ex_bruteforce(orc):
    g = synth.rng(43)
    cases = [(1, 3, 64, 64, "fp16", "fp16"), (2, 2, 128, 64, "fp32", "fp32"),
             (3, 2, 64, 32, "fp16", "bf16"), (2, 3, 128, 128, "fp32", None)]
    for M, N, K, bs, adt, bdt in cases:
        cb = synth.random_codebook(int(g.integers(100)))
        codes = g.integers(0, 16, size=(N, K), dtype=np.uint8)
        absmax = g.uniform(0.01, 0.1, size=(N, K // bs)).astype(np.float32)
        A = synth.activations(M, K, int(g.integers(1 << 30)), adt)
        b = None if bdt is None else synth.bias(N, int(g.integers(1 << 30)), bdt)
        C, S = orc.q4_gemm_ex(A, adt, synth.pack_nibbles(codes), absmax, cb, M, N, K, bs,
                              bias=b, bias_dtype=bdt or "bf16")
        bound = Fraction(_fp64_sum_bound(K + 1))
        for m in range(M):
            for n in range(N):
                terms = []
                for k in range(K):
                    w = _frac(np.float32(float(_frac(cb[codes[n, k]]) * _frac(absmax[n, k // bs]))))
                    terms.append(_frac(_act_val(A[m, k], adt)) * w)
                if b is not None:
                    terms.append(_frac(_act_val(b[n], bdt)))
                ce = sum(terms, Fraction(0))
                se = sum((abs(t) for t in terms), Fraction(0))
                assert abs(_frac(C[m, n]) - ce) <= bound * se, (adt, m, n)
                assert abs(_frac(S[m, n]) - se) <= bound * se


def pin_q4_gemm_ex_reduces_to_bf16(orc):
    M, N, K, bs = 3, 5, 192, 64
    p = synth.q4_problem(M, N, K, bs, config=98)
    args = (p["Wpacked"], p["absmax"], p["codebook"], M, N, K, bs)
    C5, S5 = orc.q4_gemm(p["A"], *args)
    C, S = orc.q4_gemm_ex(p["A"], "bf16", *args)
    assert np.array_equal(C, C5) and np.array_equal(S, S5)
    # the same values held as fp32 give the same sums
    A32 = (p["A"].astype(np.uint32) << 16).view(np.float32)
    C, S = orc.q4_gemm_ex(A32, "fp32", *args)
    assert np.array_equal(C, C5) and np.array_equal(S, S5)


def pin_q4_gemm_ex_bias_alone(orc):
    M, N, K, bs = 2, 6, 128, 64
    p = synth.q4_problem(M, N, K, bs, config=99)
    for dt in ("bf16", "fp16", "fp32"):
        b = synth.bias(N, 7, dt)
        A = np.zeros((M, K), dtype=np.float32 if dt == "fp32" else np.uint16)
        C, S = orc.q4_gemm_ex(A, dt, p["Wpacked"], p["absmax"], p["codebook"], M, N, K, bs,
                              bias=b, bias_dtype=dt)
        for n in range(N):
            assert np.all(C[:, n] == _act_val(b[n], dt)), (dt, n)
            assert np.all(S[:, n] == abs(_act_val(b[n], dt)))


# -------------------------------------------------------------------------- O11
def _int4_codebook():
    # (i - 8) / 8: every midpoint (2i - 15) / 16 is an fp32 number, so exact
    # ties can be written down
    return np.array([(i - 8) / 8.0 for i in range(16)], dtype=np.float32)


def _exact_quantize(W_vals, cb, bs):
    """Exact rationals: block absmax, then the nearest entry to w / absmax with
    ties to the lower index (brute force over all 16 entries)."""
    N, K = W_vals.shape
    codes = np.zeros((N, K), dtype=np.uint8)
    absmax = np.zeros((N, K // bs), dtype=np.float64)
    cbf = [_frac(c) for c in cb]
    for n in range(N):
        for b in range(K // bs):
            blk = [_frac(W_vals[n, k]) for k in range(b * bs, (b + 1) * bs)]
            a = max(abs(v) for v in blk)
            absmax[n, b] = float(a)
            for i, v in enumerate(blk):
                x = v / a if a != 0 else Fraction(0)
                d = [abs(x - c) for c in cbf]
                codes[n, b * bs + i] = d.index(min(d))
    return codes, absmax


def pin_quantize_bruteforce(orc):
    g = synth.rng(71)
    for N, K, bs, dt, cb in [(3, 128, 64, "fp32", synth.random_codebook(3)),
                             (2, 128, 32, "bf16", synth.nf4_style_codebook()),
                             (2, 256, 128, "fp16", synth.random_codebook(4)),
                             (1, 256, 256, "fp32", _int4_codebook())]:
        W = synth.activations(N, K, int(g.integers(1 << 30)), dt)
        vals = np.array([[_act_val(W[n, k], dt) for k in range(K)] for n in range(N)])
        codes, absmax = orc.quantize(W, dt, cb, N, K, bs)
        ce, ae = _exact_quantize(vals, cb, bs)
        assert np.array_equal(absmax.astype(np.float64), ae), dt
        assert np.array_equal(codes, ce), dt


def pin_quantize_exact_ties(orc):
    cb = _int4_codebook()
    K, bs = 64, 64
    mids = [(float(cb[i]) + float(cb[i + 1])) / 2 for i in range(15)]
    w = [1.0]  # the block's absmax is 1, so the ratio is the weight itself
    expect = [15]
    for i, m in enumerate(mids):
        m32 = np.float32(m)
        assert float(m32) == m
        w += [m, float(np.nextafter(m32, np.float32(2))), float(np.nextafter(m32, np.float32(-2)))]
        expect += [i, i + 1, i]
    w += [0.0] * (K - len(w))
    expect += [8] * (K - len(expect))
    W = np.array([w], dtype=np.float32)
    codes, absmax = orc.quantize(W, "fp32", cb, 1, K, bs)
    assert absmax[0, 0] == 1.0
    assert list(codes[0]) == expect


def pin_quantize_roundtrip_and_zero_block(orc):
    g = synth.rng(72)
    cb = synth.random_codebook(6)
    N, K, bs = 4, 256, 64
    codes = g.integers(0, 16, size=(N, K), dtype=np.uint8)
    one = int(np.nonzero(cb == 1.0)[0][0])
    codes[:, ::bs] = one  # every block holds the entry 1, so absmax is the block scale
    am = g.uniform(0.01, 0.1, size=(N, K // bs)).astype(np.float32)
    am[1, 2] = 0.0  # a block of zeros
    W = orc.dequant_f32(synth.pack_nibbles(codes), am, cb, N, K, bs)
    c2, a2 = orc.quantize(W, "fp32", cb, N, K, bs)
    assert np.array_equal(a2, am)
    zero = int(np.nonzero(cb == 0.0)[0][0])
    mask = np.ones_like(codes, dtype=bool)
    mask[1, 2 * bs:3 * bs] = False
    assert np.array_equal(c2[mask], codes[mask])
    assert np.all(c2[1, 2 * bs:3 * bs] == zero)


def pin_quantize_matches_numpy_searchsorted(orc):
    # synth's quantizer: numpy searchsorted on fp64 midpoints of w / absmax in fp64
    W = synth.weights_f32(64, 512, 17)
    for bs, cb in [(64, synth.nf4_style_codebook()), (32, synth.random_codebook(12))]:
        c1, a1 = orc.quantize(W, "fp32", cb, 64, 512, bs)
        c2, a2 = synth.quantize_blockwise(W, cb, bs)
        assert np.array_equal(a1, a2) and np.array_equal(c1, c2)


def pin_tile_layout_golden(orc):
    """O12: byte offsets worked by hand (tests/golden/tile_layout.txt)."""
    for line in golden_lines("tile_layout.txt"):
        n, j, off = (int(v) for v in line.split())
        assert orc.tile_offset(32, 256, n, j) == off, ("tile", n, j)


def pin_bf16_tile_layout(orc):
    """O13: element indices worked by hand (tests/golden/bf16_tile_layout.txt),
    a bijection, 16-row tiles of consecutive units, and pieces of 8
    consecutive k of one row."""
    for line in golden_lines("bf16_tile_layout.txt"):
        n, k, idx = (int(v) for v in line.split())
        assert orc.bf16_tile_index(32, 64, n, k) == idx, ("bf16 tile", n, k)
    N, K = 32, 96
    idx = np.array([[orc.bf16_tile_index(N, K, n, k) for k in range(K)] for n in range(N)])
    assert sorted(idx.ravel().tolist()) == list(range(N * K))
    # 8 consecutive k of a row stay consecutive (one piece) ...
    assert np.all(np.diff(idx.reshape(N, K // 8, 8), axis=2) == 1)
    # ... and the 16 rows x 32 k of (tile t, step s) fill units of 512
    # elements, (t, s) in row order with s fastest
    for t in range(N // 16):
        for s_ in range(K // 32):
            u = idx[16 * t:16 * t + 16, 32 * s_:32 * s_ + 32]
            assert u.min() == (t * (K // 32) + s_) * 512 and u.max() == u.min() + 511
    W = np.arange(N * K, dtype=np.uint16).reshape(N, K)
    T = orc.bf16_repack_tiles(W, N, K).ravel()
    assert np.array_equal(T[idx.ravel()], W.ravel())


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]
