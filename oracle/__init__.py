"""CPU oracle for the blockwise 4-bit skinny GEMM (test infrastructure only).

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The GPU library neither imports nor links
it, and the two share no code.  The arithmetic lives in ``oracle.c`` (plain C,
fp64 accumulation); this module only builds that file with gcc, loads it with
ctypes and marshals numpy arrays.

Function map (steps as numbered in the C file):
  unpack          O1  code(n,k) from the packed bytes (low nibble = even k)
  block_index     O2  which absmax scales element (n,k)
  dequant_f32     O3  codebook[code] * absmax as one fp32 multiply
  dequant_bf16    O4  O3 rounded to bf16, nearest-even
  f32_to_bf16     O4's rounding alone
  q4_gemm         O5  fp64-accumulated A * dequant(W)^T, plus S = sum |a*w|
  bf16_gemm       O6  fp64-accumulated A * W^T (+ bias), plus S
  q4_gemm_w16     O7  O5 on bf16-rounded weights (split-path diagnostic)
  gemm_f32w       O8  plain fp64 GEMM on an already dequantized fp32 W
  f16_to_double   O9  IEEE binary16 widened exactly
  f32_to_f16      O9  fp32 -> binary16, nearest-even
  dequant_f16     O9  O3 rounded to binary16
  q4_gemm_ex      O10 O5 with bf16 / fp16 / fp32 activations and a bias
  quantize        O11 blockwise absmax + nearest-entry codes (inverse of O3)
  tile_offset     O12 where byte j of packed row n sits in the tile layout
  repack_tiles    O12 the row-major packed bytes moved to the tile layout
  bf16_tile_index O13 where element k of bf16 weight row n sits in its tile layout
  bf16_repack_tiles O13 the row-major bf16 weights moved to that layout

Element types are named "bf16", "fp16", "fp32" (uint16 bit patterns for the
two 16-bit types, float32 arrays for fp32).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
CFLAGS = ["-O2", "-ffp-contract=off", "-fno-fast-math", "-fopenmp", "-fPIC", "-shared",
          "-std=c11"]


def compile_c(src: str, out: str) -> str:
    """gcc the given oracle source into a shared library (atomic replace)."""
    tmp = out + ".tmp%d" % os.getpid()
    subprocess.check_call(["gcc", *CFLAGS, src, "-o", tmp, "-lm"])
    os.replace(tmp, out)
    return out


def build(force: bool = False) -> str:
    """Compile oracle.c into liboracle.so (when missing, stale or forced)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(SOURCE):
        compile_c(SOURCE, _LIB)
    return _LIB


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


class Oracle:
    """ctypes view of one compiled oracle library."""

    def __init__(self, lib_path: str):
        lib = ctypes.CDLL(lib_path)
        P, I = ctypes.c_void_p, ctypes.c_int64
        lib.oracle_code.argtypes = [P, I, I, I]
        lib.oracle_code.restype = ctypes.c_int
        lib.oracle_unpack.argtypes = [P, I, I, P]
        lib.oracle_block_index.argtypes = [I, I, I, I]
        lib.oracle_block_index.restype = I
        lib.oracle_w32.argtypes = [P, P, P, I, I, I, I]
        lib.oracle_w32.restype = ctypes.c_float
        lib.oracle_dequant_f32.argtypes = [P, P, P, I, I, I, P]
        lib.oracle_dequant_bf16.argtypes = [P, P, P, I, I, I, P]
        lib.oracle_f32_to_bf16.argtypes = [ctypes.c_float]
        lib.oracle_f32_to_bf16.restype = ctypes.c_uint16
        lib.oracle_f32_to_bf16_array.argtypes = [P, I, P]
        lib.oracle_q4_gemm.argtypes = [P, P, P, P, I, I, I, I, P, I, P, P]
        lib.oracle_q4_gemm_w16.argtypes = [P, P, P, P, I, I, I, I, P, I, P, P]
        lib.oracle_bf16_gemm.argtypes = [P, P, P, I, I, I, P, I, P, P]
        lib.oracle_gemm_f32w.argtypes = [P, P, I, I, I, P]
        lib.oracle_f16_to_double.argtypes = [ctypes.c_uint16]
        lib.oracle_f16_to_double.restype = ctypes.c_double
        lib.oracle_f32_to_f16.argtypes = [ctypes.c_float]
        lib.oracle_f32_to_f16.restype = ctypes.c_uint16
        lib.oracle_f32_to_f16_array.argtypes = [P, I, P]
        lib.oracle_dequant_f16.argtypes = [P, P, P, I, I, I, P]
        lib.oracle_q4_gemm_ex.argtypes = [P, ctypes.c_int, P, P, P, P, ctypes.c_int, I, I, I, I,
                                          P, I, P, P]
        lib.oracle_quantize.argtypes = [P, ctypes.c_int, P, I, I, I, P, P]
        lib.oracle_max_threads.restype = ctypes.c_int
        lib.oracle_set_threads.argtypes = [ctypes.c_int]
        lib.oracle_tile_offset.argtypes = [I, I, I, I]
        lib.oracle_tile_offset.restype = I
        lib.oracle_repack_tiles.argtypes = [P, I, I, P]
        lib.oracle_bf16_tile_index.argtypes = [I, I, I, I]
        lib.oracle_bf16_tile_index.restype = I
        lib.oracle_bf16_repack_tiles.argtypes = [P, I, I, P]
        self.lib = lib
        self.path = lib_path

    def set_threads(self, n: int) -> None:
        """Threads the OpenMP loops use from now on (n >= 1)."""
        self.lib.oracle_set_threads(int(n))

    def max_threads(self) -> int:
        """Threads the OpenMP loops use (OMP_NUM_THREADS)."""
        return int(self.lib.oracle_max_threads())

    def code(self, Wpacked, K, n, k) -> int:
        Wp = _c(Wpacked, np.uint8)
        return int(self.lib.oracle_code(_ptr(Wp), K, n, k))

    def unpack(self, Wpacked, N, K) -> np.ndarray:
        Wp = _c(Wpacked, np.uint8)
        out = np.empty((N, K), dtype=np.uint8)
        self.lib.oracle_unpack(_ptr(Wp), N, K, _ptr(out))
        return out

    def block_index(self, K, bs, n, k) -> int:
        return int(self.lib.oracle_block_index(K, bs, n, k))

    def w32(self, Wpacked, absmax, codebook, K, bs, n, k) -> np.float32:
        Wp, am, cb = _c(Wpacked, np.uint8), _c(absmax, np.float32), _c(codebook, np.float32)
        return np.float32(self.lib.oracle_w32(_ptr(Wp), _ptr(am), _ptr(cb), K, bs, n, k))

    def dequant_f32(self, Wpacked, absmax, codebook, N, K, bs) -> np.ndarray:
        Wp, am, cb = _c(Wpacked, np.uint8), _c(absmax, np.float32), _c(codebook, np.float32)
        out = np.empty((N, K), dtype=np.float32)
        self.lib.oracle_dequant_f32(_ptr(Wp), _ptr(am), _ptr(cb), N, K, bs, _ptr(out))
        return out

    def dequant_bf16(self, Wpacked, absmax, codebook, N, K, bs) -> np.ndarray:
        """bf16 bit patterns (uint16) of the dequantized weights."""
        Wp, am, cb = _c(Wpacked, np.uint8), _c(absmax, np.float32), _c(codebook, np.float32)
        out = np.empty((N, K), dtype=np.uint16)
        self.lib.oracle_dequant_bf16(_ptr(Wp), _ptr(am), _ptr(cb), N, K, bs, _ptr(out))
        return out

    def f32_to_bf16(self, x) -> np.ndarray:
        """bf16 bit patterns of an fp32 array (any shape)."""
        xs = _c(x, np.float32)
        out = np.empty(xs.shape, dtype=np.uint16)
        self.lib.oracle_f32_to_bf16_array(_ptr(xs), xs.size, _ptr(out))
        return out

    @staticmethod
    def _cols(cols, N):
        if cols is None:
            return None, N
        c = _c(cols, np.int64)
        if c.size and (c.min() < 0 or c.max() >= N):
            raise ValueError("column index out of range")
        return c, c.size

    def q4_gemm(self, A_bf16, Wpacked, absmax, codebook, M, N, K, bs, cols=None):
        """(C, S) in fp64, shape [M, len(cols) or N]."""
        A = _c(A_bf16, np.uint16)
        Wp, am, cb = _c(Wpacked, np.uint8), _c(absmax, np.float32), _c(codebook, np.float32)
        c, nc = self._cols(cols, N)
        C = np.empty((M, nc), dtype=np.float64)
        S = np.empty((M, nc), dtype=np.float64)
        self.lib.oracle_q4_gemm(_ptr(A), _ptr(Wp), _ptr(am), _ptr(cb), M, N, K, bs,
                                _ptr(c), nc, _ptr(C), _ptr(S))
        return C, S

    def q4_gemm_w16(self, A_bf16, Wpacked, absmax, codebook, M, N, K, bs, cols=None):
        A = _c(A_bf16, np.uint16)
        Wp, am, cb = _c(Wpacked, np.uint8), _c(absmax, np.float32), _c(codebook, np.float32)
        c, nc = self._cols(cols, N)
        C = np.empty((M, nc), dtype=np.float64)
        S = np.empty((M, nc), dtype=np.float64)
        self.lib.oracle_q4_gemm_w16(_ptr(A), _ptr(Wp), _ptr(am), _ptr(cb), M, N, K, bs,
                                    _ptr(c), nc, _ptr(C), _ptr(S))
        return C, S

    def bf16_gemm(self, A_bf16, W_bf16, bias_bf16, M, N, K, cols=None):
        A, W = _c(A_bf16, np.uint16), _c(W_bf16, np.uint16)
        b = None if bias_bf16 is None else _c(bias_bf16, np.uint16)
        c, nc = self._cols(cols, N)
        C = np.empty((M, nc), dtype=np.float64)
        S = np.empty((M, nc), dtype=np.float64)
        self.lib.oracle_bf16_gemm(_ptr(A), _ptr(W), _ptr(b), M, N, K, _ptr(c), nc,
                                  _ptr(C), _ptr(S))
        return C, S

    DTYPES = {"bf16": (0, np.uint16), "fp32": (1, np.float32), "fp16": (2, np.uint16)}

    def f16_to_double(self, bits) -> np.ndarray:
        """fp64 values of binary16 bit patterns (uint16 array, any shape)."""
        b = _c(bits, np.uint16)
        return np.array([self.lib.oracle_f16_to_double(int(v)) for v in b.ravel()],
                        dtype=np.float64).reshape(b.shape)

    def f32_to_f16(self, x) -> np.ndarray:
        """binary16 bit patterns of an fp32 array (any shape), nearest-even."""
        xs = _c(x, np.float32)
        out = np.empty(xs.shape, dtype=np.uint16)
        self.lib.oracle_f32_to_f16_array(_ptr(xs), xs.size, _ptr(out))
        return out

    def dequant_f16(self, Wpacked, absmax, codebook, N, K, bs) -> np.ndarray:
        """binary16 bit patterns (uint16) of the dequantized weights."""
        Wp, am, cb = _c(Wpacked, np.uint8), _c(absmax, np.float32), _c(codebook, np.float32)
        out = np.empty((N, K), dtype=np.uint16)
        self.lib.oracle_dequant_f16(_ptr(Wp), _ptr(am), _ptr(cb), N, K, bs, _ptr(out))
        return out

    def q4_gemm_ex(self, A, a_dtype, Wpacked, absmax, codebook, M, N, K, bs, bias=None,
                   bias_dtype="bf16", cols=None):
        """(C, S) in fp64 for activations of a_dtype and an optional bias."""
        acode, anp = self.DTYPES[a_dtype]
        bcode, bnp = self.DTYPES[bias_dtype]
        Aa = _c(A, anp)
        b = None if bias is None else _c(bias, bnp)
        Wp, am, cb = _c(Wpacked, np.uint8), _c(absmax, np.float32), _c(codebook, np.float32)
        c, nc = self._cols(cols, N)
        C = np.empty((M, nc), dtype=np.float64)
        S = np.empty((M, nc), dtype=np.float64)
        self.lib.oracle_q4_gemm_ex(_ptr(Aa), acode, _ptr(Wp), _ptr(am), _ptr(cb), _ptr(b), bcode,
                                   M, N, K, bs, _ptr(c), nc, _ptr(C), _ptr(S))
        return C, S

    def quantize(self, W, w_dtype, codebook, N, K, bs):
        """(codes uint8 [N, K], absmax float32 [N, K/bs]) of W in w_dtype."""
        code, npt = self.DTYPES[w_dtype]
        Wa, cb = _c(W, npt), _c(codebook, np.float32)
        codes = np.empty((N, K), dtype=np.uint8)
        absmax = np.empty((N, K // bs), dtype=np.float32)
        self.lib.oracle_quantize(_ptr(Wa), code, _ptr(cb), N, K, bs, _ptr(codes), _ptr(absmax))
        return codes, absmax

    def tile_offset(self, N, K, n, j) -> int:
        return int(self.lib.oracle_tile_offset(N, K, n, j))

    def repack_tiles(self, Wpacked, N, K) -> np.ndarray:
        """uint8 [N, K/2] holding the tile layout of row-major Wpacked."""
        Wp = _c(Wpacked, np.uint8)
        out = np.empty((N, K // 2), dtype=np.uint8)
        self.lib.oracle_repack_tiles(_ptr(Wp), N, K, _ptr(out))
        return out

    def bf16_tile_index(self, N, K, n, k) -> int:
        return int(self.lib.oracle_bf16_tile_index(N, K, n, k))

    def bf16_repack_tiles(self, W_bf16, N, K) -> np.ndarray:
        """uint16 [N, K] holding the tile layout of row-major bf16 W."""
        W = _c(W_bf16, np.uint16)
        out = np.empty((N, K), dtype=np.uint16)
        self.lib.oracle_bf16_repack_tiles(_ptr(W), N, K, _ptr(out))
        return out

    def gemm_f32w(self, A_bf16, W_f32, M, N, K):
        A, W = _c(A_bf16, np.uint16), _c(W_f32, np.float32)
        C = np.empty((M, N), dtype=np.float64)
        self.lib.oracle_gemm_f32w(_ptr(A), _ptr(W), M, N, K, _ptr(C))
        return C


_default = None


def default() -> Oracle:
    global _default
    if _default is None:
        _default = Oracle(build())
    return _default


def __getattr__(name):
    # Module-level access (oracle.q4_gemm, ...) goes to the default library.
    if name.startswith("_"):
        raise AttributeError(name)
    return getattr(default(), name)
