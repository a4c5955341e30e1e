"""Python binding of the q4skinny HIP library (MI355X / gfx950).

Argument marshalling only: every step of the computation runs in the HIP
kernels of ``libq4skinny.so``.  torch provides device memory and the current
stream.  There is no CPU fallback: if the library is missing, importing the
functions below raises.

Entry points (same names as the C ABI in include/q4skinny.h):
  q4_gemm_skinny(A, Wpacked, absmax, codebook, blocksize=64, out=None, path="auto",
                 bias=None, out_dtype=None)   (q4_gemm_skinny_path / q4_gemm_skinny_ex)
  bf16_gemm_skinny(A, W, bias=None, out=None, layout="rows")   (bf16_gemm_skinny_tiles)
  bf16_repack_tiles(W, out=None)
  q4_dequant(Wpacked, absmax, codebook, blocksize=64, out_dtype=torch.bfloat16, out=None)
  q4_quantize(W, codebook, blocksize=64, out=None)   codebook: host sequence of 16 floats
  q4_codebook_preset(name)   "nf4_style" or "int4" -> numpy float32 [16]
  q4_get_crossover_m() / q4_set_crossover_m(m) / q4_release_workspace()
  q4_set_crossover_shape(N, K, m) / q4_get_crossover_shape(N, K) / q4_clear_crossover_shapes()
  q4_skinny_kparts(M, N, K)
  q4_copy_probe(src, dst) / q4_read_probe(src, sink, ...) / q4_version()
``lib()`` returns the raw ctypes handle for callers that pass pointers.
"""
from __future__ import annotations

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libq4skinny.so")

Q4_OK, Q4_ERR_INVALID_ARGUMENT, Q4_ERR_UNSUPPORTED, Q4_ERR_HIP = 0, 1, 2, 3
Q4_DTYPE_BF16, Q4_DTYPE_FP32, Q4_DTYPE_FP16 = 0, 1, 2
PATHS = {"auto": 0, "fused": 1, "split": 2}
FUSED_PASS_M = 32
CROSSOVER_MAX = 65536
Q4_NOALLOC_SCRATCH_BYTES = 64 << 20

# Every symbol include/q4skinny.h declares.
EXPORTS = (
    "q4_gemm_skinny", "q4_gemm_skinny_path", "q4_gemm_skinny_ex", "bf16_gemm_skinny", "q4_dequant",
    "q4_get_crossover_m", "q4_set_crossover_m", "q4_release_workspace", "q4_last_error",
    "q4_copy_probe", "q4_version", "q4_quantize", "q4_codebook_preset",
    "q4_set_crossover_shape", "q4_get_crossover_shape", "q4_clear_crossover_shapes",
    "q4_repack_tiles", "q4_gemm_skinny_tiles", "q4_dequant_tiles", "q4_read_probe",
    "q4_gemm_skinny_ex_noalloc", "bf16_repack_tiles", "bf16_gemm_skinny_tiles",
    "q4_skinny_kparts",
)
PRESETS = {"nf4_style": 0, "int4": 1}


class Q4Error(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__("q4skinny status %d: %s" % (status, message))
        self.status = status


_lib = None


def lib():
    """Load libq4skinny.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError("libq4skinny.so is not built; run python -m bit_dequant_skinny_amd.build")
        # torch first: its HIP runtime is then the one the library binds to
        # (same soname), so the process has a single runtime.  Loading the
        # library first pulls in a second copy that sees no device once
        # torch's has claimed it.
        _torch()
        L = ctypes.CDLL(LIB_PATH)
        P, I = ctypes.c_void_p, ctypes.c_int
        L.q4_gemm_skinny.argtypes = [P, P, P, P, I, I, I, I, P, P]
        L.q4_gemm_skinny_path.argtypes = [P, P, P, P, I, I, I, I, P, P, I]
        L.q4_gemm_skinny_ex.argtypes = [P, I, P, P, P, P, I, I, I, I, P, I, P, I]
        L.bf16_gemm_skinny.argtypes = [P, P, P, I, I, I, P, P]
        L.bf16_gemm_skinny_tiles.argtypes = [P, P, P, I, I, I, P, P]
        L.bf16_repack_tiles.argtypes = [P, P, I, I, P]
        L.q4_dequant.argtypes = [P, P, P, I, I, I, P, I, P]
        L.q4_gemm_skinny_tiles.argtypes = [P, I, P, P, P, P, I, I, I, I, P, I, P, I]
        L.q4_gemm_skinny_ex_noalloc.argtypes = [P, I, P, P, P, P, I, I, I, I, P, I, P, I]
        L.q4_dequant_tiles.argtypes = [P, P, P, I, I, I, P, I, P]
        L.q4_repack_tiles.argtypes = [P, P, I, I, P]
        L.q4_copy_probe.argtypes = [P, P, ctypes.c_size_t, P]
        L.q4_read_probe.argtypes = [P, ctypes.c_size_t, P, I, I, I, I, P]
        L.q4_set_crossover_m.argtypes = [I]
        L.q4_quantize.argtypes = [P, I, P, I, I, I, P, P, P]
        L.q4_codebook_preset.argtypes = [I, P]
        L.q4_set_crossover_shape.argtypes = [I, I, I]
        L.q4_get_crossover_shape.argtypes = [I, I]
        L.q4_get_crossover_shape.restype = ctypes.c_int
        L.q4_skinny_kparts.argtypes = [I, I, I]
        L.q4_skinny_kparts.restype = ctypes.c_int
        for name in ("q4_gemm_skinny", "q4_gemm_skinny_path", "q4_gemm_skinny_ex",
                     "q4_gemm_skinny_ex_noalloc", "q4_gemm_skinny_tiles", "q4_dequant_tiles",
                     "q4_repack_tiles",
                     "bf16_gemm_skinny", "bf16_gemm_skinny_tiles", "bf16_repack_tiles",
                     "q4_dequant",
                     "q4_copy_probe", "q4_read_probe", "q4_set_crossover_m",
                     "q4_release_workspace",
                     "q4_quantize", "q4_codebook_preset", "q4_set_crossover_shape",
                     "q4_clear_crossover_shapes"):
            getattr(L, name).restype = ctypes.c_int
        L.q4_get_crossover_m.restype = ctypes.c_int
        L.q4_last_error.restype = ctypes.c_char_p
        L.q4_version.restype = ctypes.c_char_p
        _lib = L
    return _lib


def _check(status: int):
    if status != Q4_OK:
        raise Q4Error(status, lib().q4_last_error().decode())


def _torch():
    import torch
    return torch


def _stream(t):
    """Raw handle of torch's current stream on t's device."""
    torch = _torch()
    raw = getattr(torch._C, "_cuda_getCurrentRawStream", None)
    if raw is not None:
        return raw(t.get_device())
    return torch.cuda.current_stream(t.device).cuda_stream


def _dtype_code(dtype):
    torch = _torch()
    codes = {torch.bfloat16: Q4_DTYPE_BF16, torch.float16: Q4_DTYPE_FP16,
             torch.float32: Q4_DTYPE_FP32}
    if dtype not in codes:
        raise TypeError("dtype must be torch.bfloat16, torch.float16 or torch.float32, got %s"
                        % dtype)
    return codes[dtype]


def _dev(t, name, dtype):
    """Device pointer of a contiguous GPU tensor of dtype (raises otherwise)."""
    try:
        if t.is_cuda and t.dtype is dtype and t.is_contiguous():
            return t.data_ptr()
    except AttributeError:
        pass
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if t.device.type != "cuda":
        raise ValueError("%s must be on a GPU" % name)
    if t.dtype != dtype:
        raise TypeError("%s must be %s, got %s" % (name, dtype, t.dtype))
    raise ValueError("%s must be contiguous" % name)


def q4_gemm_skinny(A, Wpacked, absmax, codebook, blocksize: int = 64, out=None, path: str = "auto",
                   bias=None, out_dtype=None, layout: str = "rows"):
    """C[M,N] = A[M,K] * dequant(W)[N,K]^T (+ bias), fp32 accumulation.

    A may be bf16, fp16 or fp32; C (and bias) have out_dtype, by default A's
    dtype.  layout "rows": Wpacked holds row-major packed rows; bf16 in and
    out without a bias calls q4_gemm_skinny_path, anything else
    q4_gemm_skinny_ex.  layout "tiles": Wpacked holds the output of
    q4_repack_tiles (same [N, K/2] shape) and q4_gemm_skinny_tiles runs."""
    if layout not in ("rows", "tiles"):
        raise ValueError("layout must be 'rows' or 'tiles'")
    torch = _torch()
    if A.dim() != 2 or Wpacked.dim() != 2:
        raise ValueError("A must be [M, K] and Wpacked [N, K/2]")
    M, K = A.shape
    N = Wpacked.shape[0]
    if Wpacked.shape[1] * 2 != K:
        raise ValueError("Wpacked must be [N, K/2]")
    if blocksize > 0 and K % blocksize == 0 and tuple(absmax.shape) != (N, K // blocksize):
        raise ValueError("absmax must be [N, K/blocksize]")
    if codebook.numel() != 16:
        raise ValueError("codebook must hold 16 entries")
    out_dtype = A.dtype if out_dtype is None else out_dtype
    a_code, c_code = _dtype_code(A.dtype), _dtype_code(out_dtype)
    if bias is not None and tuple(bias.shape) != (N,):
        raise ValueError("bias must be [N]")
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype, device=A.device)
    elif tuple(out.shape) != (M, N):
        raise ValueError("out must be [M, N]")
    if layout == "rows" and a_code == Q4_DTYPE_BF16 and c_code == Q4_DTYPE_BF16 and bias is None:
        _check(lib().q4_gemm_skinny_path(
            _dev(A, "A", torch.bfloat16), _dev(Wpacked, "Wpacked", torch.uint8),
            _dev(absmax, "absmax", torch.float32), _dev(codebook, "codebook", torch.float32),
            M, N, K, blocksize, _dev(out, "out", torch.bfloat16), _stream(A), PATHS[path]))
        return out
    bptr = None if bias is None else _dev(bias, "bias", out_dtype)
    fn = lib().q4_gemm_skinny_ex if layout == "rows" else lib().q4_gemm_skinny_tiles
    _check(fn(
        _dev(A, "A", A.dtype), a_code, _dev(Wpacked, "Wpacked", torch.uint8),
        _dev(absmax, "absmax", torch.float32), _dev(codebook, "codebook", torch.float32), bptr,
        M, N, K, blocksize, _dev(out, "out", out_dtype), c_code, _stream(A), PATHS[path]))
    return out


def bf16_gemm_skinny(A, W, bias=None, out=None, layout: str = "rows"):
    """C[M,N] = A[M,K] * W[N,K]^T (+ bias) in bf16, M <= 5.

    layout "tiles" reads weights made by bf16_repack_tiles (same shape)."""
    if layout not in ("rows", "tiles"):
        raise ValueError("layout must be 'rows' or 'tiles'")
    torch = _torch()
    if A.dim() != 2 or W.dim() != 2 or A.shape[1] != W.shape[1]:
        raise ValueError("A must be [M, K] and W [N, K]")
    M, K = A.shape
    N = W.shape[0]
    if bias is not None and tuple(bias.shape) != (N,):
        raise ValueError("bias must be [N]")
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=A.device)
    elif tuple(out.shape) != (M, N):
        raise ValueError("out must be [M, N]")
    bptr = None if bias is None else _dev(bias, "bias", torch.bfloat16)
    fn = lib().bf16_gemm_skinny if layout == "rows" else lib().bf16_gemm_skinny_tiles
    _check(fn(
        _dev(A, "A", torch.bfloat16), _dev(W, "W", torch.bfloat16), bptr, M, N, K,
        _dev(out, "out", torch.bfloat16), _stream(A)))
    return out


def bf16_repack_tiles(W, out=None):
    """The tile layout of row-major bf16 weights [N, K] (same shape: 16-row
    tiles of 1 KiB units of 32 k; N % 16 == 0, K % 32 == 0)."""
    torch = _torch()
    if W.dim() != 2:
        raise ValueError("W must be [N, K]")
    N, K = W.shape
    if out is None:
        out = torch.empty_like(W)
    elif tuple(out.shape) != (N, K):
        raise ValueError("out must be [N, K]")
    _check(lib().bf16_repack_tiles(
        _dev(W, "W", torch.bfloat16), _dev(out, "out", torch.bfloat16), N, K, _stream(W)))
    return out


def q4_dequant(Wpacked, absmax, codebook, blocksize: int = 64, out_dtype=None, out=None,
               layout: str = "rows"):
    """W[N,K] = codebook[code] * absmax, as bf16 (default), fp16 or fp32.

    layout "tiles" reads weights made by q4_repack_tiles; the output is
    row-major either way."""
    if layout not in ("rows", "tiles"):
        raise ValueError("layout must be 'rows' or 'tiles'")
    torch = _torch()
    out_dtype = torch.bfloat16 if out_dtype is None else out_dtype
    N, K = Wpacked.shape[0], Wpacked.shape[1] * 2
    if out is None:
        out = torch.empty((N, K), dtype=out_dtype, device=Wpacked.device)
    elif tuple(out.shape) != (N, K) or out.dtype != out_dtype:
        raise ValueError("out must be [N, K] of out_dtype")
    code = _dtype_code(out_dtype)
    fn = lib().q4_dequant if layout == "rows" else lib().q4_dequant_tiles
    _check(fn(
        _dev(Wpacked, "Wpacked", torch.uint8), _dev(absmax, "absmax", torch.float32),
        _dev(codebook, "codebook", torch.float32), N, K, blocksize, _dev(out, "out", out_dtype),
        code, _stream(Wpacked)))
    return out


def q4_skinny_kparts(M: int, N: int, K: int) -> int:
    """Parts the fused skinny kernel splits K into for this shape (1 = none)."""
    return int(lib().q4_skinny_kparts(M, N, K))


def q4_repack_tiles(Wpacked, out=None):
    """The tile layout of row-major packed weights [N, K/2] (uint8, same shape:
    16-row tiles of 1 KiB units; N % 16 == 0, K % 128 == 0)."""
    torch = _torch()
    if Wpacked.dim() != 2:
        raise ValueError("Wpacked must be [N, K/2]")
    N, K = Wpacked.shape[0], Wpacked.shape[1] * 2
    if out is None:
        out = torch.empty_like(Wpacked)
    elif tuple(out.shape) != (N, K // 2):
        raise ValueError("out must be [N, K/2]")
    _check(lib().q4_repack_tiles(
        _dev(Wpacked, "Wpacked", torch.uint8), _dev(out, "out", torch.uint8), N, K,
        _stream(Wpacked)))
    return out


def q4_copy_probe(src, dst):
    torch = _torch()
    nbytes = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() < nbytes:
        raise ValueError("dst too small")
    _check(lib().q4_copy_probe(_dev(src, "src", src.dtype), _dev(dst, "dst", dst.dtype), nbytes,
                               _stream(src)))
    del torch
    return dst


PROBE_NONTEMPORAL, PROBE_INTERLEAVE = 1, 2


def q4_read_probe(src, sink, threads: int = 0, unroll: int = 0, wgs_per_cu: int = 0,
                  nontemporal: bool = True, interleave: bool = True):
    """Reads all of src (a contiguous GPU tensor) once; sink is a GPU tensor of
    at least 4 bytes (written only when the folded data hits a fixed value)."""
    torch = _torch()
    nbytes = src.numel() * src.element_size()
    if sink.numel() * sink.element_size() < 4:
        raise ValueError("sink must hold 4 bytes")
    flags = (PROBE_NONTEMPORAL if nontemporal else 0) | (PROBE_INTERLEAVE if interleave else 0)
    _check(lib().q4_read_probe(_dev(src, "src", src.dtype), nbytes, _dev(sink, "sink", sink.dtype),
                               int(threads), int(unroll), int(wgs_per_cu), flags, _stream(src)))
    del torch


def q4_get_crossover_m() -> int:
    return int(lib().q4_get_crossover_m())


def q4_set_crossover_m(m: int) -> None:
    _check(lib().q4_set_crossover_m(int(m)))


def q4_set_crossover_shape(N: int, K: int, m: int) -> None:
    """Crossover for weight shape (N, K); m < 0 removes the entry."""
    _check(lib().q4_set_crossover_shape(int(N), int(K), int(m)))


def q4_get_crossover_shape(N: int, K: int) -> int:
    return int(lib().q4_get_crossover_shape(int(N), int(K)))


def q4_clear_crossover_shapes() -> None:
    _check(lib().q4_clear_crossover_shapes())


def q4_release_workspace() -> None:
    _check(lib().q4_release_workspace())


def q4_version() -> str:
    return lib().q4_version().decode()


def q4_quantize(W, codebook, blocksize: int = 64, out=None):
    """(Wpacked uint8 [N, K/2], absmax fp32 [N, K/blocksize]) of W (bf16, fp16
    or fp32 on the GPU); codebook: 16 strictly increasing floats (host)."""
    import numpy as np
    torch = _torch()
    if W.dim() != 2:
        raise ValueError("W must be [N, K]")
    N, K = W.shape
    cb = np.ascontiguousarray(np.asarray(codebook, dtype=np.float32).reshape(-1))
    if cb.size != 16:
        raise ValueError("codebook must hold 16 entries")
    if out is None:
        nb = K // blocksize if blocksize > 0 and K % blocksize == 0 else 0
        out = (torch.empty((N, K // 2), dtype=torch.uint8, device=W.device),
               torch.empty((N, nb), dtype=torch.float32, device=W.device))
    Wp, am = out
    _check(lib().q4_quantize(
        _dev(W, "W", W.dtype), _dtype_code(W.dtype), cb.ctypes.data_as(ctypes.c_void_p), N, K,
        blocksize, _dev(Wp, "Wpacked", torch.uint8), _dev(am, "absmax", torch.float32),
        _stream(W)))
    return Wp, am


def q4_codebook_preset(name: str = "nf4_style"):
    """A 16-entry fp32 table (numpy): "nf4_style" or "int4"."""
    import numpy as np
    out = np.empty(16, dtype=np.float32)
    _check(lib().q4_codebook_preset(PRESETS[name], out.ctypes.data_as(ctypes.c_void_p)))
    return out
