"""The C-ABI library on the host: it loads, exports every symbol the header
declares, and rejects invalid arguments before touching the GPU runtime.

No call here launches anything: every call either fails validation or has an
empty shape, both of which return before any HIP call.
"""
import ctypes
import os
import re
import subprocess
import sys

import pytest

import bit_dequant_skinny_amd as q4

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "q4skinny.h")

FAKE = 0x10000  # 16-byte aligned, never dereferenced on these paths
INV, UNS, OK = q4.Q4_ERR_INVALID_ARGUMENT, q4.Q4_ERR_UNSUPPORTED, q4.Q4_OK


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(q4_\w+|bf16_\w+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    L = q4.lib()
    decl = declared_functions()
    assert decl == sorted(q4.EXPORTS)
    for name in decl:
        assert hasattr(L, name), name


def test_exports_seen_by_nm():
    out = subprocess.run(["nm", "-D", "--defined-only", q4.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    syms = {line.split()[-1] for line in out.splitlines() if line.strip()}
    for name in declared_functions():
        assert name in syms, name


def test_version_and_crossover_defaults():
    assert "gfx950" in q4.q4_version()
    assert 0 <= q4.q4_get_crossover_m() <= q4.CROSSOVER_MAX


def _q4(M=1, N=16, K=128, bs=64, A=FAKE, W=FAKE, am=FAKE, cb=FAKE, C=FAKE, path=0):
    L = q4.lib()
    return L.q4_gemm_skinny_path(A, W, am, cb, M, N, K, bs, C, None, path)


@pytest.mark.parametrize("kw,expect", [
    (dict(M=-1), INV), (dict(N=-1), INV), (dict(K=-64), INV), (dict(K=0), INV),
    (dict(bs=0), INV), (dict(bs=-64), INV), (dict(bs=63), INV), (dict(K=96, bs=64), INV),
    (dict(bs=16, K=128), UNS), (dict(bs=512, K=1024), UNS), (dict(bs=48, K=96), UNS),
    (dict(A=None), INV), (dict(W=None), INV), (dict(am=None), INV), (dict(cb=None), INV),
    (dict(C=None), INV), (dict(A=FAKE + 8), INV), (dict(W=FAKE + 4), INV),
    (dict(am=FAKE + 4), INV), (dict(cb=FAKE + 2), INV), (dict(C=FAKE + 1), INV),
    (dict(path=7), INV), (dict(path=1, M=17, K=100), INV),
    (dict(M=0), OK), (dict(N=0), OK), (dict(M=0, A=None, C=None), OK),
])
def test_q4_gemm_validation(kw, expect):
    assert _q4(**kw) == expect
    msg = q4.lib().q4_last_error().decode()
    assert (msg == "") == (expect == OK)


def test_q4_gemm_auto_entry_validates_too():
    L = q4.lib()
    assert L.q4_gemm_skinny(FAKE, FAKE, FAKE, FAKE, 1, 16, 100, 64, FAKE, None) == INV
    assert L.q4_gemm_skinny(FAKE, FAKE, FAKE, FAKE, 0, 16, 128, 64, FAKE, None) == OK


@pytest.mark.parametrize("args,expect", [
    ((FAKE, FAKE, None, -1, 4, 64), INV), ((FAKE, FAKE, None, 1, 4, 0), INV),
    ((FAKE, FAKE, None, 1, 4, 12), INV), ((FAKE, FAKE, None, 6, 4, 64), UNS),
    ((None, FAKE, None, 1, 4, 64), INV), ((FAKE, None, None, 1, 4, 64), INV),
    ((FAKE + 2, FAKE, None, 1, 4, 64), INV), ((FAKE, FAKE + 8, None, 1, 4, 64), INV),
    ((FAKE, FAKE, FAKE + 1, 1, 4, 64), INV),
    ((FAKE, FAKE, None, 0, 4, 64), OK), ((FAKE, FAKE, None, 3, 0, 64), OK),
])
def test_bf16_gemm_validation(args, expect):
    A, W, b, M, N, K = args
    C = FAKE
    assert q4.lib().bf16_gemm_skinny(A, W, b, M, N, K, C, None) == expect


def test_bf16_gemm_rejects_null_output():
    assert q4.lib().bf16_gemm_skinny(FAKE, FAKE, None, 1, 4, 64, None, None) == INV


@pytest.mark.parametrize("kw,expect", [
    (dict(dtype=5), INV), (dict(N=-1), INV), (dict(K=0), INV), (dict(K=100), INV),
    (dict(bs=16, K=128), UNS), (dict(out=None), INV), (dict(out=FAKE + 4), INV),
    (dict(W=None), INV), (dict(N=0), OK),
])
def test_dequant_validation(kw, expect):
    p = dict(W=FAKE, am=FAKE, cb=FAKE, N=4, K=128, bs=64, out=FAKE, dtype=0)
    p.update(kw)
    st = q4.lib().q4_dequant(p["W"], p["am"], p["cb"], p["N"], p["K"], p["bs"], p["out"],
                             p["dtype"], None)
    assert st == expect


def test_copy_probe_validation():
    L = q4.lib()
    assert L.q4_copy_probe(FAKE, FAKE, 0, None) == OK
    assert L.q4_copy_probe(FAKE, FAKE, 24, None) == INV
    assert L.q4_copy_probe(None, FAKE, 32, None) == INV
    assert L.q4_copy_probe(FAKE + 4, FAKE, 32, None) == INV


def test_crossover_setter_range():
    L = q4.lib()
    old = L.q4_get_crossover_m()
    assert L.q4_set_crossover_m(-1) == INV
    assert L.q4_set_crossover_m(q4.CROSSOVER_MAX + 1) == INV
    assert L.q4_set_crossover_m(4) == OK and L.q4_get_crossover_m() == 4
    assert L.q4_set_crossover_m(old) == OK


def _in_subprocess(code, env_extra):
    env = dict(os.environ)
    env.update(env_extra)
    env["PYTHONPATH"] = ROOT
    return subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, env=env,
                          timeout=120)


def test_crossover_env_override():
    r = _in_subprocess("import bit_dequant_skinny_amd as q; print(q.q4_get_crossover_m())",
                       {"Q4_CROSSOVER_M": "3"})
    assert r.returncode == 0 and r.stdout.strip() == "3", r.stderr
    r = _in_subprocess("import bit_dequant_skinny_amd as q; print(q.q4_get_crossover_m())",
                       {"Q4_CROSSOVER_M": "banana"})
    assert r.returncode == 0 and int(r.stdout.strip()) == q4.q4_get_crossover_m()


def test_crossover_shape_table():
    L = q4.lib()
    q4.q4_clear_crossover_shapes()
    base = q4.q4_get_crossover_m()
    assert L.q4_set_crossover_shape(0, 64, 4) == INV
    assert L.q4_set_crossover_shape(64, -1, 4) == INV
    assert L.q4_set_crossover_shape(64, 128, q4.CROSSOVER_MAX + 1) == INV
    try:
        q4.q4_set_crossover_shape(4096, 4096, 8)
        q4.q4_set_crossover_shape(5120, 8192, 0)
        assert q4.q4_get_crossover_shape(4096, 4096) == 8
        assert q4.q4_get_crossover_shape(5120, 8192) == 0
        assert q4.q4_get_crossover_shape(8192, 4096) == base  # (N, K) is ordered
        q4.q4_set_crossover_m(3)
        assert q4.q4_get_crossover_shape(4096, 4096) == 8     # the entry wins
        assert q4.q4_get_crossover_shape(100, 100) == 3       # no entry: global
        q4.q4_set_crossover_shape(4096, 4096, -1)              # removes it
        assert q4.q4_get_crossover_shape(4096, 4096) == 3
    finally:
        q4.q4_set_crossover_m(base)
        q4.q4_clear_crossover_shapes()
    assert q4.q4_get_crossover_shape(5120, 8192) == base


def test_crossover_bucket_of_unmeasured_shapes():
    """A shape without an entry takes the smallest entry of its bucket (K
    rounded up to a power of two, tiles per compute unit in the classes 1, 2,
    3-4, 5+; 256 compute units assumed without a GPU); exact entries win."""
    base = q4.q4_get_crossover_m()
    q4.q4_clear_crossover_shapes()
    try:
        q4.q4_set_crossover_shape(28672, 8192, 300)  # 7 tiles per CU, K bucket 8192
        q4.q4_set_crossover_shape(24576, 8192, 280)  # 6 tiles per CU, same bucket
        q4.q4_set_crossover_shape(5120, 5120, 90)    # 2 tiles per CU, K bucket 8192
        assert q4.q4_get_crossover_shape(20480, 7000) == 280   # 5 tiles, K -> 8192
        assert q4.q4_get_crossover_shape(28672, 8192) == 300   # exact entry
        assert q4.q4_get_crossover_shape(8192, 6144) == 90     # 2 tiles, K -> 8192
        assert q4.q4_get_crossover_shape(8192, 16384) == base  # K bucket 16384: none
        assert q4.q4_get_crossover_shape(16384, 8192) == base  # 4 tiles: no entry
        assert q4.q4_get_crossover_shape(100, 8192) == base    # 1 tile: no entry
    finally:
        q4.q4_clear_crossover_shapes()


def test_crossover_shape_table_from_environment():
    code = ("import bit_dequant_skinny_amd as q; "
            "print(q.q4_get_crossover_shape(4096, 4096), q.q4_get_crossover_shape(64, 128), "
            "q.q4_get_crossover_shape(7, 7), q.q4_get_crossover_m())")
    r = _in_subprocess(code, {"Q4_CROSSOVER_TABLE": "4096:4096:12, bad,64:128:0,7:7:-2,5:5:5x",
                              "Q4_CROSSOVER_M": "9"})
    assert r.returncode == 0, r.stderr
    assert r.stdout.split() == ["12", "0", "9", "9"]


def test_binding_refuses_cpu_tensors():
    import torch
    A = torch.zeros(1, 128, dtype=torch.bfloat16)
    W = torch.zeros(4, 64, dtype=torch.uint8)
    am = torch.zeros(4, 2)
    cb = torch.zeros(16)
    with pytest.raises(ValueError):
        q4.q4_gemm_skinny(A, W, am, cb, out=torch.empty(1, 4, dtype=torch.bfloat16))


def _ex(M=1, N=16, K=128, bs=64, adt=0, cdt=0, A=FAKE, W=FAKE, am=FAKE, cb=FAKE, bias=None,
        C=FAKE, path=0):
    return q4.lib().q4_gemm_skinny_ex(A, adt, W, am, cb, bias, M, N, K, bs, C, cdt, None, path)


@pytest.mark.parametrize("kw,expect", [
    (dict(adt=3), INV), (dict(cdt=-1), INV), (dict(path=9), INV), (dict(M=-2), INV),
    (dict(K=96), INV), (dict(bs=16, K=128), UNS), (dict(A=None), INV), (dict(C=None), INV),
    (dict(cdt=1, C=FAKE + 2), INV), (dict(cdt=1, bias=FAKE + 2), INV), (dict(bias=FAKE + 1), INV),
    (dict(A=FAKE + 8), INV), (dict(adt=1, path=2), UNS), (dict(adt=1, M=40, path=2), UNS),
    (dict(path=1, M=17, bs=48, K=96), UNS), (dict(M=0), OK), (dict(N=0, cdt=2), OK),
    (dict(adt=1, M=0, path=1), OK),
])
def test_q4_gemm_ex_validation(kw, expect):
    assert _ex(**kw) == expect
    assert (q4.lib().q4_last_error().decode() == "") == (expect == OK)


def _quant(cb, N=4, K=128, bs=64, wdt=0, W=FAKE, Wp=FAKE, am=FAKE):
    import numpy as np
    c = None if cb is None else np.ascontiguousarray(cb, dtype=np.float32)
    ptr = None if c is None else c.ctypes.data_as(ctypes.c_void_p)
    return q4.lib().q4_quantize(W, wdt, ptr, N, K, bs, Wp, am, None)


def test_q4_quantize_validation():
    import numpy as np
    good = q4.q4_codebook_preset("nf4_style")
    assert _quant(good, N=0) == OK
    assert _quant(None) == INV
    assert _quant(good, wdt=7) == INV
    assert _quant(good, K=100) == INV
    assert _quant(good, bs=16, K=128) == UNS
    assert _quant(good, W=None) == INV
    assert _quant(good, Wp=FAKE + 4) == INV
    assert _quant(good, am=FAKE + 2) == INV
    bad = good.copy()
    bad[3], bad[4] = bad[4], bad[3]   # not increasing
    assert _quant(bad, N=0) == INV
    dup = good.copy()
    dup[5] = dup[6]                    # not strictly increasing
    assert _quant(dup, N=0) == INV
    nan = good.copy()
    nan[2] = np.nan
    assert _quant(nan, N=0) == INV


def test_codebook_presets():
    import numpy as np
    import synth
    nf4 = q4.q4_codebook_preset("nf4_style")
    # the same rule as the test generator's table, which uses Python's own
    # normal quantile (a different algorithm from the library's bisection)
    assert np.array_equal(nf4.view(np.uint32), synth.nf4_style_codebook().view(np.uint32))
    int4 = q4.q4_codebook_preset("int4")
    assert list(int4) == [(i - 8) / 8 for i in range(16)]
    for cb in (nf4, int4):
        assert np.all(np.diff(cb) > 0) and cb[0] == -1.0 and 0.0 in cb
    out = np.empty(16, dtype=np.float32)
    assert q4.lib().q4_codebook_preset(5, out.ctypes.data_as(ctypes.c_void_p)) == INV
    assert q4.lib().q4_codebook_preset(0, None) == INV
