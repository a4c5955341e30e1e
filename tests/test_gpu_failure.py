"""Launch-failure injection through the C ABI.

The library's test hook Q4_TEST_FAIL_LAUNCH=<kernel>[:count] makes the next
`count` launches of one kernel report a HIP failure before anything is
launched (the host-forced failure pattern of the hipBLASLt int8 cache pull
request).  Each case runs in a child process (the hook reads its variable
once per process) and checks: the call returns Q4_ERR_HIP with a message
naming the kernel, the output is untouched, and the next call succeeds with
the right result.
"""
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

CHILD = r'''
import sys
import numpy as np
import torch
import bit_dequant_skinny_amd as q4
import oracle, synth
sys.path.insert(0, "tests")
from gpu_util import assert_within_tolerance, bf16_host, host_f64, q4_to_dev, to_dev

case = sys.argv[1]
dev = torch.device("cuda:0")
M, N, K, bs = 3, 80, 512, 64
p = synth.q4_problem(M, N, K, bs, config=70)
A, Wp, am, cb = q4_to_dev(p)

def expect_failure(fn, out, kernel):
    before = out.clone()
    try:
        fn()
    except q4.Q4Error as e:
        assert e.status == q4.Q4_ERR_HIP, e.status
        assert kernel in str(e) and "injected" in str(e), str(e)
    else:
        raise AssertionError("no failure reported")
    torch.cuda.synchronize()
    assert torch.equal(out, before), "output written by a failed call"

if case in ("fused", "dequant_split", "gemm_split"):
    path = "fused" if case == "fused" else "split"
    kernel = {"fused": "fused", "dequant_split": "dequant", "gemm_split": "gemm"}[case]
    C = torch.full((M, N), 7.0, dtype=torch.bfloat16, device=dev)
    expect_failure(lambda: q4.q4_gemm_skinny(A, Wp, am, cb, bs, out=C, path=path), C, kernel)
    q4.q4_gemm_skinny(A, Wp, am, cb, bs, out=C, path=path)
    torch.cuda.synchronize()
    Cr, S = oracle.q4_gemm(p["A"], p["Wpacked"], p["absmax"], p["codebook"], M, N, K, bs)
    assert_within_tolerance(bf16_host(C), Cr, S, case)
elif case in ("plane_sum", "planes"):
    # fp32 activations: 3 tokens have their planes summed inside the skinny
    # kernel (launches "planes", "fused"); 6 go through fp32 partials and the
    # plane sum (launches "planes", "fused", "plane sum")
    Mp = 6 if case == "plane_sum" else M
    A32 = synth.activations(Mp, K, 71, "fp32")
    C = torch.full((Mp, N), 7.0, dtype=torch.float32, device=dev)
    dA = to_dev(A32, "f32")
    expect_failure(lambda: q4.q4_gemm_skinny(dA, Wp, am, cb, bs, out=C, out_dtype=torch.float32),
                   C, "plane sum" if case == "plane_sum" else "planes")
    q4.q4_gemm_skinny(dA, Wp, am, cb, bs, out=C, out_dtype=torch.float32)
    torch.cuda.synchronize()
    Cr, S = oracle.q4_gemm_ex(A32, "fp32", p["Wpacked"], p["absmax"], p["codebook"], Mp, N, K, bs)
    assert_within_tolerance(None, Cr, S, case, out="fp32", values=host_f64(C))
elif case == "dequant":
    out = torch.full((N, K), 3.0, dtype=torch.bfloat16, device=dev)
    expect_failure(lambda: q4.q4_dequant(Wp, am, cb, bs, out=out), out, "dequant")
    q4.q4_dequant(Wp, am, cb, bs, out=out)
    torch.cuda.synchronize()
    ref = oracle.dequant_bf16(p["Wpacked"], p["absmax"], p["codebook"], N, K, bs)
    assert np.array_equal(bf16_host(out), ref)
elif case == "gemm":
    W = to_dev(synth.bf16_weights(N, K, 72), "bf16")
    C = torch.full((M, N), 5.0, dtype=torch.bfloat16, device=dev)
    expect_failure(lambda: q4.bf16_gemm_skinny(A, W, None, out=C), C, "gemm")
    q4.bf16_gemm_skinny(A, W, None, out=C)
    C2 = q4.bf16_gemm_skinny(A, W, None)
    torch.cuda.synchronize()
    assert torch.equal(C, C2)
else:
    raise SystemExit("unknown case " + case)
print("ok", case)
'''

CASES = {
    "fused": "fused:1",
    "dequant_split": "dequant:1",
    "gemm_split": "gemm:1",
    "plane_sum": "plane sum:1",
    "planes": "planes:1",
    "dequant": "dequant:1",
    "gemm": "gemm:1",
}


@pytest.mark.parametrize("case", sorted(CASES))
def test_injected_launch_failure_and_recovery(case):
    env = dict(os.environ)
    env["Q4_TEST_FAIL_LAUNCH"] = CASES[case]
    env["PYTHONPATH"] = ROOT + os.pathsep + env.get("PYTHONPATH", "")
    r = subprocess.run([sys.executable, "-c", CHILD, case], cwd=ROOT, env=env,
                       capture_output=True, text=True, timeout=240)
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-4000:]
    assert ("ok " + case) in r.stdout


WS_CHILD = r'''
import sys
import numpy as np
import torch
import bit_dequant_skinny_amd as q4
import oracle, synth
sys.path.insert(0, "tests")
from gpu_util import assert_within_tolerance, bf16_host, q4_to_dev

side = torch.cuda.Stream()
bs = 64
small = synth.q4_problem(4, 64, 512, bs, config=71)
big = synth.q4_problem(4, 512, 2048, bs, config=72)
As, Wps, ams, cbs = q4_to_dev(small)
Ab, Wpb, amb, cbb = q4_to_dev(big)
with torch.cuda.stream(side):
    q4.q4_gemm_skinny(As, Wps, ams, cbs, bs, path="split")  # workspace sized for the small shape
torch.cuda.synchronize()
out = torch.zeros((4, 512), dtype=torch.bfloat16, device="cuda:0")
g = torch.cuda.CUDAGraph()
err = None
with torch.cuda.graph(g, stream=side):
    try:
        q4.q4_gemm_skinny(Ab, Wpb, amb, cbb, bs, path="split", out=out)
    except q4.Q4Error as e:
        err = e
assert err is not None and err.status == q4.Q4_ERR_HIP, err
assert "captured" in str(err), str(err)
torch.cuda.synchronize()
assert torch.count_nonzero(out).item() == 0, "output written by a refused call"
with torch.cuda.stream(side):
    q4.q4_gemm_skinny(Ab, Wpb, amb, cbb, bs, path="split", out=out)
torch.cuda.synchronize()
Cr, S = oracle.q4_gemm_w16(big["A"], big["Wpacked"], big["absmax"], big["codebook"], 4, 512, 2048, bs)
assert_within_tolerance(bf16_host(out), Cr, S, "split after a refused capture")
# now the workspace is large enough: the same call can be captured and replayed
g2 = torch.cuda.CUDAGraph()
out2 = torch.zeros_like(out)
with torch.cuda.graph(g2, stream=side):
    q4.q4_gemm_skinny(Ab, Wpb, amb, cbb, bs, path="split", out=out2)
for _ in range(3):
    out2.zero_()
    torch.cuda.synchronize()
    g2.replay()
    torch.cuda.synchronize()
    assert torch.equal(out2, out)
q4.q4_release_workspace()
print("OK")
'''


def test_workspace_growth_during_capture_is_refused():
    """A call that would grow its stream's workspace while the stream is
    being captured returns Q4_ERR_HIP (no allocation can be captured) and
    launches nothing; the same call run eagerly afterwards is correct, and
    once the workspace is large enough the call captures and replays."""
    r = subprocess.run([sys.executable, "-c", WS_CHILD], cwd=ROOT, capture_output=True, text=True,
                       timeout=300)
    assert r.returncode == 0 and "OK" in r.stdout, r.stdout + r.stderr
