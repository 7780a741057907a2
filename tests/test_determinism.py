"""Bitwise reproducibility and the residual-compensation ablation on the GPU.

The pages report all four gradients bitwise identical over five repeated calls under
fixed execution conditions ("TurboPairFormer ...", arXiv 2610.05854, Abstract).  Here
every reduction has a fixed order and there are no floating-point atomics, so five
calls must agree bit for bit on every output.
"""
import numpy as np
import pytest
import torch

import oracle
from tri_synth import WORKLOADS, make_inputs, workload_inputs

from ._util import f64, inputs64, rrmse, run_gpu

pytestmark = pytest.mark.gpu

OUTS = ("o", "lse", "res", "dq", "dk", "dv", "dbias")


def _five_calls_identical(inp):
    first = run_gpu(inp)
    for _ in range(4):
        again = run_gpu(inp)
        for n in OUTS:
            assert torch.equal(first[n].view(torch.uint8) if first[n].dtype != torch.float32 else first[n].view(torch.int32),
                               again[n].view(torch.uint8) if again[n].dtype != torch.float32 else again[n].view(torch.int32)), n


@pytest.mark.parametrize("shape", [(1, 64, 4, 16), (1, 200, 2, 32), (2, 130, 3, 16)])
def test_five_calls_bitwise_small(shape):
    B, N, H, D = shape
    _five_calls_identical(make_inputs(B, N, H, D, seed=N, bias_std=4.0))


def test_five_calls_bitwise_wide_bias_768():
    # crop 768, d = 16, bias ~ N(0, 4^2): the workload the reproducibility claim is checked on
    _five_calls_identical(workload_inputs(WORKLOADS["n768_h4_d16_bias4"]))


@pytest.mark.parametrize("name", ["n768_h4_d32", "n640_h4_d16_mask64"])
def test_five_calls_bitwise_full_size(name):
    # the other full-size workloads (both head dimensions, with and without the key mask), each
    # kernel at the benchmark's launch configuration
    _five_calls_identical(workload_inputs(WORKLOADS[name]))


def test_compensation_ablation_small():
    """dv does not depend on the correction D, so it is bitwise identical with and without the
    residual; the gradients that do (dq, dk, dbias) are reported against FP64 both ways."""
    inp = make_inputs(1, 128, 4, 32, seed=11, bias_std=1.0)
    a = run_gpu(inp, residual=True)
    b = run_gpu(inp, residual=False)
    assert torch.equal(a["dv"].view(torch.int16), b["dv"].view(torch.int16))
    assert torch.equal(a["o"].view(torch.int16), b["o"].view(torch.int16))
    x = inputs64(inp)
    dq64, dk64, _, db64 = oracle.backward64(x["q"], x["k"], x["v"], x["bias"], x["dO"])
    with_r = dict(dq=rrmse(f64(a["dq"]), dq64), dk=rrmse(f64(a["dk"]), dk64), dbias=rrmse(f64(a["dbias"]), db64))
    without = dict(dq=rrmse(f64(b["dq"]), dq64), dk=rrmse(f64(b["dk"]), dk64), dbias=rrmse(f64(b["dbias"]), db64))
    print("rel-RMSE with residual", with_r, "without", without, flush=True)
    # the compensated correction must not be worse on the gradient that sees D most directly
    assert with_r["dbias"] <= without["dbias"]


def test_bitwise_with_concurrent_work_on_another_stream():
    """Results do not depend on what else the GPU runs: the same call while another stream keeps
    the device busy with unrelated products (both streams at the default priority)."""
    inp = make_inputs(1, 200, 2, 32, seed=5, bias_std=2.0)
    ref = run_gpu(inp)
    x = torch.randn(2048, 2048, device="cuda")
    side, main = torch.cuda.Stream(), torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    main.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        y = x
        for _ in range(40):
            y = torch.tanh(y @ x)  # float32, contiguous operands
    with torch.cuda.stream(main):
        out = run_gpu(inp)
    torch.cuda.synchronize()
    assert torch.isfinite(y).all()
    for n in OUTS:
        a, b = ref[n], out[n]
        va = a.view(torch.int32) if a.dtype == torch.float32 else a.view(torch.int16)
        vb = b.view(torch.int32) if b.dtype == torch.float32 else b.view(torch.int16)
        assert torch.equal(va, vb), n
