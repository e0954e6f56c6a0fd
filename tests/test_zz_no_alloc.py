"""mx_gemm_noalloc, the allocation-free variant of mx_gemm: split-K partials
go to the library's static device scratch instead of a caller workspace.
Called through the C ABI (ctypes) and checked against mx_gemm with a
workspace (bitwise: same kernels, same split) and against the oracle (the
GEMM bound), on two calls in a row, the second with a smaller input, so the
second call runs on the scratch the first one left behind."""
import ctypes

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from helpers import check_gemm, cuda_bf16, host

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

import fp8_quantized_linear_amd as mxl  # noqa: E402

FMT = {"mxfp4": 0, "mxfp8": 1}
ELEM = {"mxfp4": "e2m1", "mxfp8": "e4m3"}
W_RULE = {"mxfp4": "even", "mxfp8": "floor"}
P = ctypes.c_void_p


def call_noalloc(fmt, aq, as_, wq, ws, m, n, k, y, f32):
    stream = P(torch.cuda.current_stream().cuda_stream)
    return mxl.lib.mx_gemm_noalloc(FMT[fmt], FMT[fmt], P(aq.data_ptr()), P(as_.data_ptr()), P(wq.data_ptr()),
                                   P(ws.data_ptr()), m, n, k, P(y.data_ptr()), 1 if f32 else 0, stream)


@pytest.mark.parametrize("fmt,big,small", [("mxfp4", (300, 2048, 200), (100, 1024, 130)),
                                           ("mxfp8", (300, 2048, 200), (64, 5120, 96))])
def test_noalloc_matches_mx_gemm(fmt, big, small):
    for (m, k, n) in (big, small):
        need = mxl.mx_gemm_workspace_size(fmt, fmt, m, n, k)
        print(f"noalloc {fmt} {m}x{k}x{n}: split-K partials {need} B of scratch", flush=True)
        assert 0 < need <= (24 << 20)
        a_bits = W.activations_entry_outliers(m, k)
        w_bits = W.normal_bf16(n, k, 0.02, 1)
        aq, as_ = mxl.mx_quantize_act(cuda_bf16(a_bits), fmt, "ceil")
        wq, wsc = mxl.mx_pack_weights(cuda_bf16(w_bits), fmt, W_RULE[fmt])
        raq, ras = oracle.mx_quantize(ELEM[fmt], "ceil", a_bits)
        rwq, rws = oracle.mx_quantize(ELEM[fmt], W_RULE[fmt], w_bits)
        y_ref, s = oracle.gemm_dq(oracle.mx_dequantize(ELEM[fmt], raq, ras, m, k),
                                  oracle.mx_dequantize(ELEM[fmt], rwq, rws, n, k))
        for f32 in (False, True):
            y = torch.empty((m, n), dtype=torch.float32 if f32 else torch.bfloat16, device="cuda")
            assert call_noalloc(fmt, aq, as_, wq, wsc, m, n, k, y, f32) == 0
            y_ws = mxl.mx_gemm(aq, as_, wq, wsc, k, fmt, fmt, out_f32=f32)   # with a workspace
            torch.cuda.synchronize()
            assert torch.equal(y, y_ws), f"{fmt} {m}x{k}x{n} f32={f32}: noalloc != mx_gemm with a workspace"
            yh = host(y.float()) if not f32 else host(y)
            check_gemm(yh, y_ref, s, not f32, f"noalloc {fmt} {m}x{k}x{n} f32={f32}")


def test_noalloc_without_split():
    # a shape whose tiles fill the GPU needs no scratch: same as mx_gemm
    m, k, n = 1100, 1152, 1090
    a_bits = W.activations_entry_outliers(m, k)
    w_bits = W.normal_bf16(n, k, 0.02, 1)
    aq, as_ = mxl.mx_quantize_act(cuda_bf16(a_bits))
    wq, wsc = mxl.mx_pack_weights(cuda_bf16(w_bits))
    y = mxl.mx_gemm_noalloc(aq, as_, wq, wsc, k)
    torch.cuda.synchronize()
    assert torch.equal(y, mxl.mx_gemm(aq, as_, wq, wsc, k))
