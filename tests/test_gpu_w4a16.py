"""GPU parity of the weight-only mode (mx_gemm_w4a16): bf16 activations times
packed MXFP4 or NVFP4 weights, against the oracle's fp64 product of the
activations with the dequantized weights (oracle.w4a16_gemm).

The weights are packed on the GPU and must equal the oracle's packing byte
for byte; the product is then checked per element with the GEMM bound of
helpers.check_gemm (1e-4 * sum_k |a_k dq(w)_k|, plus half a bf16 ulp for
bf16 output).  Shapes cover the decode kernel (M <= 16, K % 512 == 0, ragged
N) and the general kernel (larger M, K with a partial last stage, NVFP4 K %
32 == 16); the decode configuration is checked on sampled columns."""
import sys

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


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def pack(w_bits, fmt):
    w = cuda_bf16(w_bits)
    if fmt == "mxfp4":
        wq, ws = mxl.mx_pack_weights(w, fmt="mxfp4", rule="even")
        rq, rs = oracle.mx_quantize("e2m1", "even", w_bits)
        g = None
    else:
        g = oracle.nv_global_scale(oracle.bf16_amax(w_bits))
        wq, ws = mxl.mx_pack_weights(w, fmt="nvfp4", global_scale=float(g))
        rq, rs = oracle.nv_quantize(w_bits, g)
    torch.cuda.synchronize()
    assert np.array_equal(host(wq), rq) and np.array_equal(host(ws), rs), "packing differs from the oracle"
    return wq, ws, rq, rs, g


def alpha_of(g):
    return 1.0 if g is None else float(np.float32(1.0) / np.float32(g))


CASES = [
    # per-wave streamed decode kernel: M <= 2, K % 1024 == 0, LDS within 64 KiB
    (1, 1024, 300), (2, 5120, 100), (1, 6144, 33), (2, 3072, 17),
    # two-group streamed decode kernel: M <= 16, K % 1024 == 0, K <= 8192,
    # where the one above does not fit (M > 2; NVFP4 at (2, 5120) and (1, 6144))
    (3, 1024, 100), (8, 2048, 33), (16, 5120, 200), (5, 8192, 70), (12, 3072, 31), (16, 1024, 32),
    # decode kernel: M <= 16, K % 512 == 0
    (1, 512, 16), (16, 512, 300), (9, 1536, 48),
    # general kernel
    (17, 512, 130), (130, 96, 257), (200, 416, 300), (64, 1056, 64),
]


@pytest.mark.parametrize("fmt", ["mxfp4", "nvfp4"])
@pytest.mark.parametrize("m,k,n", CASES)
def test_w4a16_full(fmt, m, k, n):
    plan = mxl.mx_gemm_w4a16_plan(fmt, m, n, k)
    say(f"w4a16 {fmt} m={m} k={k} n={n}: {plan}")
    # the streamed kernel holds W codes, A and the W scale block in 64 KiB of LDS
    lds = 16 * (k // 2) + m * k * 2 + 16 * (k // (16 if fmt == "nvfp4" else 32))
    if m <= 2 and k % 1024 == 0 and lds <= 65536:
        assert "w4a16_decode_stream_kernel<" in plan
    elif m <= 16 and k % 1024 == 0 and k <= 8192:
        assert "w4a16_decode_stream2_kernel<" in plan
    elif m <= 16 and k % 512 == 0:
        assert "w4a16_decode_kernel<" in plan
    a_bits = W.activations_entry_outliers(m, k)
    w_bits = W.normal_bf16(n, k, 0.02, 1)
    wq, ws, rq, rs, g = pack(w_bits, fmt)
    y_ref, s = oracle.w4a16_gemm(a_bits, rq, rs, n, k, fmt, g)
    a = cuda_bf16(a_bits)
    for out_f32 in (False, True):
        y = mxl.mx_gemm_w4a16(a, wq, ws, fmt, alpha_of(g), out_f32=out_f32)
        torch.cuda.synchronize()
        yh = host(y.float()) if not out_f32 else host(y)
        check_gemm(yh, y_ref, s, not out_f32, f"w4a16 {fmt} {m}x{k}x{n} f32={out_f32}")


# 4 to 5 sixteen-row W groups per compute unit (NVFP4 from 8 rows of A): one
# workgroup per CU over an even share of them (4 or 5; rows past a share read
# as zero and are not stored), at even (N = 16384) and ragged shares
@pytest.mark.parametrize("fmt,m,n", [("mxfp4", 3, 16384), ("mxfp4", 8, 16400), ("mxfp4", 16, 17408),
                                     ("mxfp4", 5, 20470), ("nvfp4", 8, 16384), ("nvfp4", 9, 16400),
                                     ("nvfp4", 16, 17408), ("nvfp4", 12, 20470)])
def test_w4a16_partitioned(fmt, m, n):
    k = 1024
    plan = mxl.mx_gemm_w4a16_plan(fmt, m, n, k)
    say(f"w4a16 partitioned {fmt} m={m} k={k} n={n}: {plan[:70]}")
    assert "one workgroup per compute unit" in plan
    a_bits = W.activations_entry_outliers(m, k, seed=9 + m)
    w_bits = W.normal_bf16(n, k, 0.02, 10)
    wq, ws, rq, rs, g = pack(w_bits, fmt)
    y_ref, s = oracle.w4a16_gemm(a_bits, rq, rs, n, k, fmt, g)
    a = cuda_bf16(a_bits)
    for out_f32 in (False, True):
        y = mxl.mx_gemm_w4a16(a, wq, ws, fmt, alpha_of(g), out_f32=out_f32)
        torch.cuda.synchronize()
        yh = host(y.float()) if not out_f32 else host(y)
        check_gemm(yh, y_ref, s, not out_f32, f"w4a16 partitioned {fmt} {m}x{k}x{n} f32={out_f32}")


@pytest.mark.parametrize("fmt", ["mxfp4", "nvfp4"])
def test_w4a16_nvfp4_odd_k_and_small_n(fmt):
    # NVFP4 with K % 32 == 16 and N = 1 (general kernel); MXFP4 with N = 1
    m, k, n = (5, 400, 1) if fmt == "nvfp4" else (5, 96, 1)
    a_bits = W.normal_bf16(m, k, 1.0, 3)
    w_bits = W.normal_bf16(n, k, 0.02, 4)
    wq, ws, rq, rs, g = pack(w_bits, fmt)
    y_ref, s = oracle.w4a16_gemm(a_bits, rq, rs, n, k, fmt, g)
    y = mxl.mx_gemm_w4a16(cuda_bf16(a_bits), wq, ws, fmt, alpha_of(g), out_f32=True)
    torch.cuda.synchronize()
    check_gemm(host(y), y_ref, s, False, f"w4a16 {fmt} {m}x{k}x{n}")


@pytest.mark.parametrize("fmt", ["mxfp4", "nvfp4"])
@pytest.mark.parametrize("m", [1, 8])
def test_w4a16_decode_config_sampled(fmt, m):
    # the decode-shaped projection (K = 5120, N = 17408) on 512 sampled columns
    cfg = [c for c in W.DECODE if c.m == m][0]
    a_bits, w_bits = cfg.activations(), cfg.weights()
    k, n = cfg.k, cfg.n
    w = cuda_bf16(w_bits)
    if fmt == "mxfp4":
        wq, ws = mxl.mx_pack_weights(w, fmt="mxfp4", rule="even")
        g = None
    else:
        g = oracle.nv_global_scale(oracle.bf16_amax(w_bits))
        wq, ws = mxl.mx_pack_weights(w, fmt="nvfp4", global_scale=float(g))
    y = mxl.mx_gemm_w4a16(cuda_bf16(a_bits), wq, ws, fmt, alpha_of(g))
    torch.cuda.synchronize()
    say(f"w4a16 decode {fmt} m={m}: {mxl.mx_gemm_w4a16_plan(fmt, m, n, k)}")
    rng = np.random.default_rng(7)
    cols = np.unique(np.concatenate([rng.choice(n, 500, replace=False), [0, 15, 16, n - 16, n - 1]]))
    wsub = w_bits[cols]
    if fmt == "mxfp4":
        rq, rs = oracle.mx_quantize("e2m1", "even", wsub)
    else:
        rq, rs = oracle.nv_quantize(wsub, g)
    assert np.array_equal(host(wq)[cols], rq) and np.array_equal(host(ws)[cols], rs)
    y_ref, s = oracle.w4a16_gemm(a_bits, rq, rs, len(cols), k, fmt, g)
    check_gemm(host(y.float())[:, cols], y_ref, s, True, f"w4a16 decode {fmt} m={m}")


def test_w4a16_equals_w4a4_on_representable_activations():
    # activations that are exactly dequantized MXFP4 values: W4A16 of their
    # bf16 values and W4A4 of their codes compute the same products; both
    # are within the bound of the same exact result, and on the GPU they must
    # agree to fp32 accumulation order
    m, k, n = 16, 1024, 64
    a_bits = W.normal_bf16(m, k, 1.0, 5)
    w_bits = W.normal_bf16(n, k, 0.02, 6)
    a = cuda_bf16(a_bits)
    wq, ws = mxl.mx_pack_weights(cuda_bf16(w_bits), fmt="mxfp4", rule="even")
    aq, as_ = mxl.mx_quantize_act(a, fmt="mxfp4", rule="ceil")
    y4 = mxl.mx_gemm(aq, as_, wq, ws, k, "mxfp4", "mxfp4", out_f32=True)
    rq, rs = oracle.mx_quantize("e2m1", "ceil", a_bits)
    ad = oracle.mx_dequantize("e2m1", rq, rs, m, k)
    ad_bits = torch.from_numpy(ad.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    y16 = mxl.mx_gemm_w4a16(cuda_bf16(ad_bits), wq, ws, "mxfp4", out_f32=True)
    torch.cuda.synchronize()
    rqw, rsw = oracle.mx_quantize("e2m1", "even", w_bits)
    assert np.array_equal(host(wq), rqw) and np.array_equal(host(ws), rsw)
    y_ref, s = oracle.w4a16_gemm(ad_bits, rqw, rsw, n, k, "mxfp4")
    check_gemm(host(y16), y_ref, s, False, "w4a16 on representable A")
    check_gemm(host(y4), y_ref, s, False, "w4a4 on the same values")
