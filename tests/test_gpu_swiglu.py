"""GPU parity of the gated-MLP epilogue: SwiGLU of the gate_up projection,
quantized to MXFP4 (CEIL) for the down projection, both fused into the FP4
GEMM (mx_gemm_swiglu_quant) and standalone (mx_swiglu_quant).

SwiGLU runs on the hardware exp2 and reciprocal, and the oracle evaluates it
in fp64, so codes near a rounding boundary may legitimately differ.  Every
output is therefore checked to be the CEIL MXFP4 quantization of some h
within a derived bound of the oracle's exact h (helpers
check_mxfp4_ceil_intervals), at least 98% of codes and scales must equal the
quantization of the oracle's h rounded to bf16, and the fused and unfused
GPU paths must agree bit for bit.  Sources: vLLM's fused gate_up_proj
(Qwen3.8-27B-MXFP8Attn-MXFP4MLP-lmheadMXFP4, section 2) and the per-token
CEIL activation rule (Qwen3.5-9B-MXFP4-QAD-W4A4-LR1e-5-s3000, "Training
mode")."""
import sys

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from helpers import check_mxfp4_ceil_intervals, cuda_bf16, half_ulp_bf16, host

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

import fp8_quantized_linear_amd as mxl  # noqa: E402


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def bf16_bits_of(x: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.asarray(x, np.float64)).to(torch.float32).to(torch.bfloat16) \
        .view(torch.int16).numpy().view(np.uint16)


def bits_to_f64(b: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.ascontiguousarray(b).view(np.int16)).view(torch.bfloat16).double().numpy()


def swiglu_tol(g, u, dg, du):
    """Bound on |h_gpu - h| for h = swiglu(g, u) exact, when the GPU starts
    from gate and up within dg, du of g, u: |silu'| <= 1.1 carries the input
    error; the fp32 chain adds |g| * 2^-24 relative through the rounded exp2
    argument plus a few ulp (taken as 2^-20 + |g| 2^-23); a reciprocal
    that flushes a subnormal result (1 + e^-g > 2^126) to zero adds up to
    |g u| 2^-126; the final bf16 rounding adds half a bf16 ulp (of a bound on
    |h_gpu|)."""
    h = oracle.swiglu(g, u)
    sil = np.abs(oracle.swiglu(g, 1.0))
    t = 1.1 * dg * (np.abs(u) + du) + sil * du
    t = t + np.abs(h) * (2.0 ** -20 + np.abs(g) * 2.0 ** -23)
    t = t + (np.abs(g) + dg) * (np.abs(u) + du) * 2.0 ** -125
    return h, t + half_ulp_bf16(2 * (np.abs(h) + t))


def check(q, s, h, tol, what, min_exact=0.98):
    check_mxfp4_ceil_intervals(q, s, h - tol, h + tol, what)
    rq, rs = oracle.mx_quantize("e2m1", "ceil", bf16_bits_of(h))
    frac_q = float((q == rq).mean())
    frac_s = float((s == rs).mean())
    say(f"{what}: code bytes equal {frac_q:.5f}, scales equal {frac_s:.5f}")
    assert frac_q >= min_exact and frac_s >= min_exact, what


def gpu_q(fn, *args, **kw):
    q, s = fn(*args, **kw)
    torch.cuda.synchronize()
    return host(q), host(s)


def test_standalone_against_oracle():
    rng = np.random.default_rng(60)
    m, inter = 96, 160
    g = rng.standard_normal((m, inter)) * 3
    u = rng.standard_normal((m, inter))
    g[0] = np.linspace(-120, 120, inter)     # exp2 overflow (zero), saturation to g * u
    g[1, :32] = 0.0
    u[2, :32] = 0.0
    g[3] *= 1e-30                            # tiny gate: h ~ g * u / 2
    u[4, 32:64] *= 1e20
    gb, ub = bf16_bits_of(g), bf16_bits_of(u)
    x = np.concatenate([gb, ub], axis=1)
    q, s = gpu_q(mxl.mx_swiglu_quant, cuda_bf16(x))
    h, tol = swiglu_tol(bits_to_f64(gb), bits_to_f64(ub), 0.0, 0.0)
    check(q, s, h, tol, "standalone")


def _pack_gate_up(m, inter, k, seed):
    rng = np.random.default_rng(seed)
    a = bf16_bits_of(rng.standard_normal((m, k)))
    w = bf16_bits_of(rng.standard_normal((2 * inter, k)) * 0.05)
    aq, a_s = mxl.mx_quantize_act(cuda_bf16(a), "mxfp4", "ceil")
    wq, ws = mxl.mx_pack_weights(cuda_bf16(w), "mxfp4", "even")
    return a, w, aq, a_s, wq, ws


@pytest.mark.parametrize("m,inter,k", [(300, 160, 512), (17, 96, 384), (256, 640, 256)])
def test_fused_against_oracle(m, inter, k):
    say(f"fused swiglu m={m} inter={inter} k={k}")
    a, w, aq, a_s, wq, ws = _pack_gate_up(m, inter, k, 61)
    q, s = gpu_q(mxl.mx_gemm_swiglu_quant, aq, a_s, mxl.interleave_gate_up(wq), mxl.interleave_gate_up(ws), k)
    oaq, oas = oracle.mx_quantize("e2m1", "ceil", a)
    owq, ows = oracle.mx_quantize("e2m1", "even", w)
    _, gate, up, sg, su = oracle.mlp_swiglu(oaq, oas, owq, ows, m, inter, k)
    dg = 1e-4 * sg + half_ulp_bf16(2 * (np.abs(gate) + 1e-4 * sg))
    du = 1e-4 * su + half_ulp_bf16(2 * (np.abs(up) + 1e-4 * su))
    h, tol = swiglu_tol(gate, up, dg, du)
    check(q, s, h, tol, f"fused {m}x{inter}x{k}")


@pytest.mark.parametrize("m,inter,k", [(1024, 640, 512), (1100, 608, 384)])
def test_fused_equals_unfused(m, inter, k):
    say(f"fused vs unfused m={m} inter={inter} k={k}")
    assert "prefill" in mxl.mx_gemm_plan("mxfp4", "mxfp4", m, 2 * inter, k)
    _, _, aq, a_s, wq, ws = _pack_gate_up(m, inter, k, 62)
    y = mxl.mx_gemm(aq, a_s, wq, ws, k)
    q0, s0 = gpu_q(mxl.mx_swiglu_quant, y)
    q1, s1 = gpu_q(mxl.mx_gemm_swiglu_quant, aq, a_s, mxl.interleave_gate_up(wq), mxl.interleave_gate_up(ws), k)
    assert np.array_equal(s0, s1) and np.array_equal(q0, q1)


def test_mlp_workload_sampled_rows():
    cfg = W.MLP_GATE_UP
    inter = cfg.n // 2
    say(f"mlp gate_up {cfg.name}: plan {mxl.mx_gemm_swiglu_quant_plan(cfg.m, inter, cfg.k)}")
    a_bits, w_bits = cfg.activations(), cfg.weights()
    aq, a_s = mxl.mx_quantize_act(cuda_bf16(a_bits), "mxfp4", "ceil")
    wq, ws = mxl.mx_pack_weights(cuda_bf16(w_bits), "mxfp4", "even")
    q, s = gpu_q(mxl.mx_gemm_swiglu_quant, aq, a_s, mxl.interleave_gate_up(wq), mxl.interleave_gate_up(ws), cfg.k)
    # unfused on the same GPU: bit for bit
    y = mxl.mx_gemm(aq, a_s, wq, ws, cfg.k)
    q0, s0 = gpu_q(mxl.mx_swiglu_quant, y)
    del y
    assert np.array_equal(s0, s) and np.array_equal(q0, q)
    rows = np.unique(np.concatenate([np.random.default_rng(5).integers(0, cfg.m, 10), [0, cfg.m - 1]]))
    oaq, oas = oracle.mx_quantize("e2m1", "ceil", np.ascontiguousarray(a_bits[rows]))
    owq, ows = oracle.mx_quantize("e2m1", "even", w_bits)
    _, gate, up, sg, su = oracle.mlp_swiglu(oaq, oas, owq, ows, len(rows), inter, cfg.k)
    dg = 1e-4 * sg + half_ulp_bf16(2 * (np.abs(gate) + 1e-4 * sg))
    du = 1e-4 * su + half_ulp_bf16(2 * (np.abs(up) + 1e-4 * su))
    h, tol = swiglu_tol(gate, up, dg, du)
    check(q[rows], s[rows], h, tol, "mlp sampled rows")
