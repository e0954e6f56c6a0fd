"""GPU parity of the fake-quantization op (mx_fake_quant: the serving
quantizer's codes, dequantized, rounded once to bf16) against the CPU oracle,
bit for bit, for MXFP4 / MXFP8 under every scale rule and for NVFP4 under
several global scales.  Training runs this op on weights (EVEN) and per-token
activations (CEIL) of every quantized linear
(Qwen3.5-27B-MXFP4-QAD-W4A4-LR1e-5-s1000, "How this checkpoint was produced",
Training row; Qwen3.5-9B-MXFP4-QAD-W4A4-LR1e-5-s3000, "Training mode")."""
import sys

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from helpers import bf16_bits, cuda_bf16, double_rounding_trap_scales, host

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

import fp8_quantized_linear_amd as mxl  # noqa: E402

ELEM = {"mxfp4": "e2m1", "mxfp8": "e4m3"}


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def gpu_fake(bits, fmt, rule, g=1.0):
    y = mxl.mx_fake_quant(cuda_bf16(bits), fmt, rule, g)
    torch.cuda.synchronize()
    return bf16_bits(y)


def assert_bits(got, ref, what):
    assert got.shape == ref.shape, what
    bad = got != ref
    if bad.any():
        i = np.argwhere(bad)[:4].tolist()
        raise AssertionError(f"{what}: {int(bad.sum())} of {got.size} differ; first at {i}: "
                             f"got {[hex(int(got[tuple(j)])) for j in i]} "
                             f"want {[hex(int(ref[tuple(j)])) for j in i]}")


def edge_rows(k: int) -> np.ndarray:
    """Rows that reach the op's edge cases: bf16 subnormal inputs (clamped
    scales, subnormal outputs), values near the bf16 maximum (dequantized
    values beyond it become infinity under CEIL), zeros of both signs."""
    rng = np.random.default_rng(31)
    x = rng.standard_normal((4, k)).astype(np.float32)
    x[0] *= np.float32(1e-39)
    x[1] = np.clip(rng.standard_normal(k), -3.3, 3.3) * np.float32(1e38)   # finite in bf16
    x[1, ::32] = np.float32(3.3e38)
    x[2] = 0.0
    x[2, 1::2] = -0.0
    x[3, : k // 2] *= np.float32(1e-30)
    return torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


@pytest.mark.parametrize("fmt", ["mxfp4", "mxfp8"])
@pytest.mark.parametrize("rule", ["floor", "ceil", "even"])
def test_mx_small_ragged_and_edges(fmt, rule):
    cases = [W.SMALL.activations(), W.SMALL.weights(), W.normal_bf16(1, 32, 1.0, 3),
             W.normal_bf16(7, 2080, 1.0, 5), W.fuzz_bf16(5, 4128, seed=11), edge_rows(8224)]
    for i, bits in enumerate(cases):
        say(f"fake {fmt} {rule} case {i} shape {bits.shape}")
        assert_bits(gpu_fake(bits, fmt, rule), oracle.fake_quant(fmt, rule, bits), f"{fmt}/{rule} case {i}")


@pytest.mark.parametrize("fmt,rule", [("mxfp4", "ceil"), ("mxfp4", "even"), ("mxfp8", "ceil")])
def test_mx_fuzz_corpus(fmt, rule):
    bits = W.fuzz_bf16(1024, 7168, seed=2024)
    say(f"fake fuzz {fmt} {rule} {bits.size} elements")
    assert_bits(gpu_fake(bits, fmt, rule), oracle.fake_quant(fmt, rule, bits), f"fuzz {fmt}/{rule}")


def test_nvfp4_global_scales_and_traps():
    fz = W.fuzz_bf16(64, 1024, seed=9)
    traps = double_rounding_trap_scales(4)
    # blocks whose scale is 1 and whose second element codes to 1 under a trap
    # scale g: the output is the single rounding of 1/g, which an fp32 quotient
    # rounded again to bf16 gets wrong
    tb = np.zeros((2, 64), np.float32)
    for j, g in enumerate(traps):
        tb[:, 16 * j] = 6.0 / float(g)
        tb[:, 16 * j + 1] = -1.0 / float(g)
        tb[1, 16 * j + 2] = 3.0 / float(g)
    tbits = torch.from_numpy(tb).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    for g in (1.0, 0.37, 1e5, 3.0e-3, 3.0e30, float(oracle.nv_global_scale(oracle.bf16_amax(fz)))):
        say(f"fake nvfp4 fuzz g={g}")
        assert_bits(gpu_fake(fz, "nvfp4", None, g), oracle.fake_quant("nvfp4", None, fz, g), f"nvfp4 g={g}")
    for g in traps:
        say(f"fake nvfp4 trap g={g}")
        assert_bits(gpu_fake(tbits, "nvfp4", None, g), oracle.fake_quant("nvfp4", None, tbits, g),
                    f"nvfp4 trap g={g}")
    ragged = W.normal_bf16(3, 48, 2.0, 6)
    assert_bits(gpu_fake(ragged, "nvfp4", None, 7.0), oracle.fake_quant("nvfp4", None, ragged, 7.0), "ragged")
    e = edge_rows(1040)
    assert_bits(gpu_fake(e, "nvfp4", None, 0.5), oracle.fake_quant("nvfp4", None, e, 0.5), "edges")
    for g in (1.0, 0.5, 64.0, 2.0 ** -30):
        tb = W.nvfp4_tie_bf16(64, 1024, g, seed=13)
        say(f"fake nvfp4 ties g={g}")
        assert_bits(gpu_fake(tb, "nvfp4", None, g), oracle.fake_quant("nvfp4", None, tb, g), f"nvfp4 ties g={g}")


def test_nvfp4_fake_large_fuzz():
    # the fake quantization's bracketed bf16 rounding over 4M adversarial
    # elements and global scales across the range
    fz = W.fuzz_bf16(1024, 4096, seed=33)
    rng = np.random.default_rng(6)
    gs = [1.0, 0.37, 3.7e-3, 2.5e4, 1e-20, 1e20] + [float(v) for v in np.exp(rng.uniform(-30, 30, 4))]
    for g in gs:
        g = float(np.float32(g))
        say(f"fake nvfp4 fuzz 1024x4096 g={g:.4g}")
        assert_bits(gpu_fake(fz, "nvfp4", None, g), oracle.fake_quant("nvfp4", None, fz, g), f"nvfp4 fuzz g={g}")


def test_nvfp4_workload():
    cfg = W.NVFP4
    a_bits = cfg.activations()
    amax = float(mxl.mx_tensor_amax(cuda_bf16(a_bits)).item())
    g = mxl.mx_nv_global_scale(amax)
    say(f"fake nvfp4 {cfg.name} activations {a_bits.shape} g={g}")
    got = gpu_fake(a_bits, "nvfp4", None, g)
    rows = np.unique(np.concatenate([np.random.default_rng(2).integers(0, a_bits.shape[0], 256),
                                     [0, a_bits.shape[0] - 1]]))
    assert_bits(got[rows], oracle.fake_quant("nvfp4", None, np.ascontiguousarray(a_bits[rows]), g),
                "nvfp4 sampled rows")


@pytest.mark.parametrize("cfg,which,fmt,rule", [
    (W.PREFILL_UP, "a", "mxfp4", "ceil"),
    (W.PREFILL_DOWN, "w", "mxfp4", "even"),
])
def test_full_size_sampled_rows(cfg, which, fmt, rule):
    bits = cfg.activations() if which == "a" else cfg.weights()
    say(f"fake full {cfg.name} {which} {bits.shape} {fmt}/{rule}")
    got = gpu_fake(bits, fmt, rule)
    rows = np.unique(np.concatenate([np.random.default_rng(3).integers(0, bits.shape[0], 512),
                                     [0, bits.shape[0] - 1]]))
    assert_bits(got[rows], oracle.fake_quant(fmt, rule, np.ascontiguousarray(bits[rows])),
                f"{cfg.name} {which} sampled rows")


def test_same_codes_as_the_serving_quantizer():
    """The fake output decodes from exactly the codes mx_quantize_act writes:
    re-deriving it test-side from those codes (E2M1 table times 2^(s-127),
    fp64, then bf16) gives the same patterns."""
    bits = W.fuzz_bf16(32, 2048, seed=41)
    x = cuda_bf16(bits)
    q, s = mxl.mx_quantize_act(x, "mxfp4", "ceil")
    q, s = host(q), host(s)
    lat = np.array([0, .5, 1, 1.5, 2, 3, 4, 6, -0.0, -.5, -1, -1.5, -2, -3, -4, -6])
    codes = np.stack([q & 0xF, q >> 4], axis=-1).reshape(q.shape[0], -1)
    val = lat[codes] * np.ldexp(1.0, np.repeat(s.astype(np.int64) - 127, 32, axis=1))
    want = torch.from_numpy(val).to(torch.float32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert_bits(gpu_fake(bits, "mxfp4", "ceil"), want, "fake vs serving codes")


def test_straight_through_gradient_and_errors():
    x = cuda_bf16(W.normal_bf16(4, 64, 1.0, 8)).requires_grad_(True)
    y = mxl.FakeQuantSTE.apply(x, "mxfp4", "ceil", 1.0)
    g = torch.randn_like(y)
    y.backward(g)
    assert torch.equal(x.grad, g)
    with pytest.raises(mxl.MXError):
        mxl.mx_fake_quant(cuda_bf16(W.normal_bf16(2, 48, 1.0, 9)), "mxfp4", "ceil")
    xx = cuda_bf16(W.normal_bf16(2, 64, 1.0, 9))
    with pytest.raises(mxl.MXError):
        mxl.mx_fake_quant(xx, "mxfp4", "ceil", out=xx)   # in place is rejected
