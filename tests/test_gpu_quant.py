"""GPU parity of the quantizers (mx_quantize_act / mx_pack_weights, MX and
NVFP4) against the CPU oracle: codes and scale bytes must match bit for bit.

The fuzz case mirrors the quantizer fuzz on the Qwen3.5-9B-MXFP4-QAD card
("Training mode": a GPU fuzz with zero mismatches over 7,248,896 elements):
here at least that many codes, over adversarial blocks, for every rule."""
import sys

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from helpers import cuda_bf16, host

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

import fp8_quantized_linear_amd as mxl  # noqa: E402

ELEM = {"mxfp4": "e2m1", "mxfp8": "e4m3"}


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def gpu_quant(bits, fmt, rule, weights=False, g=1.0):
    x = cuda_bf16(bits)
    fn = mxl.mx_pack_weights if weights else mxl.mx_quantize_act
    q, s = fn(x, fmt=fmt, rule=rule, global_scale=g)
    torch.cuda.synchronize()
    return host(q), host(s)


def assert_same(got, ref, what):
    gq, gs = got
    rq, rs = ref
    assert gs.shape == rs.shape and gq.shape == rq.shape, what
    ms = int((gs != rs).sum())
    mq = int((gq != rq).sum())
    if ms or mq:
        i = np.argwhere(gs != rs)[:3] if ms else np.argwhere(gq != rq)[:3]
        raise AssertionError(f"{what}: {mq} code bytes and {ms} scale bytes differ; first at {i.tolist()}")


@pytest.mark.parametrize("fmt", ["mxfp4", "mxfp8"])
@pytest.mark.parametrize("rule", ["floor", "ceil", "even"])
def test_small_config_and_ragged(fmt, rule):
    cases = [W.SMALL.activations(), W.SMALL.weights(),
             W.normal_bf16(1, 32, 1.0, 3), W.normal_bf16(3, 96, 5.0, 4),
             W.normal_bf16(7, 2080, 1.0, 5), W.fuzz_bf16(5, 4128, seed=11)]
    for i, bits in enumerate(cases):
        say(f"quant {fmt} {rule} case {i} shape {bits.shape}")
        assert_same(gpu_quant(bits, fmt, rule), oracle.mx_quantize(ELEM[fmt], rule, bits),
                    f"{fmt}/{rule} case {i}")


@pytest.mark.parametrize("fmt,rule", [("mxfp4", "ceil"), ("mxfp4", "even"), ("mxfp4", "floor"),
                                      ("mxfp8", "floor"), ("mxfp8", "ceil"), ("mxfp8", "even")])
def test_fuzz_corpus(fmt, rule):
    bits = W.fuzz_bf16(1024, 7168, seed=2024)  # 7,340,032 codes per rule
    say(f"fuzz {fmt} {rule} {bits.size} elements")
    got = gpu_quant(bits, fmt, rule)
    ref = oracle.mx_quantize(ELEM[fmt], rule, bits)
    assert_same(got, ref, f"fuzz {fmt}/{rule}")
    assert bits.size >= 7_248_896


def test_pack_and_quantize_are_the_same_operation():
    bits = W.fuzz_bf16(8, 1024, seed=5)
    a = gpu_quant(bits, "mxfp4", "even", weights=True)
    b = gpu_quant(bits, "mxfp4", "even", weights=False)
    assert_same(a, b, "pack vs quantize")


@pytest.mark.parametrize("cfg,which,fmt,rule", [
    (W.DECODE[2], "a", "mxfp4", "ceil"),
    (W.DECODE[0], "w", "mxfp4", "even"),
    (W.PREFILL_UP, "a", "mxfp4", "ceil"),
    (W.PREFILL_DOWN, "a", "mxfp4", "ceil"),
    (W.PREFILL_DOWN, "w", "mxfp4", "even"),
    (W.MXFP8_ATTN, "a", "mxfp8", "ceil"),
    (W.MXFP8_ATTN, "w", "mxfp8", "floor"),
])
def test_full_size_configs(cfg, which, fmt, rule):
    bits = cfg.activations() if which == "a" else cfg.weights()
    say(f"full {cfg.name} {which} {bits.shape} {fmt}/{rule}")
    assert_same(gpu_quant(bits, fmt, rule, weights=which == "w"),
                oracle.mx_quantize(ELEM[fmt], rule, bits), f"{cfg.name} {which}")


def test_vocab_weights_sampled_rows():
    cfg = W.MXFP4_VOCAB
    bits = cfg.weights()
    say(f"vocab weights {bits.shape}")
    gq, gs = gpu_quant(bits, "mxfp4", "even", weights=True)
    rows = np.unique(np.concatenate([np.random.default_rng(1).integers(0, cfg.n, 2048),
                                     [0, cfg.n - 1]]))
    rq, rs = oracle.mx_quantize("e2m1", "even", np.ascontiguousarray(bits[rows]))
    assert_same((gq[rows], gs[rows]), (rq, rs), "vocab weights sampled rows")


def test_amax_and_nvfp4_quantization():
    cfg = W.NVFP4
    # activation global scale: running max over the 8 calibration batches
    run = 0.0
    for b in cfg.calibration_batches():
        amax_gpu = float(mxl.mx_tensor_amax(cuda_bf16(b)).item())
        assert amax_gpu == oracle.bf16_amax(b)
        run = max(run, amax_gpu)
    g_a = mxl.mx_nv_global_scale(run)
    assert np.float32(g_a) == oracle.nv_global_scale(run)
    a_bits, w_bits = cfg.activations(), cfg.weights()
    g_w = mxl.mx_nv_global_scale(float(mxl.mx_tensor_amax(cuda_bf16(w_bits)).item()))
    for bits, g, weights in ((a_bits, g_a, False), (w_bits, g_w, True)):
        say(f"nvfp4 quant {bits.shape} g={g}")
        assert_same(gpu_quant(bits, "nvfp4", "ceil", weights=weights, g=g),
                    oracle.nv_quantize(bits, g), "nvfp4")
    # adversarial blocks and several global scales, including ones that push
    # block scales into E4M3 subnormals and saturation
    fz = W.fuzz_bf16(64, 1024, seed=9)
    for g in (1.0, 0.37, 1e5, 3.0e-3, float(oracle.nv_global_scale(oracle.bf16_amax(fz)))):
        assert_same(gpu_quant(fz, "nvfp4", "ceil", g=g), oracle.nv_quantize(fz, g), f"nvfp4 g={g}")
    ragged = W.normal_bf16(3, 48, 2.0, 6)
    assert_same(gpu_quant(ragged, "nvfp4", "ceil", g=7.0), oracle.nv_quantize(ragged, 7.0), "ragged")
    # elements on the E2M1 midpoints of exact E4M3 block scales and one bf16
    # step either side (the encoder's fallback decides these)
    for g in (1.0, 0.5, 64.0, 2.0 ** -30):
        tb = W.nvfp4_tie_bf16(64, 1024, g, seed=12)
        assert_same(gpu_quant(tb, "nvfp4", "ceil", g=g), oracle.nv_quantize(tb, g), f"nvfp4 ties g={g}")


def test_nvfp4_quantization_large_fuzz():
    # 4M adversarial elements under global scales across the whole range,
    # plus normal data under its own scale: every code and scale bit for bit
    # (the encoder's fast roundings and its exact fallback alike)
    fz = W.fuzz_bf16(1024, 4096, seed=31)
    rng = np.random.default_rng(5)
    gs = [1.0, 0.37, 3.7e-3, 2.5e4, 1e-20, 1e20] + [float(v) for v in np.exp(rng.uniform(-30, 30, 4))]
    for g in gs:
        g = float(np.float32(g))
        say(f"nvfp4 quant fuzz 1024x4096 g={g:.4g}")
        assert_same(gpu_quant(fz, "nvfp4", "ceil", g=g), oracle.nv_quantize(fz, g), f"nvfp4 fuzz g={g}")
    nb = W.normal_bf16(1024, 4096, 1.0, 32)
    g = float(oracle.nv_global_scale(oracle.bf16_amax(nb)))
    assert_same(gpu_quant(nb, "nvfp4", "ceil", g=g), oracle.nv_quantize(nb, g), "nvfp4 normal")


def test_deterministic():
    bits = W.fuzz_bf16(64, 2048, seed=3)
    a = gpu_quant(bits, "mxfp4", "ceil")
    b = gpu_quant(bits, "mxfp4", "ceil")
    assert_same(a, b, "repeat")
