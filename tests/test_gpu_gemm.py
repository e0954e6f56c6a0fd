"""GPU parity of the GEMMs (mx_gemm, mx_gemm_fused, nv_gemm) against the CPU
oracle's fp64 product of the dequantized operands.

Bound per element (stated in helpers.check_gemm): |y - y_ref| <= 1e-4 *
sum_k |a_k w_k|, plus half a bf16 ulp when Y is written as bf16.  Full-size
configurations are checked on sampled outputs (random pairs plus tile-edge
rows and columns), computed one by one by the oracle from the quantized rows;
smaller shapes that still span several tiles and a ragged tail are checked in
full."""
import sys

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from helpers import check_gemm, cuda_bf16, flushed_terms, host, sample_pairs, underflow_allowance

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

import fp8_quantized_linear_amd as mxl  # noqa: E402

ELEM = {"mxfp4": "e2m1", "mxfp8": "e4m3"}
W_RULE = {"mxfp4": "even", "mxfp8": "floor"}


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def run_mx(a_bits, w_bits, fmt="mxfp4", out_f32=False, fused=False):
    a, w = cuda_bf16(a_bits), cuda_bf16(w_bits)
    k = a_bits.shape[1]
    wq, ws = mxl.mx_pack_weights(w, fmt=fmt, rule=W_RULE[fmt])
    aq, as_ = mxl.mx_quantize_act(a, fmt=fmt, rule="ceil")
    y = mxl.mx_gemm(aq, as_, wq, ws, k, fmt, fmt, out_f32=out_f32, split_k=False)
    yf = mxl.mx_gemm_fused(a, wq, ws, fmt, "ceil", fmt, out_f32=out_f32) if fused else None
    torch.cuda.synchronize()
    return y, yf, (aq, as_), (wq, ws)


def oracle_full(a_bits, w_bits, fmt):
    m, k = a_bits.shape
    n = w_bits.shape[0]
    aq, as_ = oracle.mx_quantize(ELEM[fmt], "ceil", a_bits)
    wq, ws = oracle.mx_quantize(ELEM[fmt], W_RULE[fmt], w_bits)
    ad = oracle.mx_dequantize(ELEM[fmt], aq, as_, m, k)
    wd = oracle.mx_dequantize(ELEM[fmt], wq, ws, n, k)
    y, s = oracle.gemm_dq(ad, wd)
    return y, s, (aq, as_), (wq, ws)


def y_host(y):
    return host(y.float()) if y.dtype == torch.bfloat16 else host(y)


SHAPES = [(16, 256, 256), (200, 416, 300), (1, 32, 1), (129, 160, 257), (33, 5120, 96),
          (64, 1056, 130), (260, 384, 520)]


@pytest.mark.parametrize("fmt", ["mxfp4", "mxfp8"])
@pytest.mark.parametrize("m,k,n", SHAPES)
def test_gemm_full_small_shapes(fmt, m, k, n):
    say(f"gemm {fmt} m={m} k={k} n={n}")
    a_bits = W.activations_entry_outliers(m, k)
    w_bits = W.normal_bf16(n, k, 0.02, 1)
    y_ref, s, (raq, ras), (rwq, rws) = oracle_full(a_bits, w_bits, fmt)
    for out_f32 in (False, True):
        y, yf, (aq, as_), (wq, ws) = run_mx(a_bits, w_bits, fmt, out_f32=out_f32, fused=True)
        assert np.array_equal(host(aq), raq) and np.array_equal(host(as_), ras)
        assert np.array_equal(host(wq), rwq) and np.array_equal(host(ws), rws)
        check_gemm(y_host(y), y_ref, s, not out_f32, f"{fmt} {m}x{k}x{n} f32={out_f32}")
        # the fused prologue quantizes exactly like the standalone quantizer
        # and feeds the same matrix-core sequence: bitwise equal outputs
        # (both unsplit)
        assert torch.equal(y, yf), "fused != standalone"
        # the default call, which splits K where the tiles leave the GPU idle
        ys = mxl.mx_gemm(aq, as_, wq, ws, k, fmt, fmt, out_f32=out_f32)
        torch.cuda.synchronize()
        check_gemm(y_host(ys), y_ref, s, not out_f32, f"{fmt} {m}x{k}x{n} f32={out_f32} split-K default")


@pytest.mark.parametrize("m,k,n", [(129, 160, 257), (200, 416, 300), (33, 5120, 96)])
def test_mxfp8_fast_path_within_its_documented_bound(m, k, n):
    # MX_FP8_FAST contracts on the FP8 matrix cores, whose internal
    # accumulation is inexact (measured up to ~2e-4 * sum|a*b|); its
    # documented bound is 5e-4 * sum|a*b|.  The default path must meet 1e-4.
    a_bits = W.activations_entry_outliers(m, k)
    w_bits = W.normal_bf16(n, k, 0.02, 1)
    y_ref, s, _, _ = oracle_full(a_bits, w_bits, "mxfp8")
    a, w = cuda_bf16(a_bits), cuda_bf16(w_bits)
    wq, ws = mxl.mx_pack_weights(w, fmt="mxfp8", rule="floor")
    aq, as_ = mxl.mx_quantize_act(a, fmt="mxfp8", rule="ceil")
    y = mxl.mx_gemm(aq, as_, wq, ws, k, "mxfp8", "mxfp8", out_f32=True, fp8_fast=True, split_k=False)
    ys = mxl.mx_gemm(aq, as_, wq, ws, k, "mxfp8", "mxfp8", out_f32=True, fp8_fast=True)
    yf = mxl.mx_gemm_fused(a, wq, ws, "mxfp8", "ceil", "mxfp8", out_f32=True, fp8_fast=True)
    torch.cuda.synchronize()
    # scale the error down by 5 so that check_gemm's 1e-4 bound reads as 5e-4
    rel = check_gemm(0.2 * (y_host(y) - y_ref) + y_ref, y_ref, s, False, f"fast fp8 {m}x{k}x{n}")
    check_gemm(0.2 * (y_host(ys) - y_ref) + y_ref, y_ref, s, False, f"fast fp8 {m}x{k}x{n} split-K default")
    assert torch.equal(y, yf)
    say(f"fast fp8 {m}x{k}x{n}: max err/S = {rel * 5.0:.2e}")


def test_integer_exact_tiny():
    # lattice-valued operands with unit scales: every partial sum is an exact
    # binary fraction, so the fp32 result must equal the oracle exactly
    rng = np.random.default_rng(8)
    lat = np.array([0, .5, 1, 1.5, 2, 3, 4, 6], np.float32)
    for (m, k, n) in [(16, 128, 16), (32, 64, 48), (5, 96, 7)]:
        a = (lat[rng.integers(0, 8, (m, k))] * rng.choice([-1, 1], (m, k))).astype(np.float32)
        w = (lat[rng.integers(0, 8, (n, k))] * rng.choice([-1, 1], (n, k))).astype(np.float32)
        # each block holds a 4, so its max is 4 or 6 and every rule picks
        # scale 2^0: the codes are the lattice values themselves
        a[:, ::32] = 4.0
        w[:, ::32] = 4.0
        ab, wb = W._to_bf16_bits(a), W._to_bf16_bits(w)
        y_ref, s, _, _ = oracle_full(ab, wb, "mxfp4")
        y, _, _, _ = run_mx(ab, wb, "mxfp4", out_f32=True)
        assert np.array_equal(y_host(y), y_ref.astype(np.float32)), (m, k, n)


# Exact MXFP8 dequantization inside the GEMM, read back through a selection
# matrix: W row n holds the code of 1.0 (scale 2^0) at position n and zeros
# elsewhere, so Y[m, n] = dequant(A)[m, n] with a single product.  A takes every
# finite E4M3 code and scale exponents from -127 upwards.  The kernels hold
# operands in bf16: every value must come back as the bf16 nearest to the
# oracle's exact dequantized value (ties to even), which is the value itself
# from 2^-126 up and a rounded bf16 subnormal below.  The rounding is torch's
# fp32 -> bf16 conversion of the exact value (exact in fp32: 4 significant
# bits, at least 2^-136).  K = 256 takes the 128 x 128 kernel's scales as
# aligned dwords (K % 128 == 0), K = 160 as bytes; 4352 x 4096 x 4096 runs the
# 256 x 256 tile kernel (256 tiles and 16 tail halves).
@pytest.mark.parametrize("m,k", [(96, 256), (96, 160), (4352, 4096)])
def test_mxfp8_exact_dequantization_by_selection(m, k):
    plan = mxl.mx_gemm_plan("mxfp8", "mxfp8", m, k, k)
    say(f"mxfp8 selection {m}x{k}x{k}: {plan[:60]}")
    if m > 1024:
        assert "mx8_gemm_tile_kernel" in plan
    rng = np.random.default_rng(31)
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8)   # finite E4M3
    aq = codes[rng.integers(0, codes.size, (m, k))]
    a_s = rng.choice(np.array([0, 0, 0, 1, 2, 5, 9, 100, 127, 130], np.uint8), (m, k // 32))
    a_s[0, :] = 0                                   # a whole row of 2^-127 blocks
    wq = np.zeros((k, k), np.uint8)
    wq[np.arange(k), np.arange(k)] = 0x38            # E4M3 1.0
    ws = np.full((k, k // 32), 127, np.uint8)
    ad = oracle.mx_dequantize("e4m3", aq, a_s, m, k)
    ad32 = ad.astype(np.float32)
    assert np.array_equal(ad32.astype(np.float64), ad)
    want = torch.from_numpy(ad32).to(torch.bfloat16).float().numpy().astype(np.float64)
    normal = np.abs(ad) >= 2.0 ** -126
    assert normal.any() and (~normal & (ad != 0)).any() and (~normal & (want != ad)).any()
    dev = torch.device("cuda")
    y = mxl.mx_gemm(torch.from_numpy(aq).to(dev), torch.from_numpy(a_s).to(dev), torch.from_numpy(wq).to(dev),
                    torch.from_numpy(ws).to(dev), k, "mxfp8", "mxfp8", out_f32=True, split_k=False)
    torch.cuda.synchronize()
    yh = host(y).astype(np.float64)
    tiny = ~normal & (ad != 0)
    say(f"  {int(normal.sum())} normal-range values, {int((normal & (yh == ad)).sum())} exact; "
        f"{int(tiny.sum())} nonzero values below 2^-126: {int((tiny & (yh == want)).sum())} equal to the "
        f"nearest bf16, {int((tiny & (yh == 0)).sum())} zero")
    bad = np.argwhere(yh != want)
    assert bad.size == 0, f"{bad.shape[0]} values differ from the nearest bf16, first at {bad[0]}: " \
                          f"{yh[tuple(bad[0])]} vs {want[tuple(bad[0])]} (exact {ad[tuple(bad[0])]}, " \
                          f"code {aq[tuple(bad[0])]:#x}, scale byte {a_s[bad[0][0], bad[0][1] // 32]})"


def test_decode_shapes_full():
    for cfg in W.DECODE:
        say(f"decode {cfg.name}")
        a_bits, w_bits = cfg.activations(), cfg.weights()
        y_ref, s, _, _ = oracle_full(a_bits, w_bits, "mxfp4")
        y, yf, _, _ = run_mx(a_bits, w_bits, "mxfp4", fused=True)
        check_gemm(y_host(y), y_ref, s, True, cfg.name)
        assert torch.equal(y, yf)


# Decode-shaped calls (M <= 32 here) pick one of four kernels by K: per-wave
# streamed K quarters (K % 1024 == 0, K <= 8192; whole quarters in LDS for
# M <= 8 where they fit, else a ring of pair slots), whole-row LDS blocks (other
# K % 512 == 0 while the block fits 64 KiB of LDS), K-chunked direct loads
# (other K % 128 == 0) and the generic split-K kernel.  Each is checked in
# full against the oracle at ragged N and at the edges of its K range.
DECODE_KINDS = [("mx_decode_stream_kernel<", 1024), ("mx_decode_stream_kernel<", 5120),
                ("mx_decode_stream_kernel<", 6144), ("mx_decode_stream_kernel<", 8192),
                ("mx_decode_kernel<", 512), ("mx_decode_kernel<", 6656), ("mx_decode_kernel<", 2560),
                ("mx_decode_direct_kernel<", 384), ("mx_decode_direct_kernel<", 3200),
                ("mx_decode_direct_kernel<", 16384),
                ("mx_decode_generic_kernel<", 96), ("mx_decode_generic_kernel<", 4128)]


@pytest.mark.parametrize("m", [1, 8, 17, 32])
@pytest.mark.parametrize("kernel,k", DECODE_KINDS)
def test_decode_kernel_kinds(kernel, k, m):
    n = 300 if k <= 8192 else 70
    say(f"decode kind {kernel} m={m} k={k} n={n}")
    assert mxl.mx_gemm_plan("mxfp4", "mxfp4", m, n, k).split(" ", 1)[1].startswith(kernel)
    a_bits = W.activations_entry_outliers(m, k, seed=3 + m)
    w_bits = W.normal_bf16(n, k, 0.02, 4)
    y_ref, s, _, _ = oracle_full(a_bits, w_bits, "mxfp4")
    for out_f32 in (False, True):
        y, _, _, _ = run_mx(a_bits, w_bits, "mxfp4", out_f32=out_f32)
        check_gemm(y_host(y), y_ref, s, not out_f32, f"{kernel} {m}x{k}x{n} f32={out_f32}")


# M = 9 .. 32 with 4 to 5 sixteen-row W groups per compute unit: one
# workgroup per CU over an even share of the groups (4 or 5 each; rows past a
# workgroup's share read as zero and are not stored).  Full outputs against
# the oracle at even shares (N = 16384, 20480) and ragged ones.
@pytest.mark.parametrize("m", [9, 16, 17, 32])
@pytest.mark.parametrize("n", [16384, 16400, 17408, 20470])
def test_decode_partitioned(m, n):
    k = 1024
    plan = mxl.mx_gemm_plan("mxfp4", "mxfp4", m, n, k)
    say(f"decode partitioned m={m} k={k} n={n}: {plan[:70]}")
    assert "one workgroup per compute unit" in plan
    a_bits = W.activations_entry_outliers(m, k, seed=5 + m)
    w_bits = W.normal_bf16(n, k, 0.02, 6)
    y_ref, s, _, _ = oracle_full(a_bits, w_bits, "mxfp4")
    for out_f32 in (False, True):
        y, _, _, _ = run_mx(a_bits, w_bits, "mxfp4", out_f32=out_f32)
        check_gemm(y_host(y), y_ref, s, not out_f32, f"decode partitioned {m}x{k}x{n} f32={out_f32}")


# M = 33 .. 48 runs the decode kernels with three 16-row A fragments (the
# whole-row LDS block where it fits 64 KiB, else the generic kernel).
@pytest.mark.parametrize("m", [33, 40, 48])
@pytest.mark.parametrize("k", [512, 5120, 6656, 384, 4128])
def test_decode_wide_m(m, k):
    n = 300
    plan = mxl.mx_gemm_plan("mxfp4", "mxfp4", m, n, k)
    say(f"decode wide m={m} k={k} n={n}: {plan[:60]}")
    assert plan.split(" ", 1)[1].startswith("mx_decode")
    a_bits = W.activations_entry_outliers(m, k, seed=3 + m)
    w_bits = W.normal_bf16(n, k, 0.02, 4)
    y_ref, s, _, _ = oracle_full(a_bits, w_bits, "mxfp4")
    for out_f32 in (False, True):
        y, _, _, _ = run_mx(a_bits, w_bits, "mxfp4", out_f32=out_f32)
        check_gemm(y_host(y), y_ref, s, not out_f32, f"decode wide {m}x{k}x{n} f32={out_f32}")


def sampled_check(cfg, fmt, fused=True, count=4096):
    a_bits, w_bits = cfg.activations(), cfg.weights()
    say(f"sampled {cfg.name}: generated inputs")
    y, yf, (aq, as_), (wq, ws) = run_mx(a_bits, w_bits, fmt, fused=fused)
    mi, ni = sample_pairs(cfg.m, cfg.n, count)
    ur, ir = np.unique(mi, return_inverse=True)
    uc, ic = np.unique(ni, return_inverse=True)
    raq, ras = oracle.mx_quantize(ELEM[fmt], "ceil", np.ascontiguousarray(a_bits[ur]))
    rwq, rws = oracle.mx_quantize(ELEM[fmt], W_RULE[fmt], np.ascontiguousarray(w_bits[uc]))
    assert np.array_equal(host(aq)[ur], raq) and np.array_equal(host(as_)[ur], ras)
    assert np.array_equal(host(wq)[uc], rwq) and np.array_equal(host(ws)[uc], rws)
    ad = oracle.mx_dequantize(ELEM[fmt], raq, ras, len(ur), cfg.k)
    wd = oracle.mx_dequantize(ELEM[fmt], rwq, rws, len(uc), cfg.k)
    y_ref, s = oracle.gemm_dq_pairs(ad, wd, ir, ic)
    yv = y[torch.from_numpy(mi).cuda(), torch.from_numpy(ni).cuda()]
    check_gemm(y_host(yv), y_ref, s, True, cfg.name)
    if fused:
        assert torch.equal(y, yf), f"{cfg.name}: fused != standalone"
    return y


def test_prefill_up_sampled():
    sampled_check(W.PREFILL_UP, "mxfp4")


def test_prefill_down_sampled():
    sampled_check(W.PREFILL_DOWN, "mxfp4")


def test_mxfp8_attention_sampled():
    sampled_check(W.MXFP8_ATTN, "mxfp8")


def test_vocab_projection_sampled():
    sampled_check(W.MXFP4_VOCAB, "mxfp4", fused=False)


# The prefill kernel on shapes that reach its edges: an odd number of 128-K
# sub-stages (K % 256 == 128, a half pair at the end), ragged M and N, a main
# launch with no tail, a tail-only launch, and a main launch plus a tail.
# Sampled outputs against the oracle, bf16 and fp32 output.
PREFILL_EDGE = [
    ("odd sub-stages, main only", 2148, 1408, 4146),      # 9 x 17 = 153 tiles: no tail
    ("tail only", 1024, 1152, 1100),                      # 4 x 5 = 20 tiles: all as halves
    ("main + tail", 1300, 2560, 33000),                   # 6 x 129 = 774 tiles: 6 tail tiles
]


@pytest.mark.parametrize("what,m,k,n", PREFILL_EDGE)
def test_prefill_kernel_edges(what, m, k, n):
    assert mxl.mx_gemm_plan("mxfp4", "mxfp4", m, n, k).split(" ", 1)[1].startswith("mx_gemm_prefill_kernel<")
    cfg = W.Gemm(f"prefill edge {what}", m, k, n)
    y = sampled_check(cfg, "mxfp4", fused=False, count=3000)
    a_bits, w_bits = cfg.activations(), cfg.weights()
    _, _, (aq, as_), (wq, ws) = run_mx(a_bits, w_bits, "mxfp4", fused=False)
    yf = mxl.mx_gemm(aq, as_, wq, ws, k, out_f32=True)
    # the bf16 output is the RNE of the fp32 one, element by element
    assert torch.equal(yf.to(torch.bfloat16), y)


# Full-output parity of the headline prefill kernels: every element of Y
# against the oracle, on shapes whose tile grid takes both launches (a main
# launch of 256 x 256 tiles and a tail launch of 256 x 128 halves), for the
# standalone GEMM and for the quantize-once fused path, bf16 and fp32 output.
# The first shape has one 256-K pair per tile; the second has ragged M and N,
# 4.5 pairs (two scale windows, a half pair at the end) and ragged last tiles.
PREFILL_FULL = [("one pair, main + tail", 2048, 256, 10240),
                ("ragged, 4.5 pairs, main + tail", 4300, 1152, 4000)]


def prefill_launches(m: int, n: int):
    """Tiles of the main and of the tail launch, as the library splits them
    for this GPU's compute-unit count."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    t = ((m + 255) // 256) * ((n + 255) // 256)
    rem = t % cus
    tail = rem if rem and 2 * rem <= cus else 0
    return t - tail, tail


@pytest.mark.parametrize("what,m,k,n", PREFILL_FULL)
def test_prefill_full_output(what, m, k, n):
    main, tail = prefill_launches(m, n)
    say(f"prefill full output {what}: {m}x{k}x{n}, {main} main tiles + {tail} tail tiles")
    assert main > 0 and tail > 0
    assert mxl.mx_gemm_plan("mxfp4", "mxfp4", m, n, k).split(" ", 1)[1].startswith("mx_gemm_prefill_kernel<")
    assert "mx_gemm_prefill_fq_kernel" in mxl.mx_gemm_plan("mxfp4", "mxfp4", m, n, k, fused=True, in_gemm=True)
    a_bits = W.activations_entry_outliers(m, k)
    w_bits = W.normal_bf16(n, k, 0.02, 1)
    y_ref, s, (raq, ras), (rwq, rws) = oracle_full(a_bits, w_bits, "mxfp4")
    a, w = cuda_bf16(a_bits), cuda_bf16(w_bits)
    wq, wsc = mxl.mx_pack_weights(w, "mxfp4", "even")
    aq, as_ = mxl.mx_quantize_act(a, "mxfp4", "ceil")
    wsz = mxl.mx_gemm_fused_workspace_size("mxfp4", "mxfp4", m, n, k, in_gemm=True)
    assert wsz > 0
    for out_f32 in (False, True):
        y = mxl.mx_gemm(aq, as_, wq, wsc, k, out_f32=out_f32)
        ws = torch.empty(wsz, dtype=torch.uint8, device="cuda")
        yq = mxl.mx_gemm_fused(a, wq, wsc, "mxfp4", "ceil", "mxfp4", out_f32=out_f32, workspace=ws,
                               in_gemm=True)
        torch.cuda.synchronize()
        if not out_f32:
            assert np.array_equal(host(aq), raq) and np.array_equal(host(as_), ras)
            assert np.array_equal(host(wq), rwq) and np.array_equal(host(wsc), rws)
        rel = check_gemm(y_host(y), y_ref, s, not out_f32, f"prefill {what} f32={out_f32}")
        check_gemm(y_host(yq), y_ref, s, not out_f32, f"quantize-once {what} f32={out_f32}")
        assert torch.equal(y, yq), "quantize-once != standalone"
        say(f"  f32={out_f32}: max err/S {rel:.2e}")


# Full-output parity of the large-tile exact MXFP8 kernel (at least 256
# tiles of 256 x 256, K % 128 == 0): 4352 x 4096 is 17 x 16 = 272 tiles, a
# main launch and a tail of 16 tiles as 256 x 128 halves; K = 1152 is 9
# pairs of 128 (two scale windows, the second with one pair).  Seeded
# activations with outliers, and fuzz-corpus operands with many tiny blocks
# (scale 2^-127 included); bf16 and fp32 output.  The
# fused call quantizes A into its workspace and runs the same kernel, so it
# is bitwise equal to the standalone pair.
@pytest.mark.parametrize("data", ["outliers", "fuzz"])
def test_mxfp8_tile_full_output(data):
    m, k, n = 4352, 1152, 4096
    main, tail = prefill_launches(m, n)
    plan = mxl.mx_gemm_plan("mxfp8", "mxfp8", m, n, k)
    say(f"mxfp8 tile full output ({data}) {m}x{k}x{n}: {main} + {tail} tiles; {plan[:40]}")
    assert main > 0 and tail > 0 and "mx8_gemm_tile_kernel" in plan
    if data == "fuzz":
        a_bits, w_bits = fuzz_operands(m, k, n)
    else:
        a_bits, w_bits = W.activations_entry_outliers(m, k), W.normal_bf16(n, k, 0.02, 1)
    raq, ras = oracle.mx_quantize("e4m3", "ceil", a_bits)
    rwq, rws = oracle.mx_quantize("e4m3", "floor", w_bits)
    ad = oracle.mx_dequantize("e4m3", raq, ras, m, k)
    wd = oracle.mx_dequantize("e4m3", rwq, rws, n, k)
    y_ref, s = oracle.gemm_dq(ad, wd)
    fl, u = (flushed_terms(ad, wd), underflow_allowance(k)) if data == "fuzz" else (None, 0.0)
    a, w = cuda_bf16(a_bits), cuda_bf16(w_bits)
    aq, as_ = mxl.mx_quantize_act(a, "mxfp8", "ceil")
    wq, wsc = mxl.mx_pack_weights(w, "mxfp8", "floor")
    assert np.array_equal(host(aq), raq) and np.array_equal(host(as_), ras)
    assert np.array_equal(host(wq), rwq) and np.array_equal(host(wsc), rws)
    if data == "fuzz":
        say(f"  blocks with scale 2^-127: A {int((ras == 0).sum())}, W {int((rws == 0).sum())}")
    for out_f32 in (False, True):
        y = mxl.mx_gemm(aq, as_, wq, wsc, k, "mxfp8", "mxfp8", out_f32=out_f32)
        yf = mxl.mx_gemm_fused(a, wq, wsc, "mxfp8", "ceil", "mxfp8", out_f32=out_f32)
        torch.cuda.synchronize()
        rel = check_gemm(y_host(y), y_ref, s, not out_f32, f"mxfp8 tile {data} f32={out_f32}", fl, u)
        assert torch.equal(y, yf), "fused != standalone"
        say(f"  f32={out_f32}: max err/S {rel:.2e}")


# GEMM parity on adversarial operands: fuzz-corpus activations (blocks in
# binades -135 .. 60, E2M1/E4M3 ties, rule thresholds, zero and -0 blocks,
# mixed magnitudes) against fuzz-corpus weights (binades -20 .. 2), so that
# tiny blocks meet large weights and scales reach 2^-127.  Ranges keep every
# product and sum inside fp32.  The contract's bound for operands below the
# fp32 normal range applies: 1e-4 * S, plus the terms with an operand value
# below 2^-126 (helpers.flushed_terms) and an accumulation underflow
# allowance of (K/16 + 1) * 2^-126.  Outputs that needed more than 1e-4 * S
# are counted and printed.
FUZZ_SHAPES = [(200, 416, 300), (1100, 1152, 1090)]     # the second runs the prefill kernel (MXFP4)


def fuzz_operands(m, k, n):
    a_bits = W.fuzz_bf16(m, k, seed=23, emax=60, mix=(-60, 60))
    w_bits = W.fuzz_bf16(n, k, seed=29, emin=-20, emax=2, mix=(-20, 3))
    return a_bits, w_bits


def report_fuzz(what, y, y_ref, s, fl, bf16_out):
    yv = y_host(y).astype(np.float64)
    err = np.abs(yv - y_ref)
    beyond = int((err > 1e-4 * s + (0 if not bf16_out else np.abs(y_ref) * 2.0 ** -8)).sum())
    say(f"  {what}: {beyond} outputs beyond 1e-4*S; flushed-term allowance nonzero at "
        f"{int((fl > 0).sum())} of {fl.size}")


@pytest.mark.parametrize("fmt", ["mxfp4", "mxfp8"])
@pytest.mark.parametrize("m,k,n", FUZZ_SHAPES)
def test_gemm_fuzz_operands(fmt, m, k, n):
    say(f"fuzz gemm {fmt} {m}x{k}x{n}: {mxl.mx_gemm_plan(fmt, fmt, m, n, k)[:50]}")
    a_bits, w_bits = fuzz_operands(m, k, n)
    aq, as_ = oracle.mx_quantize(ELEM[fmt], "ceil", a_bits)
    wq, ws = oracle.mx_quantize(ELEM[fmt], W_RULE[fmt], w_bits)
    ad = oracle.mx_dequantize(ELEM[fmt], aq, as_, m, k)
    wd = oracle.mx_dequantize(ELEM[fmt], wq, ws, n, k)
    y_ref, s = oracle.gemm_dq(ad, wd)
    fl = flushed_terms(ad, wd)
    u = underflow_allowance(k)
    for out_f32 in (False, True):
        y, yf, (gaq, gas), (gwq, gws) = run_mx(a_bits, w_bits, fmt, out_f32=out_f32, fused=True)
        assert np.array_equal(host(gaq), aq) and np.array_equal(host(gas), as_)
        assert np.array_equal(host(gwq), wq) and np.array_equal(host(gws), ws)
        check_gemm(y_host(y), y_ref, s, not out_f32, f"fuzz {fmt} {m}x{k}x{n} f32={out_f32}", fl, u)
        assert torch.equal(y, yf), "fused != standalone"
        report_fuzz(f"{fmt} f32={out_f32}", y, y_ref, s, fl, not out_f32)


@pytest.mark.parametrize("m,k,n", [(8, 1024, 300), (130, 416, 200)])
@pytest.mark.parametrize("w_fmt", ["mxfp4", "nvfp4"])
def test_w4a16_fuzz_operands(w_fmt, m, k, n):
    a_bits, w_bits = fuzz_operands(m, k, n)
    say(f"fuzz w4a16 {w_fmt} {m}x{k}x{n}: {mxl.mx_gemm_w4a16_plan(w_fmt, m, n, k)[:40]}")
    a = cuda_bf16(a_bits)
    if w_fmt == "mxfp4":
        wq, ws = oracle.mx_quantize("e2m1", "even", w_bits)
        wd = oracle.mx_dequantize("e2m1", wq, ws, n, k)
        g_w, alpha = None, 1.0
    else:
        g_w = oracle.nv_global_scale(oracle.bf16_amax(w_bits))
        wq, ws = oracle.nv_quantize(w_bits, g_w)
        wd = oracle.nv_dequantize(wq, ws, n, k, g_w)
        alpha = float(np.float32(1.0) / np.float32(g_w))
    ad = oracle.bf16_to_f64(a_bits)
    y_ref, s = oracle.gemm_dq(ad, wd)
    # the GEMM consumes the weights before the global scale: e2m1 * s_w
    w_cons = wd if w_fmt == "mxfp4" else wd * float(g_w)
    fl = flushed_terms(ad, w_cons) * (1.0 if w_fmt == "mxfp4" else 1.0 / float(g_w))
    u = underflow_allowance(k)
    dev = torch.device("cuda")
    for out_f32 in (False, True):
        y = mxl.mx_gemm_w4a16(a, torch.from_numpy(wq).to(dev), torch.from_numpy(ws).to(dev), w_fmt, alpha,
                              out_f32=out_f32)
        torch.cuda.synchronize()
        check_gemm(y_host(y), y_ref, s, not out_f32, f"fuzz w4a16 {w_fmt} {m}x{k}x{n} f32={out_f32}", fl, u)
        report_fuzz(f"w4a16 {w_fmt} f32={out_f32}", y, y_ref, s, fl, not out_f32)


def test_nvfp4_fuzz_operands():
    m, k, n = 200, 416, 300
    a_bits, w_bits = fuzz_operands(m, k, n)
    g_a = oracle.nv_global_scale(oracle.bf16_amax(a_bits))
    g_w = oracle.nv_global_scale(oracle.bf16_amax(w_bits))
    aq, as_ = oracle.nv_quantize(a_bits, g_a)
    wq, ws = oracle.nv_quantize(w_bits, g_w)
    y_ref, s = oracle.gemm_dq(oracle.nv_dequantize(aq, as_, m, k, g_a), oracle.nv_dequantize(wq, ws, n, k, g_w))
    u = underflow_allowance(k)
    for out_f32 in (False, True):
        y, (gaq, gas), (gwq, gws) = nv_case(a_bits, w_bits, g_a, g_w, out_f32)
        assert np.array_equal(host(gaq), aq) and np.array_equal(host(gas), as_)
        assert np.array_equal(host(gwq), wq) and np.array_equal(host(gws), ws)
        # e2m1 * s_e4m3 products are exact in f16: no operand leaves its range
        check_gemm(y_host(y), y_ref, s, not out_f32, f"fuzz nvfp4 f32={out_f32}", None, u)


# The quantize-once fused paths (large MXFP4 shapes and exact MXFP8 on the
# 128 x 128 kernel, with a workspace).  By default A is quantized into the
# workspace by the standalone quantizer and mx_gemm's kernel runs; with
# MX_FUSED_IN_GEMM the GEMM's workgroups quantize A once into the workspace
# (claiming 32-row chunks from a pool) and the tiles read the codes from
# there.  Both must leave exactly mx_quantize_act's codes and scales in the
# workspace and give Y bitwise equal to the standalone pair.  For the
# in-GEMM variant:  The workspace
# must then hold exactly mx_quantize_act's codes and scales (which also shows
# that this path ran), the pool and every block's done counter must show all
# chunks, the error word must be clear, and Y must equal both the standalone
# pair and the in-tile prologue bit for bit, for every rule.  The first shape
# has a ragged last block (1100 rows: 76 rows) and only tail tiles (25 tiles
# as 256 x 128 halves), the second a main launch plus a tail, the third odd m
# and odd k/128 (its code plane ends off a cache line, so the scale plane
# starts at the next 256-byte boundary).  The exact MXFP8 GEMM does the same
# with 128-row blocks (1100 rows: a ragged 76-row block).
FQ_CASES = [("mxfp4", 1100, 1152, 1090), ("mxfp4", 1300, 2560, 33000), ("mxfp4", 1025, 1152, 1090),
            ("mxfp8", 1100, 1152, 1090), ("mxfp8", 300, 2048, 700), ("mxfp8", 1025, 1152, 1090)]


def up256(v: int) -> int:
    return (v + 255) // 256 * 256


@pytest.mark.parametrize("fmt,m,k,n", FQ_CASES)
def test_fused_quantize_once(fmt, m, k, n):
    wsz = mxl.mx_gemm_fused_workspace_size(fmt, fmt, m, n, k, in_gemm=True)
    qsz = mxl.mx_gemm_fused_workspace_size(fmt, fmt, m, n, k)
    say(f"fused quantize-once {fmt} m={m} k={k} n={n}: workspace {wsz} B in the GEMM, {qsz} B via the quantizer")
    assert wsz > 0 and qsz == m * (k // 2 if fmt == "mxfp4" else k) + m * k // 32
    a_bits = W.activations_entry_outliers(m, k)
    w_bits = W.normal_bf16(n, k, 0.02, 1)
    a, w = cuda_bf16(a_bits), cuda_bf16(w_bits)
    wq, wsc = mxl.mx_pack_weights(w, fmt=fmt, rule=W_RULE[fmt])
    cpr = k // 2 if fmt == "mxfp4" else k           # code bytes per row
    bm = 256 if fmt == "mxfp4" else 128             # rows per block
    qb, sb = m * cpr, m * k // 32
    so = up256(qb)                                  # scale plane offset
    cnt = up256(so + sb)                            # state offset
    for rule in ("ceil", "floor", "even"):
        for out_f32 in (False, True):
            ws = torch.full((wsz,), 0xA5, dtype=torch.uint8, device="cuda")
            y = mxl.mx_gemm_fused(a, wq, wsc, fmt, rule, fmt, out_f32=out_f32, workspace=ws, in_gemm=True)
            wsq = torch.full((qsz,), 0x5A, dtype=torch.uint8, device="cuda")
            yq = mxl.mx_gemm_fused(a, wq, wsc, fmt, rule, fmt, out_f32=out_f32, workspace=wsq)
            aq, as_ = mxl.mx_quantize_act(a, fmt, rule)
            y_ref = mxl.mx_gemm(aq, as_, wq, wsc, k, fmt, fmt, out_f32=out_f32, split_k=False)
            y_tile = mxl.mx_gemm_fused(a, wq, wsc, fmt, rule, fmt, out_f32=out_f32, quantize_once=False)
            torch.cuda.synchronize()
            assert torch.equal(wsq[:qb].view(m, cpr), aq) and torch.equal(wsq[qb:].view(m, k // 32), as_), \
                f"{rule}: quantizer-path workspace"
            assert torch.equal(yq, y_ref), f"{rule} f32={out_f32}: quantizer path != standalone"
            assert torch.equal(ws[:qb].view(m, cpr), aq), f"{rule}: workspace codes"
            assert torch.equal(ws[so:so + sb].view(m, k // 32), as_), f"{rule}: workspace scales"
            nb = (m + bm - 1) // bm
            st = ws[cnt:cnt + 4 * (nb + 2)].view(torch.int32).cpu().numpy()
            assert st[0] >= (bm // 32) * nb, "chunk pool"
            assert np.all(st[1:nb + 1] == bm // 32), "done counters"
            assert st[nb + 1] == 0, "error word"
            assert torch.equal(y, y_ref), f"{rule} f32={out_f32}: quantize-once != standalone"
            assert torch.equal(y, y_tile), f"{rule} f32={out_f32}: quantize-once != in-tile prologue"
    rq, rs = oracle.mx_quantize(ELEM[fmt], "even", a_bits)
    assert np.array_equal(host(ws[:qb].view(m, cpr)), rq) and np.array_equal(host(ws[so:so + sb].view(m, k // 32)), rs)


# Mixed MX pairs (MXFP8 activations with MXFP4 weights and the reverse):
# the default path dequantizes each operand exactly to bf16 (bound 1e-4 * S),
# MX_FP8_FAST runs the block-scaled FP8 x FP4 matrix cores (documented bound
# 5e-4 * S), and mx_gemm_fused quantizes A into its workspace and runs the
# same GEMM (bitwise equal to mx_quantize_act + unsplit mx_gemm).  Full
# outputs against the oracle, ragged shapes, both K tilings (K % 128 == 0
# takes the scales as row dwords) and a split-K shape.
MIXED_SHAPES = [(200, 416, 300), (129, 512, 257), (33, 5120, 96)]


@pytest.mark.parametrize("a_fmt,w_fmt", [("mxfp8", "mxfp4"), ("mxfp4", "mxfp8")])
@pytest.mark.parametrize("m,k,n", MIXED_SHAPES)
def test_mixed_pairs(a_fmt, w_fmt, m, k, n):
    say(f"mixed {a_fmt} x {w_fmt} {m}x{k}x{n}: {mxl.mx_gemm_plan(a_fmt, w_fmt, m, n, k)[:60]}")
    a_bits = W.activations_entry_outliers(m, k)
    w_bits = W.normal_bf16(n, k, 0.02, 1)
    raq, ras = oracle.mx_quantize(ELEM[a_fmt], "ceil", a_bits)
    rwq, rws = oracle.mx_quantize(ELEM[w_fmt], W_RULE[w_fmt], w_bits)
    y_ref, s = oracle.gemm_dq(oracle.mx_dequantize(ELEM[a_fmt], raq, ras, m, k),
                              oracle.mx_dequantize(ELEM[w_fmt], rwq, rws, n, k))
    a, w = cuda_bf16(a_bits), cuda_bf16(w_bits)
    aq, as_ = mxl.mx_quantize_act(a, a_fmt, "ceil")
    wq, wsc = mxl.mx_pack_weights(w, w_fmt, W_RULE[w_fmt])
    for out_f32 in (False, True):
        y = mxl.mx_gemm(aq, as_, wq, wsc, k, a_fmt, w_fmt, out_f32=out_f32)
        y1 = mxl.mx_gemm(aq, as_, wq, wsc, k, a_fmt, w_fmt, out_f32=out_f32, split_k=False)
        yf = mxl.mx_gemm_fused(a, wq, wsc, a_fmt, "ceil", w_fmt, out_f32=out_f32)
        yfast = mxl.mx_gemm(aq, as_, wq, wsc, k, a_fmt, w_fmt, out_f32=True, fp8_fast=True, split_k=False)
        torch.cuda.synchronize()
        check_gemm(y_host(y), y_ref, s, not out_f32, f"mixed {a_fmt}x{w_fmt} {m}x{k}x{n} f32={out_f32}")
        check_gemm(y_host(y1), y_ref, s, not out_f32, f"mixed unsplit {a_fmt}x{w_fmt} f32={out_f32}")
        assert torch.equal(yf, y1), "fused mixed != quantize + unsplit GEMM"
        # the fast path against its documented 5e-4 bound (error scaled by 1/5)
        rel = check_gemm(0.2 * (y_host(yfast) - y_ref) + y_ref, y_ref, s, False, f"mixed fast {a_fmt}x{w_fmt}")
        say(f"  fast path max err/S = {rel * 5:.2e}")


def test_deterministic():
    a_bits = W.activations_entry_outliers(300, 1024)
    w_bits = W.normal_bf16(700, 1024, 0.02, 1)
    y1, _, _, _ = run_mx(a_bits, w_bits)
    y2, _, _, _ = run_mx(a_bits, w_bits)
    assert torch.equal(y1, y2)


# ---------------------------------------------------------------- NVFP4
def nv_case(a_bits, w_bits, g_a, g_w, out_f32=False):
    a, w = cuda_bf16(a_bits), cuda_bf16(w_bits)
    k = a_bits.shape[1]
    aq, as_ = mxl.mx_quantize_act(a, fmt="nvfp4", global_scale=g_a)
    wq, ws = mxl.mx_pack_weights(w, fmt="nvfp4", global_scale=g_w)
    alpha = float(np.float32(1.0) / (np.float32(g_a) * np.float32(g_w)))
    y = mxl.nv_gemm(aq, as_, wq, ws, k, alpha, out_f32=out_f32)
    torch.cuda.synchronize()
    return y, (aq, as_), (wq, ws)


# K % 64 == 0 (scales fetched as row dwords), K % 64 == 32 (byte scales),
# K % 32 == 16 (8-byte aligned rows, a last half chunk)
@pytest.mark.parametrize("m,k,n", [(16, 256, 256), (200, 400, 300), (1, 16, 1), (130, 5120, 96), (64, 288, 100)])
def test_nvfp4_full_small(m, k, n):
    a_bits = W.normal_bf16(m, k, 1.0, 0)
    w_bits = W.normal_bf16(n, k, 0.02, 1)
    g_a = oracle.nv_global_scale(oracle.bf16_amax(a_bits))
    g_w = oracle.nv_global_scale(oracle.bf16_amax(w_bits))
    aq, as_ = oracle.nv_quantize(a_bits, g_a)
    wq, ws = oracle.nv_quantize(w_bits, g_w)
    y_ref, s = oracle.gemm_dq(oracle.nv_dequantize(aq, as_, m, k, g_a),
                              oracle.nv_dequantize(wq, ws, n, k, g_w))
    for out_f32 in (False, True):
        y, (gaq, gas), (gwq, gws) = nv_case(a_bits, w_bits, g_a, g_w, out_f32)
        assert np.array_equal(host(gaq), aq) and np.array_equal(host(gas), as_)
        assert np.array_equal(host(gwq), wq) and np.array_equal(host(gws), ws)
        check_gemm(y_host(y), y_ref, s, not out_f32, f"nvfp4 {m}x{k}x{n}")


# Full-output parity of the 8-wave NVFP4 kernel (at least 256 tiles of 256 x
# 256, K % 256 == 0): 4352 x 4096 is 17 x 16 = 272 tiles, a main launch and
# a tail of 16 tiles as 256 x 128 halves; K = 1280 is 5 pairs of 256 (three
# scale windows of 2 pairs, the last with one).  Normal activations as in
# the NVFP4 workload, and fuzz-corpus operands whose E4M3 block scales reach
# the subnormal ones; bf16 and fp32 output.
@pytest.mark.parametrize("data", ["normal", "fuzz"])
def test_nvfp4_tile_full_output(data):
    m, k, n = 4352, 1280, 4096
    plan = mxl.mx_gemm_plan("nvfp4", "nvfp4", m, n, k)
    say(f"nvfp4 tile full output ({data}) {m}x{k}x{n}: {plan[:60]}")
    assert "dq8w_gemm_tile_kernel" in plan
    if data == "normal":
        a_bits, w_bits = W.normal_bf16(m, k, 1.0, 0), W.normal_bf16(n, k, 0.02, 1)
    else:
        a_bits, w_bits = fuzz_operands(m, k, n)
    g_a = oracle.nv_global_scale(oracle.bf16_amax(a_bits))
    g_w = oracle.nv_global_scale(oracle.bf16_amax(w_bits))
    aq, as_ = oracle.nv_quantize(a_bits, g_a)
    wq, ws = oracle.nv_quantize(w_bits, g_w)
    if data == "fuzz":
        say(f"  E4M3 block scales below 2^-6 (subnormal): A {int(((as_ & 0x78) == 0).sum())}, "
            f"W {int(((ws & 0x78) == 0).sum())}")
    y_ref, s = oracle.gemm_dq(oracle.nv_dequantize(aq, as_, m, k, g_a), oracle.nv_dequantize(wq, ws, n, k, g_w))
    u = underflow_allowance(k) if data == "fuzz" else 0.0
    for out_f32 in (False, True):
        y, (gaq, gas), (gwq, gws) = nv_case(a_bits, w_bits, g_a, g_w, out_f32)
        assert np.array_equal(host(gaq), aq) and np.array_equal(host(gas), as_)
        assert np.array_equal(host(gwq), wq) and np.array_equal(host(gws), ws)
        rel = check_gemm(y_host(y), y_ref, s, not out_f32, f"nvfp4 tile {data} f32={out_f32}", None, u)
        say(f"  f32={out_f32}: max err/S {rel:.2e}")


def test_nvfp4_config_sampled():
    cfg = W.NVFP4
    run = max(oracle.bf16_amax(b) for b in cfg.calibration_batches())
    g_a = oracle.nv_global_scale(run)
    a_bits, w_bits = cfg.activations(), cfg.weights()
    g_w = oracle.nv_global_scale(oracle.bf16_amax(w_bits))
    say(f"nvfp4 config g_a={g_a} g_w={g_w}")
    y, _, _ = nv_case(a_bits, w_bits, g_a, g_w)
    mi, ni = sample_pairs(cfg.m, cfg.n, 4096)
    ur, ir = np.unique(mi, return_inverse=True)
    uc, ic = np.unique(ni, return_inverse=True)
    aq, as_ = oracle.nv_quantize(np.ascontiguousarray(a_bits[ur]), g_a)
    wq, ws = oracle.nv_quantize(np.ascontiguousarray(w_bits[uc]), g_w)
    y_ref, s = oracle.gemm_dq_pairs(oracle.nv_dequantize(aq, as_, len(ur), cfg.k, g_a),
                                    oracle.nv_dequantize(wq, ws, len(uc), cfg.k, g_w), ir, ic)
    yv = y[torch.from_numpy(mi).cuda(), torch.from_numpy(ni).cuda()]
    check_gemm(y_host(yv), y_ref, s, True, cfg.name)


# split-K: few output tiles and a long K, so the library splits K over
# workgroups (mx_gemm_workspace_size > 0) and sums fp32 partials in order.
# (M <= 48 MXFP4 runs the decode kernels, which do not split; so does MXFP8
# at M <= 16 when K is a multiple of 1024 up to 8192, hence K = 4608 at M = 1.)
SPLIT_SHAPES = [(300, 2048, 200), (64, 5120, 96), (1, 4608, 48), (513, 1536, 130)]
SPLIT_CASES = [(f, m, k, n) for (m, k, n) in SPLIT_SHAPES for f in ("mxfp4", "mxfp8") if not (f == "mxfp4" and m <= 48)]
# 141 tiles of 128 x 128: the dequantizing kernel still splits K in two
SPLIT_CASES += [("mxfp8", 300, 1024, 6000)]


@pytest.mark.parametrize("fmt,m,k,n", SPLIT_CASES)
def test_gemm_split_k(fmt, m, k, n):
    ws = mxl.mx_gemm_workspace_size(fmt, fmt, m, n, k)
    plan = mxl.mx_gemm_plan(fmt, fmt, m, n, k)
    say(f"split-K {fmt} m={m} k={k} n={n}: workspace {ws} B, plan {plan}")
    assert ws > 0 and "split-K" in plan
    a_bits = W.activations_entry_outliers(m, k)
    w_bits = W.normal_bf16(n, k, 0.02, 1)
    y_ref, s, _, _ = oracle_full(a_bits, w_bits, fmt)
    a, w = cuda_bf16(a_bits), cuda_bf16(w_bits)
    wq, wsc = mxl.mx_pack_weights(w, fmt=fmt, rule=W_RULE[fmt])
    aq, as_ = mxl.mx_quantize_act(a, fmt=fmt, rule="ceil")
    for out_f32 in (False, True):
        ys = mxl.mx_gemm(aq, as_, wq, wsc, k, fmt, fmt, out_f32=out_f32)
        y1 = mxl.mx_gemm(aq, as_, wq, wsc, k, fmt, fmt, out_f32=out_f32, split_k=False)
        ys2 = mxl.mx_gemm(aq, as_, wq, wsc, k, fmt, fmt, out_f32=out_f32)
        torch.cuda.synchronize()
        check_gemm(y_host(ys), y_ref, s, not out_f32, f"split {fmt} {m}x{k}x{n} f32={out_f32}")
        check_gemm(y_host(y1), y_ref, s, not out_f32, f"unsplit {fmt} {m}x{k}x{n} f32={out_f32}")
        assert torch.equal(ys, ys2), "split-K is deterministic"


def test_nvfp4_and_w4a16_split_k():
    m, k, n = 96, 4096, 160
    a_bits = W.normal_bf16(m, k, 1.0, 3)
    w_bits = W.normal_bf16(n, k, 0.02, 4)
    g_a = oracle.nv_global_scale(oracle.bf16_amax(a_bits))
    g_w = oracle.nv_global_scale(oracle.bf16_amax(w_bits))
    assert mxl.mx_gemm_workspace_size("nvfp4", "nvfp4", m, n, k) > 0
    aq, as_ = mxl.mx_quantize_act(cuda_bf16(a_bits), "nvfp4", global_scale=float(g_a))
    wq, ws = mxl.mx_pack_weights(cuda_bf16(w_bits), "nvfp4", global_scale=float(g_w))
    alpha = float(np.float32(1.0) / (np.float32(g_a) * np.float32(g_w)))
    y = mxl.nv_gemm(aq, as_, wq, ws, k, alpha, out_f32=True)
    torch.cuda.synchronize()
    raq, ras = oracle.nv_quantize(a_bits, g_a)
    rwq, rws = oracle.nv_quantize(w_bits, g_w)
    ad = oracle.nv_dequantize(raq, ras, m, k, g_a)
    wd = oracle.nv_dequantize(rwq, rws, n, k, g_w)
    y_ref, s = oracle.gemm_dq(ad, wd)
    check_gemm(y_host(y), y_ref, s, False, "nvfp4 split-K")
    # W4A16 general kernel (M > 16 runs it) with the same weights
    say("w4a16 split-K: " + mxl.mx_gemm_w4a16_plan("nvfp4", m, n, k))
    yw = mxl.mx_gemm_w4a16(cuda_bf16(a_bits), wq, ws, "nvfp4", alpha=float(np.float32(1.0) / np.float32(g_w)),
                           out_f32=True)
    torch.cuda.synchronize()
    yw_ref = oracle.w4a16_gemm(a_bits, rwq, rws, n, k, "nvfp4", g_w=g_w)
    check_gemm(y_host(yw), yw_ref[0], yw_ref[1], False, "w4a16 split-K")


# The fused prologue's own quantization, dumped by MX_DEBUG_DUMP_AQ, against
# the oracle bit for bit: MXFP4 on the 128 x 128 and 256 x 256 fused kernels
# (ragged M and N), MXFP8 on the exact (dequantizing) and the fast fused paths.
@pytest.mark.parametrize("fmt,fast,m,k,n", [("mxfp4", False, 200, 416, 300), ("mxfp4", False, 1100, 1152, 1090),
                                            ("mxfp8", False, 130, 544, 260), ("mxfp8", True, 130, 544, 260)])
def test_fused_prologue_codes_dumped(fmt, fast, m, k, n):
    say(f"fused dump {fmt} fast={fast} m={m} k={k} n={n}")
    a_bits = W.fuzz_bf16(m, k, seed=17)
    w_bits = W.normal_bf16(n, k, 0.02, 1)
    a, w = cuda_bf16(a_bits), cuda_bf16(w_bits)
    wq, ws = mxl.mx_pack_weights(w, fmt=fmt, rule=W_RULE[fmt])
    y, (dq, ds) = mxl.mx_gemm_fused(a, wq, ws, fmt, "ceil", fmt, fp8_fast=fast, dump_aq=True)
    y0 = mxl.mx_gemm_fused(a, wq, ws, fmt, "ceil", fmt, fp8_fast=fast)
    torch.cuda.synchronize()
    rq, rs = oracle.mx_quantize(ELEM[fmt], "ceil", a_bits)
    assert np.array_equal(host(ds), rs), "prologue scales"
    assert np.array_equal(host(dq), rq), "prologue codes"
    assert torch.equal(y, y0), "the dump does not change the product"


# The decode-shaped exact MXFP8 and NVFP4 GEMMs (dq_decode_stream_kernel: M <=
# 32, one launch per 16 rows of A; K % 1024 == 0, K <= 8192) against the
# oracle in full: one chunk ring
# slot (NVFP4 K = 1024), a ring shorter than the quarter (K = 5120), the
# largest K; ragged N; normal operands and fuzz-corpus operands whose block
# scales reach 2^-127 (MXFP8) or the subnormal E4M3 scales (NVFP4); bf16 and
# fp32 output.
DQ_DECODE_CASES = [(1, 1024, 300), (3, 5120, 200), (8, 5120, 17), (16, 8192, 130), (16, 2048, 1),
                   (17, 5120, 130), (32, 2048, 300), (29, 8192, 33),   # above 16 rows: two launches
                   (2, 1024, 65600)]   # wide enough for the tile kernels, which the decode kernel precedes


@pytest.mark.parametrize("data", ["normal", "fuzz"])
@pytest.mark.parametrize("m,k,n", DQ_DECODE_CASES)
def test_mxfp8_decode_kernel(m, k, n, data):
    plan = mxl.mx_gemm_plan("mxfp8", "mxfp8", m, n, k)
    say(f"mxfp8 decode {data} {m}x{k}x{n}: {plan[:60]}")
    assert "dq_decode_stream_kernel<mxfp8" in plan
    if data == "normal":
        a_bits, w_bits = W.activations_entry_outliers(m, k, seed=5 + m), W.normal_bf16(n, k, 0.02, 6)
    else:
        a_bits, w_bits = fuzz_operands(m, k, n)
    y_ref, s, (raq, ras), (rwq, rws) = oracle_full(a_bits, w_bits, "mxfp8")
    fl = flushed_terms(oracle.mx_dequantize("e4m3", raq, ras, m, k), oracle.mx_dequantize("e4m3", rwq, rws, n, k))
    for out_f32 in (False, True):
        y, _, (aq, as_), (wq, ws) = run_mx(a_bits, w_bits, "mxfp8", out_f32=out_f32)
        assert np.array_equal(host(aq), raq) and np.array_equal(host(wq), rwq)
        check_gemm(y_host(y), y_ref, s, not out_f32, f"mxfp8 decode {data} {m}x{k}x{n} f32={out_f32}", fl,
                   underflow_allowance(k) if data == "fuzz" else 0.0)


@pytest.mark.parametrize("data", ["normal", "fuzz"])
@pytest.mark.parametrize("m,k,n", DQ_DECODE_CASES)
def test_nvfp4_decode_kernel(m, k, n, data):
    plan = mxl.mx_gemm_plan("nvfp4", "nvfp4", m, n, k)
    say(f"nvfp4 decode {data} {m}x{k}x{n}: {plan[:60]}")
    assert "dq_decode_stream_kernel<nvfp4" in plan
    if data == "normal":
        a_bits, w_bits = W.normal_bf16(m, k, 1.0, 7), W.normal_bf16(n, k, 0.02, 8)
    else:
        a_bits, w_bits = fuzz_operands(m, k, n)
    g_a = oracle.nv_global_scale(oracle.bf16_amax(a_bits))
    g_w = oracle.nv_global_scale(oracle.bf16_amax(w_bits))
    aq, as_ = oracle.nv_quantize(a_bits, g_a)
    wq, ws = oracle.nv_quantize(w_bits, g_w)
    y_ref, s = oracle.gemm_dq(oracle.nv_dequantize(aq, as_, m, k, g_a), oracle.nv_dequantize(wq, ws, n, k, g_w))
    u = underflow_allowance(k) if data == "fuzz" else 0.0
    for out_f32 in (False, True):
        y, (gaq, gas), (gwq, gws) = nv_case(a_bits, w_bits, g_a, g_w, out_f32)
        assert np.array_equal(host(gaq), aq) and np.array_equal(host(gas), as_)
        assert np.array_equal(host(gwq), wq) and np.array_equal(host(gws), ws)
        check_gemm(y_host(y), y_ref, s, not out_f32, f"nvfp4 decode {data} {m}x{k}x{n} f32={out_f32}", None, u)
