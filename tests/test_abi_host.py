"""Host-side checks of libmxlinear.so that need no GPU: the library loads,
exports every entry point that include/mxlinear.h declares, validates its
arguments before touching the HIP runtime, and its host helpers agree with
the oracle."""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mxlinear.h")

mxl = pytest.importorskip("fp8_quantized_linear_amd")
L = mxl.lib

OK, INVALID, SHAPE, ALIGN, WORKSPACE, UNSUPPORTED, HIPERR = range(7)
P = ctypes.c_void_p
GOOD = P(0x10000)      # 16-byte aligned, never dereferenced by validation failures
BAD_ALIGN = P(0x10008)


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^[A-Za-z_][\w\s\*]*?\b([a-z_][a-z0-9_]*)\s*\(", text, flags=re.M)
    return sorted(set(n for n in names if n not in ("if", "defined")))


def test_header_declares_expected_entry_points():
    names = declared_functions()
    for n in ("mx_pack_weights", "mx_quantize_act", "mx_gemm", "mx_gemm_fused", "nv_gemm",
              "mx_gemm_w4a16", "mx_gemm_w4a16_plan", "mx_fake_quant",
              "mx_gemm_swiglu_quant", "mx_gemm_swiglu_quant_plan", "mx_swiglu_quant",
              "mx_gemm_workspace_size", "mx_gemm_w4a16_workspace_size", "mx_gemm_fused_workspace_size",
              "mx_tensor_amax", "mx_nv_global_scale", "mx_gemm_plan", "mx_status_string",
              "mx_abi_version"):
        assert n in names


def test_library_exports_every_declared_symbol():
    for n in declared_functions():
        assert hasattr(L, n), f"{n} declared in mxlinear.h but not exported"


def test_abi_version_matches_header():
    m = re.search(r"#define MXLINEAR_ABI_VERSION (\d+)", open(HEADER).read())
    assert L.mx_abi_version() == int(m.group(1))


def test_status_strings():
    for s in range(7):
        assert L.mx_status_string(s)
    assert b"unknown" in L.mx_status_string(99)


def q(fn, fmt=0, rule=1, x=GOOD, rows=4, k=64, g=1.0, qp=GOOD, sp=GOOD):
    return fn(fmt, rule, x, rows, k, g, qp, sp, None)


@pytest.mark.parametrize("fn", [L.mx_quantize_act, L.mx_pack_weights])
def test_quantize_validation(fn):
    assert q(fn, fmt=7) == INVALID
    assert q(fn, rule=9) == INVALID
    assert q(fn, fmt=2, rule=9, g=0.5) != INVALID  # NVFP4 ignores the rule
    assert q(fn, x=None) == INVALID
    assert q(fn, qp=None) == INVALID
    assert q(fn, sp=None) == INVALID
    assert q(fn, rows=0) == SHAPE
    assert q(fn, k=0) == SHAPE
    assert q(fn, k=48) == SHAPE              # MX needs k % 32
    assert q(fn, fmt=2, k=40, g=1.0) == SHAPE  # NVFP4 needs k % 16
    assert q(fn, fmt=2, k=48, g=0.0) == INVALID  # global scale must be > 0
    assert q(fn, fmt=2, k=48, g=float("nan")) == INVALID
    assert q(fn, x=BAD_ALIGN) == ALIGN
    # valid arguments reach the device check: without a GPU that is a HIP error
    st = q(fn)
    assert st in (OK, UNSUPPORTED, HIPERR)


def g(**kw):
    a = dict(a_fmt=0, w_fmt=0, aq=GOOD, as_=GOOD, wq=GOOD, ws=GOOD, m=16, n=16, k=64, y=GOOD,
             flags=0)
    a.update(kw)
    return L.mx_gemm(a["a_fmt"], a["w_fmt"], a["aq"], a["as_"], a["wq"], a["ws"], a["m"], a["n"],
                     a["k"], a["y"], a["flags"], None, 0, None)


def test_gemm_validation():
    assert g(a_fmt=2) == INVALID          # NVFP4 goes through nv_gemm
    assert g(w_fmt=5) == INVALID
    assert g(aq=None) == INVALID
    assert g(y=None) == INVALID
    assert g(flags=0x80) == INVALID
    assert g(m=0) == SHAPE
    assert g(n=0) == SHAPE
    assert g(k=48) == SHAPE
    assert g(k=1 << 31) == SHAPE
    assert g(a_fmt=0, w_fmt=1) == UNSUPPORTED  # mixed element types
    assert g(ws=BAD_ALIGN) == ALIGN
    assert g(n=96) in (OK, UNSUPPORTED, HIPERR)  # N < 128 is accepted (validation passes)
    assert g(n=1, m=1, k=32) in (OK, UNSUPPORTED, HIPERR)


def test_fused_and_nv_validation():
    f = L.mx_gemm_fused
    assert f(0, 9, GOOD, 0, GOOD, GOOD, 4, 4, 64, GOOD, 0, None, 0, None) == INVALID
    assert f(0, 1, None, 0, GOOD, GOOD, 4, 4, 64, GOOD, 0, None, 0, None) == INVALID
    assert f(0, 1, GOOD, 0, GOOD, GOOD, 4, 4, 40, GOOD, 0, None, 0, None) == SHAPE
    assert f(1, 1, GOOD, 0, GOOD, GOOD, 4, 4, 64, GOOD, 0, None, 0, None) == UNSUPPORTED
    nv = L.nv_gemm
    assert nv(GOOD, GOOD, GOOD, GOOD, 4, 4, 40, 1.0, GOOD, 0, None, 0, None) == SHAPE
    assert nv(GOOD, GOOD, GOOD, GOOD, 4, 4, 48, float("inf"), GOOD, 0, None, 0, None) == INVALID
    assert nv(None, GOOD, GOOD, GOOD, 4, 4, 48, 1.0, GOOD, 0, None, 0, None) == INVALID
    assert L.mx_tensor_amax(None, 10, GOOD, None) == INVALID
    assert L.mx_tensor_amax(GOOD, 0, GOOD, None) == SHAPE
    assert L.mx_tensor_amax(GOOD, 10, P(0x10002), None) == ALIGN


def test_w4a16_validation():
    w = L.mx_gemm_w4a16
    def g(fmt=0, a=GOOD, wq=GOOD, ws=GOOD, m=4, n=4, k=64, alpha=1.0, y=GOOD, flags=0):
        return w(fmt, a, wq, ws, m, n, k, alpha, y, flags, None, 0, None)
    assert g(fmt=7) == INVALID
    assert g(fmt=1) == UNSUPPORTED          # MXFP8 weights: no W4A16 mode
    assert g(a=None) == INVALID
    assert g(flags=0x80) == INVALID
    assert g(alpha=float("nan")) == INVALID
    assert g(k=48) == SHAPE                  # MXFP4 needs k % 32 == 0
    assert g(fmt=2, k=40) == SHAPE           # NVFP4 needs k % 16 == 0
    assert g(m=0) == SHAPE
    assert g(wq=BAD_ALIGN) == ALIGN
    assert g(fmt=2, k=48) in (OK, UNSUPPORTED, HIPERR)   # validation passes


def test_fake_quant_validation():
    f = L.mx_fake_quant
    def g(fmt=0, rule=1, x=GOOD, rows=4, k=64, gs=1.0, y=P(0x20000)):
        return f(fmt, rule, x, rows, k, gs, y, None)
    assert g(fmt=7) == INVALID
    assert g(rule=9) == INVALID
    assert g(fmt=2, rule=9) in (OK, UNSUPPORTED, HIPERR)   # NVFP4 ignores the rule
    assert g(x=None) == INVALID
    assert g(y=None) == INVALID
    assert g(fmt=2, gs=0.0) == INVALID
    assert g(fmt=2, gs=float("inf")) == INVALID
    assert g(y=P(0x10000 + 64 * 4 * 2 - 16)) == INVALID      # y overlaps the end of x
    assert g(k=48) == SHAPE
    assert g(fmt=2, k=40) == SHAPE
    assert g(rows=0) == SHAPE
    assert g(x=BAD_ALIGN) == ALIGN
    assert g(y=P(0x20008)) == ALIGN
    assert g(y=P(0x10000 + 64 * 4 * 2)) in (OK, UNSUPPORTED, HIPERR)  # adjacent, not overlapping


def test_swiglu_validation():
    f = L.mx_gemm_swiglu_quant
    def g(aq=GOOD, a_s=GOOD, wq=GOOD, ws=GOOD, m=4, inter=64, k=256, hq=GOOD, hs=GOOD):
        return f(aq, a_s, wq, ws, m, inter, k, hq, hs, None)
    assert g(aq=None) == INVALID
    assert g(hs=None) == INVALID
    assert g(inter=48) == SHAPE
    assert g(inter=0) == SHAPE
    assert g(k=48) == SHAPE
    assert g(m=0) == SHAPE
    assert g(k=96) == UNSUPPORTED          # the fused kernel needs k % 128 == 0
    assert g(hq=BAD_ALIGN) == ALIGN
    assert g() in (OK, UNSUPPORTED, HIPERR)
    s = L.mx_swiglu_quant
    assert s(None, 4, 64, GOOD, GOOD, None) == INVALID
    assert s(GOOD, 4, 40, GOOD, GOOD, None) == SHAPE
    assert s(GOOD, 0, 64, GOOD, GOOD, None) == SHAPE
    assert s(BAD_ALIGN, 4, 64, GOOD, GOOD, None) == ALIGN
    assert "swiglu" in mxl.mx_gemm_swiglu_quant_plan(8192, 17408, 5120)
    with pytest.raises(mxl.MXError):
        mxl.mx_gemm_swiglu_quant_plan(16, 64, 96)


def test_workspace_sizes():
    # few tiles and a long K: split-K with S fp32 partials of M x N
    assert mxl.mx_gemm_workspace_size("mxfp8", "mxfp8", 64, 96, 5120) == 10 * 64 * 96 * 4
    assert mxl.mx_gemm_workspace_size("mxfp4", "mxfp4", 512, 2048, 5120) == 4 * 512 * 2048 * 4
    assert mxl.mx_gemm_workspace_size("nvfp4", "nvfp4", 96, 160, 4096) > 0
    # tiles that fill the GPU, the decode kernel, the prefill kernel: none
    assert mxl.mx_gemm_workspace_size("mxfp4", "mxfp4", 8192, 17408, 5120) == 0
    # fused, quantize-once: A codes and scales of the 8192 x 5120 activations,
    # then at a 256-byte boundary a chunk pool counter, a done counter per
    # 256-row block and an error word, rounded up to 256 bytes
    assert mxl.mx_gemm_fused_workspace_size("mxfp4", "mxfp4", 8192, 17408, 5120) == 8192 * 2560 + 8192 * 160 + 256
    assert mxl.mx_gemm_fused_workspace_size("mxfp4", "mxfp4", 1100, 1090, 1152) == \
        ((1100 * 576 + 1100 * 36 + 255) // 256) * 256 + 256
    assert mxl.mx_gemm_fused_workspace_size("mxfp4", "mxfp4", 512, 2048, 5120) == 0     # not a large shape
    assert "mx_gemm_prefill_fq_kernel<" in mxl.mx_gemm_plan("mxfp4", "mxfp4", 8192, 17408, 5120, fused=True)
    # exact MXFP8: codes [m, k] and scales, then the pool counter, a done
    # counter per 128-row block and an error word; none for the fast path
    assert mxl.mx_gemm_fused_workspace_size("mxfp8", "mxfp8", 8192, 17408, 5120) == 8192 * 5120 + 8192 * 160 + 512
    assert mxl.mx_gemm_fused_workspace_size("mxfp8", "mxfp8", 8192, 17408, 5120, fp8_fast=True) == 0
    assert mxl.mx_gemm_fused_workspace_size("mxfp8", "mxfp8", 64, 96, 5120) == 0        # n <= 256
    b2 = ctypes.c_size_t(7)
    assert L.mx_gemm_fused_workspace_size(0, 0, 8192, 17408, 5120, 0x4, ctypes.byref(b2)) == OK and b2.value == 0
    assert L.mx_gemm_fused_workspace_size(0, 2, 64, 64, 64, 0, ctypes.byref(b2)) == INVALID
    assert mxl.mx_gemm_workspace_size("mxfp4", "mxfp4", 8, 17408, 5120) == 0
    assert mxl.mx_gemm_workspace_size("mxfp8", "mxfp8", 4096, 6144, 5120) == 0
    # short K: no split
    assert mxl.mx_gemm_workspace_size("mxfp8", "mxfp8", 64, 96, 256) == 0
    b = ctypes.c_size_t(7)
    assert L.mx_gemm_workspace_size(0, 2, 4, 4, 64, 0, ctypes.byref(b)) == INVALID   # mixed NVFP4
    assert L.mx_gemm_workspace_size(0, 0, 4, 4, 48, 0, ctypes.byref(b)) == SHAPE
    assert L.mx_gemm_workspace_size(0, 0, 4, 4, 64, 0, None) == INVALID
    assert L.mx_gemm_w4a16_workspace_size(1, 4, 4, 64, ctypes.byref(b)) == UNSUPPORTED
    assert L.mx_gemm_w4a16_workspace_size(2, 8, 512, 5120, ctypes.byref(b)) == OK and b.value == 0  # decode
    assert L.mx_gemm_w4a16_workspace_size(2, 96, 160, 4096, ctypes.byref(b)) == OK and b.value > 0
    # a misaligned workspace is rejected before any HIP call
    assert L.mx_gemm(0, 0, GOOD, GOOD, GOOD, GOOD, 4, 4, 64, GOOD, 0, BAD_ALIGN, 64, None) == ALIGN
    assert "split-K" in mxl.mx_gemm_plan("mxfp8", "mxfp8", 64, 96, 5120)


def test_fused_dump_validation():
    f = L.mx_gemm_fused
    def g(flags=0x4, ws=P(0x40000), wsb=1 << 20, k=64):
        return f(0, 1, GOOD, 0, GOOD, GOOD, 4, 4, k, GOOD, flags, ws, wsb, None)
    assert g(flags=0x8) == INVALID
    assert g(ws=None) == WORKSPACE
    assert g(wsb=4 * 32 + 4 * 2 - 1) == WORKSPACE          # codes 4 x 32 B + scales 4 x 2 B
    assert g(ws=BAD_ALIGN) == ALIGN
    assert g(wsb=4 * 32 + 4 * 2) in (OK, UNSUPPORTED, HIPERR)


def test_gate_up_interleave_index():
    idx = mxl.gate_up_interleave_index(96).tolist()
    assert sorted(idx) == list(range(192))
    assert idx[:32] == list(range(0, 32)) and idx[32:64] == list(range(96, 128))
    assert idx[64:96] == list(range(32, 64)) and idx[160:192] == list(range(160, 192))


def test_plan_names_the_kernel():
    s = mxl.mx_gemm_plan("mxfp4", "mxfp4", 8192, 17408, 5120)
    assert "mfma" in s and "mxfp4" in s
    assert "f16 mfma" in mxl.mx_gemm_plan("nvfp4", "nvfp4", 4096, 5120, 5120)
    assert "fused" in mxl.mx_gemm_plan("mxfp4", "mxfp4", 64, 64, 64, fused=True)
    assert mxl.mx_gemm_plan("mxfp8", "mxfp8", 16, 96, 5120)  # N = 96 is a valid plan
    with pytest.raises(mxl.MXError):
        mxl.mx_gemm_plan("mxfp4", "mxfp4", 16, 16, 40)
    assert "w4a16_decode_kernel" in mxl.mx_gemm_w4a16_plan("mxfp4", 1, 17408, 5120)
    assert "w4a16_decode_kernel" in mxl.mx_gemm_w4a16_plan("nvfp4", 16, 17408, 5120)
    assert "dq_gemm_kernel" in mxl.mx_gemm_w4a16_plan("mxfp4", 17, 17408, 5120)
    assert "dq_gemm_kernel" in mxl.mx_gemm_w4a16_plan("nvfp4", 1, 512, 400)


def test_global_scale_helper_matches_oracle():
    rng = np.random.default_rng(0)
    vals = np.concatenate([np.ldexp(rng.random(3000) + 0.5, rng.integers(-100, 100, 3000)),
                           [1.0, 3.0, 7.0, 2688.0, 6.0, 448.0, 1e-38, 3e38]]).astype(np.float32)
    for v in vals:
        assert np.float32(L.mx_nv_global_scale(float(v))) == oracle.nv_global_scale(float(v)), v
    assert L.mx_nv_global_scale(0.0) == 1.0
