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

# The validation tests call the entry points with fake device pointers.
# Calls whose arguments pass validation go on to the device check and, on a
# machine with a GPU, would launch kernels on those pointers; so these tests
# run only where no GPU is visible (counting devices initialises none).  On
# a GPU machine only the pure host logic below them runs.
import torch  # noqa: E402

NO_GPU = torch.cuda.device_count() == 0
fake_pointers = pytest.mark.skipif(not NO_GPU, reason="calls with fake device pointers run only without a GPU")


def passes_validation(call) -> bool:
    """True if call() gets past argument validation (reaching the device
    check, which fails without a GPU)."""
    assert NO_GPU
    return call() in (OK, UNSUPPORTED, HIPERR)
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


@fake_pointers
@pytest.mark.parametrize("fn", [L.mx_quantize_act, L.mx_pack_weights])
def test_quantize_validation(fn):
    assert q(fn, fmt=7) == INVALID
    assert q(fn, rule=9) == INVALID
    assert passes_validation(lambda: q(fn, fmt=2, rule=9, g=0.5))  # NVFP4 ignores the rule
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
    assert passes_validation(lambda: st)


def g(**kw):
    a = dict(a_fmt=0, w_fmt=0, aq=GOOD, as_=GOOD, wq=GOOD, ws=GOOD, m=16, n=16, k=64, y=GOOD,
             flags=0, work=None, wsb=0)
    a.update(kw)
    return L.mx_gemm(a["a_fmt"], a["w_fmt"], a["aq"], a["as_"], a["wq"], a["ws"], a["m"], a["n"],
                     a["k"], a["y"], a["work"], a["wsb"], a["flags"], None)


@fake_pointers
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
    assert passes_validation(lambda: g(a_fmt=0, w_fmt=1))   # mixed pairs pass validation
    assert passes_validation(lambda: g(a_fmt=1, w_fmt=0, flags=0x2))
    assert g(ws=BAD_ALIGN) == ALIGN
    assert passes_validation(lambda: g(n=96))  # N < 128 is accepted (validation passes)
    assert passes_validation(lambda: g(n=1, m=1, k=32))


@fake_pointers
def test_fused_and_nv_validation():
    f = L.mx_gemm_fused   # (a_fmt, w_fmt, a_bf16, a_rule, w_q, w_s, m, n, k, y, workspace, ws_bytes, flags, stream)
    assert f(0, 0, GOOD, 9, GOOD, GOOD, 4, 4, 64, GOOD, None, 0, 0, None) == INVALID
    assert f(0, 0, None, 1, GOOD, GOOD, 4, 4, 64, GOOD, None, 0, 0, None) == INVALID
    assert f(0, 0, GOOD, 1, GOOD, GOOD, 4, 4, 40, GOOD, None, 0, 0, None) == SHAPE
    # mixed pairs quantize A into the workspace: required, codes + scales
    assert f(1, 0, GOOD, 1, GOOD, GOOD, 4, 4, 64, GOOD, None, 0, 0, None) == WORKSPACE
    assert f(1, 0, GOOD, 1, GOOD, GOOD, 4, 4, 64, GOOD, P(0x40000), 4 * 64 + 4 * 2 - 1, 0, None) == WORKSPACE
    assert passes_validation(lambda: f(1, 0, GOOD, 1, GOOD, GOOD, 4, 4, 64, GOOD, P(0x40000), 4 * 64 + 4 * 2, 0,
                                       None))
    nv = L.nv_gemm
    assert nv(GOOD, GOOD, GOOD, GOOD, 4, 4, 40, 1.0, GOOD, None, 0, 0, None) == SHAPE
    assert nv(GOOD, GOOD, GOOD, GOOD, 4, 4, 48, float("inf"), GOOD, None, 0, 0, None) == INVALID
    assert nv(None, GOOD, GOOD, GOOD, 4, 4, 48, 1.0, GOOD, None, 0, 0, None) == INVALID
    assert L.mx_tensor_amax(None, 10, GOOD, None) == INVALID
    assert L.mx_tensor_amax(GOOD, 0, GOOD, None) == SHAPE
    assert L.mx_tensor_amax(GOOD, 10, P(0x10002), None) == ALIGN


@fake_pointers
def test_w4a16_validation():
    w = L.mx_gemm_w4a16
    def g(fmt=0, a=GOOD, wq=GOOD, ws=GOOD, m=4, n=4, k=64, alpha=1.0, y=GOOD, flags=0):
        return w(fmt, a, wq, ws, m, n, k, alpha, y, None, 0, flags, None)
    assert g(fmt=7) == INVALID
    assert g(fmt=1) == UNSUPPORTED          # MXFP8 weights: no W4A16 mode
    assert g(a=None) == INVALID
    assert g(flags=0x80) == INVALID
    assert g(alpha=float("nan")) == INVALID
    assert g(k=48) == SHAPE                  # MXFP4 needs k % 32 == 0
    assert g(fmt=2, k=40) == SHAPE           # NVFP4 needs k % 16 == 0
    assert g(m=0) == SHAPE
    assert g(wq=BAD_ALIGN) == ALIGN
    assert passes_validation(lambda: g(fmt=2, k=48))   # validation passes


@fake_pointers
def test_fake_quant_validation():
    f = L.mx_fake_quant
    def g(fmt=0, rule=1, x=GOOD, rows=4, k=64, gs=1.0, y=P(0x20000)):
        return f(fmt, rule, x, rows, k, gs, y, None)
    assert g(fmt=7) == INVALID
    assert g(rule=9) == INVALID
    assert passes_validation(lambda: g(fmt=2, rule=9))   # NVFP4 ignores the rule
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
    assert passes_validation(lambda: g(y=P(0x10000 + 64 * 4 * 2)))  # adjacent, not overlapping


@fake_pointers
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
    assert passes_validation(lambda: g())
    s = L.mx_swiglu_quant
    assert s(None, 4, 64, GOOD, GOOD, None) == INVALID
    assert s(GOOD, 4, 40, GOOD, GOOD, None) == SHAPE
    assert s(GOOD, 0, 64, GOOD, GOOD, None) == SHAPE
    assert s(BAD_ALIGN, 4, 64, GOOD, GOOD, None) == ALIGN
    assert "swiglu" in mxl.mx_gemm_swiglu_quant_plan(8192, 17408, 5120)
    with pytest.raises(mxl.MXError):
        mxl.mx_gemm_swiglu_quant_plan(16, 64, 96)


@fake_pointers
def test_workspace_sizes():
    # few tiles and a long K: split-K with S fp32 partials of M x N
    assert mxl.mx_gemm_workspace_size("mxfp8", "mxfp8", 64, 96, 5120) == 10 * 64 * 96 * 4
    assert mxl.mx_gemm_workspace_size("mxfp4", "mxfp4", 512, 2048, 5120) == 4 * 512 * 2048 * 4
    assert mxl.mx_gemm_workspace_size("nvfp4", "nvfp4", 96, 160, 4096) > 0
    # tiles that fill the GPU, the decode kernel, the prefill kernel: none
    assert mxl.mx_gemm_workspace_size("mxfp4", "mxfp4", 8192, 17408, 5120) == 0
    # fused on a quantize-once shape: by default A's codes and scales for the
    # standalone quantizer; with MX_FUSED_IN_GEMM the codes, the scales at
    # the next 256-byte boundary, then at the next one a chunk pool counter,
    # a done counter per 256-row block and an error word, rounded up to 256
    # bytes
    def up256(v):
        return (v + 255) // 256 * 256
    assert mxl.mx_gemm_fused_workspace_size("mxfp4", "mxfp4", 8192, 17408, 5120) == 8192 * 2560 + 8192 * 160
    assert mxl.mx_gemm_fused_workspace_size("mxfp4", "mxfp4", 8192, 17408, 5120, in_gemm=True) == \
        8192 * 2560 + 8192 * 160 + 256
    assert mxl.mx_gemm_fused_workspace_size("mxfp4", "mxfp4", 1100, 1090, 1152, in_gemm=True) == \
        up256(up256(1100 * 576) + 1100 * 36) + 256
    # odd m and odd k/128: the scale plane no longer starts on a cache line
    # after the codes, so it is moved to the next 256-byte boundary
    assert mxl.mx_gemm_fused_workspace_size("mxfp4", "mxfp4", 1025, 1090, 1152, in_gemm=True) == \
        up256(up256(1025 * 576) + 1025 * 36) + 256
    # mixed pairs: A's codes and scales
    assert mxl.mx_gemm_fused_workspace_size("mxfp8", "mxfp4", 100, 300, 512) == 100 * 512 + 100 * 16
    assert mxl.mx_gemm_fused_workspace_size("mxfp4", "mxfp8", 100, 300, 512) == 100 * 256 + 100 * 16
    assert mxl.mx_gemm_fused_workspace_size("mxfp4", "mxfp4", 512, 2048, 5120) == 0     # not a large shape
    assert mxl.mx_gemm_fused_workspace_size("mxfp4", "mxfp4", 512, 2048, 5120, in_gemm=True) == 0
    plan = mxl.mx_gemm_plan("mxfp4", "mxfp4", 8192, 17408, 5120, fused=True)
    assert "mx_quantize_act into it" in plan and "mx_gemm_prefill_kernel<" in plan
    assert "mx_gemm_prefill_fq_kernel<" in mxl.mx_gemm_plan("mxfp4", "mxfp4", 8192, 17408, 5120, fused=True,
                                                           in_gemm=True)
    # exact MXFP8 on the large-tile kernel's shapes (at least 256 tiles of
    # 256 x 256): A's codes [m, k] and scales, quantized by the standalone
    # quantizer; on smaller shapes the quantize-once pool: codes, scales at a
    # 256-byte boundary, then the pool counter, a done counter per 128-row
    # block and an error word; none for the fast path
    assert mxl.mx_gemm_fused_workspace_size("mxfp8", "mxfp8", 8192, 17408, 5120) == 8192 * 5120 + 8192 * 160
    assert "mx8_gemm_tile_kernel" in mxl.mx_gemm_plan("mxfp8", "mxfp8", 4096, 6144, 5120)
    assert "workspace, then" in mxl.mx_gemm_plan("mxfp8", "mxfp8", 4096, 6144, 5120, fused=True)
    assert mxl.mx_gemm_fused_workspace_size("mxfp8", "mxfp8", 1100, 1090, 1152) == 1100 * 1152 + 1100 * 36
    assert mxl.mx_gemm_fused_workspace_size("mxfp8", "mxfp8", 1100, 1090, 1152, in_gemm=True) == \
        up256(up256(1100 * 1152) + 1100 * 36) + 256
    assert "dq_gemm_kernel" in mxl.mx_gemm_plan("mxfp8", "mxfp8", 1100, 1090, 1152)
    assert mxl.mx_gemm_fused_workspace_size("mxfp8", "mxfp8", 8192, 17408, 5120, fp8_fast=True) == 0
    assert mxl.mx_gemm_fused_workspace_size("mxfp8", "mxfp8", 64, 96, 5120) == 0        # n <= 256
    b2 = ctypes.c_size_t(7)
    assert L.mx_gemm_fused_workspace_size(0, 0, 8192, 17408, 5120, 0x4, ctypes.byref(b2)) == OK and \
        b2.value == 8192 * 2560 + 8192 * 160                     # the dump
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
    # mixed pairs split like the exact MXFP8 kernel
    assert mxl.mx_gemm_workspace_size("mxfp8", "mxfp4", 64, 96, 5120) == 10 * 64 * 96 * 4
    # a misaligned workspace is rejected before any HIP call
    assert L.mx_gemm(0, 0, GOOD, GOOD, GOOD, GOOD, 4, 4, 64, GOOD, BAD_ALIGN, 64, 0, None) == ALIGN
    assert "split-K" in mxl.mx_gemm_plan("mxfp8", "mxfp8", 64, 96, 5120)


@fake_pointers
def test_workspace_too_small_is_an_error():
    # a non-NULL workspace smaller than the size query's answer: MX_ERR_WORKSPACE
    # (NULL always runs the variant that needs none)
    need = mxl.mx_gemm_workspace_size("mxfp8", "mxfp8", 64, 96, 5120)
    assert g(a_fmt=1, w_fmt=1, m=64, n=96, k=5120, work=P(0x40000), wsb=need - 1) == WORKSPACE
    assert g(a_fmt=1, w_fmt=1, m=64, n=96, k=5120, work=P(0x40000), wsb=0) == WORKSPACE
    assert passes_validation(lambda: g(a_fmt=1, w_fmt=1, m=64, n=96, k=5120, work=P(0x40000), wsb=need))
    assert passes_validation(lambda: g(a_fmt=1, w_fmt=1, m=64, n=96, k=5120))
    need4 = mxl.mx_gemm_workspace_size("mxfp4", "mxfp4", 512, 2048, 5120)
    assert g(m=512, n=2048, k=5120, work=P(0x40000), wsb=need4 - 16) == WORKSPACE
    # shapes that never split ignore the workspace
    assert passes_validation(lambda: g(m=8192, n=17408, k=5120, work=P(0x40000), wsb=16))
    nvneed = mxl.mx_gemm_workspace_size("nvfp4", "nvfp4", 96, 160, 4096)
    assert L.nv_gemm(GOOD, GOOD, GOOD, GOOD, 96, 160, 4096, 1.0, GOOD, P(0x40000), nvneed - 1, 0, None) == WORKSPACE
    wneed = ctypes.c_size_t(0)
    L.mx_gemm_w4a16_workspace_size(2, 96, 160, 4096, ctypes.byref(wneed))
    assert L.mx_gemm_w4a16(2, GOOD, GOOD, GOOD, 96, 160, 4096, 1.0, GOOD, P(0x40000), wneed.value - 1, 0,
                           None) == WORKSPACE
    f = L.mx_gemm_fused
    IN_GEMM = mxl.MX_FUSED_IN_GEMM
    qneed = mxl.mx_gemm_fused_workspace_size("mxfp4", "mxfp4", 1100, 1090, 1152)
    assert f(0, 0, GOOD, 1, GOOD, GOOD, 1100, 1090, 1152, GOOD, P(0x40000), qneed - 1, 0, None) == WORKSPACE
    assert passes_validation(lambda: f(0, 0, GOOD, 1, GOOD, GOOD, 1100, 1090, 1152, GOOD, P(0x40010), qneed, 0,
                                       None))
    fneed = mxl.mx_gemm_fused_workspace_size("mxfp4", "mxfp4", 1100, 1090, 1152, in_gemm=True)
    assert f(0, 0, GOOD, 1, GOOD, GOOD, 1100, 1090, 1152, GOOD, P(0x40000), fneed - 1, IN_GEMM, None) == WORKSPACE
    # the quantize-once workspace must be 256-byte aligned (its blocks own whole cache lines)
    assert f(0, 0, GOOD, 1, GOOD, GOOD, 1100, 1090, 1152, GOOD, P(0x40010), fneed, IN_GEMM, None) == ALIGN
    assert passes_validation(lambda: f(0, 0, GOOD, 1, GOOD, GOOD, 1100, 1090, 1152, GOOD, P(0x40100), fneed,
                                       IN_GEMM, None))
    pneed = mxl.mx_gemm_fused_workspace_size("mxfp8", "mxfp8", 1100, 1090, 1152, in_gemm=True)
    assert f(1, 1, GOOD, 1, GOOD, GOOD, 1100, 1090, 1152, GOOD, P(0x40080), pneed, IN_GEMM, None) == ALIGN
    assert f(0, 0, GOOD, 1, GOOD, GOOD, 1100, 1090, 1152, GOOD, P(0x40100), fneed, 0x10, None) == INVALID


@fake_pointers
def test_operands_beyond_32bit_offsets_are_rejected():
    # the tile and decode kernels address operands with 32-bit byte offsets:
    # a call that would take them with an operand of 2 GiB or more is refused
    # instead of computing with wrapped offsets
    # MXFP8 fast path, W = 65536 x 32768 E4M3 codes = 2 GiB
    assert g(a_fmt=1, w_fmt=1, m=64, n=65536, k=32768, flags=0x2) == UNSUPPORTED
    # the same shape on the exact MXFP8 path (64-bit offsets) passes validation
    assert passes_validation(lambda: g(a_fmt=1, w_fmt=1, m=64, n=65536, k=32768))
    # MXFP4 decode, W = 262144 x 16384 codes (2 GiB)
    assert g(m=8, n=262144, k=32768) == UNSUPPORTED
    # the fused in-tile kernel reads bf16 A: 32768 x 32768 x 2 B = 2 GiB
    f = L.mx_gemm_fused
    assert f(0, 0, GOOD, 1, GOOD, GOOD, 32768, 512, 32768, GOOD, None, 0, 0, None) == UNSUPPORTED
    # shapes below the limit pass validation
    assert passes_validation(lambda: g(m=8, n=17408, k=5120))


@fake_pointers
def test_fused_dump_validation():
    f = L.mx_gemm_fused
    def g(flags=0x4, ws=P(0x40000), wsb=1 << 20, k=64):
        return f(0, 0, GOOD, 1, GOOD, GOOD, 4, 4, k, GOOD, ws, wsb, flags, None)
    assert g(flags=0x10) == INVALID
    assert g(ws=None) == WORKSPACE
    assert g(wsb=4 * 32 + 4 * 2 - 1) == WORKSPACE          # codes 4 x 32 B + scales 4 x 2 B
    assert g(ws=BAD_ALIGN) == ALIGN
    assert passes_validation(lambda: g(wsb=4 * 32 + 4 * 2))


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
    assert "mxfp8xmxfp4 dq_gemm_kernel<mxfp8 x mxfp4" in mxl.mx_gemm_plan("mxfp8", "mxfp4", 4096, 5120, 5120)
    assert "mxfp4xmxfp8 dq_gemm_kernel" in mxl.mx_gemm_plan("mxfp4", "mxfp8", 4096, 5120, 5120)
    assert "mx_gemm_kernel<tile 128x128" in mxl.mx_gemm_plan("mxfp8", "mxfp4", 4096, 5120, 5120, fp8_fast=True)
    assert "workspace" in mxl.mx_gemm_plan("mxfp8", "mxfp4", 4096, 5120, 5120, fused=True)
    assert "w4a16_decode_stream_kernel" in mxl.mx_gemm_w4a16_plan("mxfp4", 1, 17408, 5120)
    assert "w4a16_decode_stream_kernel" in mxl.mx_gemm_w4a16_plan("nvfp4", 1, 17408, 5120)
    assert "w4a16_decode_stream2_kernel" in mxl.mx_gemm_w4a16_plan("nvfp4", 16, 17408, 5120)
    assert "one workgroup per compute unit" in mxl.mx_gemm_w4a16_plan("nvfp4", 16, 17408, 5120)
    assert "32 W rows per workgroup" in mxl.mx_gemm_w4a16_plan("mxfp4", 8, 4096, 5120)
    assert "32 W rows per workgroup" in mxl.mx_gemm_w4a16_plan("nvfp4", 4, 17408, 5120)
    assert "one workgroup per compute unit" in mxl.mx_gemm_w4a16_plan("mxfp4", 4, 17408, 5120)
    assert "w4a16_decode_stream2_kernel" in mxl.mx_gemm_w4a16_plan("mxfp4", 3, 17408, 8192)
    assert "w4a16_decode_kernel" in mxl.mx_gemm_w4a16_plan("mxfp4", 8, 17408, 2560)
    assert "mx_decode_stream_kernel" in mxl.mx_gemm_plan("mxfp4", "mxfp4", 32, 17408, 5120)
    # 9-32 rows over 4-5 sixteen-row W groups per compute unit: one workgroup per CU
    assert "one workgroup per compute unit" in mxl.mx_gemm_plan("mxfp4", "mxfp4", 32, 17408, 5120)
    assert "one workgroup per compute unit" in mxl.mx_gemm_plan("mxfp4", "mxfp4", 9, 17408, 5120)
    assert "one workgroup per compute unit" not in mxl.mx_gemm_plan("mxfp4", "mxfp4", 8, 17408, 5120)
    assert "one workgroup per compute unit" not in mxl.mx_gemm_plan("mxfp4", "mxfp4", 32, 151936, 5120)
    assert "mx_decode_kernel" in mxl.mx_gemm_plan("mxfp4", "mxfp4", 8, 17408, 2560)
    assert "dq_gemm_kernel" in mxl.mx_gemm_w4a16_plan("mxfp4", 17, 17408, 5120)
    assert "dq_gemm_kernel" in mxl.mx_gemm_w4a16_plan("nvfp4", 1, 512, 400)
    # decode shapes with a vocabulary-sized N stream W before the tile kernels
    # are considered (MXFP8 up to 16 rows, NVFP4 up to 32), and W beyond the
    # decode kernel's 32-bit offsets goes to the tile kernels
    for fmt, m in (("mxfp8", 1), ("mxfp8", 16), ("nvfp4", 1), ("nvfp4", 32)):
        assert "dq_decode_stream_kernel" in mxl.mx_gemm_plan(fmt, fmt, m, 151936, 5120), (fmt, m)
    assert "mx8_gemm_tile_kernel" in mxl.mx_gemm_plan("mxfp8", "mxfp8", 17, 151936, 5120)
    assert "dq_decode_stream_kernel" not in mxl.mx_gemm_plan("mxfp8", "mxfp8", 1, 300000, 8192)
    assert "dq_decode_stream_kernel" not in mxl.mx_gemm_plan("nvfp4", "nvfp4", 1, 600000, 8192)


def test_plan_names_fit_their_buffers():
    # the binding passes its buffer's real length: a long plan name is cut
    # by snprintf inside the buffer, never past it
    for fmt in ("mxfp4", "nvfp4"):
        assert len(mxl.mx_gemm_w4a16_plan(fmt, 96, 160, 4096)) < 512
    small = ctypes.create_string_buffer(16)
    assert L.mx_gemm_w4a16_plan(0, 96, 160, 4096, small, 16) == OK
    assert len(small.value) == 15
    assert L.mx_gemm_plan(0, 0, 8192, 17408, 5120, 0, 0, small, 16) == OK and len(small.value) == 15


def test_global_scale_helper_matches_oracle():
    rng = np.random.default_rng(0)
    vals = np.concatenate([np.ldexp(rng.random(3000) + 0.5, rng.integers(-100, 100, 3000)),
                           [1.0, 3.0, 7.0, 2688.0, 6.0, 448.0, 1e-38, 3e38]]).astype(np.float32)
    for v in vals:
        assert np.float32(L.mx_nv_global_scale(float(v))) == oracle.nv_global_scale(float(v)), v
    assert L.mx_nv_global_scale(0.0) == 1.0
