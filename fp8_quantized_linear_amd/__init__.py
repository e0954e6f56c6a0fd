"""fp8_quantized_linear_amd -- Python binding of libmxlinear.so, the gfx950
(MI355X) library for the W4A4 microscaling linear layer.

The binding only marshals arguments: it checks tensor dtypes, shapes and
devices, allocates outputs with torch (device memory is torch's job here) and
passes raw pointers plus the current HIP stream to the C ABI declared in
``include/mxlinear.h``.  Every step of the computation runs in the library's
HIP kernels; there is no fallback path.  If the library is missing, importing
this package raises.

Entry points (same names as the C ABI):
    mx_pack_weights, mx_quantize_act, mx_gemm, mx_gemm_fused, nv_gemm,
    mx_tensor_amax, mx_nv_global_scale, mx_gemm_plan
"""
from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
# MXL_SANITIZED=1 loads the build whose host layer runs under ASan and UBSan
# (build.build_sanitized); the process must preload clang's ASan runtime.
LIB_PATH = os.path.join(_PKG, "libmxlinear_san.so" if os.environ.get("MXL_SANITIZED") == "1" else "libmxlinear.so")

FORMATS = {"mxfp4": 0, "mxfp8": 1, "nvfp4": 2}
RULES = {"floor": 0, "ceil": 1, "even": 2}
MX_OUT_F32 = 0x1
MX_FP8_FAST = 0x2
MX_DEBUG_DUMP_AQ = 0x4
MX_FUSED_IN_GEMM = 0x8
STATUS = {0: "MX_OK", 1: "MX_ERR_INVALID_ARG", 2: "MX_ERR_SHAPE", 3: "MX_ERR_ALIGN",
          4: "MX_ERR_WORKSPACE", 5: "MX_ERR_UNSUPPORTED", 6: "MX_ERR_HIP"}


class MXError(RuntimeError):
    def __init__(self, status: int, where: str, message: str):
        super().__init__(f"{where}: {STATUS.get(status, status)} ({message})")
        self.status = status


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it first (python -c 'import __graft_entry__ as g; g.build()' "
            "or python fp8_quantized_linear_amd/build.py)")
    L = ctypes.CDLL(LIB_PATH)
    P, i32, i64, u32, f32, sz = (ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_uint,
                                 ctypes.c_float, ctypes.c_size_t)
    L.mx_abi_version.restype, L.mx_abi_version.argtypes = i32, []
    L.mx_status_string.restype, L.mx_status_string.argtypes = ctypes.c_char_p, [i32]
    for f in (L.mx_quantize_act, L.mx_pack_weights):
        f.restype, f.argtypes = i32, [i32, i32, P, i64, i64, f32, P, P, P]
    L.mx_gemm.restype = i32
    L.mx_gemm.argtypes = [i32, i32, P, P, P, P, i64, i64, i64, P, P, sz, u32, P]
    L.mx_gemm_noalloc.restype = i32
    L.mx_gemm_noalloc.argtypes = [i32, i32, P, P, P, P, i64, i64, i64, P, u32, P]
    L.mx_gemm_fused.restype = i32
    L.mx_gemm_fused.argtypes = [i32, i32, P, i32, P, P, i64, i64, i64, P, P, sz, u32, P]
    L.nv_gemm.restype = i32
    L.nv_gemm.argtypes = [P, P, P, P, i64, i64, i64, f32, P, P, sz, u32, P]
    L.mx_gemm_w4a16.restype = i32
    L.mx_gemm_w4a16.argtypes = [i32, P, P, P, i64, i64, i64, f32, P, P, sz, u32, P]
    L.mx_gemm_w4a16_plan.restype = i32
    L.mx_gemm_w4a16_plan.argtypes = [i32, i64, i64, i64, ctypes.c_char_p, sz]
    L.mx_gemm_swiglu_quant.restype = i32
    L.mx_gemm_swiglu_quant.argtypes = [P, P, P, P, i64, i64, i64, P, P, P]
    L.mx_gemm_swiglu_quant_plan.restype = i32
    L.mx_gemm_swiglu_quant_plan.argtypes = [i64, i64, i64, ctypes.c_char_p, sz]
    L.mx_swiglu_quant.restype = i32
    L.mx_swiglu_quant.argtypes = [P, i64, i64, P, P, P]
    L.mx_gemm_fused_workspace_size.restype = i32
    L.mx_gemm_fused_workspace_size.argtypes = [i32, i32, i64, i64, i64, u32, ctypes.POINTER(sz)]
    L.mx_gemm_workspace_size.restype = i32
    L.mx_gemm_workspace_size.argtypes = [i32, i32, i64, i64, i64, u32, ctypes.POINTER(sz)]
    L.mx_gemm_w4a16_workspace_size.restype = i32
    L.mx_gemm_w4a16_workspace_size.argtypes = [i32, i64, i64, i64, ctypes.POINTER(sz)]
    L.mx_fake_quant.restype = i32
    L.mx_fake_quant.argtypes = [i32, i32, P, i64, i64, f32, P, P]
    L.mx_tensor_amax.restype, L.mx_tensor_amax.argtypes = i32, [P, i64, P, P]
    L.mx_nv_global_scale.restype, L.mx_nv_global_scale.argtypes = f32, [f32]
    L.mx_gemm_plan.restype = i32
    L.mx_gemm_plan.argtypes = [i32, i32, i64, i64, i64, i32, u32, ctypes.c_char_p, sz]
    return L


lib = _load()
ABI_VERSION = lib.mx_abi_version()


def _check(status: int, where: str):
    if status != 0:
        raise MXError(status, where, lib.mx_status_string(status).decode())


def _stream(t: torch.Tensor):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _ptr(t: torch.Tensor | None):
    return ctypes.c_void_p(0 if t is None else t.data_ptr())


def _need(t: torch.Tensor, dtype, name: str):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _fmt(f):
    return FORMATS[f] if isinstance(f, str) else int(f)


def _rule(r):
    if r is None:  # NVFP4 takes no rule
        return 0
    return RULES[r] if isinstance(r, str) else int(r)


def codes_per_row(fmt: str, k: int) -> int:
    """Bytes of codes per row of k elements."""
    return k if fmt == "mxfp8" else k // 2


def scales_per_row(fmt: str, k: int) -> int:
    return k // 16 if fmt == "nvfp4" else k // 32


def _quantize(entry, x: torch.Tensor, fmt: str, rule: str, global_scale: float, out=None):
    _need(x, torch.bfloat16, "input")
    if x.dim() != 2:
        raise ValueError("input must be [rows, k]")
    rows, k = x.shape
    if out is None:
        q = torch.empty((rows, codes_per_row(fmt, k)), dtype=torch.uint8, device=x.device)
        s = torch.empty((rows, scales_per_row(fmt, k)), dtype=torch.uint8, device=x.device)
    else:
        q, s = out
    st = entry(_fmt(fmt), _rule(rule), _ptr(x), rows, k, float(global_scale), _ptr(q), _ptr(s),
               _stream(x))
    _check(st, entry.__name__)
    return q, s


def mx_quantize_act(a: torch.Tensor, fmt: str = "mxfp4", rule: str = "ceil",
                    global_scale: float = 1.0, out=None):
    """Dynamic per-token activation quantization of bf16 a[m, k] -> (codes, scales)."""
    return _quantize(lib.mx_quantize_act, a, fmt, rule, global_scale, out)


def mx_pack_weights(w: torch.Tensor, fmt: str = "mxfp4", rule: str = "even",
                    global_scale: float = 1.0, out=None):
    """Round-to-nearest packing of bf16 w[n, k] -> (codes, scales)."""
    return _quantize(lib.mx_pack_weights, w, fmt, rule, global_scale, out)


def _gemm_out(m, n, device, out_f32, y):
    if y is not None:
        return y
    return torch.empty((m, n), dtype=torch.float32 if out_f32 else torch.bfloat16, device=device)


def _flags(out_f32, fp8_fast):
    return (MX_OUT_F32 if out_f32 else 0) | (MX_FP8_FAST if fp8_fast else 0)


def _workspace(query, device, *args):
    """Split-K scratch of the size the library asks for (None when 0), from
    torch's caching allocator on the call's stream."""
    n = ctypes.c_size_t(0)
    _check(query(*args, ctypes.byref(n)), query.__name__)
    if n.value == 0:
        return None, 0
    return torch.empty(n.value, dtype=torch.uint8, device=device), n.value


def mx_gemm_workspace_size(a_fmt: str, w_fmt: str, m: int, n: int, k: int, fp8_fast: bool = False) -> int:
    b = ctypes.c_size_t(0)
    _check(lib.mx_gemm_workspace_size(_fmt(a_fmt), _fmt(w_fmt), m, n, k, _flags(False, fp8_fast), ctypes.byref(b)),
           "mx_gemm_workspace_size")
    return b.value


def mx_gemm(a_q, a_s, w_q, w_s, k: int, a_fmt: str = "mxfp4", w_fmt: str = "mxfp4",
            out_f32: bool = False, y=None, fp8_fast: bool = False, split_k: bool = True):
    """Y[m, n] = A W^T on MX codes/scales (bf16 out, or fp32 with out_f32).
    a_fmt and w_fmt may differ (mixed MXFP8 x MXFP4 pairs).  fp8_fast selects
    the FP8 matrix cores for pairs with an MXFP8 operand (inexact
    accumulation).  split_k passes the split-K workspace the library asks
    for on this shape."""
    for t, nm in ((a_q, "a_q"), (a_s, "a_s"), (w_q, "w_q"), (w_s, "w_s")):
        _need(t, torch.uint8, nm)
    m, n = a_q.shape[0], w_q.shape[0]
    if a_q.shape[1] != codes_per_row(a_fmt, k) or w_q.shape[1] != codes_per_row(w_fmt, k):
        raise ValueError("code tensors do not match k")
    if a_s.shape != (m, k // 32) or w_s.shape != (n, k // 32):
        raise ValueError("scale tensors do not match k")
    y = _gemm_out(m, n, a_q.device, out_f32, y)
    ws, wsb = _workspace(lib.mx_gemm_workspace_size, a_q.device, _fmt(a_fmt), _fmt(w_fmt), m, n, k,
                         _flags(out_f32, fp8_fast)) if split_k else (None, 0)
    st = lib.mx_gemm(_fmt(a_fmt), _fmt(w_fmt), _ptr(a_q), _ptr(a_s), _ptr(w_q), _ptr(w_s), m, n, k,
                     _ptr(y), _ptr(ws), wsb, _flags(out_f32, fp8_fast), _stream(a_q))
    _check(st, "mx_gemm")
    return y


def mx_gemm_noalloc(a_q, a_s, w_q, w_s, k: int, a_fmt: str = "mxfp4", w_fmt: str = "mxfp4",
                    out_f32: bool = False, y=None, fp8_fast: bool = False):
    """mx_gemm without a workspace argument: split-K partials go to the
    library's static device scratch (for callers that cannot allocate; calls
    overlapping on one GPU race).  Pass `y` to allocate nothing here either."""
    for t, nm in ((a_q, "a_q"), (a_s, "a_s"), (w_q, "w_q"), (w_s, "w_s")):
        _need(t, torch.uint8, nm)
    m, n = a_q.shape[0], w_q.shape[0]
    if a_q.shape[1] != codes_per_row(a_fmt, k) or w_q.shape[1] != codes_per_row(w_fmt, k):
        raise ValueError("code tensors do not match k")
    if a_s.shape != (m, k // 32) or w_s.shape != (n, k // 32):
        raise ValueError("scale tensors do not match k")
    y = _gemm_out(m, n, a_q.device, out_f32, y)
    st = lib.mx_gemm_noalloc(_fmt(a_fmt), _fmt(w_fmt), _ptr(a_q), _ptr(a_s), _ptr(w_q), _ptr(w_s), m, n, k,
                             _ptr(y), _flags(out_f32, fp8_fast), _stream(a_q))
    _check(st, "mx_gemm_noalloc")
    return y


def mx_gemm_fused_workspace_size(a_fmt: str, w_fmt: str, m: int, n: int, k: int, fp8_fast: bool = False,
                                 in_gemm: bool = False) -> int:
    b = ctypes.c_size_t(0)
    flags = _flags(False, fp8_fast) | (MX_FUSED_IN_GEMM if in_gemm else 0)
    _check(lib.mx_gemm_fused_workspace_size(_fmt(a_fmt), _fmt(w_fmt), m, n, k, flags, ctypes.byref(b)),
           "mx_gemm_fused_workspace_size")
    return b.value


def mx_gemm_fused(a: torch.Tensor, w_q, w_s, a_fmt: str = "mxfp4", a_rule: str = "ceil",
                  w_fmt: str = "mxfp4", out_f32: bool = False, y=None, fp8_fast: bool = False,
                  dump_aq: bool = False, quantize_once: bool = True, workspace=None, in_gemm: bool = False):
    """mx_gemm with the activation quantization done inside the GEMM from bf16 a[m, k].
    dump_aq also returns the codes and scales the prologue computed:
    (y, (a_q, a_s)).  quantize_once passes the workspace the library asks for
    (large shapes: A is quantized once into it, by the standalone quantizer
    or, with in_gemm, by the GEMM's own workgroups, instead of once per tile
    column; mixed pairs: required); `workspace` (uint8, on a's device,
    256-byte aligned as torch allocates) is used instead when given."""
    _need(a, torch.bfloat16, "a")
    _need(w_q, torch.uint8, "w_q")
    _need(w_s, torch.uint8, "w_s")
    m, k = a.shape
    n = w_q.shape[0]
    if w_q.shape[1] != codes_per_row(w_fmt, k) or w_s.shape != (n, k // 32):
        raise ValueError("weight tensors do not match k")
    y = _gemm_out(m, n, a.device, out_f32, y)
    flags = _flags(out_f32, fp8_fast) | (MX_FUSED_IN_GEMM if in_gemm else 0)
    ws, wsb, qb = None, 0, m * codes_per_row(a_fmt, k)
    if dump_aq:
        wsb = qb + m * (k // 32)
        ws = torch.empty(wsb, dtype=torch.uint8, device=a.device)
        flags |= MX_DEBUG_DUMP_AQ
    elif workspace is not None:
        _need(workspace, torch.uint8, "workspace")
        ws, wsb = workspace, workspace.numel()
    elif quantize_once or a_fmt != w_fmt:
        ws, wsb = _workspace(lib.mx_gemm_fused_workspace_size, a.device, _fmt(a_fmt), _fmt(w_fmt), m, n, k, flags)
    st = lib.mx_gemm_fused(_fmt(a_fmt), _fmt(w_fmt), _ptr(a), _rule(a_rule), _ptr(w_q), _ptr(w_s),
                           m, n, k, _ptr(y), _ptr(ws), wsb, flags, _stream(a))
    _check(st, "mx_gemm_fused")
    if dump_aq:
        return y, (ws[:qb].view(m, codes_per_row(a_fmt, k)), ws[qb:].view(m, k // 32))
    return y


def nv_gemm(a_q, a_s, w_q, w_s, k: int, alpha: float, out_f32: bool = False, y=None, split_k: bool = True):
    """NVFP4 GEMM: Y = alpha * sum_k dq(A) dq(W) with E4M3 block-16 scales."""
    for t, nm in ((a_q, "a_q"), (a_s, "a_s"), (w_q, "w_q"), (w_s, "w_s")):
        _need(t, torch.uint8, nm)
    m, n = a_q.shape[0], w_q.shape[0]
    if a_q.shape[1] != k // 2 or w_q.shape[1] != k // 2 or a_s.shape != (m, k // 16) \
            or w_s.shape != (n, k // 16):
        raise ValueError("NVFP4 tensors do not match k")
    y = _gemm_out(m, n, a_q.device, out_f32, y)
    ws, wsb = _workspace(lib.mx_gemm_workspace_size, a_q.device, FORMATS["nvfp4"], FORMATS["nvfp4"], m, n, k,
                         0) if split_k else (None, 0)
    st = lib.nv_gemm(_ptr(a_q), _ptr(a_s), _ptr(w_q), _ptr(w_s), m, n, k, float(alpha), _ptr(y),
                     _ptr(ws), wsb, MX_OUT_F32 if out_f32 else 0, _stream(a_q))
    _check(st, "nv_gemm")
    return y


def mx_gemm_w4a16(a: torch.Tensor, w_q, w_s, w_fmt: str = "mxfp4", alpha: float = 1.0,
                  out_f32: bool = False, y=None, split_k: bool = True):
    """Weight-only quantized linear (W4A16): Y = alpha * A_bf16 dq(W)^T with
    MXFP4 (E8M0 per 32) or NVFP4 (E4M3 per 16; alpha = 1 / g_w) weights."""
    _need(a, torch.bfloat16, "a")
    _need(w_q, torch.uint8, "w_q")
    _need(w_s, torch.uint8, "w_s")
    if w_fmt not in ("mxfp4", "nvfp4"):
        raise ValueError("W4A16 weights are mxfp4 or nvfp4")
    m, k = a.shape
    n = w_q.shape[0]
    if w_q.shape[1] != k // 2 or w_s.shape != (n, scales_per_row(w_fmt, k)):
        raise ValueError("weight tensors do not match k")
    y = _gemm_out(m, n, a.device, out_f32, y)
    ws, wsb = _workspace(lib.mx_gemm_w4a16_workspace_size, a.device, _fmt(w_fmt), m, n, k) if split_k \
        else (None, 0)
    st = lib.mx_gemm_w4a16(_fmt(w_fmt), _ptr(a), _ptr(w_q), _ptr(w_s), m, n, k, float(alpha), _ptr(y),
                           _ptr(ws), wsb, MX_OUT_F32 if out_f32 else 0, _stream(a))
    _check(st, "mx_gemm_w4a16")
    return y


def mx_gemm_w4a16_plan(w_fmt: str, m: int, n: int, k: int) -> str:
    """Name of the kernel mx_gemm_w4a16 would launch for this shape."""
    buf = ctypes.create_string_buffer(512)
    _check(lib.mx_gemm_w4a16_plan(_fmt(w_fmt), m, n, k, buf, len(buf)), "mx_gemm_w4a16_plan")
    return buf.value.decode()


def gate_up_interleave_index(inter: int, device=None) -> torch.Tensor:
    """Row order that turns a [gate; up] weight ([2*inter, k], gate rows
    first) into the layout mx_gemm_swiglu_quant reads: 32 gate rows, then
    the 32 up rows of the same columns, and so on."""
    if inter % 32 != 0:
        raise ValueError("inter must be a multiple of 32")
    c = torch.arange(inter // 32, device=device).repeat_interleave(64) * 32
    r = torch.arange(64, device=device).repeat(inter // 32)
    return torch.where(r < 32, c + r, inter + c + r - 32)


def interleave_gate_up(w: torch.Tensor) -> torch.Tensor:
    """Rows of a [gate; up] tensor (bf16 weights, or packed codes or scales,
    since packing is row-local) in the order mx_gemm_swiglu_quant reads."""
    return w.index_select(0, gate_up_interleave_index(w.shape[0] // 2, w.device)).contiguous()


def mx_swiglu_quant(x: torch.Tensor, out=None):
    """x [m, 2*inter] bf16 (gate columns, then up) -> MXFP4 codes [m, inter/2]
    and CEIL scales [m, inter/32] of SwiGLU(gate, up)."""
    _need(x, torch.bfloat16, "input")
    if x.dim() != 2 or x.shape[1] % 2:
        raise ValueError("input must be [m, 2*inter]")
    m, inter = x.shape[0], x.shape[1] // 2
    if out is None:
        q = torch.empty((m, inter // 2), dtype=torch.uint8, device=x.device)
        s = torch.empty((m, inter // 32), dtype=torch.uint8, device=x.device)
    else:
        q, s = out
    _check(lib.mx_swiglu_quant(_ptr(x), m, inter, _ptr(q), _ptr(s), _stream(x)), "mx_swiglu_quant")
    return q, s


def mx_gemm_swiglu_quant(a_q, a_s, w_q, w_s, k: int, out=None):
    """Fused gate_up GEMM + SwiGLU + CEIL MXFP4 quantization of h.  w_q/w_s
    are the interleaved [2*inter, k] weights (interleave_gate_up)."""
    for t, nm in ((a_q, "a_q"), (a_s, "a_s"), (w_q, "w_q"), (w_s, "w_s")):
        _need(t, torch.uint8, nm)
    m, inter = a_q.shape[0], w_q.shape[0] // 2
    if a_q.shape[1] != k // 2 or w_q.shape != (2 * inter, k // 2):
        raise ValueError("code tensors do not match k")
    if a_s.shape != (m, k // 32) or w_s.shape != (2 * inter, k // 32):
        raise ValueError("scale tensors do not match k")
    if out is None:
        q = torch.empty((m, inter // 2), dtype=torch.uint8, device=a_q.device)
        s = torch.empty((m, inter // 32), dtype=torch.uint8, device=a_q.device)
    else:
        q, s = out
    _check(lib.mx_gemm_swiglu_quant(_ptr(a_q), _ptr(a_s), _ptr(w_q), _ptr(w_s), m, inter, k, _ptr(q), _ptr(s),
                                    _stream(a_q)), "mx_gemm_swiglu_quant")
    return q, s


def mx_gemm_swiglu_quant_plan(m: int, inter: int, k: int) -> str:
    buf = ctypes.create_string_buffer(512)
    _check(lib.mx_gemm_swiglu_quant_plan(m, inter, k, buf, len(buf)), "mx_gemm_swiglu_quant_plan")
    return buf.value.decode()


def mx_fake_quant(x: torch.Tensor, fmt: str = "mxfp4", rule: str = "ceil", global_scale: float = 1.0,
                  out: torch.Tensor | None = None) -> torch.Tensor:
    """Quantize -> dequantize -> bf16 with the serving quantizer's codes
    (mx_fake_quant of the C ABI).  x [rows, k] bf16; returns [rows, k] bf16."""
    _need(x, torch.bfloat16, "input")
    if x.dim() != 2:
        raise ValueError("input must be [rows, k]")
    y = torch.empty_like(x) if out is None else out
    _need(y, torch.bfloat16, "out")
    if y.shape != x.shape:
        raise ValueError("out must have the input's shape")
    st = lib.mx_fake_quant(_fmt(fmt), _rule(rule), _ptr(x), x.shape[0], x.shape[1], float(global_scale),
                           _ptr(y), _stream(x))
    _check(st, "mx_fake_quant")
    return y


class FakeQuantSTE(torch.autograd.Function):
    """mx_fake_quant forward with the straight-through gradient (identity)."""

    @staticmethod
    def forward(ctx, x, fmt="mxfp4", rule="ceil", global_scale=1.0):
        return mx_fake_quant(x, fmt, rule, global_scale)

    @staticmethod
    def backward(ctx, grad):
        return grad, None, None, None


def mx_tensor_amax(x: torch.Tensor) -> torch.Tensor:
    """Largest |x| of a bf16 tensor, as a 1-element fp32 GPU tensor."""
    _need(x, torch.bfloat16, "x")
    out = torch.empty(1, dtype=torch.float32, device=x.device)
    _check(lib.mx_tensor_amax(_ptr(x), x.numel(), _ptr(out), _stream(x)), "mx_tensor_amax")
    return out


def mx_nv_global_scale(amax: float) -> float:
    """g = RNE_fp32(448 * 6 / amax) (host helper)."""
    return float(lib.mx_nv_global_scale(float(amax)))


def mx_gemm_plan(a_fmt: str, w_fmt: str, m: int, n: int, k: int, fused: bool = False,
                 fp8_fast: bool = False, in_gemm: bool = False) -> str:
    """Name of the kernel/tile configuration the GEMM would launch for this shape."""
    buf = ctypes.create_string_buffer(512)
    flags = _flags(False, fp8_fast) | (MX_FUSED_IN_GEMM if in_gemm else 0)
    _check(lib.mx_gemm_plan(_fmt(a_fmt), _fmt(w_fmt), m, n, k, int(fused), flags, buf, len(buf)),
           "mx_gemm_plan")
    return buf.value.decode()
