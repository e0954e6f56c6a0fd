"""CPU oracle for the W4A4 microscaling linear layer -- TEST INFRASTRUCTURE.

This package is the plain, slow, exact definition that the GPU library is
checked against.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import it.  The GPU library
(``fp8_quantized_linear_amd``) never imports it, and the two share no code.

The arithmetic lives in ``mx_oracle.c`` (plain C, fp64, OpenMP over rows);
this module only builds it with gcc and marshals numpy arrays through ctypes.
Every function states the passage it follows in the C source; in short:

* element codes: E2M1 / E4M3 / E8M0 of the OCP Microscaling specification,
  which the Qwen3.8-27B-MXFP8Attn-MXFP4MLP-lmheadMXFP4 card (section 7) names;
* scale rules: EVEN for weights (Qwen3.5-27B-MXFP4-QAD-W4A4-LR1e-5-s1000,
  "How this checkpoint was produced"), CEIL for activations
  (Qwen3.5-9B-MXFP4-QAD-W4A4-LR1e-5-s3000, "Training mode"), FLOOR (OCP);
* NVFP4 global and block scales (Qwen3.5-27B-NVFP4-RTN-weight-only and
  Qwen3.5-27B-NVFP4-GPTQ, introductions);
* the SwiGLU activation of the gated MLP (fused gate_up projection);
* fake quantization, the quantize -> dequantize round trip rounded to bf16
  (Qwen3.5-9B-MXFP4-QAD-W4A4-LR1e-5-s3000, "Training mode";
  Qwen3.5-27B-MXFP4-QAD-W4A4-LR1e-5-s1000, "How this checkpoint was
  produced", Training row);
* the GEMM as a dot product of dequantized operands in fp64.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "mx_oracle.c")
# MXL_SANITIZED=1 selects the AddressSanitizer + UndefinedBehaviorSanitizer
# build (build(sanitize=True)); the process must then preload clang's ASan
# runtime, as tests/test_sanitized_host.py does.
_SANITIZED = os.environ.get("MXL_SANITIZED") == "1"
_LIB = os.path.join(_HERE, "libmxoracle_san.so" if _SANITIZED else "libmxoracle.so")
_CLANG = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "llvm", "bin", "clang")

E2M1, E4M3 = 0, 1
FLOOR, CEIL, EVEN = 0, 1, 2
ELEMS = {"e2m1": E2M1, "e4m3": E4M3, "mxfp4": E2M1, "mxfp8": E4M3}
RULES = {"floor": FLOOR, "ceil": CEIL, "even": EVEN}

_lib = None


def build(force: bool = True, sanitize: bool = False) -> str:
    """Compile mx_oracle.c with gcc (-O2, no fast-math, OpenMP).  With
    sanitize, into libmxoracle_san.so with clang, AddressSanitizer and
    UndefinedBehaviorSanitizer (any finding aborts), against the shared ASan
    runtime."""
    out = os.path.join(_HERE, "libmxoracle_san.so" if sanitize else "libmxoracle.so")
    if force or not os.path.exists(out) or os.path.getmtime(out) < os.path.getmtime(_SRC):
        tmp = out + ".tmp"
        if sanitize:
            llvm_lib = os.path.join(os.path.dirname(os.path.dirname(_CLANG)), "lib")
            cmd = [_CLANG, "-O1", "-g", "-std=c11", "-Wall", "-fopenmp", "-fPIC", "-shared",
                   "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer",
                   "-shared-libsan", f"-Wl,-rpath,{llvm_lib}", "-o", tmp, _SRC, "-lm"]
        else:
            cmd = ["gcc", "-O2", "-std=c11", "-Wall", "-fopenmp", "-fPIC", "-shared", "-o", tmp, _SRC, "-lm"]
        subprocess.check_call(cmd)
        os.replace(tmp, out)
    return out


def _nthreads(n=None) -> int:
    if n:
        return int(n)
    env = os.environ.get("OMP_NUM_THREADS")
    return int(env) if env else (os.cpu_count() or 1)


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build(force=True, sanitize=_SANITIZED)
        L = ctypes.CDLL(_LIB)
        d, i32, i64, u16, f32 = (ctypes.c_double, ctypes.c_int, ctypes.c_int64, ctypes.c_uint16,
                                 ctypes.c_float)
        P = ctypes.c_void_p
        L.orc_bf16_value.restype, L.orc_bf16_value.argtypes = d, [u16]
        for f in (L.orc_e2m1_value, L.orc_e4m3_value, L.orc_e8m0_value):
            f.restype, f.argtypes = d, [i32]
        L.orc_encode.restype, L.orc_encode.argtypes = i32, [i32, d]
        L.orc_scale_exponent.restype, L.orc_scale_exponent.argtypes = i32, [d, i32, i32]
        L.orc_mx_quantize.restype = i32
        L.orc_mx_quantize.argtypes = [i32, i32, P, i64, i64, P, P, i32]
        L.orc_mx_dequantize.restype = i32
        L.orc_mx_dequantize.argtypes = [i32, P, P, i64, i64, P, i32]
        L.orc_bf16_amax.restype, L.orc_bf16_amax.argtypes = d, [P, i64]
        L.orc_nv_global_scale.restype, L.orc_nv_global_scale.argtypes = f32, [d]
        L.orc_nv_quantize.restype = i32
        L.orc_nv_quantize.argtypes = [P, i64, i64, f32, P, P, i32]
        L.orc_nv_dequantize.restype = i32
        L.orc_nv_dequantize.argtypes = [P, P, i64, i64, f32, P, i32]
        L.orc_gemm_dq.restype = i32
        L.orc_gemm_dq.argtypes = [P, P, i64, i64, i64, P, P, i32]
        L.orc_gemm_dq_pairs.restype = i32
        L.orc_gemm_dq_pairs.argtypes = [P, P, i64, P, P, i64, P, P, i32]
        L.orc_bf16_nearest_ratio.restype, L.orc_bf16_nearest_ratio.argtypes = u16, [d, d]
        L.orc_fake_quant.restype = i32
        L.orc_fake_quant.argtypes = [i32, i32, P, i64, i64, f32, P, i32]
        L.orc_mx_gemm.restype = i32
        L.orc_mx_gemm.argtypes = [i32, P, P, i32, P, P, i64, i64, i64, P, P, i32]
        _lib = L
    return _lib


def _ptr(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"], "oracle inputs must be C-contiguous"
    return a.ctypes.data_as(ctypes.c_void_p)


def _elem(e) -> int:
    return ELEMS[e] if isinstance(e, str) else int(e)


def _rule(r) -> int:
    return RULES[r] if isinstance(r, str) else int(r)


# ---------------------------------------------------------------- scalars
def bf16_value(bits: int) -> float:
    return lib().orc_bf16_value(int(bits))


def e2m1_value(code: int) -> float:
    return lib().orc_e2m1_value(int(code))


def e4m3_value(code: int) -> float:
    return lib().orc_e4m3_value(int(code))


def e8m0_value(code: int) -> float:
    return lib().orc_e8m0_value(int(code))


def encode(elem, r: float) -> int:
    """Code of the exact real r (RNE onto the grid, ties to the even code)."""
    return lib().orc_encode(_elem(elem), float(r))


def scale_exponent(amax: float, elem, rule) -> int:
    """Block scale exponent e (scale 2^e) for a block with maximum |x| = amax."""
    return lib().orc_scale_exponent(float(amax), _elem(elem), _rule(rule))


# ---------------------------------------------------------------- tensors
def _u16(x) -> np.ndarray:
    x = np.ascontiguousarray(x)
    assert x.dtype == np.uint16 and x.ndim == 2, "bf16 bit patterns as uint16 [rows, k]"
    return x


def mx_quantize(elem, rule, x_bf16: np.ndarray, nthreads=None):
    """bf16 bits [rows, k] -> (codes, E8M0 scales).  E2M1 codes are nibble
    packed [rows, k/2] (element 2j in the low nibble); E4M3 codes are
    [rows, k]; scales are [rows, k/32]."""
    x = _u16(x_bf16)
    rows, k = x.shape
    e = _elem(elem)
    q = np.zeros((rows, k // 2 if e == E2M1 else k), np.uint8)
    s = np.zeros((rows, k // 32), np.uint8)
    rc = lib().orc_mx_quantize(e, _rule(rule), _ptr(x), rows, k, _ptr(q), _ptr(s),
                               _nthreads(nthreads))
    if rc != 0:
        raise ValueError("k must be a multiple of 32")
    return q, s


def mx_dequantize(elem, q: np.ndarray, s: np.ndarray, rows: int, k: int, nthreads=None):
    out = np.empty((rows, k), np.float64)
    q = np.ascontiguousarray(q)
    s = np.ascontiguousarray(s)
    rc = lib().orc_mx_dequantize(_elem(elem), _ptr(q), _ptr(s), rows, k, _ptr(out),
                                 _nthreads(nthreads))
    if rc != 0:
        raise ValueError("k must be a multiple of 32")
    return out


def bf16_amax(x_bf16: np.ndarray) -> float:
    x = np.ascontiguousarray(x_bf16)
    return lib().orc_bf16_amax(_ptr(x), x.size)


def nv_global_scale(amax: float) -> np.float32:
    """g = RNE_fp32(448 * 6 / amax), 1 when amax is 0."""
    return np.float32(lib().orc_nv_global_scale(float(amax)))


def nv_quantize(x_bf16: np.ndarray, g: float, nthreads=None):
    """bf16 bits [rows, k] -> (E2M1 nibbles [rows, k/2], E4M3 scales [rows, k/16])."""
    x = _u16(x_bf16)
    rows, k = x.shape
    q = np.zeros((rows, k // 2), np.uint8)
    s = np.zeros((rows, k // 16), np.uint8)
    rc = lib().orc_nv_quantize(_ptr(x), rows, k, float(np.float32(g)), _ptr(q), _ptr(s),
                               _nthreads(nthreads))
    if rc != 0:
        raise ValueError("k must be a multiple of 16")
    return q, s


def nv_dequantize(q, s, rows, k, g, nthreads=None):
    out = np.empty((rows, k), np.float64)
    q = np.ascontiguousarray(q)
    s = np.ascontiguousarray(s)
    rc = lib().orc_nv_dequantize(_ptr(q), _ptr(s), rows, k, float(np.float32(g)), _ptr(out),
                                 _nthreads(nthreads))
    if rc != 0:
        raise ValueError("k must be a multiple of 16")
    return out


def gemm_dq(a: np.ndarray, w: np.ndarray, nthreads=None):
    """Y = A W^T and S = |A| |W|^T-style absolute sums over dequantized fp64
    operands A [m, k], W [n, k]."""
    a = np.ascontiguousarray(a, np.float64)
    w = np.ascontiguousarray(w, np.float64)
    m, k = a.shape
    n = w.shape[0]
    y = np.empty((m, n), np.float64)
    sa = np.empty((m, n), np.float64)
    lib().orc_gemm_dq(_ptr(a), _ptr(w), m, n, k, _ptr(y), _ptr(sa), _nthreads(nthreads))
    return y, sa


def gemm_dq_pairs(a: np.ndarray, w: np.ndarray, mi, ni, nthreads=None):
    """Selected entries (mi[t], ni[t]) of Y = A W^T and of S."""
    a = np.ascontiguousarray(a, np.float64)
    w = np.ascontiguousarray(w, np.float64)
    mi = np.ascontiguousarray(mi, np.int64)
    ni = np.ascontiguousarray(ni, np.int64)
    y = np.empty(mi.shape[0], np.float64)
    sa = np.empty(mi.shape[0], np.float64)
    lib().orc_gemm_dq_pairs(_ptr(a), _ptr(w), a.shape[1], _ptr(mi), _ptr(ni), mi.shape[0],
                            _ptr(y), _ptr(sa), _nthreads(nthreads))
    return y, sa


def mx_gemm(a_elem, aq, a_s, w_elem, wq, w_s, m: int, n: int, k: int, nthreads=None):
    """Y and S straight from MX codes and E8M0 scales (decoded on the fly)."""
    aq, a_s, wq, w_s = (np.ascontiguousarray(t) for t in (aq, a_s, wq, w_s))
    y = np.empty((m, n), np.float64)
    sa = np.empty((m, n), np.float64)
    rc = lib().orc_mx_gemm(_elem(a_elem), _ptr(aq), _ptr(a_s), _elem(w_elem), _ptr(wq), _ptr(w_s),
                           m, n, k, _ptr(y), _ptr(sa), _nthreads(nthreads))
    if rc != 0:
        raise ValueError("k must be a multiple of 32")
    return y, sa


def bf16_to_f64(x_bf16: np.ndarray) -> np.ndarray:
    """Exact values of bf16 bit patterns [rows, k]: a bf16 is the upper half
    of an fp32."""
    x = _u16(x_bf16)
    return (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def w4a16_gemm(a_bf16, wq, w_s, n: int, k: int, fmt: str = "mxfp4", g_w=None, nthreads=None):
    """Weight-only quantized linear (W4A16): the bf16 activations as they are
    times the dequantized packed weights, in fp64.  One packed artifact serves
    W4A4 and W4A16 (Qwen3.5-27B-MXFP4-QAD-W4A4-LR1e-5-s1000, introduction),
    and the NVFP4 weight-only checkpoint keeps its activations in bf16 with
    weight bytes identical to the W4A4 sibling
    (Qwen3.5-27B-NVFP4-RTN-weight-only, introduction).  MXFP4 weights
    dequantize as e2m1 * 2^(s - 127), NVFP4 weights as e2m1 * s_e4m3 / g_w.
    Returns (y, S) as gemm_dq does."""
    a = bf16_to_f64(a_bf16)
    if fmt == "nvfp4":
        wd = nv_dequantize(wq, w_s, n, k, g_w, nthreads)
    elif fmt == "mxfp4":
        wd = mx_dequantize("e2m1", wq, w_s, n, k, nthreads)
    else:
        raise ValueError("W4A16 weights are mxfp4 or nvfp4")
    return gemm_dq(a, wd, nthreads)


FAKE_FMT = {"mxfp4": 0, "mxfp8": 1, "nvfp4": 2}


def bf16_nearest_ratio(p: float, g: float) -> int:
    """bf16 bits (sign clear) nearest to the exact ratio p / g, ties to even."""
    return int(lib().orc_bf16_nearest_ratio(float(p), float(g)))


def fake_quant(fmt: str, rule, x_bf16: np.ndarray, g=None, nthreads=None) -> np.ndarray:
    """Quantize -> dequantize -> nearest bf16 (the training-time fake-quant
    op).  MX formats use the block rule `rule`; NVFP4 uses the global scale
    g.  Returns bf16 bit patterns [rows, k]."""
    x = _u16(x_bf16)
    rows, k = x.shape
    out = np.empty((rows, k), np.uint16)
    rc = lib().orc_fake_quant(FAKE_FMT[fmt], _rule(rule) if rule is not None else 0, _ptr(x), rows, k,
                              float(np.float32(g if g is not None else 1.0)), _ptr(out), _nthreads(nthreads))
    if rc != 0:
        raise ValueError("bad format or k not a multiple of the block")
    return out


def swiglu(gate, up) -> np.ndarray:
    """The gated MLP activation between the fused gate_up projection and the
    down projection: h = silu(gate) * up = gate * up / (1 + e^-gate),
    elementwise in fp64.  (The cards name vLLM's fused gate_up_proj,
    Qwen3.8-27B-MXFP8Attn-MXFP4MLP-lmheadMXFP4 section 2; the Qwen MLP gates
    with SiLU.)"""
    g = np.asarray(gate, np.float64)
    u = np.asarray(up, np.float64)
    with np.errstate(over="ignore"):
        return g * u / (1.0 + np.exp(-g))


def mlp_swiglu(aq, a_s, wq, w_s, m: int, inter: int, k: int, nthreads=None):
    """The gate_up projection of MXFP4 operands followed by SwiGLU, exactly:
    W is [2 * inter, k] with the gate rows first, then the up rows.  Returns
    (h, gate, up, S_gate, S_up) with S the absolute sums of the products."""
    y, sa = mx_gemm("e2m1", aq, a_s, "e2m1", wq, w_s, m, 2 * inter, k, nthreads)
    gate, up = y[:, :inter], y[:, inter:]
    return swiglu(gate, up), gate, up, sa[:, :inter], sa[:, inter:]


# ---------------------------------------------------------------- compositions
def mx_linear(a_bf16, w_bf16, a_elem="e2m1", w_elem="e2m1", a_rule="ceil", w_rule="even",
              nthreads=None):
    """The whole MX path on the CPU: pack W, quantize A, dequantized fp64 GEMM.
    Returns (y, S, (aq, as), (wq, ws))."""
    aq, a_s = mx_quantize(a_elem, a_rule, a_bf16, nthreads)
    wq, w_s = mx_quantize(w_elem, w_rule, w_bf16, nthreads)
    m, k = a_bf16.shape
    n = w_bf16.shape[0]
    ad = mx_dequantize(a_elem, aq, a_s, m, k, nthreads)
    wd = mx_dequantize(w_elem, wq, w_s, n, k, nthreads)
    y, sa = gemm_dq(ad, wd, nthreads)
    return y, sa, (aq, a_s), (wq, w_s)
