"""Shared helpers for the GPU parity tests: moving seeded inputs to the GPU,
running the oracle on sampled rows, and the GEMM acceptance bound.

Acceptance bound (per output element), from the per-element error bound
|err| <= 1e-4 * sum_k |a_k w_k| that the GEMM must meet: with an fp32 output
the bound applies as is; with a bf16 output the final rounding of Y to bf16
adds at most half a bf16 ulp of the larger of |y_ref| and |y_gpu|.  If the
absolute sum S is 0 the output must be exactly 0.
"""
from __future__ import annotations

import numpy as np
import torch

import oracle


def cuda_bf16(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def host(t: torch.Tensor) -> np.ndarray:
    return t.cpu().numpy()


def half_ulp_bf16(v: np.ndarray) -> np.ndarray:
    a = np.abs(v)
    out = np.zeros_like(a)
    nz = a > 0
    e = np.floor(np.log2(a[nz]))
    e = np.maximum(e, -126)  # subnormal spacing below the normal range
    out[nz] = np.ldexp(1.0, (e - 8).astype(np.int64))
    return out


FP32_MIN_NORMAL = 2.0 ** -126


def underflow_allowance(k: int) -> float:
    """Absolute allowance for fp32 underflow in a K-long accumulation: each of
    at most K/16 fp32 additions (one per 16-wide matrix-core step at the
    narrowest) can lose a value below the smallest normal fp32 if the
    hardware flushes it."""
    return (k // 16 + 1) * FP32_MIN_NORMAL


def flushed_terms(a_dq: np.ndarray, w_dq: np.ndarray) -> np.ndarray:
    """F[m, n] = sum_k |a_k w_k| over the k where an operand value lies below
    the smallest normal fp32 (2^-126): the terms that the dequantizing GEMMs
    may round or flush.  Computed by the oracle as S minus the same sum over
    the operands with those values zeroed (fp64 cancellation is ~1e-16 S)."""
    _, s_all = oracle.gemm_dq(a_dq, w_dq)
    a_n = np.where(np.abs(a_dq) >= FP32_MIN_NORMAL, a_dq, 0.0)
    w_n = np.where(np.abs(w_dq) >= FP32_MIN_NORMAL, w_dq, 0.0)
    _, s_norm = oracle.gemm_dq(a_n, w_n)
    return np.maximum(s_all - s_norm, 0.0)


def check_gemm(y_gpu: np.ndarray, y_ref: np.ndarray, s_abs: np.ndarray, bf16_out: bool, what: str,
               flushed=None, underflow: float = 0.0):
    """Asserts |y_gpu - y_ref| <= 1e-4 * S (+ half a bf16 ulp for bf16 Y).
    Where operands reach below the fp32 normal range, the GEMM's contract
    adds the sum of the affected terms (`flushed`, from flushed_terms) and an
    accumulation underflow allowance (`underflow`, underflow_allowance(K));
    both default to 0, the contract for operands in the normal range."""
    y_gpu = y_gpu.astype(np.float64)
    err = np.abs(y_gpu - y_ref)
    bound = 1e-4 * s_abs
    if bf16_out:
        bound = bound + half_ulp_bf16(np.maximum(np.abs(y_ref), np.abs(y_gpu)))
    if flushed is not None:
        bound = bound + flushed
    bound = bound + underflow
    bad = ~(err <= bound)
    zero_s = s_abs == 0
    bad |= zero_s & (y_gpu != 0)
    nbad = int(bad.sum())
    if nbad:
        i = np.argwhere(bad)[0]
        i = tuple(i)
        raise AssertionError(f"{what}: {nbad}/{bad.size} outside bound; first at {i}: gpu={y_gpu[i]!r} "
                             f"ref={y_ref[i]!r} S={s_abs[i]!r} bound={bound[i]!r}")
    rel = float((err / np.where(s_abs > 0, s_abs, 1)).max()) if err.size else 0.0
    return rel


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def tile_edges(size: int, tiles=(128, 256)) -> list[int]:
    """Every first and last index of every tile of each size in `tiles`
    (the GEMM kernels tile by 128 and by 256), plus 0 and size - 1."""
    out = {0, size - 1}
    for t in tiles:
        for e in range(t, size, t):
            out.add(e - 1)
            out.add(e)
    return sorted(out)


def sample_pairs(m: int, n: int, count: int, seed: int = 0, tiles=(128, 256)):
    """Output positions to check against the oracle: `count` random (row,
    col) pairs, plus every pair of a tile-edge row and a tile-edge column --
    the first and last row and column of every 128- and 256-wide tile, and
    the last row and column of the output."""
    rng = np.random.default_rng(seed)
    mi = list(rng.integers(0, m, count))
    ni = list(rng.integers(0, n, count))
    em, en = tile_edges(m, tiles), tile_edges(n, tiles)
    gm, gn = np.meshgrid(np.array(em, np.int64), np.array(en, np.int64), indexing="ij")
    mi.extend(gm.ravel().tolist())
    ni.extend(gn.ravel().tolist())
    return np.array(mi, np.int64), np.array(ni, np.int64)


def oracle_rows_mx(elem, rule, bits: np.ndarray, rows: np.ndarray):
    """Oracle quantization of selected rows (row-local, so a sample suffices)."""
    return oracle.mx_quantize(elem, rule, np.ascontiguousarray(bits[rows]))


def double_rounding_trap_scales(count: int = 4, seed: int = 0) -> list[np.float32]:
    """fp32 values g in [1, 2) for which rounding 1/g to fp32 and then to bf16
    gives a different bf16 than rounding 1/g once: the fp32 reciprocal lands
    exactly on a midpoint between two bf16 values, and the even one of the
    two lies on the other side of 1/g.  m * g with the midpoint m (9
    significant bits) and g (24) is exact in fp64, so 1 <=> m * g decides on
    which side of the midpoint 1/g lies."""
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < count:
        mant = rng.integers(1, 1 << 23, 1 << 20, dtype=np.int64)
        g = (1.0 + mant / float(1 << 23)).astype(np.float32)
        r32 = (1.0 / g.astype(np.float64)).astype(np.float32)
        bits = r32.view(np.uint32)
        on_mid = (bits & 0xFFFF) == 0x8000
        above = 1.0 > r32.astype(np.float64) * g.astype(np.float64)   # 1/g above the midpoint
        lower_even = ((bits >> 16) & 1) == 0                           # tie would go down
        pick = on_mid & (above == lower_even)
        out.extend(g[pick][: count - len(out)])
    return out


# ------------------------------------------------------------- quantized-output validity
E2M1_VALS = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
_E2M1_MIDS = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])


def e2m1_values(q: np.ndarray) -> np.ndarray:
    """Signed values of nibble-packed E2M1 codes [rows, k/2] -> [rows, k]."""
    codes = np.stack([q & 0xF, q >> 4], axis=-1).reshape(q.shape[0], -1).astype(np.int64)
    v = E2M1_VALS[codes & 7]
    return np.where(codes & 8, -v, v)


def _rne_bounds(x: np.ndarray):
    """Lowest and highest signed E2M1 lattice values that round-to-nearest of
    the real x can give, either way at an exact midpoint (saturating at 6)."""
    a = np.abs(x)
    strict = (a[..., None] > _E2M1_MIDS).sum(-1)      # midpoints passed
    loose = (a[..., None] >= _E2M1_MIDS).sum(-1)      # ... or reached
    lo = np.where(x < 0, -E2M1_VALS[loose], E2M1_VALS[strict])
    hi = np.where(x < 0, -E2M1_VALS[strict], E2M1_VALS[loose])
    return lo, hi


def check_mxfp4_ceil_intervals(q: np.ndarray, s: np.ndarray, lo: np.ndarray, hi: np.ndarray, what: str):
    """The codes q [rows, k/2] and E8M0 scales s [rows, k/32] must be the
    CEIL-rule MXFP4 quantization of SOME values h with lo <= h <= hi
    elementwise: each block's exponent lies between the CEIL exponents of
    the smallest and the largest possible block maximum, and each code is a
    rounding of some admissible value at that exponent.  Used where the
    quantized values come from arithmetic the oracle can only bound."""
    rows, k = lo.shape
    nb = k // 32
    mag_lo = np.where((lo <= 0) & (hi >= 0), 0.0, np.minimum(np.abs(lo), np.abs(hi)))
    mag_hi = np.maximum(np.abs(lo), np.abs(hi))
    amin = mag_lo.reshape(rows, nb, 32).max(-1)
    amax = mag_hi.reshape(rows, nb, 32).max(-1)
    e = s.astype(np.int64) - 127
    bad = 0
    for r in range(rows):
        for b in range(nb):
            e_lo = oracle.scale_exponent(float(amin[r, b]), "e2m1", "ceil")
            e_hi = oracle.scale_exponent(float(amax[r, b]), "e2m1", "ceil")
            bad += not (e_lo <= e[r, b] <= e_hi)
    assert bad == 0, f"{what}: {bad} block scales outside their admissible range"
    scale = np.ldexp(1.0, np.repeat(e, 32, axis=1))
    vlo, _ = _rne_bounds(lo / scale)
    _, vhi = _rne_bounds(hi / scale)
    v = e2m1_values(q)
    ok = (v >= vlo) & (v <= vhi)
    if not ok.all():
        i = np.argwhere(~ok)[:3].tolist()
        raise AssertionError(f"{what}: {int((~ok).sum())} codes outside their admissible range; first at {i}")
