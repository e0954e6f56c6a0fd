"""Seeded synthetic inputs for the W4A4 microscaling linear layer.

This module is shared by the tests, the smoke check and the benchmark.  It
draws random bf16 tensors and holds the workload shapes; it contains none of
the quantization or GEMM arithmetic.

Recipe (the model-card pages publish no tensors, so these stand in for the
layers they describe: the MLP and lm_head projections of the 27B-class models
and the attention projections of the AutoRound card):

* draws come from ``numpy.random.default_rng(seed)`` (PCG64) as float32 and
  are rounded once to bf16 (round to nearest even, via torch);
* activations A ~ N(0, 1) with seed 0; weights W ~ N(0, 0.02) with seed 1;
* "entry outliers": exactly round(0.01 * M * K) entries of A, picked with
  seed 2 without replacement, are multiplied by 20 before the bf16 rounding;
* "channel outliers": round(0.005 * K) whole columns (input channels) of A,
  picked with seed 2, are multiplied by 30;
* heavy-tailed weights: Student-t with 4 degrees of freedom scaled to a
  standard deviation of 0.02 (t4 has variance 2, so the factor is 0.02/sqrt 2);
* NVFP4 calibration batches b = 1..8 use seeds 100 + b, each N(0, 1) of the
  evaluated activation's shape.

Large tensors are drawn in row chunks from one stream, which gives the same
numbers as a single draw.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np
import torch

SEED_A, SEED_W, SEED_OUTLIER = 0, 1, 2
_CHUNK = 1 << 24  # elements per draw


def _to_bf16_bits(x32: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(x32, np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def _draw(shape, seed: int, kind: str = "normal", std: float = 1.0, dof: float = 4.0) -> np.ndarray:
    """float32 draws of the given shape, chunked along the flat index."""
    rng = np.random.default_rng(seed)
    total = int(np.prod(shape))
    out = np.empty(total, np.float32)
    pos = 0
    while pos < total:
        cnt = min(_CHUNK, total - pos)
        if kind == "normal":
            out[pos:pos + cnt] = rng.standard_normal(cnt, dtype=np.float32)
        elif kind == "t":
            out[pos:pos + cnt] = rng.standard_t(dof, cnt).astype(np.float32)
        else:
            raise ValueError(kind)
        pos += cnt
    out *= np.float32(std)
    return out.reshape(shape)


def normal_bf16(rows: int, cols: int, std: float = 1.0, seed: int = SEED_A) -> np.ndarray:
    return _to_bf16_bits(_draw((rows, cols), seed, "normal", std))


def student_t_bf16(rows: int, cols: int, std: float = 0.02, dof: float = 4.0,
                   seed: int = SEED_W) -> np.ndarray:
    # Var(t_nu) = nu / (nu - 2); scale so the standard deviation is `std`
    scale = std / math.sqrt(dof / (dof - 2.0))
    return _to_bf16_bits(_draw((rows, cols), seed, "t", scale, dof))


def activations_entry_outliers(m: int, k: int, frac: float = 0.01, factor: float = 20.0,
                               seed: int = SEED_A, outlier_seed: int = SEED_OUTLIER) -> np.ndarray:
    x = _draw((m, k), seed, "normal", 1.0)
    count = int(round(frac * m * k))
    idx = np.random.default_rng(outlier_seed).choice(m * k, size=count, replace=False)
    x.reshape(-1)[idx] *= np.float32(factor)
    return _to_bf16_bits(x)


def activations_channel_outliers(m: int, k: int, frac: float = 0.005, factor: float = 30.0,
                                 seed: int = SEED_A, outlier_seed: int = SEED_OUTLIER) -> np.ndarray:
    x = _draw((m, k), seed, "normal", 1.0)
    count = int(round(frac * k))
    cols = np.random.default_rng(outlier_seed).choice(k, size=count, replace=False)
    x[:, cols] *= np.float32(factor)
    return _to_bf16_bits(x)


# --------------------------------------------------------------------------- workloads
@dataclass
class Gemm:
    """One linear layer Y[M, N] = A[M, K] W[N, K]^T and how its inputs are drawn."""
    name: str
    m: int
    k: int
    n: int
    a_fmt: str = "mxfp4"          # mxfp4 | mxfp8 | nvfp4
    w_fmt: str = "mxfp4"
    a_dist: str = "entry_outliers"  # entry_outliers | channel_outliers | normal
    w_dist: str = "normal"          # normal | student_t
    extra: dict = field(default_factory=dict)

    @property
    def flops(self) -> int:
        return 2 * self.m * self.n * self.k

    def activations(self, m: int | None = None) -> np.ndarray:
        m = self.m if m is None else m
        if self.a_dist == "entry_outliers":
            return activations_entry_outliers(m, self.k)
        if self.a_dist == "channel_outliers":
            return activations_channel_outliers(m, self.k)
        return normal_bf16(m, self.k, 1.0, SEED_A)

    def weights(self, n: int | None = None) -> np.ndarray:
        n = self.n if n is None else n
        if self.w_dist == "student_t":
            return student_t_bf16(n, self.k, 0.02, 4.0, SEED_W)
        return normal_bf16(n, self.k, 0.02, SEED_W)

    def calibration_batches(self):
        """NVFP4 activation calibration: 8 batches, seeds 101..108."""
        for b in range(1, 9):
            yield normal_bf16(self.m, self.k, 1.0, 100 + b)


SMALL = Gemm("mxfp4_small_16x256x256", 16, 256, 256)
DECODE = [Gemm(f"mxfp4_decode_m{m}_k5120_n17408", m, 5120, 17408, a_dist="channel_outliers",
               w_dist="student_t") for m in (1, 8, 32)]
PREFILL_UP = Gemm("mxfp4_prefill_up_8192x5120x17408", 8192, 5120, 17408)
PREFILL_DOWN = Gemm("mxfp4_prefill_down_8192x17408x5120", 8192, 17408, 5120)
NVFP4 = Gemm("nvfp4_4096x5120x5120", 4096, 5120, 5120, "nvfp4", "nvfp4", a_dist="normal")
MXFP8_ATTN = Gemm("mxfp8_attn_4096x5120x6144", 4096, 5120, 6144, "mxfp8", "mxfp8")
MXFP4_VOCAB = Gemm("mxfp4_vocab_4096x5120x151936", 4096, 5120, 151936)
# the gated MLP's fused gate_up projection (gate rows, then up rows: 2 x
# 17408) whose SwiGLU output feeds PREFILL_DOWN
MLP_GATE_UP = Gemm("mxfp4_mlp_gate_up_8192x5120x34816", 8192, 5120, 34816)

ALL = [SMALL, *DECODE, PREFILL_UP, PREFILL_DOWN, NVFP4, MXFP8_ATTN, MXFP4_VOCAB]


# --------------------------------------------------------------------------- fuzz corpus
_E2M1_POINTS = np.array([0.25, 0.5, 0.75, 1.0, 1.25, 1.5, 1.75, 2.0, 2.5, 3.0, 3.5, 4.0, 5.0, 6.0],
                        np.float64)  # lattice points and the midpoints between them


def _e4m3_points():
    mags = []
    for ef in range(16):
        for m in range(8):
            if ef == 15 and m == 7:
                continue
            mags.append(m * 2.0 ** -9 if ef == 0 else (1 + m / 8) * 2.0 ** (ef - 7))
    mags = np.array(mags)
    return np.concatenate([mags, (mags[:-1] + mags[1:]) / 2])


_AMAX_MANTISSAS = np.array([1.0, 1.0078125, 1.4921875, 1.5, 1.5078125, 1.7421875, 1.75, 1.7578125,
                            1.9296875, 1.9375, 1.9453125, 1.9921875])


def nvfp4_tie_bf16(rows: int, k: int, g: float, seed: int = 11) -> np.ndarray:
    """NVFP4 blocks (16 along k) on the E2M1 rounding midpoints of a known
    E4M3 block scale, for a power-of-two global scale g.

    Each block draws a positive E4M3 value s (subnormals included); its max
    element is 6 s / g, so the block scale is s exactly, and the other 15 are
    lattice points or midpoints of E2M1 times s / g, each with a random sign,
    a third of them then moved one bf16 step up or down.  Every value is
    exact in bf16.
    """
    assert k % 16 == 0 and g > 0 and np.frexp(g)[0] == 0.5, "k % 16 == 0, g a power of two"
    rng = np.random.default_rng(seed)
    nblk = rows * k // 16
    mags = np.array([m * 2.0 ** -9 for m in range(1, 8)] +
                    [(1 + m / 8) * 2.0 ** (ef - 7) for ef in range(1, 16) for m in range(8) if (ef, m) != (15, 7)])
    s = mags[rng.integers(0, len(mags), nblk)][:, None] / g
    sign = np.where(rng.random((nblk, 16)) < 0.5, -1.0, 1.0)
    out = _E2M1_POINTS[rng.integers(0, len(_E2M1_POINTS), (nblk, 16))] * s * sign
    out[:, 0] = 6.0 * s[:, 0] * sign[:, 0]
    b = _to_bf16_bits(out.astype(np.float32)).reshape(nblk, 16).astype(np.int32)
    bump = rng.random((nblk, 16)) < 1 / 3
    bump[:, 0] = False
    step = np.where(rng.random((nblk, 16)) < 0.5, 1, -1).astype(np.int32)
    mag = b & 0x7FFF
    b = np.where(bump & (mag != 0), (b & 0x8000) | np.clip(mag + step, 0, 0x7F7F), b)
    return b.astype(np.uint16).reshape(rows, k)


def fuzz_bf16(rows: int, k: int, seed: int = 7, emin: int = -135, emax: int = 120,
              mix: tuple[int, int] = (-60, 60)) -> np.ndarray:
    """Adversarial bf16 blocks (32 along k) for quantizer fuzzing.

    Every block draws a binade E in [emin, emax] (default [-135, 120]) and
    one of six shapes:
    random normals; E2M1 rounding ties (the block max is 2^(E+2), so every
    scale rule picks exponent E, and the other elements sit on lattice points,
    midpoints, or one bf16 step either side of them); E4M3 ties (max
    2^(E+8)); a block max with a mantissa at a rule threshold; all-zero or
    negative-zero blocks; mixed huge and tiny values (binades drawn from
    `mix`).  Values are built exactly in bf16, so the final rounding changes
    nothing.  GEMM tests narrow the ranges so that no product or sum leaves
    the fp32 range.
    """
    rng = np.random.default_rng(seed)
    nblk = rows * k // 32
    out = np.zeros((nblk, 32), np.float64)
    kind = rng.integers(0, 6, nblk)
    E = rng.integers(emin, emax + 1, nblk)
    p2 = np.ldexp(1.0, E)[:, None]
    sign = np.where(rng.random((nblk, 32)) < 0.5, -1.0, 1.0)
    # 0: normals
    out[kind == 0] = (rng.standard_normal((nblk, 32)) * p2)[kind == 0]
    # 1: E2M1 ties
    t = _E2M1_POINTS[rng.integers(0, len(_E2M1_POINTS), (nblk, 32))] * p2 * sign
    t[:, 0] = np.ldexp(1.0, E + 2)
    out[kind == 1] = t[kind == 1]
    # 2: E4M3 ties
    pts = _e4m3_points()
    t8 = pts[rng.integers(0, len(pts), (nblk, 32))] * p2 * sign
    t8[:, 0] = np.ldexp(1.0, E + 8)
    out[kind == 2] = t8[kind == 2]
    # 3: block max on a threshold mantissa
    tm = rng.standard_normal((nblk, 32)) * p2 * 0.3
    tm[:, 5] = _AMAX_MANTISSAS[rng.integers(0, len(_AMAX_MANTISSAS), nblk)] * p2[:, 0] * sign[:, 5]
    out[kind == 3] = tm[kind == 3]
    # 4: zeros, some negative
    z = np.where(rng.random((nblk, 32)) < 0.5, -0.0, 0.0)
    out[kind == 4] = z[kind == 4]
    # 5: mixed magnitudes
    mixed = rng.standard_normal((nblk, 32)) * np.ldexp(1.0, rng.integers(mix[0], mix[1], (nblk, 32)))
    out[kind == 5] = mixed[kind == 5]
    # keep everything finite in bf16 and round to bf16 exactly once
    out = np.clip(out, -3.0e38, 3.0e38).astype(np.float32)
    bits = _to_bf16_bits(out.reshape(rows, k))
    # one bf16 step either side of a tie for a quarter of the tie blocks
    bump = (rng.random((nblk, 32)) < 0.25) & ((kind == 1) | (kind == 2))[:, None]
    bump[:, 0] = False
    step = np.where(rng.random((nblk, 32)) < 0.5, 1, -1).astype(np.int32)
    b = bits.reshape(nblk, 32).astype(np.int32)
    mag = b & 0x7FFF
    newmag = np.clip(mag + step, 0, 0x7F7F)
    b = np.where(bump & (mag != 0), (b & 0x8000) | newmag, b)
    return b.astype(np.uint16).reshape(rows, k)
