"""Pins for the CPU oracle: each test checks the oracle against something other
than itself -- the format tables of the OCP MX specification, torch's own
float8 codecs, closed forms and invariants of the scale rules, brute force in
exact rational arithmetic, hand-worked examples, and numpy's fp64 matmul.

Sources: the QAD cards Qwen3.5-27B-MXFP4-QAD-W4A4-LR1e-5-s1000 (EVEN weight
rule) and Qwen3.5-9B-MXFP4-QAD-W4A4-LR1e-5-s3000 (CEIL activation rule), the
NVFP4 cards Qwen3.5-27B-NVFP4-RTN-weight-only / -GPTQ (per-tensor global
scales), and the AutoRound card Qwen3.8-27B-MXFP8Attn-MXFP4MLP-lmheadMXFP4
(E4M3/E2M1 + E8M0 per 32, OCP MX).
"""
import json
import math
import os
from fractions import Fraction as F

import numpy as np
import pytest
import torch

import oracle

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def lattice():
    vals = {}
    for line in open(os.path.join(GOLD, "e2m1_lattice.txt")):
        if line.startswith("#") or not line.strip():
            continue
        c, v = line.split()
        vals[int(c)] = float(v)
    return vals


LAT = lattice()
POS = [LAT[c] for c in range(8)]


def all_bf16_positive_finite():
    bits = np.arange(0x0001, 0x7F80, dtype=np.uint16)  # +subnormals .. largest finite
    vals = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).double().numpy()
    return bits, vals


def torch_e4m3_table():
    return torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()


E4M3_POS = [F(float(v)) for v in torch_e4m3_table()[:127]]


# ------------------------------------------------------------------ decoders
def test_e2m1_decode_matches_ocp_table():
    for c in range(16):
        v = oracle.e2m1_value(c)
        assert v == LAT[c]
        assert math.copysign(1.0, v) == math.copysign(1.0, LAT[c])  # code 8 is -0


def test_e4m3_decode_matches_torch():
    ref = torch_e4m3_table()
    for c in range(256):
        v = oracle.e4m3_value(c)
        if np.isnan(ref[c]):
            assert math.isnan(v)
        else:
            assert v == ref[c] and math.copysign(1, v) == math.copysign(1, ref[c]), c


def test_e8m0_decode_matches_torch():
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e8m0fnu).double().numpy()
    for c in range(256):
        v = oracle.e8m0_value(c)
        if np.isnan(ref[c]):
            assert math.isnan(v) and c == 255
        else:
            assert v == ref[c], c


def test_bf16_decode_matches_torch():
    bits = np.arange(0, 65536, 97, dtype=np.uint16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).double().numpy()
    for b, r in zip(bits, ref):
        v = oracle.bf16_value(int(b))
        assert (math.isnan(v) and math.isnan(r)) or v == r


# ------------------------------------------------------------------ encoders
def brute_e2m1(x: F, neg: bool) -> int:
    """Nearest lattice magnitude by exhaustive distance, ties to the even code;
    anything beyond 6 saturates (the nearest lattice point is then 6)."""
    a = abs(x)
    best = min(range(8), key=lambda c: (abs(a - F(POS[c])), c % 2))
    return best | (8 if neg else 0)


def test_e2m1_encode_bruteforce_dense_grid():
    vals = [F(i, 64) for i in range(0, 64 * 9)]  # 0 .. 9 step 1/64: every midpoint and tie
    for v in vals:
        for neg in (False, True):
            r = -float(v) if neg else float(v)
            if v == 0 and neg:
                r = -0.0
            assert oracle.encode("e2m1", r) == brute_e2m1(v, neg), (r,)


def test_e2m1_encode_bf16_values():
    bits, vals = all_bf16_positive_finite()
    sel = vals[vals < 16.0]
    for v in sel[:: max(1, len(sel) // 3000)]:
        assert oracle.encode("e2m1", float(v)) == brute_e2m1(F(float(v)), False)
        assert oracle.encode("e2m1", -float(v)) == brute_e2m1(F(float(v)), True)


def test_e2m1_threshold_table():
    # closed form of RNE onto {0,.5,1,1.5,2,3,4,6}: <=.25,<.75,<=1.25,<1.75,<=2.5,<3.5,<=5
    def table(a):
        return ((a > 0.25) + (a >= 0.75) + (a > 1.25) + (a >= 1.75) + (a > 2.5) + (a >= 3.5)
                + (a > 5.0))
    for i in range(0, 2000):
        a = i / 256.0
        assert oracle.encode("e2m1", a) == table(a)


def test_e4m3_encode_matches_torch_in_range():
    # torch's float32 -> float8_e4m3fn cast is round-to-nearest-even; below the
    # 448/480 midpoint it must agree with the oracle exactly.
    tab = torch_e4m3_table()
    pos = tab[:127]
    mids = (pos[:-1] + pos[1:]) / 2
    probes = np.concatenate([pos, mids, mids * (1 + 2 ** -20), mids * (1 - 2 ** -20),
                             np.linspace(0, 463.9, 5001)])
    probes = probes[probes < 464]
    probes32 = probes.astype(np.float32)
    ref = torch.from_numpy(probes32).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    refn = torch.from_numpy(-probes32).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    for p, r, rn in zip(probes32, ref, refn):
        assert oracle.encode("e4m3", float(p)) == int(r), p
        assert oracle.encode("e4m3", -float(p)) == int(rn), p


def test_e4m3_encode_saturates():
    for v in (448.0, 460.0, 464.0, 479.0, 480.0, 1e6, 3e38):
        assert oracle.encode("e4m3", v) == 0x7E
        assert oracle.encode("e4m3", -v) == 0xFE


def test_roundtrip_all_codes():
    for c in range(16):
        assert oracle.encode("e2m1", oracle.e2m1_value(c)) == c
    for c in range(256):
        if c & 0x7F == 0x7F:
            continue
        assert oracle.encode("e4m3", oracle.e4m3_value(c)) == c


# ------------------------------------------------------------------ scale rules
def closed_form(amax: float, elem: str, rule: str) -> int:
    """Closed forms from the mantissa M in [1,2) and exponent E of amax."""
    m, x = math.frexp(amax)
    M, E = 2 * m, x - 1
    emax, maxm, evenm = (2, 1.5, 1.75) if elem == "e2m1" else (8, 1.75, 1.9375)
    if rule == "floor":
        e = E - emax
    elif rule == "ceil":
        e = E - emax + (1 if M > maxm else 0)
    else:
        e = E - emax + (1 if M >= evenm else 0)
    return max(-127, min(127, e))


@pytest.mark.parametrize("elem", ["e2m1", "e4m3"])
@pytest.mark.parametrize("rule", ["floor", "ceil", "even"])
def test_scale_rule_closed_form_all_bf16(elem, rule):
    _, vals = all_bf16_positive_finite()
    for v in vals:
        assert oracle.scale_exponent(float(v), elem, rule) == closed_form(float(v), elem, rule), v
    assert oracle.scale_exponent(0.0, elem, rule) == -127


@pytest.mark.parametrize("elem,rule,lo,lo_open,hi,hi_open", [
    ("e2m1", "ceil", 3.0, True, 6.0, False),      # CEIL never clips: r in (3, 6]
    ("e2m1", "floor", 4.0, False, 8.0, True),     # OCP FLOOR: r in [4, 8)
    ("e2m1", "even", 3.5, False, 7.0, True),      # EVEN: r in [3.5, 7)
    ("e4m3", "ceil", 224.0, True, 448.0, False),
    ("e4m3", "floor", 256.0, False, 512.0, True),
])
def test_scale_rule_invariants(elem, rule, lo, lo_open, hi, hi_open):
    _, vals = all_bf16_positive_finite()
    for v in vals:
        e = oracle.scale_exponent(float(v), elem, rule)
        if e == -127:
            continue  # clamped
        r = F(float(v)) / F(2) ** e
        assert (r > lo if lo_open else r >= lo) and (r < hi if hi_open else r <= hi), (v, e)


def test_ceil_is_smallest_unclipped_power():
    # brute force: smallest e with amax <= 6 * 2^e, over exact rationals
    _, vals = all_bf16_positive_finite()
    for v in vals[::7]:
        a = F(float(v))
        e = -140
        while a > 6 * F(2) ** e:
            e += 1
        assert oracle.scale_exponent(float(v), "e2m1", "ceil") == max(-127, e)


def test_even_rule_second_characterisation():
    # EVEN (E2M1) = the smallest e at which amax/2^e, rounded to nearest-even on
    # the E2M1 grid continued upward (..., 4, 6, 8, 12, 16, ...), is at most 6.
    def rne_extended(r: F) -> F:
        if r == 0:
            return r
        E = math.floor(math.log2(r))
        while F(2) ** E > r:
            E -= 1
        while F(2) ** (E + 1) <= r:
            E += 1
        step = F(2) ** (E - 1)
        q = r / step
        fl = q.numerator // q.denominator
        frac = q - fl
        if frac > F(1, 2) or (frac == F(1, 2) and fl % 2 == 1):
            fl += 1
        return fl * step
    _, vals = all_bf16_positive_finite()
    for v in vals[::5]:
        a = F(float(v))
        e = -140
        while rne_extended(a / F(2) ** e) > 6:
            e += 1
        assert oracle.scale_exponent(float(v), "e2m1", "even") == max(-127, e), v


# ------------------------------------------------------------------ block quantization
def bits_of(values):
    t = torch.tensor(values, dtype=torch.float32).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def test_worked_examples_mx():
    ex = json.load(open(os.path.join(GOLD, "worked_examples.json")))
    for case in ex["mx_blocks"]:
        row = np.zeros((1, 32), np.uint16)
        b = bits_of(case["values"])
        row[0, :len(b)] = b
        q, s = oracle.mx_quantize(case["elem"], case["rule"], row)
        assert int(s[0, 0]) == case["scale_byte"], case["why"]
        nb = len(case["first_bytes"])
        assert [int(x) for x in q[0, :nb]] == case["first_bytes"], case["why"]
        if case["elem"] == "e2m1":
            codes = [(int(q[0, i // 2]) >> (4 * (i % 2))) & 0xF for i in range(len(case["codes"]))]
        else:
            codes = [int(q[0, i]) for i in range(len(case["codes"]))]
        assert codes == case["codes"], case["why"]


def brute_block(vals, elem, rule):
    """Reference quantization of one block with exact rationals: the exponent
    from the closed form, elements by exhaustive nearest search."""
    amax = max(abs(F(float(v))) for v in vals)
    e = -127 if amax == 0 else closed_form(float(amax), elem, rule)
    grid = [F(p) for p in POS] if elem == "e2m1" else E4M3_POS
    out = []
    for v in vals:
        r = F(float(v)) / F(2) ** e
        mag = min(range(len(grid)), key=lambda c: (abs(abs(r) - grid[c]), c % 2))
        neg = math.copysign(1.0, float(v)) < 0
        out.append(mag | ((8 if elem == "e2m1" else 128) if neg else 0))
    return e + 127, out


@pytest.mark.parametrize("elem", ["e2m1", "e4m3"])
@pytest.mark.parametrize("rule", ["floor", "ceil", "even"])
def test_quantize_bruteforce_random_blocks(elem, rule):
    rng = np.random.default_rng(1234)
    rows, k = 6, 96
    x = rng.standard_normal((rows, k)).astype(np.float32)
    x[1] *= 1e-3
    x[2, :32] = 0.0
    x[2, 40] = -0.0
    x[3] *= rng.choice([1, 20, 1e-30], size=k).astype(np.float32)
    x[4, :32] = np.float32(0.25) * rng.integers(-24, 25, 32)  # E2M1 ties
    x[5, 32:64] = rng.standard_normal(32) * np.float32(3e37)
    xb = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    vals = torch.from_numpy(xb.view(np.int16)).view(torch.bfloat16).double().numpy()
    q, s = oracle.mx_quantize(elem, rule, xb)
    for r in range(rows):
        for b in range(k // 32):
            blk = [vals[r, b * 32 + i] if not (xb[r, b * 32 + i] == 0x8000) else -0.0
                   for i in range(32)]
            sb, codes = brute_block(blk, elem, rule)
            assert int(s[r, b]) == sb
            for i in range(32):
                j = b * 32 + i
                got = ((int(q[r, j // 2]) >> (4 * (j % 2))) & 0xF) if elem == "e2m1" else int(q[r, j])
                assert got == codes[i], (r, b, i, blk[i])


def test_dequantize_matches_table():
    rng = np.random.default_rng(7)
    x = torch.from_numpy(rng.standard_normal((3, 64)).astype(np.float32)).to(torch.bfloat16)
    xb = x.view(torch.int16).numpy().view(np.uint16)
    q, s = oracle.mx_quantize("e2m1", "ceil", xb)
    d = oracle.mx_dequantize("e2m1", q, s, 3, 64)
    for r in range(3):
        for j in range(64):
            c = (int(q[r, j // 2]) >> (4 * (j % 2))) & 0xF
            assert d[r, j] == LAT[c] * 2.0 ** (int(s[r, j // 32]) - 127)


# ------------------------------------------------------------------ NVFP4
def brute_global_scale(amax: float) -> np.float32:
    if amax == 0:
        return np.float32(1.0)
    q = F(2688) / F(amax)
    fmax = np.finfo(np.float32).max
    if q > F(float(fmax)):
        return fmax  # saturating reading for tensors below ~8e-36
    c = np.float32(float(q))
    cands = [c, np.nextafter(c, np.float32(0)), np.nextafter(c, np.float32(np.inf))]
    def key(v):
        return (abs(F(float(v)) - q), int(np.array(v).view(np.uint32)) & 1)
    return min(cands, key=key)


def test_nv_global_scale_bruteforce():
    _, vals = all_bf16_positive_finite()
    for v in list(vals[::11]) + [3.0, 7.0, 2688.0, 1.0, 0.0]:
        assert oracle.nv_global_scale(float(v)) == brute_global_scale(float(v)), v
    assert oracle.nv_global_scale(3.0) == np.float32(896.0)
    assert oracle.nv_global_scale(0.0) == np.float32(1.0)


def brute_nv_block(vals, g):
    amax = max(abs(F(float(v))) for v in vals)
    target = amax * F(float(g)) / 6
    sc = min(range(127), key=lambda c: (abs(target - E4M3_POS[c]), c % 2))
    s = E4M3_POS[sc]
    out = []
    for v in vals:
        neg = math.copysign(1.0, float(v)) < 0
        if s == 0:
            mag = 0
        else:
            r = abs(F(float(v))) * F(float(g)) / s
            mag = min(range(8), key=lambda c: (abs(r - F(POS[c])), c % 2))
        out.append(mag | (8 if neg else 0))
    return sc, out


def test_worked_examples_nv():
    ex = json.load(open(os.path.join(GOLD, "worked_examples.json")))
    for case in ex["nv_blocks"]:
        row = np.zeros((1, 16), np.uint16)
        b = bits_of(case["values"])
        row[0, :len(b)] = b
        q, s = oracle.nv_quantize(row, case["g"])
        assert int(s[0, 0]) == case["scale_byte"], case["why"]
        codes = [(int(q[0, i // 2]) >> (4 * (i % 2))) & 0xF for i in range(len(case["codes"]))]
        assert codes == case["codes"], case["why"]


def test_nv_quantize_bruteforce():
    rng = np.random.default_rng(99)
    rows, k = 5, 64
    x = rng.standard_normal((rows, k)).astype(np.float32)
    x[1] *= 1e-4
    x[2, :16] = 0
    x[3] *= 40
    xb = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    vals = torch.from_numpy(xb.view(np.int16)).view(torch.bfloat16).double().numpy()
    for g in (oracle.nv_global_scale(float(np.abs(vals).max())), np.float32(1.0),
              np.float32(1e5), np.float32(0.37)):
        q, s = oracle.nv_quantize(xb, g)
        for r in range(rows):
            for b in range(k // 16):
                sc, codes = brute_nv_block(list(vals[r, b * 16:(b + 1) * 16]), g)
                assert int(s[r, b]) == sc, (g, r, b)
                for i in range(16):
                    j = b * 16 + i
                    assert ((int(q[r, j // 2]) >> (4 * (j % 2))) & 0xF) == codes[i], (g, r, b, i)


def test_nv_quantize_ties_bruteforce():
    # blocks whose elements sit on the E2M1 rounding midpoints of an exact
    # E4M3 block scale (and one bf16 step either side): the brute-force block
    # rule decides every tie, and the inputs do hold ties
    import workloads as W
    mids = {F(1, 4), F(3, 4), F(5, 4), F(7, 4), F(5, 2), F(7, 2), F(5)}
    for g in (1.0, 0.5, 64.0):
        xb = W.nvfp4_tie_bf16(3, 64, g, seed=21)
        vals = torch.from_numpy(xb.view(np.int16)).view(torch.bfloat16).double().numpy()
        q, s = oracle.nv_quantize(xb, np.float32(g))
        ties = 0
        for r in range(3):
            for b in range(4):
                blk = list(vals[r, b * 16:(b + 1) * 16])
                sc, codes = brute_nv_block(blk, np.float32(g))
                assert int(s[r, b]) == sc and E4M3_POS[sc] == abs(F(float(blk[0]))) * F(g) / 6, (g, r, b)
                ties += sum(abs(F(float(v))) * F(g) / E4M3_POS[sc] in mids for v in blk)
                for i in range(16):
                    j = b * 16 + i
                    assert ((int(q[r, j // 2]) >> (4 * (j % 2))) & 0xF) == codes[i], (g, r, b, i)
        assert ties >= 40, (g, ties)


def _torch_amax(bits: np.ndarray) -> float:
    # torch decodes the bf16 patterns independently of the oracle
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16)
    return float(t.double().abs().max()) if bits.size else 0.0


def test_bf16_amax_against_torch_decode():
    # orc_bf16_amax feeds every NVFP4 global scale (the per-tensor amax of the
    # weights, the running max of the activation batches).  Pinned against
    # torch's bf16 decode on tensors built so that a dropped fabs, a signed
    # compare, a skipped element or a subnormal flush each gives a wrong value:
    # the extreme magnitude is negative, sits at the first or the last index,
    # or is a subnormal among -0 and smaller subnormals.
    rng = np.random.default_rng(41)
    cases = []
    x = rng.standard_normal(4099).astype(np.float32)
    x[1234] = -37.5                                     # extreme value negative, mid-tensor
    cases.append(x)
    y = rng.standard_normal(513).astype(np.float32)
    y[0] = -9.0e3                                       # first element
    cases.append(y)
    z = rng.standard_normal(777).astype(np.float32)
    z[-1] = -6.5e4                                      # last element
    cases.append(z)
    cases.append(np.array([-3.0e38, 1.0, -0.0], np.float32))   # near the largest finite bf16
    for xs in cases:
        bits = torch.from_numpy(xs).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        assert oracle.bf16_amax(bits) == _torch_amax(bits)
        assert oracle.bf16_amax(bits) > float(np.max(torch.from_numpy(bits.view(np.int16)).view(
            torch.bfloat16).double().numpy())), "the extreme is negative: a signed max is smaller"
    # subnormals only, with -0: the largest magnitude is the negative subnormal 0x807F
    sub = np.array([0x8000, 0x0001, 0x807F, 0x0040, 0x8003, 0x0000], np.uint16)
    assert oracle.bf16_amax(sub) == _torch_amax(sub) == 127 * 2.0 ** -133
    # zeros of both signs: amax 0 (the NVFP4 global scale is then 1)
    zeros = np.array([0x8000, 0x0000, 0x8000], np.uint16)
    assert oracle.bf16_amax(zeros) == 0.0
    assert oracle.nv_global_scale(oracle.bf16_amax(zeros)) == np.float32(1.0)
    # every positive finite bf16 once, shuffled, negated: the maximum is the
    # largest finite bf16 whatever the order
    bits, vals = all_bf16_positive_finite()
    perm = rng.permutation(bits.size)
    neg = (bits[perm] | 0x8000).astype(np.uint16)
    assert oracle.bf16_amax(neg) == vals.max() == _torch_amax(neg)
    # one element
    assert oracle.bf16_amax(np.array([0xC2F7], np.uint16)) == 123.5


def test_nv_invariants():
    rng = np.random.default_rng(3)
    x = torch.from_numpy(rng.standard_normal((64, 256)).astype(np.float32)).to(torch.bfloat16)
    xb = x.view(torch.int16).numpy().view(np.uint16)
    amax = oracle.bf16_amax(xb)
    g = oracle.nv_global_scale(amax)
    q, s = oracle.nv_quantize(xb, g)
    sv = torch_e4m3_table()[s]
    assert (sv <= 448).all() and (sv >= 0).all()
    # the tensor's own amax maps to a block scale of exactly 448 (no clipping)
    assert sv.max() == 448.0
    # every element is within half a lattice step of its dequantized value
    d = oracle.nv_dequantize(q, s, 64, 256, g)
    xv = x.double().numpy()
    step = np.repeat(sv, 16, axis=1) / float(g)  # largest E2M1 gap is 2*s/g
    assert (np.abs(d - xv) <= step + 1e-30).all()


# ------------------------------------------------------------------ GEMM
def test_gemm_integer_exact():
    rng = np.random.default_rng(5)
    a = rng.integers(-7, 8, (5, 13)).astype(np.float64)
    w = rng.integers(-7, 8, (3, 13)).astype(np.float64)
    y, sa = oracle.gemm_dq(a, w)
    for i in range(5):
        for j in range(3):
            assert y[i, j] == sum(int(a[i, t]) * int(w[j, t]) for t in range(13))
            assert sa[i, j] == sum(abs(int(a[i, t]) * int(w[j, t])) for t in range(13))


@pytest.mark.parametrize("a_elem,w_elem", [("e2m1", "e2m1"), ("e4m3", "e4m3"), ("e4m3", "e2m1")])
def test_mx_gemm_matches_numpy_on_dequantized(a_elem, w_elem):
    rng = np.random.default_rng(11)
    m, n, k = 7, 5, 96  # distinct sizes: a transposed operand cannot pass
    a = torch.from_numpy(rng.standard_normal((m, k)).astype(np.float32)).to(torch.bfloat16)
    w = torch.from_numpy((rng.standard_normal((n, k)) * 0.02).astype(np.float32)).to(torch.bfloat16)
    ab = a.view(torch.int16).numpy().view(np.uint16)
    wb = w.view(torch.int16).numpy().view(np.uint16)
    aq, a_s = oracle.mx_quantize(a_elem, "ceil", ab)
    wq, w_s = oracle.mx_quantize(w_elem, "even", wb)
    y, sa = oracle.mx_gemm(a_elem, aq, a_s, w_elem, wq, w_s, m, n, k)

    def deq(elem, q, s, rows):
        out = np.zeros((rows, k))
        for r in range(rows):
            for j in range(k):
                if elem == "e2m1":
                    v = LAT[(int(q[r, j // 2]) >> (4 * (j % 2))) & 0xF]
                else:
                    v = torch_e4m3_table()[q[r, j]]
                out[r, j] = v * 2.0 ** (int(s[r, j // 32]) - 127)
        return out
    ad, wd = deq(a_elem, aq, a_s, m), deq(w_elem, wq, w_s, n)
    ref = ad @ wd.T
    np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-300)
    np.testing.assert_allclose(sa, np.abs(ad) @ np.abs(wd).T, rtol=1e-12)
    # dequantized + gemm_dq path agrees with the on-the-fly path
    y2, _ = oracle.gemm_dq(ad, wd)
    np.testing.assert_allclose(y2, ref, rtol=1e-12)
    # selected pairs
    mi = np.array([0, 6, 3]); ni = np.array([4, 0, 2])
    yp, sp = oracle.gemm_dq_pairs(ad, wd, mi, ni)
    np.testing.assert_allclose(yp, ref[mi, ni], rtol=1e-12)


def test_quantization_error_bound_end_to_end():
    # the dequantized CEIL activations stay within half a lattice step of A:
    # |a - dq(a)| <= 2^e (the largest E2M1 gap, 2, times 2^e / 2)
    rng = np.random.default_rng(21)
    a = torch.from_numpy(rng.standard_normal((8, 128)).astype(np.float32) * 3).to(torch.bfloat16)
    ab = a.view(torch.int16).numpy().view(np.uint16)
    q, s = oracle.mx_quantize("e2m1", "ceil", ab)
    d = oracle.mx_dequantize("e2m1", q, s, 8, 128)
    bound = np.repeat(2.0 ** (s.astype(np.float64) - 127), 32, axis=1)
    assert (np.abs(d - a.double().numpy()) <= bound).all()


# ------------------------------------------------------------------ W4A16
def _bf16_bits(x):
    return torch.from_numpy(np.asarray(x, np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


@pytest.mark.parametrize("fmt,k", [("mxfp4", 64), ("nvfp4", 48)])
def test_w4a16_bruteforce_tiny(fmt, k):
    # every term decoded on its own (torch for bf16 and E4M3, the OCP lattice
    # file for E2M1) and summed in exact rationals
    rng = np.random.default_rng(31)
    m, n = 3, 2   # distinct sizes: a transposed operand cannot pass
    ab = _bf16_bits(rng.standard_normal((m, k)) * 4)
    wq = rng.integers(0, 256, (n, k // 2)).astype(np.uint8)
    if fmt == "mxfp4":
        ws = rng.integers(118, 136, (n, k // 32)).astype(np.uint8)
        g = None
    else:
        ws = rng.integers(0x20, 0x60, (n, k // 16)).astype(np.uint8)
        g = np.float32(3.0)
    y, sa = oracle.w4a16_gemm(ab, wq, ws, n, k, fmt, g)
    av = torch.from_numpy(ab.view(np.int16)).view(torch.bfloat16).double().numpy()
    e4 = torch_e4m3_table()
    for i in range(m):
        for j in range(n):
            acc, aabs = F(0), F(0)
            for t in range(k):
                code = (int(wq[j, t // 2]) >> (4 * (t % 2))) & 0xF
                if fmt == "mxfp4":
                    wv = F(LAT[code]) * F(2) ** (int(ws[j, t // 32]) - 127)
                else:
                    wv = F(LAT[code]) * F(float(e4[ws[j, t // 16]])) / F(float(g))
                term = F(float(av[i, t])) * wv
                acc += term
                aabs += abs(term)
            # fp64 dequantization (NVFP4 divides by g) and summation round
            # at most a few ulps of the absolute sum
            assert abs(F(y[i, j]) - acc) <= aabs * F(1, 2 ** 46) + F(1, 2 ** 1000)
            assert abs(F(sa[i, j]) - aabs) <= aabs * F(1, 2 ** 46) + F(1, 2 ** 1000)


def test_w4a16_equals_w4a4_on_representable_activations():
    # activations that are already dequantized MXFP4 values (exact in bf16)
    # give the W4A4 product of their codes
    rng = np.random.default_rng(32)
    m, n, k = 5, 7, 128
    ab = _bf16_bits(rng.standard_normal((m, k)))
    wb = _bf16_bits(rng.standard_normal((n, k)) * 0.02)
    aq, a_s = oracle.mx_quantize("e2m1", "ceil", ab)
    wq, ws = oracle.mx_quantize("e2m1", "even", wb)
    ad = oracle.mx_dequantize("e2m1", aq, a_s, m, k)
    ad_bits = _bf16_bits(ad)
    assert np.array_equal(oracle.bf16_to_f64(ad_bits), ad)   # exact in bf16
    y16, s16 = oracle.w4a16_gemm(ad_bits, wq, ws, n, k, "mxfp4")
    y4, s4 = oracle.mx_gemm("e2m1", aq, a_s, "e2m1", wq, ws, m, n, k)
    np.testing.assert_allclose(y16, y4, rtol=1e-13, atol=1e-300)
    np.testing.assert_allclose(s16, s4, rtol=1e-13)


def test_w4a16_nvfp4_closed_form():
    # every weight element 1.0 (E2M1 code 2) with E4M3 scale 1.0 (0x38) and
    # g_w = 4: each output is sum_k a / 4
    rng = np.random.default_rng(33)
    m, n, k = 4, 3, 80
    ab = _bf16_bits(rng.standard_normal((m, k)))
    wq = np.full((n, k // 2), 0x22, np.uint8)
    ws = np.full((n, k // 16), 0x38, np.uint8)
    y, sa = oracle.w4a16_gemm(ab, wq, ws, n, k, "nvfp4", np.float32(4.0))
    av = oracle.bf16_to_f64(ab)
    for j in range(n):
        np.testing.assert_allclose(y[:, j], av.sum(axis=1) / 4, rtol=1e-14)
        np.testing.assert_allclose(sa[:, j], np.abs(av).sum(axis=1) / 4, rtol=1e-14)


# ------------------------------------------------------------------ fake quantization
# Training-time fake quantization (Qwen3.5-9B-MXFP4-QAD-W4A4-LR1e-5-s3000,
# "Training mode"; Qwen3.5-27B-MXFP4-QAD-W4A4-LR1e-5-s1000, "How this
# checkpoint was produced", Training row): the codes of the serving
# quantizer, dequantized, rounded once to bf16.
_BITS, _VALS = all_bf16_positive_finite()           # patterns 0x0001 .. 0x7F7F, ascending
_TOP = F(float(_VALS[-1]))
_HALF_ULP_TOP = F(2) ** (127 - 8)


def _bf16_val(c: int) -> F:
    return F(0) if c == 0 else F(float(_VALS[c - 1]))


def brute_bf16_nearest(q: F) -> int:
    """Nearest bf16 pattern to the rational q >= 0 by search over the sorted
    table of every positive finite bf16; ties to the even pattern; from the
    largest finite value plus half an ulp upward, infinity."""
    if q >= _TOP + _HALF_ULP_TOP:
        return 0x7F80
    i = int(np.searchsorted(_VALS, float(q)))
    cands = [0] + [int(_BITS[j]) for j in range(max(0, i - 2), min(len(_VALS), i + 2))]
    return min(cands, key=lambda c: (abs(_bf16_val(c) - q), c & 1))


def test_bf16_nearest_ratio_bruteforce():
    rng = np.random.default_rng(17)
    e4 = [float(v) for v in E4M3_POS[1:]]
    for _ in range(3000):
        p = float(rng.choice(POS[1:])) * float(rng.choice(e4))
        g = float(np.float32(np.exp(rng.uniform(-60, 60))))
        assert oracle.bf16_nearest_ratio(p, g) == brute_bf16_nearest(F(p) / F(g)), (p, g)
    # exact midpoints between neighbouring patterns of both parities: ties to even
    for c in (0x3F80, 0x3F81, 0x0001, 0x0002, 0x7F7E, 0x0080):
        mid = (_bf16_val(c) + _bf16_val(c + 1)) / 2
        for g in (1.0, 3.0, float(np.float32(0.1)), float(np.float32(1e-20))):
            p = float(mid * F(g))
            assert F(p) == mid * F(g)                       # 9 + 24 bits: exact in a double
            assert oracle.bf16_nearest_ratio(p, g) == (c if c % 2 == 0 else c + 1), hex(c)
    # overflow boundary: top + half ulp rounds to infinity, anything below to the top
    edge = float(_TOP + _HALF_ULP_TOP)
    assert oracle.bf16_nearest_ratio(edge, 1.0) == 0x7F80
    assert oracle.bf16_nearest_ratio(np.nextafter(edge, 0.0), 1.0) == 0x7F7F
    assert oracle.bf16_nearest_ratio(0.0, 5.0) == 0
    assert oracle.bf16_nearest_ratio(2.0 ** -134, 1.0) == 0      # half the smallest subnormal: tie -> 0
    assert oracle.bf16_nearest_ratio(3 * 2.0 ** -134, 1.0) == 2  # 1.5 subnormal steps: tie -> even 2


def test_bf16_nearest_ratio_single_rounding():
    """Where rounding to fp32 first lands on a bf16 midpoint, the result is
    still the single rounding of the exact quotient."""
    from helpers import double_rounding_trap_scales
    for g in double_rounding_trap_scales(8):
        q = F(1) / F(float(g))
        want = brute_bf16_nearest(q)
        assert oracle.bf16_nearest_ratio(1.0, float(g)) == want
        twice = int(torch.tensor(float(np.float32(1.0 / float(g))), dtype=torch.float32)
                    .to(torch.bfloat16).view(torch.int16)) & 0xFFFF
        assert twice != want  # the trap is real: rounding twice goes the other way


def _signed(bits: int, neg: bool) -> int:
    return bits | (0x8000 if neg else 0)


@pytest.mark.parametrize("elem,fmt", [("e2m1", "mxfp4"), ("e4m3", "mxfp8")])
@pytest.mark.parametrize("rule", ["floor", "ceil", "even"])
def test_fake_quant_mx_bruteforce(elem, fmt, rule):
    rng = np.random.default_rng(77)
    rows, k = 5, 96
    x = rng.standard_normal((rows, k)).astype(np.float32)
    x[1] *= 1e-38                                    # subnormal bf16 inputs, clamped scales
    x[2, :32] = 0.0
    x[2, 33] = -0.0
    x[3, :32] = np.clip(rng.standard_normal(32), -3.3, 3.3) * np.float32(1e38)   # codes near the top
    x[3, 7] = 3.3e38   # CEIL: scale 2^126, code 4 -> 2^128, beyond bf16
    x[4, :32] = np.float32(0.25) * rng.integers(-24, 25, 32)
    xb = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    vals = torch.from_numpy(xb.view(np.int16)).view(torch.bfloat16).double().numpy()
    got = oracle.fake_quant(fmt, rule, xb)
    grid = [F(p) for p in POS] if elem == "e2m1" else E4M3_POS
    infs = 0
    for r in range(rows):
        for b in range(k // 32):
            blk = [-0.0 if xb[r, b * 32 + i] == 0x8000 else vals[r, b * 32 + i] for i in range(32)]
            sb, codes = brute_block(blk, elem, rule)
            for i in range(32):
                c = codes[i]
                neg = bool(c & (8 if elem == "e2m1" else 128))
                mag = grid[c & (7 if elem == "e2m1" else 127)] * F(2) ** (sb - 127)
                want = _signed(brute_bf16_nearest(mag), neg)
                infs += (want & 0x7FFF) == 0x7F80
                assert int(got[r, b * 32 + i]) == want, (r, b, i, blk[i])
    if rule == "ceil" and elem == "e2m1":
        assert infs > 0  # the near-top block overflows bf16 under CEIL


def test_fake_quant_nv_bruteforce():
    from helpers import double_rounding_trap_scales
    rng = np.random.default_rng(78)
    rows, k = 4, 64
    x = rng.standard_normal((rows, k)).astype(np.float32)
    x[1] *= 1e-4
    x[2, :16] = 0.0
    x[3] *= 40
    traps = double_rounding_trap_scales(4)
    # blocks built so that s = 1 and one element codes to 1: its output is the
    # single rounding of 1/g (a double-rounding trap for an fp32 path)
    for j, gt in enumerate(traps[:2]):
        x[0, 16 * j:16 * j + 16] = 0.0
        x[0, 16 * j] = 6.0 / float(gt)
        x[0, 16 * j + 1] = -1.0 / float(gt)
    xb = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    vals = torch.from_numpy(xb.view(np.int16)).view(torch.bfloat16).double().numpy()
    for g in (oracle.nv_global_scale(float(np.abs(vals).max())), np.float32(0.37), traps[0], traps[1]):
        got = oracle.fake_quant("nvfp4", None, xb, g)
        for r in range(rows):
            for b in range(k // 16):
                sc, codes = brute_nv_block(list(vals[r, b * 16:(b + 1) * 16]), g)
                for i in range(16):
                    v = F(POS[codes[i] & 7]) * E4M3_POS[sc] / F(float(g))
                    want = _signed(brute_bf16_nearest(v), bool(codes[i] & 8))
                    assert int(got[r, b * 16 + i]) == want, (g, r, b, i)


def test_fake_quant_identity_on_lattice():
    """Values already on a block's lattice come back unchanged."""
    rng = np.random.default_rng(79)
    # MXFP4 EVEN: a block whose amax is 6 * 2^e has scale 2^e (mantissa 1.5)
    e = rng.integers(-20, 20, 4)
    x = np.zeros((4, 32), np.float64)
    for r in range(4):
        x[r] = rng.choice(POS, 32) * rng.choice([-1, 1], 32) * 2.0 ** e[r]
        x[r, 5] = 6.0 * 2.0 ** e[r]
    xb = _bf16_bits(x)
    assert np.array_equal(oracle.fake_quant("mxfp4", "even", xb), xb)
    # NVFP4 with g = 1: block amax 6 * s with s on the E4M3 lattice
    s = 1.25
    y = rng.choice(POS, (2, 16)) * rng.choice([-1, 1], (2, 16)) * s
    y[:, 0] = 6.0 * s
    yb = _bf16_bits(y)
    assert np.array_equal(oracle.fake_quant("nvfp4", None, yb, np.float32(1.0)), yb)


def test_fake_quant_matches_dequantized_codes():
    """Outputs agree with the fp64 dequantization of the serving quantizer's
    codes wherever that value is a bf16 (always for MX, exactly-divisible
    NVFP4 cases otherwise)."""
    rng = np.random.default_rng(80)
    x = torch.from_numpy(rng.standard_normal((6, 128)).astype(np.float32)).to(torch.bfloat16)
    xb = x.view(torch.int16).numpy().view(np.uint16)
    q, s = oracle.mx_quantize("e2m1", "ceil", xb)
    d = oracle.mx_dequantize("e2m1", q, s, 6, 128)
    want = torch.from_numpy(d).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = oracle.fake_quant("mxfp4", "ceil", xb)
    # -0 codes dequantize to -0.0; numpy keeps the sign, so patterns compare directly
    assert np.array_equal(got, want)
    assert np.array_equal(torch.from_numpy(d).float().numpy(),
                          torch.from_numpy(got.view(np.int16)).view(torch.bfloat16).float().numpy())


# ------------------------------------------------------------------ SwiGLU
def test_swiglu_matches_torch_silu():
    rng = np.random.default_rng(90)
    g = rng.standard_normal(4000) * 6
    u = rng.standard_normal(4000) * 3
    want = (torch.nn.functional.silu(torch.from_numpy(g)) * torch.from_numpy(u)).numpy()
    np.testing.assert_allclose(oracle.swiglu(g, u), want, rtol=1e-14, atol=1e-300)


def test_swiglu_special_values():
    # sigmoid(1) = 1 / (1 + 1/e) = 0.7310585786300049 (tabulated value)
    assert abs(oracle.swiglu(1.0, 1.0) - 0.7310585786300049) < 1e-15
    assert oracle.swiglu(0.0, 5.0) == 0.0
    g = np.array([40.0, 50.0, 100.0])
    np.testing.assert_array_equal(oracle.swiglu(g, 3.0), 3.0 * g)       # e^-g below half an ulp
    assert oracle.swiglu(-1000.0, 2.0) == 0.0                            # e^1000 overflows to inf
    # silu(-x) = silu(x) - x
    x = np.linspace(-9, 9, 37)
    np.testing.assert_allclose(oracle.swiglu(-x, 1.0), oracle.swiglu(x, 1.0) - x, rtol=1e-13, atol=1e-14)


def test_mlp_swiglu_composes_gate_and_up():
    rng = np.random.default_rng(91)
    m, inter, k = 5, 64, 96
    a = _bf16_bits(rng.standard_normal((m, k)))
    w = _bf16_bits(rng.standard_normal((2 * inter, k)) * 0.1)
    aq, a_s = oracle.mx_quantize("e2m1", "ceil", a)
    wq, w_s = oracle.mx_quantize("e2m1", "even", w)
    h, gate, up, sg, su = oracle.mlp_swiglu(aq, a_s, wq, w_s, m, inter, k)
    ad = oracle.mx_dequantize("e2m1", aq, a_s, m, k)
    wd = oracle.mx_dequantize("e2m1", wq, w_s, 2 * inter, k)
    np.testing.assert_allclose(gate, ad @ wd[:inter].T, rtol=1e-12, atol=1e-300)   # gate rows first
    np.testing.assert_allclose(up, ad @ wd[inter:].T, rtol=1e-12, atol=1e-300)
    np.testing.assert_allclose(sg, np.abs(ad) @ np.abs(wd[:inter]).T, rtol=1e-12)
    np.testing.assert_allclose(h, oracle.swiglu(gate, up), rtol=0)
