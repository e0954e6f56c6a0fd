// quant.hip -- block quantizers for gfx950: MX (E2M1 / E4M3 elements with an
// E8M0 scale per 32) and NVFP4 (E2M1 with an E4M3 scale per 16 and an fp32
// per-tensor global scale), plus the tensor amax used for NVFP4 global scales.
//
// Operations (model-card pages):
//  - Qwen3.5-9B-MXFP4-QAD-W4A4-LR1e-5-s3000, "Training mode": per-token block-32
//    E2M1 activations with CEIL-rule UE8M0 scales, computed at run time.
//  - Qwen3.5-27B-MXFP4-QAD-W4A4-LR1e-5-s1000, "How this checkpoint was
//    produced": block-32 E2M1 weights with EVEN-rule E8M0 scales, rounded to
//    nearest (Qwen3.5-27B-NVFP4-RTN-weight-only: "rounded to the lattice").
//  - Qwen3.8-27B-MXFP8Attn-MXFP4MLP-lmheadMXFP4, introduction and section 2:
//    MXFP8 = E4M3 elements with an E8M0 scale per group of 32.
//  - Qwen3.5-27B-NVFP4-RTN-weight-only / Qwen3.5-27B-NVFP4-GPTQ, introductions:
//    NVFP4 with per-tensor global scales.
//
// Layout: since k is a multiple of the block, block b of a [rows, k] tensor
// is elements [B*b, B*b + B) of the flat array and its scale is byte b of the
// flat scale plane.  The kernels therefore run over the flat arrays: rows
// never appear.
//
// Work mapping (MX): a wave covers 2048 consecutive elements (4 KiB of bf16)
// with 4 loads of 16 B per lane; load j of lane i reads the 8-element group
// 64*j + i, so every load instruction is one contiguous 1 KiB read.  The 32
// elements of a block sit in a lane quad; its amax is a quad reduction over
// DPP.  Codes go out as one contiguous 256 B (E2M1) or 512 B (E4M3) store per
// load; scales as 16 consecutive bytes per load.
#include "mx_device.h"

namespace mxl {

constexpr int QUANT_THREADS = 256;
constexpr int ELEMS_PER_WAVE = 2048;
constexpr int ELEMS_PER_BLOCK = ELEMS_PER_WAVE * (QUANT_THREADS / 64);

// 16-byte loads and stores marked non-temporal, for data touched once and
// streamed past the caches.  The quantizers, the SwiGLU quantizer and the
// tensor amax read their inputs this way (the MXFP4 quantizer on the 285 MB
// down-projection activations went from 5.4 to 6.3 TB/s) and store their
// codes normally, since a GEMM reads them next.  The NVFP4 fake quantization
// (bound by its vector work) is faster with both its load and its store
// non-temporal, the MXFP4 one with neither (same-box A/B).
typedef unsigned int nt_u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 ld_nt(const uint4* p)
{
    const nt_u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const nt_u32x4*>(p));
    return make_uint4(v[0], v[1], v[2], v[3]);
}
__device__ __forceinline__ void st_nt(uint4* p, uint4 v)
{
    __builtin_nontemporal_store(nt_u32x4{v.x, v.y, v.z, v.w}, reinterpret_cast<nt_u32x4*>(p));
}

template <int ELEM, int RULE>
__global__ __launch_bounds__(QUANT_THREADS) void mx_quantize_kernel(const uint4* __restrict__ x,
                                                                     int64_t total,
                                                                     uint8_t* __restrict__ q,
                                                                     uint8_t* __restrict__ s)
{
    const int lane = threadIdx.x & 63;
    const int64_t wave_base = ((int64_t)blockIdx.x * (QUANT_THREADS / 64) + (threadIdx.x >> 6)) * ELEMS_PER_WAVE;
    uint4 v[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int64_t g = wave_base / 8 + 64 * j + lane;  // 8-element group index
        if (g * 8 < total) v[j] = ld_nt(&x[g]);   // read once: streamed past the caches
        else v[j] = make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int64_t g = wave_base / 8 + 64 * j + lane;
        const uint32_t amax = quad_max_u32(amax_bits8(v[j]));
        const int e = scale_exponent<ELEM, RULE>(amax);
        if (g * 8 < total) {
            if (ELEM == ELEM_E2M1) {
                reinterpret_cast<uint32_t*>(q)[g] = encode8_e2m1(v[j], e);
            } else {
                reinterpret_cast<uint2*>(q)[g] = encode8_e4m3(v[j], e);
            }
            if ((lane & 3) == 0) s[g >> 2] = (uint8_t)(e + 127);
        }
    }
}

// NVFP4: a block of 16 is a lane pair.  The block scale and the element codes
// are roundings of exact reals (amax * g / 6 and x * g / s), each decided by
// a bracket where it can be, else exactly:
//  * Bracket.  With r an approximation of the real value within 2^-21.5
//    (relative), the hardware converters round r (1 - 2^-20) and r (1 +
//    2^-20), which strictly bracket the real value.  Rounding is monotonic,
//    so where the two codes agree they are the real value's code; a
//    midpoint inside the bracket makes them differ.  Values below 2^-100
//    lose the relative bound but lie far below the formats' first nonzero
//    rounding midpoint, and round to zero either way.
//  * Scale: r = amax * g * fl(1/6) in fp32 (three roundings), clamped to 448
//    (the format's saturation), rounded to E4M3 by v_cvt_scalef32_pk_fp8_f32
//    (round to nearest even, subnormals included).  Exactly otherwise: amax *
//    g is exact in fp64 (8 + 24 significant bits); its quotient by 6 is
//    evaluated in fp64 and can only meet an E4M3 rounding midpoint when the
//    quotient is exactly that midpoint, which fp64 then represents exactly.
//  * Elements: r = x * g * rcp(s) (v_rcp_f32, within 1 ulp; four roundings
//    in all), rounded to E2M1 by v_cvt_scalef32_pk_fp4_f32 (round to nearest
//    even, saturating at 6, sign kept), when s > 0, c = g * rcp(s) >= 2^-100
//    and amax * c (1 + 2^-20) <= 2^30 (no overflow).  Exactly otherwise, and
//    in every lane whose two codes differ: x * g <=> t * s for each
//    threshold t by the sign of one fma (e2m1_rne_fma).
// Returns the 8 codes of the lane's group (element i in nibble i) and the
// block's scale code and value.
__device__ __forceinline__ uint32_t nv_encode8(uint4 v, float gscale, uint32_t& sc, float& sf)
{
    const uint32_t amax = pair_max_u32(amax_bits8(v));
    const float af = bf16_bits_to_float(amax);
    {
        const float r = af * gscale * (1.0f / 6.0f);
        short2_t pk = {0, 0};
        pk = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(pk, __builtin_fminf(r * (1.0f - 0x1p-20f), 448.0f),
                                                      __builtin_fminf(r * (1.0f + 0x1p-20f), 448.0f), 1.0f, false);
        const uint32_t pw = __builtin_bit_cast(uint32_t, pk);
        if ((pw & 0xFFu) == ((pw >> 8) & 0xFFu)) {
            sc = pw & 0xFFu;
        } else {
            const double ag = (double)af * (double)gscale;   // exact
            sc = e4m3_rne_f64(ag / 6.0);
        }
    }
    sf = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(sc, 1.0f, false)[0];   // exact
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
    const float c = gscale * __builtin_amdgcn_rcpf(sf);
    const float c_lo = c * (1.0f - 0x1p-20f), c_hi = c * (1.0f + 0x1p-20f);
    uint32_t lo = 0, hi = 0;
#define MXL_NV_PAIR(J)                                                                               \
    {                                                                                                \
        const float x0 = __uint_as_float(w[J] << 16), x1 = __uint_as_float(w[J] & 0xFFFF0000u);     \
        lo = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(lo, x0 * c_lo, x1 * c_lo, 1.0f, J);            \
        hi = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(hi, x0 * c_hi, x1 * c_hi, 1.0f, J);            \
    }
    MXL_NV_PAIR(0) MXL_NV_PAIR(1) MXL_NV_PAIR(2) MXL_NV_PAIR(3)
#undef MXL_NV_PAIR
    const bool fast = sf > 0.0f && c >= 0x1p-100f && af * c_hi <= 0x1p30f;
    if (fast && lo == hi) return lo;
    float t[7];
    e2m1_thresholds(sf, t);
    uint32_t codes = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const uint32_t b = (w[i / 2] >> (16 * (i % 2))) & 0xFFFFu;
        const uint32_t cd = e2m1_rne_fma(bf16_bits_to_float(b & 0x7FFFu), gscale, t);
        const uint32_t mag = sf == 0.0f ? 0u : cd;   // s == 0: signed zeros
        codes |= (mag | ((b >> 15) << 3)) << (4 * i);
    }
    return codes;
}

__global__ __launch_bounds__(QUANT_THREADS) void nv_quantize_kernel(const uint4* __restrict__ x,
                                                                     int64_t total, float gscale,
                                                                     uint8_t* __restrict__ q,
                                                                     uint8_t* __restrict__ s)
{
    const int lane = threadIdx.x & 63;
    const int64_t wave_base = ((int64_t)blockIdx.x * (QUANT_THREADS / 64) + (threadIdx.x >> 6)) * ELEMS_PER_WAVE;
    uint4 v[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int64_t gi = wave_base / 8 + 64 * j + lane;
        v[j] = (gi * 8 < total) ? ld_nt(&x[gi]) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int64_t gi = wave_base / 8 + 64 * j + lane;
        uint32_t sc;
        float sf;
        const uint32_t codes = nv_encode8(v[j], gscale, sc, sf);
        if (gi * 8 < total) {
            reinterpret_cast<uint32_t*>(q)[gi] = codes;
            if ((lane & 1) == 0) s[gi >> 1] = (uint8_t)sc;
        }
    }
}

// ---------------------------------------------------------------- fake quantization
// The quantize -> dequantize round trip written back as bf16, the op that
// runs in the training forward in place of the serving quantizer
// (Qwen3.5-9B-MXFP4-QAD-W4A4-LR1e-5-s3000, "Training mode": the training
// quantizer is bit-identical to the serving one).  The codes are produced by
// the same encoders as the quantizer kernels above, then decoded; each output
// is the bf16 nearest to the exact dequantized value, ties to even.

// 8 decoded element values (scale 1, exact in fp32) of the codes of one
// 8-element group.
template <int ELEM>
__device__ __forceinline__ void decode8(uint4 v, int e, float f[8])
{
    if (ELEM == ELEM_E2M1) {
        const uint32_t c = encode8_e2m1(v, e);
        const float2_t f0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c, 1.0f, 0);
        const float2_t f1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c, 1.0f, 1);
        const float2_t f2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c, 1.0f, 2);
        const float2_t f3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c, 1.0f, 3);
        f[0] = f0[0]; f[1] = f0[1]; f[2] = f1[0]; f[3] = f1[1];
        f[4] = f2[0]; f[5] = f2[1]; f[6] = f3[0]; f[7] = f3[1];
    } else {
        const uint2 c = encode8_e4m3(v, e);
        const float2_t f0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(c.x, 1.0f, false);
        const float2_t f1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(c.x, 1.0f, true);
        const float2_t f2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(c.y, 1.0f, false);
        const float2_t f3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(c.y, 1.0f, true);
        f[0] = f0[0]; f[1] = f0[1]; f[2] = f1[0]; f[3] = f1[1];
        f[4] = f2[0]; f[5] = f2[1]; f[6] = f3[0]; f[7] = f3[1];
    }
}

// MX: element value times 2^e is exact in fp32 (ldexp keeps subnormal
// results and overflows to infinity), so one fp32 -> bf16 rounding gives the
// nearest bf16.  Same work mapping as mx_quantize_kernel; each group of 8
// goes out as one 16-byte store.
template <int ELEM, int RULE>
__global__ __launch_bounds__(QUANT_THREADS) void mx_fake_quant_kernel(const uint4* __restrict__ x,
                                                                       int64_t total,
                                                                       uint4* __restrict__ y)
{
    const int lane = threadIdx.x & 63;
    const int64_t wave_base = ((int64_t)blockIdx.x * (QUANT_THREADS / 64) + (threadIdx.x >> 6)) * ELEMS_PER_WAVE;
    uint4 v[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int64_t g = wave_base / 8 + 64 * j + lane;
        v[j] = (g * 8 < total) ? x[g] : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int64_t g = wave_base / 8 + 64 * j + lane;
        const int e = scale_exponent<ELEM, RULE>(quad_max_u32(amax_bits8(v[j])));
        float f[8];
        decode8<ELEM>(v[j], e, f);
        uint32_t o[4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
            o[i] = bf16x2_rne(__builtin_amdgcn_ldexpf(f[2 * i], e), __builtin_amdgcn_ldexpf(f[2 * i + 1], e));
        if (g * 8 < total) y[g] = make_uint4(o[0], o[1], o[2], o[3]);
    }
}

// bf16 pattern (sign clear) nearest to p / g for p >= 0 and g > 0, ties to
// even.  q = p * (1/g), with 1/g a normal fp32 (ginv; DIV divides instead,
// for g beyond 2^126), is within 2 ulp of the quotient, far closer than the
// bf16 spacing, so the answer is the bf16 truncation lo of q or lo + 1; the
// midpoint m between them (9 significant bits) decides, compared as
// m * g <=> p through one fused multiply-add: its result is negative exactly
// when the quotient lies above m, and +0 exactly on a tie.  A quotient
// beyond the fp32 range (q = inf, lo = 0x7F80) stays infinity.
template <bool DIV>
__device__ __forceinline__ uint32_t bf16_nearest_quotient(float p, float g, float ginv)
{
    const float q = DIV ? p / g : p * ginv;
    const uint32_t lo = __float_as_uint(q) >> 16;
    const float m = __uint_as_float((lo << 16) | 0x8000u);
    const uint32_t rb = __float_as_uint(__builtin_fmaf(m, g, -p));
    const uint32_t up = (rb >> 31) + (rb == 0u ? (lo & 1u) : 0u);
    const uint32_t r = lo + up;
    return r < 0x7F80u ? r : 0x7F80u;
}

// NVFP4: the dequantized value p / g, p = e2m1 * s, is rounded once to
// bf16; p comes from the codes through the hardware decoder (scale 1) and
// one multiply, both exact.  Where p (1/g) (1 - 2^-21) and p (1/g) (1 +
// 2^-21) are normal and round to the same bf16 (hardware RNE), that is the
// rounding of p / g, by the bracket argument of nv_encode8; otherwise
// bf16_nearest_quotient decides.  Same mapping as nv_quantize_kernel; the
// quotient's form is chosen once per launch.
template <bool DIV>
__device__ __forceinline__ void nv_fake_quant_body(const uint4* __restrict__ x, int64_t total, float gscale,
                                                   uint4* __restrict__ y)
{
    const int lane = threadIdx.x & 63;
    const int64_t wave_base = ((int64_t)blockIdx.x * (QUANT_THREADS / 64) + (threadIdx.x >> 6)) * ELEMS_PER_WAVE;
    const float ginv = DIV ? 0.0f : 1.0f / gscale;
    const float g_lo = ginv * (1.0f - 0x1p-21f), g_hi = ginv * (1.0f + 0x1p-21f);
    uint4 v[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int64_t gi = wave_base / 8 + 64 * j + lane;
        v[j] = (gi * 8 < total) ? ld_nt(&x[gi]) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int64_t gi = wave_base / 8 + 64 * j + lane;
        uint32_t sc;
        float sf;
        const uint32_t codes = nv_encode8(v[j], gscale, sc, sf);
        float f[8];
        {
            const float2_t f0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, 1.0f, 0);
            const float2_t f1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, 1.0f, 1);
            const float2_t f2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, 1.0f, 2);
            const float2_t f3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, 1.0f, 3);
            f[0] = f0[0]; f[1] = f0[1]; f[2] = f1[0]; f[3] = f1[1];
            f[4] = f2[0]; f[5] = f2[1]; f[6] = f3[0]; f[7] = f3[1];
        }
        const uint32_t w[4] = {v[j].x, v[j].y, v[j].z, v[j].w};
        // the bracket of nv_encode8 once more: bf16 RNE of p (1/g) (1 -+ 2^-21)
        // where both are normal (the smallest nonzero p is s / 2) and agree
        const bool qfast = !DIV && sf * 0.5f * g_lo >= 0x1p-125f;
        uint32_t o[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float p0 = __builtin_fabsf(f[2 * i]) * sf, p1 = __builtin_fabsf(f[2 * i + 1]) * sf;
            uint32_t r = bf16x2_rne(p0 * g_lo, p1 * g_lo);
            if (!(qfast && r == bf16x2_rne(p0 * g_hi, p1 * g_hi)))
                r = bf16_nearest_quotient<DIV>(p0, gscale, ginv) | (bf16_nearest_quotient<DIV>(p1, gscale, ginv) << 16);
            o[i] = r | (w[i] & 0x80008000u);   // the input's signs are the codes' signs
        }
        if (gi * 8 < total) st_nt(&y[gi], make_uint4(o[0], o[1], o[2], o[3]));
    }
}

__global__ __launch_bounds__(QUANT_THREADS) void nv_fake_quant_kernel(const uint4* __restrict__ x,
                                                                       int64_t total, float gscale,
                                                                       uint4* __restrict__ y)
{
    if (gscale < 0x1p126f) nv_fake_quant_body<false>(x, total, gscale, y);
    else nv_fake_quant_body<true>(x, total, gscale, y);
}

// ---------------------------------------------------------------- SwiGLU + quantization
// The unfused step between the gate_up projection and the down projection:
// x is [rows, 2 * inter] bf16 with gate columns [0, inter) and up columns
// [inter, 2 * inter); h = bf16(swiglu_f32(gate, up)) is quantized to MXFP4
// with CEIL-rule scales: codes [rows, inter/2], scales [rows, inter/32].
// Work mapping as mx_quantize_kernel over the flat h array (inter % 32 == 0,
// so a lane quad is one block of one row); each lane reads its 8 gate and 8
// up values with one 16-byte load each.
__global__ __launch_bounds__(QUANT_THREADS) void swiglu_quant_kernel(const uint4* __restrict__ x,
                                                                      int64_t total, int inter,
                                                                      uint8_t* __restrict__ q,
                                                                      uint8_t* __restrict__ s)
{
    const int lane = threadIdx.x & 63;
    const int64_t wave_base = ((int64_t)blockIdx.x * (QUANT_THREADS / 64) + (threadIdx.x >> 6)) * ELEMS_PER_WAVE;
    const int gpr = inter / 8;   // 8-element groups per row of h
    uint4 gv[4], uv[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int64_t gi = wave_base / 8 + 64 * j + lane;
        const int64_t row = gi / gpr, c = gi - row * gpr;
        const int64_t src = row * (2 * (int64_t)gpr) + c;   // uint4 index of the gate group
        const bool ok = gi * 8 < total;
        gv[j] = ok ? ld_nt(&x[src]) : make_uint4(0, 0, 0, 0);
        uv[j] = ok ? ld_nt(&x[src + gpr]) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int64_t gi = wave_base / 8 + 64 * j + lane;
        const uint32_t gw[4] = {gv[j].x, gv[j].y, gv[j].z, gv[j].w};
        const uint32_t uw[4] = {uv[j].x, uv[j].y, uv[j].z, uv[j].w};
        uint32_t hw[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float h0 = swiglu_f32(__uint_as_float(gw[i] << 16), __uint_as_float(uw[i] << 16));
            const float h1 = swiglu_f32(__uint_as_float(gw[i] & 0xFFFF0000u), __uint_as_float(uw[i] & 0xFFFF0000u));
            hw[i] = bf16x2_rne(h0, h1);
        }
        const uint4 h = make_uint4(hw[0], hw[1], hw[2], hw[3]);
        const int e = scale_exponent<ELEM_E2M1, RULE_CEIL>(quad_max_u32(amax_bits8(h)));
        const uint32_t codes = encode8_e2m1(h, e);
        if (gi * 8 < total) {
            reinterpret_cast<uint32_t*>(q)[gi] = codes;
            if ((lane & 3) == 0) s[gi >> 2] = (uint8_t)(e + 127);
        }
    }
}

// amax of a bf16 tensor into *out (fp32 bits; non-negative floats order like
// unsigned integers, so an integer atomic max is a float max).
__global__ void amax_init_kernel(uint32_t* out) { *out = 0u; }

__global__ __launch_bounds__(256) void amax_kernel(const uint16_t* __restrict__ x, int64_t count,
                                                   uint32_t* __restrict__ out)
{
    uint32_t m = 0;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    const int64_t nvec = count / 8;
    const uint4* xv = reinterpret_cast<const uint4*>(x);
    int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    // four independent 16-byte loads in flight per lane
    for (; i + 3 * stride < nvec; i += 4 * stride) {
        const uint4 v0 = ld_nt(&xv[i]), v1 = ld_nt(&xv[i + stride]), v2 = ld_nt(&xv[i + 2 * stride]),
                    v3 = ld_nt(&xv[i + 3 * stride]);
        const uint32_t a = max(max(amax_bits8(v0), amax_bits8(v1)), max(amax_bits8(v2), amax_bits8(v3)));
        m = m > a ? m : a;
    }
    for (; i < nvec; i += stride) {
        const uint32_t a = amax_bits8(xv[i]);
        m = m > a ? m : a;
    }
    for (int64_t i = nvec * 8 + (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < count; i += stride) {
        uint32_t a = x[i] & 0x7FFFu;
        m = m > a ? m : a;
    }
    // wave reduction, then across the block's waves through LDS, then one
    // atomic per block: atomics on a single address serialize, so their
    // count (the grid is capped at 512 blocks) must stay small
    for (int off = 32; off > 0; off >>= 1) {
        uint32_t o = (uint32_t)__shfl_xor((int)m, off, 64);
        m = m > o ? m : o;
    }
    __shared__ uint32_t wmax[4];
    if ((threadIdx.x & 63) == 0) wmax[threadIdx.x >> 6] = m;
    __syncthreads();
    if (threadIdx.x == 0) {
        m = wmax[0];
        for (int w = 1; w < 4; ++w) m = m > wmax[w] ? m : wmax[w];
        atomicMax(out, m << 16);
    }
}

} // namespace mxl

// ---------------------------------------------------------------- launchers
using namespace mxl;

extern "C" hipError_t mxl_launch_mx_quantize(int elem, int rule, const void* x, int64_t total,
                                             void* q, void* s, hipStream_t stream)
{
    const int64_t blocks = (total + ELEMS_PER_BLOCK - 1) / ELEMS_PER_BLOCK;
    dim3 grid((unsigned)blocks), block(QUANT_THREADS);
    const uint4* xv = static_cast<const uint4*>(x);
    uint8_t* qb = static_cast<uint8_t*>(q);
    uint8_t* sb = static_cast<uint8_t*>(s);
#define MXL_Q(E, R) hipLaunchKernelGGL((mx_quantize_kernel<E, R>), grid, block, 0, stream, xv, total, qb, sb)
    if (elem == ELEM_E2M1) {
        if (rule == RULE_FLOOR) MXL_Q(ELEM_E2M1, RULE_FLOOR);
        else if (rule == RULE_CEIL) MXL_Q(ELEM_E2M1, RULE_CEIL);
        else MXL_Q(ELEM_E2M1, RULE_EVEN);
    } else {
        if (rule == RULE_FLOOR) MXL_Q(ELEM_E4M3, RULE_FLOOR);
        else if (rule == RULE_CEIL) MXL_Q(ELEM_E4M3, RULE_CEIL);
        else MXL_Q(ELEM_E4M3, RULE_EVEN);
    }
#undef MXL_Q
    return hipGetLastError();
}

extern "C" hipError_t mxl_launch_nv_quantize(const void* x, int64_t total, float g, void* q, void* s,
                                             hipStream_t stream)
{
    const int64_t blocks = (total + ELEMS_PER_BLOCK - 1) / ELEMS_PER_BLOCK;
    hipLaunchKernelGGL(nv_quantize_kernel, dim3((unsigned)blocks), dim3(QUANT_THREADS), 0, stream,
                       static_cast<const uint4*>(x), total, g, static_cast<uint8_t*>(q),
                       static_cast<uint8_t*>(s));
    return hipGetLastError();
}

extern "C" hipError_t mxl_launch_amax(const void* x, int64_t count, float* out, hipStream_t stream)
{
    hipLaunchKernelGGL(amax_init_kernel, dim3(1), dim3(1), 0, stream, reinterpret_cast<uint32_t*>(out));
    int64_t blocks = (count / 8 + 255) / 256;
    if (blocks < 1) blocks = 1;
    if (blocks > 512) blocks = 512;
    hipLaunchKernelGGL(amax_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                       static_cast<const uint16_t*>(x), count, reinterpret_cast<uint32_t*>(out));
    return hipGetLastError();
}

extern "C" hipError_t mxl_launch_mx_fake_quant(int elem, int rule, const void* x, int64_t total, void* y,
                                               hipStream_t stream)
{
    const int64_t blocks = (total + ELEMS_PER_BLOCK - 1) / ELEMS_PER_BLOCK;
    dim3 grid((unsigned)blocks), block(QUANT_THREADS);
    const uint4* xv = static_cast<const uint4*>(x);
    uint4* yv = static_cast<uint4*>(y);
#define MXL_F(E, R) hipLaunchKernelGGL((mx_fake_quant_kernel<E, R>), grid, block, 0, stream, xv, total, yv)
    if (elem == ELEM_E2M1) {
        if (rule == RULE_FLOOR) MXL_F(ELEM_E2M1, RULE_FLOOR);
        else if (rule == RULE_CEIL) MXL_F(ELEM_E2M1, RULE_CEIL);
        else MXL_F(ELEM_E2M1, RULE_EVEN);
    } else {
        if (rule == RULE_FLOOR) MXL_F(ELEM_E4M3, RULE_FLOOR);
        else if (rule == RULE_CEIL) MXL_F(ELEM_E4M3, RULE_CEIL);
        else MXL_F(ELEM_E4M3, RULE_EVEN);
    }
#undef MXL_F
    return hipGetLastError();
}

extern "C" hipError_t mxl_launch_nv_fake_quant(const void* x, int64_t total, float g, void* y,
                                               hipStream_t stream)
{
    const int64_t blocks = (total + ELEMS_PER_BLOCK - 1) / ELEMS_PER_BLOCK;
    hipLaunchKernelGGL(nv_fake_quant_kernel, dim3((unsigned)blocks), dim3(QUANT_THREADS), 0, stream,
                       static_cast<const uint4*>(x), total, g, static_cast<uint4*>(y));
    return hipGetLastError();
}

extern "C" hipError_t mxl_launch_swiglu_quant(const void* x, int64_t rows, int64_t inter, void* q, void* s,
                                              hipStream_t stream)
{
    const int64_t total = rows * inter;
    const int64_t blocks = (total + ELEMS_PER_BLOCK - 1) / ELEMS_PER_BLOCK;
    hipLaunchKernelGGL(swiglu_quant_kernel, dim3((unsigned)blocks), dim3(QUANT_THREADS), 0, stream,
                       static_cast<const uint4*>(x), total, (int)inter, static_cast<uint8_t*>(q),
                       static_cast<uint8_t*>(s));
    return hipGetLastError();
}
