// mx_device.h -- device-side building blocks shared by the gfx950 kernels of
// libmxlinear: bf16 bit handling, wave-level reductions, the block-scale
// rules on bf16 bit patterns, and the element encoders.
//
// Formats (OCP Microscaling v1.0, which the AutoRound card
// Qwen3.8-27B-MXFP8Attn-MXFP4MLP-lmheadMXFP4 names in section 7):
//   E2M1: sign bit 3, exponent bits 2..1 (bias 1), mantissa bit 0; magnitudes
//         0, .5, 1, 1.5, 2, 3, 4, 6.
//   E4M3: sign bit 7, exponent bits 6..3 (bias 7), mantissa 2..0; max 448,
//         S.1111.111 is NaN.
//   E8M0: biased exponent, value 2^(c - 127).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace mxl {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef short short2_t __attribute__((ext_vector_type(2)));
typedef float float2_t __attribute__((ext_vector_type(2)));
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef float float16_t __attribute__((ext_vector_type(16)));
typedef int int4_t __attribute__((ext_vector_type(4)));
typedef int int8_t_ __attribute__((ext_vector_type(8)));
typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));

enum : int { ELEM_E2M1 = 0, ELEM_E4M3 = 1 };
enum : int { RULE_FLOOR = 0, RULE_CEIL = 1, RULE_EVEN = 2 };

__device__ __forceinline__ float bf16_bits_to_float(uint32_t b16) { return __uint_as_float(b16 << 16); }

// Workgroup barrier for LDS hand-offs only.  __syncthreads() also fences
// global memory, which makes every wave wait for all of its outstanding
// global loads (vmcnt(0)) at each barrier and defeats register prefetching.
// Here each wave waits only for its own LDS operations (lgkmcnt(0)) before the
// hardware barrier; the empty asm statements keep the compiler from moving
// memory accesses across it.  Global loads into registers are still waited for
// precisely by the compiler where their registers are used.
__device__ __forceinline__ void lds_barrier()
{
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0); vmcnt and expcnt left at their maxima
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// Max over the 4 lanes of a lane quad (lanes 4q .. 4q+3) via DPP quad permutes.
__device__ __forceinline__ uint32_t quad_max_u32(uint32_t v)
{
    uint32_t o = (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, false); // [1,0,3,2]
    v = v > o ? v : o;
    o = (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xF, 0xF, false);          // [2,3,0,1]
    return v > o ? v : o;
}
// Max over lane pairs (2p, 2p+1).
__device__ __forceinline__ uint32_t pair_max_u32(uint32_t v)
{
    uint32_t o = (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, false);
    return v > o ? v : o;
}

// Largest |x| of 8 bf16 values packed in a uint4, as a 15-bit magnitude
// pattern.  Non-negative floats order like their bit patterns, so the
// maximum is an integer maximum of the sign-cleared halves.
__device__ __forceinline__ uint32_t amax_bits8(uint4 v)
{
    uint32_t m = 0;
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        uint32_t lo = w[i] & 0x7FFFu, hi = (w[i] >> 16) & 0x7FFFu;
        m = m > lo ? m : lo;
        m = m > hi ? m : hi;
    }
    return m;
}

// Scale exponent e (scale 2^e) of a block from its amax bf16 magnitude bits.
// amax = M * 2^E with M in [1, 2):
//   FLOOR e = E - emax
//   CEIL  e = E - emax + [M > max_elem / 2^emax]   (1.5 for E2M1, 1.75 for E4M3)
//   EVEN  e = E - emax + [M >= 2 - 2^-(mbits+1)]   (1.75 for E2M1, 1.9375 for E4M3)
// clamped to [-127, 127].  A zero or subnormal bf16 amax always lands on the
// lower clamp (E <= -127), so only the normal encoding is decoded here.
template <int ELEM, int RULE>
__device__ __forceinline__ int scale_exponent(uint32_t amax16)
{
    const int ef = (int)(amax16 >> 7);       // bf16 exponent field
    const uint32_t mb = amax16 & 0x7Fu;      // 7 mantissa bits
    if (ef == 0) return -127;
    const int emax = ELEM == ELEM_E2M1 ? 2 : 8;
    int bump = 0;
    if (RULE == RULE_CEIL) bump = ELEM == ELEM_E2M1 ? (mb > 0x40u) : (mb > 0x60u);
    if (RULE == RULE_EVEN) bump = ELEM == ELEM_E2M1 ? (mb >= 0x60u) : (mb >= 0x78u);
    int e = ef - 127 - emax + bump;
    e = e < -127 ? -127 : e;
    return e > 127 ? 127 : e;
}

// 2^e as an fp32 for e in [-126, 127].
__device__ __forceinline__ float pow2f(int e) { return __uint_as_float((uint32_t)(e + 127) << 23); }

// Encode 8 bf16 values (a uint4) as E2M1 codes of x / 2^e, 4 bytes, element
// 2j in the low nibble of byte j.  The gfx950 conversion rounds to nearest
// even, saturates at 6 and keeps the sign; its scale operand contributes
// only its exponent, so it is passed as the fp32 2^e.  e = -127 has no normal
// fp32, so that (rare) case pre-multiplies by 2^126 and divides by 2^-1.
__device__ __forceinline__ uint32_t encode8_e2m1(uint4 v, int e)
{
    uint32_t r = 0;
    if (e > -127) {
        const float s = pow2f(e);
        bf16x2_t p0, p1, p2, p3;
        __builtin_memcpy(&p0, &v.x, 4);
        __builtin_memcpy(&p1, &v.y, 4);
        __builtin_memcpy(&p2, &v.z, 4);
        __builtin_memcpy(&p3, &v.w, 4);
        r = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(r, p0, s, 0);
        r = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(r, p1, s, 1);
        r = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(r, p2, s, 2);
        r = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(r, p3, s, 3);
    } else {
        const float up = 0x1p126f, s = 0.5f;
#define MXL_LO(w) (bf16_bits_to_float((w) & 0xFFFFu) * up)
#define MXL_HI(w) (bf16_bits_to_float((w) >> 16) * up)
        r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, MXL_LO(v.x), MXL_HI(v.x), s, 0);
        r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, MXL_LO(v.y), MXL_HI(v.y), s, 1);
        r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, MXL_LO(v.z), MXL_HI(v.z), s, 2);
        r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, MXL_LO(v.w), MXL_HI(v.w), s, 3);
#undef MXL_LO
#undef MXL_HI
    }
    return r;
}

// Encode 8 bf16 values as E4M3 codes of x / 2^e (8 bytes).  The gfx950
// conversion rounds to nearest even but turns values beyond 464 into NaN, so
// inputs are clamped to +-448 * 2^e first (exact), giving the saturating
// behaviour of the format definition.
__device__ __forceinline__ uint2 encode8_e4m3(uint4 v, int e)
{
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
    float up = 1.0f, s;
    if (e > -127) {
        s = pow2f(e);
    } else {
        up = 0x1p126f;
        s = 0.5f;
    }
    const float lim = 448.0f * s;
    float f[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        f[2 * i] = __builtin_amdgcn_fmed3f(bf16_bits_to_float(w[i] & 0xFFFFu) * up, -lim, lim);
        f[2 * i + 1] = __builtin_amdgcn_fmed3f(bf16_bits_to_float(w[i] >> 16) * up, -lim, lim);
    }
    short2_t lo = {0, 0}, hi = {0, 0};
    lo = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(lo, f[0], f[1], s, false);
    lo = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(lo, f[2], f[3], s, true);
    hi = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(hi, f[4], f[5], s, false);
    hi = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(hi, f[6], f[7], s, true);
    uint32_t out[2];
    __builtin_memcpy(&out[0], &lo, 4);
    __builtin_memcpy(&out[1], &hi, 4);
    return make_uint2(out[0], out[1]);
}

// ---------------------------------------------------------------- NVFP4 helpers
// E4M3 value of a code (non-NaN codes), as a double.
__device__ __forceinline__ double e4m3_value_f64(uint32_t c)
{
    const uint32_t ef = (c >> 3) & 15u, m = c & 7u;
    double mag = ef == 0 ? (double)m * 0x1p-9 : (1.0 + (double)m * 0.125) * __builtin_ldexp(1.0, (int)ef - 7);
    return (c & 0x80u) ? -mag : mag;
}

// RNE_E4M3 of a non-negative double v (saturating at 448): v >= 448 -> 0x7E;
// below 2^-6 the subnormal step 2^-9 applies; otherwise the double is rounded
// to 3 mantissa bits (ties to even) on its bit pattern.
// All three forms are computed and one is selected, so the code has no branch.
__device__ __forceinline__ uint32_t e4m3_rne_f64(double v)
{
    const uint32_t sub = (uint32_t)__builtin_rint(__builtin_fmin(v, 0x1p-6) * 512.0); // 0..8; 8 is 2^-6
    uint64_t b = (uint64_t)__double_as_longlong(v);
    b += ((uint64_t)1 << 48) - 1 + ((b >> 49) & 1);              // RNE at mantissa bit 49
    const uint32_t nrm = (uint32_t)(b >> 49) - ((1023u - 7u) << 3); // exponent(11) | mantissa(3), rebiased
    return v >= 448.0 ? 0x7Eu : (v < 0x1p-6 ? sub : nrm);
}

// The 7 rounding thresholds of E2M1 (midpoints between neighbouring
// magnitudes) times a block scale s: t * s is exact in fp32 (t has at most 3
// significant bits, an E4M3 s at most 4).
__device__ __forceinline__ void e2m1_thresholds(float s, float t[7])
{
    t[0] = 0.25f * s; t[1] = 0.75f * s; t[2] = 1.25f * s; t[3] = 1.75f * s;
    t[4] = 2.5f * s;  t[5] = 3.5f * s;  t[6] = 5.0f * s;
}

// RNE_E2M1 code (magnitude) of the exact real xa * g / s for xa >= 0, g > 0,
// given the thresholds t of s > 0: the number of thresholds that xa * g
// passes, where landing exactly on one goes to the even code, so the
// thresholds below codes 1, 3, 5, 7 count only when passed strictly.  Each
// comparison is the sign bit of one fma, the exact difference rounded once:
// fma(-xa, g, t) < 0 for "xa * g > t" and fma(xa, g, -t) < 0 for
// "xa * g < t"; an exact zero difference rounds to +0, so a tie is never
// negative.  No difference rounds to zero from a nonzero value: near a
// threshold xa * g >= 2^-11 and every bit of xa * g and t lies above 2^-42,
// far from fp32's subnormal step.  An overflow of xa * g gives -inf / +inf,
// which still compare correctly.
__device__ __forceinline__ uint32_t e2m1_rne_fma(float xa, float g, const float t[7])
{
    const uint32_t above = (__float_as_uint(__builtin_fmaf(-xa, g, t[0])) >> 31) +
                           (__float_as_uint(__builtin_fmaf(-xa, g, t[2])) >> 31) +
                           (__float_as_uint(__builtin_fmaf(-xa, g, t[4])) >> 31) +
                           (__float_as_uint(__builtin_fmaf(-xa, g, t[6])) >> 31);
    const uint32_t below = (__float_as_uint(__builtin_fmaf(xa, g, -t[1])) >> 31) +
                           (__float_as_uint(__builtin_fmaf(xa, g, -t[3])) >> 31) +
                           (__float_as_uint(__builtin_fmaf(xa, g, -t[5])) >> 31);
    return above + 3u - below;
}

// fp32 -> bf16, round to nearest even, on the hardware converter
// (v_cvt_pk_bf16_f32).  For every finite input it equals the bit rule
// (u + 0x7fff + ((u >> 16) & 1)) >> 16 (checked exhaustively over all 2^32
// patterns); non-finite inputs are outside the library's contract.
__device__ __forceinline__ uint32_t bf16x2_rne(float lo, float hi)
{
    typedef float f32x2 __attribute__((ext_vector_type(2)));
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){lo, hi}, bf16x2));
}
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) { return (uint16_t)bf16x2_rne(f, 0.0f); }

// SwiGLU of bf16 gate and up values, silu(g) * u = g * u / (1 + e^-g),
// evaluated in fp32 as (g * rcp(1 + exp2(-g * log2 e))) * u on the hardware
// exp2 and reciprocal: a relative error of a few fp32 ulp, far below the
// bf16 step of the result.  Every kernel that applies SwiGLU calls this
// function, so fused and unfused paths agree bit for bit.  For g below about
// -88 the exponential is +inf and the result a signed zero.
__device__ __forceinline__ float swiglu_f32(float g, float u)
{
    const float t = __builtin_amdgcn_exp2f(-g * 1.44269504088896341f);
    return g * __builtin_amdgcn_rcpf(1.0f + t) * u;
}

// Buffer-to-LDS copies.  Each instruction writes its 64 lanes x width bytes
// contiguously at the LDS address in M0, reading each lane's bytes from the
// buffer at (voff + soff); lanes past the buffer's size read zero.  They are
// issued from inline assembly, so the compiler does not count them: callers
// wait with wait_vmcnt, whose count includes them, before a barrier that
// publishes the data.  A write of M0 needs one instruction between it and
// the load that takes its LDS address from M0 (s_nop 0 here, the offset add
// in the _at forms).
__device__ __forceinline__ void dma_b128(uint32_t lds, int voff, const int4_t& rsrc, int soff)
{
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
                 :: "s"(lds), "v"(voff), "s"(rsrc), "s"(soff) : "memory");
}
__device__ __forceinline__ void dma_b32(uint32_t lds, int voff, const int4_t& rsrc, int soff)
{
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dword %1, %2, %3 offen lds"
                 :: "s"(lds), "v"(voff), "s"(rsrc), "s"(soff) : "memory");
}
// The same copies to LDS address lds + imm from buffer offset voff + sadd
// (sadd uniform), in three instructions.  imm must fold to a constant once
// the caller is inlined and unrolled.
__device__ __forceinline__ void dma_b128_at(uint32_t lds, int imm, int voff, int sadd, const int4_t& rsrc)
{
    int off;
    asm volatile("s_add_u32 m0, %1, %5\n\tv_add_u32 %0, %2, %3\n\tbuffer_load_dwordx4 %0, %4, 0 offen lds"
                 : "=&v"(off) : "s"(lds), "s"(sadd), "v"(voff), "s"(rsrc), "i"(imm) : "memory", "scc");
}
__device__ __forceinline__ void dma_b32_at(uint32_t lds, int imm, int voff, int sadd, const int4_t& rsrc)
{
    int off;
    asm volatile("s_add_u32 m0, %1, %5\n\tv_add_u32 %0, %2, %3\n\tbuffer_load_dword %0, %4, 0 offen lds"
                 : "=&v"(off) : "s"(lds), "s"(sadd), "v"(voff), "s"(rsrc), "i"(imm) : "memory", "scc");
}
template <int N>
__device__ __forceinline__ void wait_vmcnt()
{
    static_assert(N >= 0 && N <= 63, "vmcnt range");
    asm volatile("s_waitcnt vmcnt(%0)" :: "n"(N) : "memory");
}

// Raw buffer descriptor (stride 0) over `bytes` bytes at `base`, built as
// four uniform dwords so it lives in SGPRs: base address (48 bits),
// num_records, and the dword-format word that raw buffer loads use.
__device__ __forceinline__ int4_t make_rsrc(const void* base, uint32_t bytes)
{
    const uint64_t a = (uint64_t)(uintptr_t)base;
    int4_t v;
    v[0] = __builtin_amdgcn_readfirstlane((int)(uint32_t)a);
    v[1] = __builtin_amdgcn_readfirstlane((int)((uint32_t)(a >> 32) & 0xffffu));
    v[2] = __builtin_amdgcn_readfirstlane((int)bytes);
    v[3] = 0x00020000;
    return v;
}

// Fills the part of Y[M, N] (bf16, or fp32 when f32) covered by the tile
// [m0, m0 + bm) x [n0, n0 + bn) with NaN, from all threads of the
// workgroup.  A tile whose bounded wait for another workgroup gave up writes
// this instead of its product, so the failure cannot pass for a result.
__device__ __forceinline__ void fill_tile_nan(void* y, int M, int N, int m0, int n0, int bm, int bn, bool f32)
{
    for (int idx = threadIdx.x; idx < bm * bn; idx += blockDim.x) {
        const int m = m0 + idx / bn, n = n0 + idx % bn;
        if (m < M && n < N) {
            if (f32) reinterpret_cast<uint32_t*>(y)[(size_t)m * N + n] = 0x7FC00000u;
            else reinterpret_cast<uint16_t*>(y)[(size_t)m * N + n] = (uint16_t)0x7FC0u;
        }
    }
}

// Calls f(std::integral_constant<int, i>) for i = B .. E-1 in order: a loop
// whose index is a compile-time constant in every iteration however large the
// body (unrolling by pragma stops at a size threshold, and inline-assembly
// immediates need constants).
template <int B, int E, class F>
__device__ __forceinline__ void static_for(F&& f)
{
    if constexpr (B < E) {
        f(std::integral_constant<int, B>{});
        static_for<B + 1, E>(f);
    }
}

// Tile ordering.  Workgroups are dispatched round-robin over the 8 XCDs
// (workgroup i runs on XCD i % 8), and each XCD has its own L2.  So the
// workgroup id is first remapped so that each XCD receives one contiguous
// range of the tile order, and the tile order itself walks groups of GROUP_N
// tile columns down M (N fastest inside a group): the tiles an XCD runs at
// the same time share a few A row panels and W column panels in its L2.
constexpr int NUM_XCD = 8;

template <int BM, int BN, int GROUP_N>
__device__ __forceinline__ void tile_coords(int M, int N, int id, int& tm, int& tn)
{
    const int tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
    const int total = tiles_m * tiles_n;
    const int xcd = id % NUM_XCD, j = id / NUM_XCD;
    const int q = total / NUM_XCD, r = total % NUM_XCD;
    const int t = xcd * q + (xcd < r ? xcd : r) + j;   // bijection onto [0, total)
    const int group_size = GROUP_N * tiles_m;
    const int gidx = t / group_size;
    const int first_n = gidx * GROUP_N;
    const int gn = (tiles_n - first_n) < GROUP_N ? (tiles_n - first_n) : GROUP_N;
    const int in = t % group_size;
    tm = in / gn;
    tn = first_n + in % gn;
}

} // namespace mxl
