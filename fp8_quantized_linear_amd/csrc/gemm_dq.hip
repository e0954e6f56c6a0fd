// gemm_dq.hip -- GEMMs that dequantize their operands exactly into 16-bit
// floats while staging them into LDS and contract them on f16/bf16 matrix
// cores with fp32 accumulation:
//
//   NVFP4: Y = alpha * sum_k (e2m1_a * s_a) * (e2m1_w * s_w), E4M3 scale per 16,
//          alpha = 1 / (g_a * g_w)                                   -> f16
//   MXFP8: Y = sum_k (e4m3_a * 2^ea) * (e4m3_w * 2^ew), E8M0 scale per 32 -> bf16
//   W4A16: Y = alpha * sum_k a_bf16 * dq(w), w MXFP4 (e2m1 * 2^ew, alpha = 1)
//          or NVFP4 (e2m1 * s_w, alpha = 1 / g_w)                    -> bf16
//   mixed MX pairs: A MXFP8 x W MXFP4 or A MXFP4 x W MXFP8, each operand
//          dequantized by its own format                              -> bf16
//
// Operations: the NVFP4 W4A4 path of Qwen3.5-27B-NVFP4-GPTQ and
// Qwen3.5-27B-NVFP4-RTN-weight-only (introductions: FP4 elements, per-block
// scales, per-tensor global scales), and the MXFP8 W8A8 attention projections
// of Qwen3.8-27B-MXFP8Attn-MXFP4MLP-lmheadMXFP4 (introduction, section 2);
// the weight-only mode that the same packed weights serve with bf16
// activations (Qwen3.5-27B-MXFP4-QAD-W4A4-LR1e-5-s1000 and
// Qwen3.5-27B-NVFP4-RTN-weight-only, introductions).
//
// Why these do not use the block-scaled FP4/FP8 matrix cores:
//  - NVFP4 scales are E4M3 per 16 elements; the scaled instructions accept
//    only power-of-two scales per 32.  e2m1 (2 significant bits) times an
//    E4M3 scale (4 bits, 2^-9 .. 448) is exact in f16.
//  - The FP8 matrix-core instructions of gfx950 do not accumulate exactly:
//    measured on hardware, their error reaches about 1.7e-4 (scaled 32x32x64)
//    to 3.9e-4 (unscaled 32x32x16) of sum|a*b| on operands with a wide
//    exponent spread, beyond the 1e-4 bound.  The f16/bf16 instructions stay at
//    fp32 rounding level.  An E4M3 value times its power-of-two block scale is
//    exact in bf16 (8-bit significand, fp32 exponent range) for every block
//    whose scale exponent is at least -117.  Below that (blocks with amax
//    under ~2^-110), values under 2^-126 become bf16 subnormals rounded to
//    nearest even.
//
// 16-bit matrix-core layout (32x32x16): lane l = r + 32 g holds row/column r
// and the 8 consecutive K elements [8g, 8g + 8) of the 16-wide step.
#include "mx_device.h"

#include <type_traits>

namespace mxl {

enum : int { DQ_NVFP4 = 0, DQ_MXFP8 = 1, DQ_MXFP4 = 2 };   // format of W (and of A unless A is bf16 or KA says otherwise)

constexpr int DQ_BK = 64;                 // K elements per LDS stage
constexpr int DQ_ROW_BYTES = DQ_BK * 2;   // 16-bit bytes per LDS row per stage (8 chunks)

__device__ __forceinline__ int dq_swz(int row) { return row & 7; }

template <int KIND>
struct DqTraits {
    // global bytes of one row per stage, 16-byte chunks per row per stage
    static constexpr int SRC_ROW_BYTES = KIND == DQ_MXFP8 ? DQ_BK : DQ_BK / 2;
    static constexpr int CHUNKS = SRC_ROW_BYTES / 16;
    static constexpr int ELEMS_PER_CHUNK = KIND == DQ_MXFP8 ? 16 : 32;
    static constexpr int SCALE_BLOCK = KIND == DQ_NVFP4 ? 16 : 32;
};

typedef __bf16 bf16x2_t_ __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));

// The two E4M3 codes in bits 0-15 of v as an f16 pair, by the hardware
// conversion at scale 1: exact, since every finite E4M3 value (subnormals
// included) is an f16 normal.  NaN codes never occur in valid scales.
__device__ __forceinline__ half2_t e4m3x2_to_f16x2(uint32_t v)
{
    return __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(v, 1.0f, false);
}
// the same pair as fp32 values
__device__ __forceinline__ float2_t e4m3x2_to_f32x2(uint32_t v)
{
    return __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(v, 1.0f, false);
}
// {s[i], s[i]}
__device__ __forceinline__ half2_t bcast_h2(half2_t s, int i)
{
    return i ? half2_t{s[1], s[1]} : half2_t{s[0], s[0]};
}

// 8 E2M1 codes (one dword, element 2j in the low nibble of byte j) times an
// E4M3 scale given as an f16 pair {s, s}, as 8 f16 values (exact products:
// at most 6 significant bits, magnitudes in [2^-10, 2688]).
__device__ __forceinline__ uint4 dequant8_nvfp4(uint32_t codes, half2_t s2)
{
    half2_t h[4];
    h[0] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 0) * s2;
    h[1] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 1) * s2;
    h[2] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 2) * s2;
    h[3] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 3) * s2;
    uint4 out;
    __builtin_memcpy(&out, h, 16);
    return out;
}

// 8 E4M3 codes (uint2) times 2^e, as 8 bf16 values.  The conversion reads
// the exponent field of its fp32 scale operand as an E8M0 scale, field 0
// (e = -127) included, and rounds results below 2^-126 to nearest even.
__device__ __forceinline__ uint4 dequant8_mxfp8(uint2 codes, int e)
{
    const float s = pow2f(e);
    bf16x2_t_ h[4];
    h[0] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(codes.x, s, false);
    h[1] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(codes.x, s, true);
    h[2] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(codes.y, s, false);
    h[3] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(codes.y, s, true);
    uint4 out;
    __builtin_memcpy(&out, h, 16);
    return out;
}

// 8 E2M1 codes (one dword) times 2^e, as 8 bf16 values: exact for every
// scale, 2^-127 included (e2m1 * 2^-127 is at least 2^-128, a bf16 subnormal).
__device__ __forceinline__ uint4 dequant8_mxfp4_bf16(uint32_t codes, int e)
{
    const float s = pow2f(e);
    bf16x2_t_ h[4];
    h[0] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, s, 0);
    h[1] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, s, 1);
    h[2] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, s, 2);
    h[3] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, s, 3);
    uint4 out;
    __builtin_memcpy(&out, h, 16);
    return out;
}

// 8 E2M1 codes (one dword) times an E4M3 scale s (as fp32), as 8 bf16
// values: e2m1 (2 significant bits) times s (4) is exact in bf16.
__device__ __forceinline__ uint4 dequant8_nvfp4_bf16(uint32_t codes, float s)
{
    const float2_t f0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, 1.0f, 0);
    const float2_t f1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, 1.0f, 1);
    const float2_t f2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, 1.0f, 2);
    const float2_t f3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, 1.0f, 3);
    return make_uint4(bf16x2_rne(f0[0] * s, f0[1] * s), bf16x2_rne(f1[0] * s, f1[1] * s),
                      bf16x2_rne(f2[0] * s, f2[1] * s), bf16x2_rne(f3[0] * s, f3[1] * s));
}

struct DqArgs {
    const uint8_t* a_q; const uint8_t* a_s;
    const uint8_t* w_q; const uint8_t* w_s;
    void* y;
    int M, N, K;
    float alpha;
    // split-K as in the MX tile kernel: workgroup b computes stages
    // [s * chunk, (s + 1) * chunk) (chunk even) of tile b % tiles, s = b /
    // tiles, and with splits > 1 writes its fp32 partial (without alpha) to
    // part + s * M * N
    float* part;
    int splits, chunk;
    // FUSED_A only, optional: the prologue's E4M3 codes [M, K] and E8M0
    // scales [M, K/32], written by the tiles of the first tile column
    uint8_t* dump_q;
    uint8_t* dump_s;
    // POOL only: A as bf16 [M, K], quantized once (RULE of the pool) into
    // a_q / a_s (a workspace) by the workgroups themselves; state: the chunk
    // pool counter, a done counter per 128-row block, an error word
    const uint4* a_bf16;
    int* state;
    int nb;
};

// ---------------------------------------------------------------------------
// Quantize-once for the fused MXFP8 GEMM (POOL): before its tile, a
// workgroup claims 32-row chunks of A (of any 128-row block) from the pool
// counter and quantizes them into the workspace exactly as mx_quantize_act
// does, until the pool is empty; then it waits until its own block's done
// counter shows every chunk.  It only waits for chunks that running
// workgroups have claimed and finish without waiting, so no co-residency is
// needed.  A chunk's writer waits for its stores and releases (one L2
// write-back) before counting it; readers poll with device-scope atomic loads
// and need no invalidation: a block is read only after it is done, and no L2
// holds its lines from before in this launch (blocks start on cache-line
// boundaries: the workspace is 256-byte aligned, the scale plane starts at a
// 256-byte boundary, and a block is 128 rows of k code bytes and of k/32
// scale bytes, k % 128 == 0).  Polls are bounded (about 0.5 s); a tile that
// gives up sets the error word and fills its part of Y with NaN.
// ---------------------------------------------------------------------------
constexpr int DQ_POOL_ROWS = 32;               // rows per chunk
constexpr int DQ_POOL_SPINS = 1 << 21;

// mx_quantize_act (MXFP8, rule RULE) of rows [r0, r1): consecutive threads
// take consecutive 8-element groups (lane quads hold the blocks of 32), 16
// groups per thread loaded before any is encoded.
template <int RULE, int NT>
__device__ __forceinline__ void dq_pool_quantize_rows(const uint4* __restrict__ x, int k, int r0, int r1,
                                                      uint8_t* __restrict__ q, uint8_t* __restrict__ s)
{
    constexpr int G = 16;
    const int lane = threadIdx.x & 63;
    const int64_t g_end = (int64_t)r1 * (k / 8);
    for (int64_t g0 = (int64_t)r0 * (k / 8) + threadIdx.x; g0 < g_end; g0 += G * NT) {
        uint4 v[G];
#pragma unroll
        for (int j = 0; j < G; ++j) {
            const int64_t g = g0 + NT * j;
            v[j] = x[g < g_end ? g : g0];
        }
#pragma unroll
        for (int j = 0; j < G; ++j) {
            const int64_t g = g0 + NT * j;
            const int e = scale_exponent<ELEM_E4M3, RULE>(quad_max_u32(amax_bits8(v[j])));
            const uint2 c = encode8_e4m3(v[j], e);
            if (g < g_end) {
                reinterpret_cast<uint2*>(q)[g] = c;
                if ((lane & 3) == 0) s[g >> 2] = (uint8_t)(e + 127);
            }
        }
    }
}

template <int RULE, int BM, int NT>
__device__ __forceinline__ bool dq_pool_ensure(const DqArgs& p, int tm, uint8_t* smem)
{
    constexpr int CPB = BM / DQ_POOL_ROWS;
    int* pool = p.state;
    int* done = p.state + 1;
    int* word = reinterpret_cast<int*>(smem);
    while (true) {
        __syncthreads();
        if (threadIdx.x == 0) *word = __hip_atomic_fetch_add(pool, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __syncthreads();
        const int c = *word;
        if (c >= p.nb * CPB) break;
        const int b = c / CPB, r0 = b * BM + (c % CPB) * DQ_POOL_ROWS;
        const int r1 = min(r0 + DQ_POOL_ROWS, p.M);
        if (r0 < r1)
            dq_pool_quantize_rows<RULE, NT>(p.a_bf16, p.K, r0, r1, const_cast<uint8_t*>(p.a_q),
                                            const_cast<uint8_t*>(p.a_s));
        wait_vmcnt<0>();
        __syncthreads();
        if (threadIdx.x == 0) __hip_atomic_fetch_add(done + b, 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        int v = 0;
        for (int spin = 0; spin < DQ_POOL_SPINS; ++spin) {
            v = __hip_atomic_load(done + tm, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            if (v >= CPB) break;
            __builtin_amdgcn_s_sleep(4);
        }
        if (v < CPB) __hip_atomic_store(p.state + 1 + p.nb, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        *word = v >= CPB ? 1 : 0;
    }
    __syncthreads();
    const bool ok = *word != 0;
    __syncthreads();   // the tile reuses this LDS word
    return ok;
}

// FUSED_A (MXFP8 only): A arrives as bf16 [M, K]; each 8-element chunk is
// quantized in registers (block-32 scale by A_RULE over a lane quad, E4M3
// codes) and dequantized back exactly, as mx_quantize_act would have done.
// A_RAW (W4A16): A arrives as bf16 [M, K] and is staged as it is; W is
// MXFP4 or NVFP4 and is dequantized to bf16.
// KA: the format of quantized A when it differs from W's (mixed MX pairs:
// MXFP8 A with MXFP4 W, or MXFP4 A with MXFP8 W; both scale per 32, so the
// scale layout and K tiling are shared and each operand is dequantized to
// bf16 by its own format); -1 means the same format as W.
// ODD16 (NVFP4 with K % 32 == 16): rows are only 8-byte aligned and the
// last chunk of a row holds a single block of 16 elements.  SCW (NVFP4 with
// K % 64 == 0, MXFP8 with K % 128 == 0): scale bytes are fetched as the
// aligned dword of the row that holds them (NVFP4: the stage's 4 scales,
// MXFP8: the 2 stages' 2 + 2) and extracted when the chunk is dequantized;
// the compiler waits for a byte load's zero extension right after the load,
// a dword needs none.
template <int KIND, int BM, int BN, int WM, int WN, bool OUT_F32, bool FUSED_A = false, int A_RULE = RULE_CEIL,
          bool ODD16 = false, bool SCW = false, bool A_RAW = false, bool POOL = false, int KA = -1>
__global__ __launch_bounds__(WM * WN * 64) void dq_gemm_kernel(DqArgs p)
{
    constexpr int KAQ = KA < 0 ? KIND : KA;   // format of quantized A
    static_assert(!POOL || (KIND == DQ_MXFP8 && KAQ == KIND && !FUSED_A && !A_RAW), "the pool quantizes MXFP8 A");
    using T = DqTraits<KIND>;                 // W
    using TA = DqTraits<KAQ>;                 // quantized A
    static_assert(KAQ == KIND || (KAQ != DQ_NVFP4 && KIND != DQ_NVFP4 && !FUSED_A && !A_RAW),
                  "mixed pairs are MX formats with quantized A");
    static_assert(!FUSED_A || KIND == DQ_MXFP8, "fused quantization is for MXFP8");
    static_assert(!A_RAW || KIND != DQ_MXFP8, "W4A16 weights are MXFP4 or NVFP4");
    static_assert(A_RAW || KIND != DQ_MXFP4 || KAQ != DQ_MXFP4, "MXFP4 x MXFP4 runs on the FP4 matrix cores");
    constexpr bool A_BF16 = FUSED_A || A_RAW;       // A arrives as bf16
    constexpr bool F16 = KIND == DQ_NVFP4 && !A_RAW;  // f16 matrix cores (NVFP4 W4A4), else bf16
    constexpr int NT = WM * WN * 64;
    constexpr int A_TILE = BM * DQ_ROW_BYTES, W_TILE = BN * DQ_ROW_BYTES;
    constexpr int STAGE = A_TILE + W_TILE;
    constexpr int WTM = BM / WM, WTN = BN / WN, FM = WTM / 32, FN = WTN / 32;
    constexpr int A_CPR = A_BF16 ? DQ_BK * 2 / 16 : TA::CHUNKS;  // A chunks per row per stage
    constexpr int A_CH = BM * A_CPR, W_CH = BN * T::CHUNKS;
    using KindW = std::integral_constant<int, KIND>;
    using KindA = std::integral_constant<int, KAQ>;
    static_assert(!A_BF16 || (A_CH % NT == 0 && NT % A_CPR == 0), "bf16 A tile mapping");
    constexpr int A_PER_T = (A_CH + NT - 1) / NT, W_PER_T = (W_CH + NT - 1) / NT;

    extern __shared__ __align__(16) uint8_t smem[];

    const int tiles_n = (p.N + BN - 1) / BN;
    const int tiles = ((p.M + BM - 1) / BM) * tiles_n;
    const int split = blockIdx.x / tiles, bid = blockIdx.x - split * tiles;
    const int tm = bid / tiles_n, tn = bid % tiles_n;
    const int m0 = tm * BM, n0 = tn * BN;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave / WN, wn = wave % WN;
    const int K = p.K, KS = K / T::SCALE_BLOCK;
    auto row_bytes_of = [K](int kind) { return kind == DQ_MXFP8 ? K : K / 2; };   // code bytes per row
    const int kt0 = split * p.chunk;                                // even: set parity = stage parity
    const int nk = min(p.chunk, (K + DQ_BK - 1) / DQ_BK - kt0);     // stages of this split
    if constexpr (POOL) {
        if (!dq_pool_ensure<A_RULE, BM, NT>(p, tm, smem)) {
            fill_tile_nan(p.y, p.M, p.N, m0, n0, BM, BN, OUT_F32);
            return;
        }
    }

    // two register sets of staged chunks: stage kt lives in set kt % 2.
    // Loads are branch-free and nothing loaded is used before the chunk is
    // dequantized, so a stage's loads stay in flight through the compute of
    // the stage before: an out-of-range chunk or scale byte is loaded from
    // the operand's first byte instead and dropped by its flag.
    uint4 ra[2][A_PER_T], rw[2][W_PER_T];
    uint32_t sa[2][A_PER_T][2], sw[2][W_PER_T][2];   // scale bytes of the chunk (MXFP8: one)
    uint32_t fa[2][A_PER_T], fw[2][W_PER_T];         // flags: 1 chunk, 2 its second 8 bytes, 4 second scale

    auto load_one = [&](auto kind, const uint8_t* q, const uint8_t* s, int rows_lim, int r0, int qi, int kt,
                        uint4& v, uint32_t* sc, uint32_t& fl) __attribute__((always_inline)) {
        constexpr int KK = decltype(kind)::value;
        using TK = DqTraits<KK>;
        const int row_bytes = row_bytes_of(KK);
        const int row = qi / TK::CHUNKS, c = qi % TK::CHUNKS;
        const int gr = r0 + row;
        const int kb = kt * TK::SRC_ROW_BYTES + c * 16;
        const bool ok = gr < rows_lim && kb < row_bytes;
        const size_t rb = ok ? (size_t)gr * row_bytes + kb : 0;
        if (!ODD16) {
            v = *reinterpret_cast<const uint4*>(q + rb);
            fl = ok ? 3u : 0u;
        } else {
            const bool ok_hi = ok && kb + 8 < row_bytes;
            const uint2 lo = *reinterpret_cast<const uint2*>(q + rb);
            const uint2 hi = *reinterpret_cast<const uint2*>(q + (ok_hi ? rb + 8 : 0));
            v = make_uint4(lo.x, lo.y, hi.x, hi.y);
            fl = (ok ? 1u : 0u) | (ok_hi ? 2u : 0u);
        }
        if (SCW) {
            const size_t so = KK == DQ_NVFP4 ? (size_t)gr * KS + kt * 4 : (size_t)gr * KS + (kt >> 1) * 4;
            sc[0] = *reinterpret_cast<const uint32_t*>(s + (ok ? so : 0));
            fl |= ok ? 4u : 0u;
        } else if (KK == DQ_NVFP4) {
            const int blk = kt * (DQ_BK / 16) + c * 2;
            const bool ok1 = ok && blk + 1 < KS;
            sc[0] = s[ok ? (size_t)gr * KS + blk : 0];
            sc[1] = s[ok1 ? (size_t)gr * KS + blk + 1 : 0];
            fl |= ok1 ? 4u : 0u;
        } else {
            sc[0] = s[ok ? (size_t)gr * KS + (kt * DQ_BK + c * TK::ELEMS_PER_CHUNK) / 32 : 0];
        }
    };
    auto load_stage = [&](int kt, int set) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < A_PER_T; ++i) {
            const int qi = tid + i * NT;
            if (A_BF16) {
                const int row = qi / A_CPR, c = qi % A_CPR, gm = m0 + row;
                const int kb = kt * DQ_BK * 2 + c * 16;
                const bool ok = gm < p.M && kb < K * 2;
                ra[set][i] = *reinterpret_cast<const uint4*>(p.a_q + (ok ? (size_t)gm * K * 2 + kb : 0));
                fa[set][i] = ok ? 3u : 0u;
            } else if (A_CH % NT == 0 || qi < A_CH) {
                load_one(KindA{}, p.a_q, p.a_s, p.M, m0, qi, kt, ra[set][i], sa[set][i], fa[set][i]);
            }
        }
#pragma unroll
        for (int i = 0; i < W_PER_T; ++i) {
            const int qi = tid + i * NT;
            if (W_CH % NT == 0 || qi < W_CH)
                load_one(KindW{}, p.w_q, p.w_s, p.N, n0, qi, kt, rw[set][i], sw[set][i], fw[set][i]);
        }
    };
    auto store_one = [&](auto kind, uint8_t* tile, int qi, uint4 v, const uint32_t* scb, uint32_t fl, int par)
                         __attribute__((always_inline)) {
        constexpr int KK = decltype(kind)::value;
        using TK = DqTraits<KK>;
        const int row = qi / TK::CHUNKS, c = qi % TK::CHUNKS;
        if (!(fl & 1u)) v = make_uint4(0, 0, 0, 0);
        if (!(fl & 2u)) v.z = v.w = 0;
        if (KK == DQ_NVFP4) {
            const uint32_t sc = SCW ? (fl & 1u ? __builtin_amdgcn_ubfe(scb[0], 16 * c, 16) : 0u)
                                    : (fl & 1u ? scb[0] : 0u) | (fl & 4u ? scb[1] << 8 : 0u);
            const uint32_t w[4] = {v.x, v.y, v.z, v.w};
            if (F16) {
                const half2_t sp = e4m3x2_to_f16x2(sc);
#pragma unroll
                for (int h = 0; h < 4; ++h) {   // 8 elements per dword -> one 16-B chunk of f16
                    const uint4 d = dequant8_nvfp4(w[h], bcast_h2(sp, h >> 1));
                    const int chunk = (c * 4 + h) ^ dq_swz(row);
                    *reinterpret_cast<uint4*>(tile + row * DQ_ROW_BYTES + chunk * 16) = d;
                }
            } else {
                const float2_t sp = e4m3x2_to_f32x2(sc);
                const float s0 = sp[0], s1 = sp[1];
#pragma unroll
                for (int h = 0; h < 4; ++h) {   // 8 elements per dword -> one 16-B chunk of bf16
                    const uint4 d = dequant8_nvfp4_bf16(w[h], h < 2 ? s0 : s1);
                    const int chunk = (c * 4 + h) ^ dq_swz(row);
                    *reinterpret_cast<uint4*>(tile + row * DQ_ROW_BYTES + chunk * 16) = d;
                }
            }
        } else if (KK == DQ_MXFP4) {
            const uint32_t sb = SCW ? __builtin_amdgcn_ubfe(scb[0], 16 * par + 8 * c, 8) : scb[0];
            const int e = (fl & 1u ? (int)sb : 127) - 127;
            const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int h = 0; h < 4; ++h) {
                const uint4 d = dequant8_mxfp4_bf16(w[h], e);
                const int chunk = (c * 4 + h) ^ dq_swz(row);
                *reinterpret_cast<uint4*>(tile + row * DQ_ROW_BYTES + chunk * 16) = d;
            }
        } else {
            const uint32_t sb = SCW ? __builtin_amdgcn_ubfe(scb[0], 16 * par + 8 * (c >> 1), 8) : scb[0];
            const int e = (fl & 1u ? (int)sb : 127) - 127;
            const uint4 d0 = dequant8_mxfp8(make_uint2(v.x, v.y), e);
            const uint4 d1 = dequant8_mxfp8(make_uint2(v.z, v.w), e);
            *reinterpret_cast<uint4*>(tile + row * DQ_ROW_BYTES + (((2 * c) ^ dq_swz(row)) * 16)) = d0;
            *reinterpret_cast<uint4*>(tile + row * DQ_ROW_BYTES + (((2 * c + 1) ^ dq_swz(row)) * 16)) = d1;
        }
    };
    auto store_stage = [&](int buf, int set, int kg) __attribute__((always_inline)) {
        uint8_t* a_t = smem + buf * STAGE;
        uint8_t* w_t = a_t + A_TILE;
#pragma unroll
        for (int i = 0; i < A_PER_T; ++i) {
            const int qi = tid + i * NT;
            if (A_BF16) {
                // 8 bf16 per lane; (fused) a lane quad holds one block of 32
                const int row = qi / A_CPR, c = qi % A_CPR;
                const uint4 x = fa[set][i] ? ra[set][i] : make_uint4(0, 0, 0, 0);
                uint4 d = x;
                if (FUSED_A) {
                    const uint32_t amax = quad_max_u32(amax_bits8(x));
                    const int e = scale_exponent<ELEM_E4M3, A_RULE>(amax);
                    const uint2 codes = encode8_e4m3(x, e);
                    d = dequant8_mxfp8(codes, e);
                    // debug dump of the prologue's codes (first tile column only)
                    const int grow = m0 + row, kel = kg * DQ_BK + c * 8;
                    if (p.dump_q != nullptr && tn == 0 && grow < p.M && kel < K) {
                        *reinterpret_cast<uint2*>(p.dump_q + (size_t)grow * K + kel) = codes;
                        if ((c & 3) == 0) p.dump_s[(size_t)grow * (K / 32) + kel / 32] = (uint8_t)(e + 127);
                    }
                }
                *reinterpret_cast<uint4*>(a_t + row * DQ_ROW_BYTES + ((c ^ dq_swz(row)) * 16)) = d;
            } else if (A_CH % NT == 0 || qi < A_CH) {
                store_one(KindA{}, a_t, qi, ra[set][i], sa[set][i], fa[set][i], set);
            }
        }
#pragma unroll
        for (int i = 0; i < W_PER_T; ++i) {
            const int qi = tid + i * NT;
            if (W_CH % NT == 0 || qi < W_CH) store_one(KindW{}, w_t, qi, rw[set][i], sw[set][i], fw[set][i], set);
        }
    };

    float16_t acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    const int r32 = lane & 31, g = lane >> 5;
    auto compute_stage = [&](int buf) {
        const uint8_t* a_t = smem + buf * STAGE;
        const uint8_t* w_t = a_t + A_TILE;
#pragma unroll
        for (int kk = 0; kk < DQ_BK / 16; ++kk) {
            uint4 fa[FM], fw[FN];
#pragma unroll
            for (int i = 0; i < FM; ++i) {
                const int row = wm * WTM + i * 32 + r32;
                fa[i] = *reinterpret_cast<const uint4*>(a_t + row * DQ_ROW_BYTES + (((2 * kk + g) ^ dq_swz(row)) * 16));
            }
#pragma unroll
            for (int j = 0; j < FN; ++j) {
                const int row = wn * WTN + j * 32 + r32;
                fw[j] = *reinterpret_cast<const uint4*>(w_t + row * DQ_ROW_BYTES + (((2 * kk + g) ^ dq_swz(row)) * 16));
            }
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j) {
                    if (F16) {
                        half8_t a8, b8;
                        __builtin_memcpy(&a8, &fa[i], 16);
                        __builtin_memcpy(&b8, &fw[j], 16);
                        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a8, b8, acc[i][j], 0, 0, 0);
                    } else {
                        bf16x8_t a8, b8;
                        __builtin_memcpy(&a8, &fa[i], 16);
                        __builtin_memcpy(&b8, &fw[j], 16);
                        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a8, b8, acc[i][j], 0, 0, 0);
                    }
                }
        }
    };

    // Stage kt is loaded into register set kt % 2 two stages ahead of its
    // compute: loads of stage kt + 2 go out before the compute of stage kt,
    // and stage kt + 1 (loaded one iteration earlier) is dequantized into
    // LDS after it.  The loop is unrolled by two so that the sets are static,
    // and both steps run unconditionally (stages past K load nothing and
    // dequantize to zeros in the buffer no later stage reads), so the
    // compiler's waits count exactly the loads of stage kt + 2 as newer.
    load_stage(kt0, 0);
    load_stage(kt0 + 1, 1);
    store_stage(0, 0, kt0);
    __syncthreads();
    auto iter = [&](int kt, int set) __attribute__((always_inline)) {
        load_stage(kt0 + kt + 2, set);
        compute_stage(set);
        store_stage(set ^ 1, set ^ 1, kt0 + kt + 1);
        __syncthreads();
    };
    int kt = 0;
    for (; kt + 1 < nk; kt += 2) {
        iter(kt, 0);
        iter(kt + 1, 1);
    }
    if (kt < nk) iter(kt, 0);

    if (p.splits > 1) {   // fp32 partial of this split
        float* part = p.part + (size_t)split * p.M * p.N;
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j) {
                const int n = n0 + wn * WTN + j * 32 + r32;
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int m = m0 + wm * WTM + i * 32 + (r / 4) * 8 + g * 4 + (r % 4);
                    if (m < p.M && n < p.N) part[(size_t)m * p.N + n] = acc[i][j][r];
                }
            }
        return;
    }

#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) {
            const int n = n0 + wn * WTN + j * 32 + r32;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int m = m0 + wm * WTM + i * 32 + (r / 4) * 8 + g * 4 + (r % 4);
                if (m < p.M && n < p.N) {
                    const float v = (KIND == DQ_NVFP4 || A_RAW) ? acc[i][j][r] * p.alpha : acc[i][j][r];
                    if (OUT_F32) {
                        reinterpret_cast<float*>(p.y)[(size_t)m * p.N + n] = v;
                    } else {
                        reinterpret_cast<uint16_t*>(p.y)[(size_t)m * p.N + n] = f32_to_bf16_rne(v);
                    }
                }
            }
        }
}

template <int KIND, int BM, int BN, int WM, int WN, bool OUT_F32, bool FUSED_A = false, int A_RULE = RULE_CEIL,
          bool ODD16 = false, bool SCW = false, bool A_RAW = false, bool POOL = false, int KA = -1>
hipError_t launch_dq_k(const DqArgs& a, hipStream_t stream)
{
    constexpr int LDS = 2 * (BM + BN) * DQ_ROW_BYTES;
    auto kern = dq_gemm_kernel<KIND, BM, BN, WM, WN, OUT_F32, FUSED_A, A_RULE, ODD16, SCW, A_RAW, POOL, KA>;
    static bool attr_set = false;
    if (!attr_set) {
        hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, LDS);
        if (e != hipSuccess) return e;
        attr_set = true;
    }
    const int tiles = ((a.M + BM - 1) / BM) * ((a.N + BN - 1) / BN);
    hipLaunchKernelGGL(kern, dim3(tiles * a.splits), dim3(WM * WN * 64), LDS, stream, a);
    return hipGetLastError();
}

template <int KIND, int BM, int BN, int WM, int WN, bool OUT_F32, bool FUSED_A = false, int A_RULE = RULE_CEIL,
          bool A_RAW = false, int KA = -1>
hipError_t launch_dq(const DqArgs& a, hipStream_t stream)
{
    if constexpr (KIND == DQ_NVFP4) {
        if (a.K % 32 != 0)
            return launch_dq_k<KIND, BM, BN, WM, WN, OUT_F32, FUSED_A, A_RULE, true, false, A_RAW>(a, stream);
        if (a.K % 64 == 0)
            return launch_dq_k<KIND, BM, BN, WM, WN, OUT_F32, FUSED_A, A_RULE, false, true, A_RAW>(a, stream);
    } else if (!FUSED_A) {
        if (a.K % 128 == 0)
            return launch_dq_k<KIND, BM, BN, WM, WN, OUT_F32, FUSED_A, A_RULE, false, true, A_RAW, false, KA>(a, stream);
    }
    return launch_dq_k<KIND, BM, BN, WM, WN, OUT_F32, FUSED_A, A_RULE, false, false, A_RAW, false, KA>(a, stream);
}

} // namespace mxl

using namespace mxl;

extern "C" int mxl_choose_splits(int64_t tiles, int nk, int min_stages, int even, int two_max, int* chunk);
extern "C" hipError_t mxl_launch_splitk_reduce(const float* part, int splits, int64_t mn, float alpha, void* y,
                                               int out_f32, hipStream_t stream);

// ---------------------------------------------------------------- decode
// Decode-shaped exact MXFP8 and NVFP4 GEMMs (16 rows of A per launch, at
// most two launches; K % 1024 == 0, K <= 8192): a stream over W, built like
// the MXFP4 decode kernel (mx_decode_stream_kernel): one workgroup of 4 waves
// owns 16 W rows, wave w a contiguous quarter of K.  W is consumed in chunks
// of 128 code bytes per row (one stage of 128 K for MXFP8, two for NVFP4):
//  * Each wave copies its own chunks, rows 8 h .. 8 h + 7 x 128 bytes per
//    copy (8 full cache lines; non-temporal (NT) in the last launch, which
//    reads W for the last time, and with the default policy in a first of
//    two, whose W the second partly finds in the last-level cache), through a ring
//    of 3 chunk slots in its own LDS region, and computes each chunk once
//    its two copies have landed (exact vmcnt); the slot is refilled when its
//    LDS reads have returned.  Inside a copy, row q's 16-byte chunk L sits at
//    L ^ ((q >> 1) & 7), so the 16 rows of a lane group cover all banks.
//  * The wave's A codes (and, NVFP4, its A scales) go to registers first
//    (rows past M read as zero), then the scale block of the 16 W rows (and,
//    MXFP8, of A's 16 rows) to LDS (256-byte copies spread over the waves,
//    one barrier), all before the W copies.
//  * Dequantization as in the tile kernels, in registers: MXFP8 codes to
//    bf16 by v_cvt_scalef32_pk_bf16_fp8 with the E8M0 scale in the exponent
//    field; NVFP4 codes to f16 (scale 1) times the E4M3 block scale as an
//    f16 pair (exact).  Then v_mfma_f32_16x16x32_{bf16,f16}: lane (r, g)
//    supplies row r and, in step j of a stage, elements [32 g + 8 j, +8) of
//    it, for A and W alike, so each step sums 32 distinct K.
//  * The four K quarters are summed through LDS; Y = alpha * sum.
template <bool NT>
__device__ __forceinline__ void dq_dma_b128(uint32_t lds, int voff, const int4_t& rsrc, int soff)
{
    if (NT)
        asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, %3 offen nt lds"
                     :: "s"(lds), "v"(voff), "s"(rsrc), "s"(soff) : "memory");
    else
        asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
                     :: "s"(lds), "v"(voff), "s"(rsrc), "s"(soff) : "memory");
}
__device__ __forceinline__ int4_t dq_lds_v4(uint32_t addr)
{
    return *reinterpret_cast<const __attribute__((address_space(3))) int4_t*>((size_t)addr);
}
__device__ __forceinline__ uint32_t dq_lds_u32(uint32_t addr)
{
    return *reinterpret_cast<const __attribute__((address_space(3))) uint32_t*>((size_t)addr);
}
// s_waitcnt vmcnt(n) for an even n <= 6 that folds to a constant once loops
// are unrolled
__device__ __forceinline__ void dq_wait_vmcnt_n(int n)
{
    switch (n) {
    case 0: wait_vmcnt<0>(); break;
    case 2: wait_vmcnt<2>(); break;
    case 4: wait_vmcnt<4>(); break;
    case 6: wait_vmcnt<6>(); break;
    default: wait_vmcnt<0>(); break;
    }
}

constexpr int DQD_RS = 3;   // ring slots (chunks) per wave

template <int KIND, int QC, bool OUT_F32, bool NT>
__global__ __launch_bounds__(256) void dq_decode_stream_kernel(DqArgs p)
{
    static_assert(KIND == DQ_MXFP8 || KIND == DQ_NVFP4, "decode formats");
    constexpr bool NV = KIND == DQ_NVFP4;
    constexpr int WAVES = 4, RSB = DQD_RS < QC ? DQD_RS : QC;
    constexpr int K = NV ? QC * 1024 : QC * 512;          // QC chunks of 128 code bytes per wave
    constexpr int ROWB = NV ? K / 2 : K;                  // code bytes per row
    constexpr int KS = NV ? K / 16 : K / 32;              // scale bytes per row
    constexpr int QB = ROWB / WAVES;                      // code bytes per row per wave (128 QC)
    constexpr int SPC = NV ? 2 : 1;                       // stages (128 K) per chunk
    constexpr int NST = QC * SPC;                         // stages per wave
    constexpr bool AS_REG = NV;                           // A scales in registers (else in LDS)
    constexpr int SCOP = (AS_REG ? 1 : 2) * 16 * KS / 256; // scale block copies: W, then (MXFP8) A
    extern __shared__ __align__(16) uint8_t dsm[];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int r = lane & 15, g = lane >> 4;
    const int n0 = blockIdx.x * 16;
    const int st0 = wave * QC * SPC;                      // this wave's first stage
    const uint32_t lds0 = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)dsm);
    const uint32_t lds_w = lds0 + (uint32_t)(wave * RSB * 2048);
    const uint32_t sw_lds = lds0 + (uint32_t)(WAVES * RSB * 2048), sa_lds = sw_lds + (uint32_t)(16 * KS);

    // this wave's A codes, 32 bytes per lane and chunk: row r, K [32 g, +32)
    // of each stage (MXFP8: 32 codes of the chunk's stage; NVFP4: 16 bytes of
    // each of its two stages)
    const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc((void*)p.a_q, (short)0, p.M * ROWB, 0x00020000);
    int4_t af[QC][2];
#pragma unroll
    for (int c = 0; c < QC; ++c)
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int off = NV ? (st0 + SPC * c + i) * 64 + g * 16 : (st0 + c) * 128 + g * 32 + i * 16;
            af[c][i] = __builtin_amdgcn_raw_buffer_load_b128(ra, r * ROWB + off, 0, 0);
        }
    // NVFP4: this wave's A scales, one dword per stage: row r, the dword
    // that holds lane group g's bytes (blocks 8 st + 2 g, + 1, at byte
    // 2 (g & 1)); rows past M read as zero
    uint32_t asr[AS_REG ? NST : 1];
    if (AS_REG) {
        const __amdgpu_buffer_rsrc_t ras = __builtin_amdgcn_make_buffer_rsrc((void*)p.a_s, (short)0, p.M * KS, 0x00020000);
#pragma unroll
        for (int i = 0; i < NST; ++i)
            asr[i] = __builtin_amdgcn_raw_buffer_load_b32(ras, r * KS + 8 * (st0 + i) + 4 * (g >> 1), 0, 0);
    }
    // the scale block [16 rows][KS] of W (MXFP8: then A's), spread over the waves
    {
        const int4_t rws = make_rsrc(p.w_s, (uint32_t)p.N * KS);
        const int4_t ras = make_rsrc(p.a_s, (uint32_t)p.M * KS);
#pragma unroll
        for (int j = 0; j < SCOP; ++j)
            if (j % WAVES == wave) {
                if (j < 16 * KS / 256) dma_b32(sw_lds + j * 256, n0 * KS + j * 256 + lane * 4, rws, 0);
                else dma_b32(sw_lds + j * 256, (j - 16 * KS / 256) * 256 + lane * 4, ras, 0);
            }
    }
    // W chunks: chunk c (copies h = 0, 1: rows 8 h .. 8 h + 7) into slot c % RSB
    const int4_t rw = make_rsrc(p.w_q, (uint32_t)p.N * ROWB);
    int voffh[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int q = 8 * h + (lane >> 3);
        voffh[h] = (n0 + q) * ROWB + (((lane & 7) ^ ((q >> 1) & 7)) * 16);
    }
    auto copy_chunk = [&](int c) __attribute__((always_inline)) {
#pragma unroll
        for (int h = 0; h < 2; ++h)
            dq_dma_b128<NT>(lds_w + (uint32_t)((c % RSB) * 2048 + h * 1024), voffh[h], rw, wave * QB + c * 128);
    };
#pragma unroll
    for (int c = 0; c < RSB; ++c) copy_chunk(c);
    // the scale copies (and the A loads before them) have landed once at
    // most the W copies are outstanding; the barrier publishes the scales
    wait_vmcnt<2 * RSB>();
    lds_barrier();

    float4_t acc = {0.f, 0.f, 0.f, 0.f};
    const uint32_t rd = lds_w + (uint32_t)((r >> 3) * 1024 + (r & 7) * 128);
    const int rsw = (r >> 1) & 7;
    const uint32_t srw = sw_lds + (uint32_t)(r * KS), sra = sa_lds + (uint32_t)(r * KS);
#pragma unroll
    for (int c = 0; c < QC; ++c) {
        {
            const int last = c - 1 + RSB < QC - 1 ? c - 1 + RSB : QC - 1;
            dq_wait_vmcnt_n(2 * (last - c));
        }
        const uint32_t slot = rd + (uint32_t)((c % RSB) * 2048);
#pragma unroll
        for (int hf = 0; hf < SPC; ++hf) {
            const int st = st0 + SPC * c + hf;   // global stage (128 K)
            uint32_t wd[8], ad[8];
            if (NV) {
                // 32 codes of block pair (2 g, 2 g + 1) of 16: one 16-byte chunk
                const int4_t w4 = dq_lds_v4(slot + (uint32_t)(((4 * hf + g) ^ rsw) * 16));
                for (int i = 0; i < 4; ++i) { wd[i] = (uint32_t)w4[i]; ad[i] = (uint32_t)af[c][hf][i]; }
            } else {
                // 32 codes: logical chunks 2 g and 2 g + 1
                const int4_t w0 = dq_lds_v4(slot + (uint32_t)(((2 * g) ^ rsw) * 16));
                const int4_t w1 = dq_lds_v4(slot + (uint32_t)(((2 * g + 1) ^ rsw) * 16));
                for (int i = 0; i < 4; ++i) {
                    wd[i] = (uint32_t)w0[i]; wd[4 + i] = (uint32_t)w1[i];
                    ad[i] = (uint32_t)af[c][0][i]; ad[4 + i] = (uint32_t)af[c][1][i];
                }
            }
            if (NV) {
                // E4M3 scales of blocks 8 st + 2 g, + 1 (two bytes of the row's dword)
                const uint32_t wsp = dq_lds_u32(srw + (uint32_t)(8 * st + 4 * (g >> 1))) >> (16 * (g & 1));
                const half2_t wsc = e4m3x2_to_f16x2(wsp);
                const half2_t asc = e4m3x2_to_f16x2(asr[SPC * c + hf] >> (16 * (g & 1)));
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const uint4 bw = dequant8_nvfp4(wd[j], bcast_h2(wsc, j >> 1));
                    const uint4 ba = dequant8_nvfp4(ad[j], bcast_h2(asc, j >> 1));
                    acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8_t, ba),
                                                                 __builtin_bit_cast(half8_t, bw), acc, 0, 0, 0);
                }
            } else {
                // E8M0 scale of block 4 st + g
                const int sb = 4 * st + g;
                const int ew = (int)((dq_lds_u32(srw + (uint32_t)(sb & ~3)) >> (8 * (sb & 3))) & 0xFFu) - 127;
                const int ea = (int)((dq_lds_u32(sra + (uint32_t)(sb & ~3)) >> (8 * (sb & 3))) & 0xFFu) - 127;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const uint4 bw = dequant8_mxfp8(make_uint2(wd[2 * j], wd[2 * j + 1]), ew);
                    const uint4 ba = dequant8_mxfp8(make_uint2(ad[2 * j], ad[2 * j + 1]), ea);
                    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, ba),
                                                                  __builtin_bit_cast(bf16x8_t, bw), acc, 0, 0, 0);
                }
            }
        }
        if (c + RSB < QC) {
            __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0): the slot's LDS reads have returned
            copy_chunk(c + RSB);
        }
    }
    __syncthreads();   // every wave is done with its LDS region
    float4_t* red = reinterpret_cast<float4_t*>(dsm);   // [WAVES][64]
    red[wave * 64 + lane] = acc;
    __syncthreads();
    // lane l of the first wave finishes output rows 4 (l / 16) + i, column n0 + l % 16
    if (tid < 64) {
        float4_t v = red[tid];
#pragma unroll
        for (int w = 1; w < WAVES; ++w) {
            const float4_t x = red[w * 64 + tid];
            v = float4_t{v[0] + x[0], v[1] + x[1], v[2] + x[2], v[3] + x[3]};
        }
        const int nn = n0 + (tid & 15);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int m = 4 * (tid >> 4) + i;
            if (m < p.M && nn < p.N) {
                const float o = v[i] * p.alpha;
                if (OUT_F32) reinterpret_cast<float*>(p.y)[(size_t)m * p.N + nn] = o;
                else reinterpret_cast<uint16_t*>(p.y)[(size_t)m * p.N + nn] = f32_to_bf16_rne(o);
            }
        }
    }
}

static size_t dq_decode_lds_bytes(int kind, int64_t k)
{
    const int64_t ks = kind == DQ_NVFP4 ? k / 16 : k / 32;
    const int64_t qc = kind == DQ_NVFP4 ? k / 1024 : k / 512;
    const int64_t rs = qc < DQD_RS ? qc : DQD_RS;
    return (size_t)(4 * rs * 2048 + (kind == DQ_NVFP4 ? 1 : 2) * 16 * ks);
}

// whether dq_decode_stream_kernel serves this shape (kind: DQ_NVFP4 or DQ_MXFP8):
// one launch per 16 rows of A, at most two; W's bytes within the 32-bit
// buffer ranges and offsets the kernel uses
static bool dq_decode_ok(int kind, int64_t m, int64_t n, int64_t k)
{
    const int64_t rowb = kind == DQ_NVFP4 ? k / 2 : k;
    return m <= 32 && k % 1024 == 0 && k >= 1024 && k <= 8192 && dq_decode_lds_bytes(kind, k) <= 65536 &&
           (n + 16) * rowb < ((int64_t)1 << 31);
}

template <int KIND, int QC, bool OUT_F32>
static void launch_dq_decode_qc(const DqArgs& a, bool nt, hipStream_t stream)
{
    if (nt)
        hipLaunchKernelGGL((dq_decode_stream_kernel<KIND, QC, OUT_F32, true>), dim3((a.N + 15) / 16), dim3(256),
                           dq_decode_lds_bytes(KIND, a.K), stream, a);
    else
        hipLaunchKernelGGL((dq_decode_stream_kernel<KIND, QC, OUT_F32, false>), dim3((a.N + 15) / 16), dim3(256),
                           dq_decode_lds_bytes(KIND, a.K), stream, a);
}

template <int KIND, bool OUT_F32>
static hipError_t launch_dq_decode_rows(const DqArgs& a, bool nt, hipStream_t stream)
{
    const int qc = KIND == DQ_NVFP4 ? a.K / 1024 : a.K / 512;
    switch (qc) {
    case 1: if constexpr (KIND == DQ_NVFP4) launch_dq_decode_qc<KIND, 1, OUT_F32>(a, nt, stream); break;
    case 2: launch_dq_decode_qc<KIND, 2, OUT_F32>(a, nt, stream); break;
    case 3: if constexpr (KIND == DQ_NVFP4) launch_dq_decode_qc<KIND, 3, OUT_F32>(a, nt, stream); break;
    case 4: launch_dq_decode_qc<KIND, 4, OUT_F32>(a, nt, stream); break;
    case 5: if constexpr (KIND == DQ_NVFP4) launch_dq_decode_qc<KIND, 5, OUT_F32>(a, nt, stream); break;
    case 6: launch_dq_decode_qc<KIND, 6, OUT_F32>(a, nt, stream); break;
    case 7: if constexpr (KIND == DQ_NVFP4) launch_dq_decode_qc<KIND, 7, OUT_F32>(a, nt, stream); break;
    case 8: launch_dq_decode_qc<KIND, 8, OUT_F32>(a, nt, stream); break;
    case 10: if constexpr (KIND == DQ_MXFP8) launch_dq_decode_qc<KIND, 10, OUT_F32>(a, nt, stream); break;
    case 12: if constexpr (KIND == DQ_MXFP8) launch_dq_decode_qc<KIND, 12, OUT_F32>(a, nt, stream); break;
    case 14: if constexpr (KIND == DQ_MXFP8) launch_dq_decode_qc<KIND, 14, OUT_F32>(a, nt, stream); break;
    case 16: if constexpr (KIND == DQ_MXFP8) launch_dq_decode_qc<KIND, 16, OUT_F32>(a, nt, stream); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

// Rows 16 j .. 16 j + 15 of A and Y per launch (W streamed once per launch).
template <int KIND, bool OUT_F32>
static hipError_t launch_dq_decode(const DqArgs& a0, hipStream_t stream)
{
    const size_t rowb = KIND == DQ_NVFP4 ? (size_t)a0.K / 2 : (size_t)a0.K;
    const size_t ks = KIND == DQ_NVFP4 ? (size_t)a0.K / 16 : (size_t)a0.K / 32;
    for (int r0 = 0; r0 < a0.M; r0 += 16) {
        DqArgs a = a0;
        a.a_q = a0.a_q + r0 * rowb;
        a.a_s = a0.a_s + r0 * ks;
        a.y = static_cast<uint8_t*>(a0.y) + (size_t)r0 * a0.N * (OUT_F32 ? 4 : 2);
        a.M = a0.M - r0 < 16 ? a0.M - r0 : 16;
        const hipError_t e = launch_dq_decode_rows<KIND, OUT_F32>(a, r0 + 16 >= a0.M, stream);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

// The decode kernel goes before the tile kernels (a wide N with few rows of A
// is a stream over W), except for MXFP8 above 16 rows: its two launches read
// W twice, which at N = 151936, K = 5120 (778 MB, beyond the last-level
// cache) took 337 us against 258 us for the tile kernel at M = 32, while at
// M = 1 and 8 the decode kernel took 118 and 143 us against 276 and 271.
// NVFP4 (389 MB) gains at every M up to 32: 76 / 90 / 230 us against 279.
static bool dq8_decode_first(int64_t m, int64_t n, int64_t k)
{
    return m <= 16 && dq_decode_ok(DQ_MXFP8, m, n, k);
}

extern "C" int mxl_dq_decode_ok(int nv, int64_t m, int64_t n, int64_t k)
{
    return dq_decode_ok(nv ? DQ_NVFP4 : DQ_MXFP8, m, n, k) ? 1 : 0;
}

// Split-K plan of the 128 x 128 dequantizing kernel: at least 8 stages of 64
// per split and an even stage count; two splits up to 192 tiles (M = 32 to
// 128 at N = 17408, K = 5120: 63.8 -> 50 and 57.9 µs for MXFP8; at 240
// tiles the split no longer pays).
static int dq_splits(int64_t m, int64_t n, int64_t k, int* chunk)
{
    const int64_t tiles = ((m + 127) / 128) * ((n + 127) / 128);
    return mxl_choose_splits(tiles, (int)((k + DQ_BK - 1) / DQ_BK), 8, 1, 192, chunk);
}

extern "C" size_t mxl_dq_workspace(int64_t m, int64_t n, int64_t k)
{
    int chunk;
    const int s = dq_splits(m, n, k, &chunk);
    return s > 1 ? (size_t)s * m * n * sizeof(float) : 0;
}

extern "C" int mxl_dq_splits(int64_t m, int64_t n, int64_t k)
{
    int chunk;
    return dq_splits(m, n, k, &chunk);
}

// Runs `launch(args, out_f32)` either as one pass or, when a large enough
// workspace is given and the tiles alone leave the machine idle, as split-K
// partials plus the ordered reduction (which applies alpha).
template <class F>
static hipError_t dq_run(DqArgs a, int out_f32, void* work, size_t work_bytes, hipStream_t stream, F launch)
{
    a.part = nullptr;
    a.splits = 1;
    a.chunk = 1 << 30;
    int chunk;
    const int splits = dq_splits(a.M, a.N, a.K, &chunk);
    if (work && splits > 1 && work_bytes >= (size_t)splits * a.M * a.N * sizeof(float)) {
        a.part = static_cast<float*>(work);
        a.splits = splits;
        a.chunk = chunk;
        const hipError_t e = launch(a, 1);
        if (e != hipSuccess) return e;
        return mxl_launch_splitk_reduce(a.part, splits, (int64_t)a.M * a.N, a.alpha, a.y, out_f32, stream);
    }
    return launch(a, out_f32);
}

extern "C" int mxl_dq8w_ok(int fmt, int64_t m, int64_t n, int64_t k);
extern "C" hipError_t mxl_launch_dq8w(int fmt, const void* aq, const void* as, const void* wq, const void* ws,
                                      int64_t m, int64_t n, int64_t k, float alpha, void* y, int out_f32,
                                      hipStream_t stream);
extern "C" const char* mxl_dq8w_config_name(void);
constexpr int DQ8W_FMT_NVFP4 = 2;

// The 8-wave NVFP4 tile kernel above 128 rows of A: below that the 128 x 128
// kernel is faster even where N alone fills the tile count (N = 151936, K =
// 5120: M = 64 / 128 take 276 / 300 us there against 326 / 330 us in the
// tile kernel; M = 256: 574 against 361).
static bool nv_tile_ok(int64_t m, int64_t n, int64_t k)
{
    return m > 128 && mxl_dq8w_ok(DQ8W_FMT_NVFP4, m, n, k);
}

extern "C" hipError_t mxl_launch_nv_gemm(const void* aq, const void* as, const void* wq, const void* ws,
                                         int64_t m, int64_t n, int64_t k, float alpha, void* y,
                                         int out_f32, void* work, size_t work_bytes, hipStream_t stream)
{
    DqArgs a{static_cast<const uint8_t*>(aq), static_cast<const uint8_t*>(as),
             static_cast<const uint8_t*>(wq), static_cast<const uint8_t*>(ws), y,
             (int)m, (int)n, (int)k, alpha};
    if (dq_decode_ok(DQ_NVFP4, m, n, k))   // before the tile kernel: a wide N with few rows is a W stream
        return out_f32 ? launch_dq_decode<DQ_NVFP4, true>(a, stream) : launch_dq_decode<DQ_NVFP4, false>(a, stream);
    if (nv_tile_ok(m, n, k))
        return mxl_launch_dq8w(DQ8W_FMT_NVFP4, aq, as, wq, ws, m, n, k, alpha, y, out_f32, stream);
    return dq_run(a, out_f32, work, work_bytes, stream, [&](const DqArgs& x, int f32) {
        if (f32) return launch_dq<DQ_NVFP4, 128, 128, 2, 2, true>(x, stream);
        return launch_dq<DQ_NVFP4, 128, 128, 2, 2, false>(x, stream);
    });
}

extern "C" int mxl_mx8_tile_ok(int64_t m, int64_t n, int64_t k);
extern "C" hipError_t mxl_launch_mx8_tile(const void* aq, const void* as, const void* wq, const void* ws, int64_t m,
                                          int64_t n, int64_t k, void* y, int out_f32, hipStream_t stream);
extern "C" const char* mxl_mx8_tile_config_name(void);

extern "C" hipError_t mxl_launch_mxfp8_exact_gemm(const void* aq, const void* as, const void* wq,
                                                  const void* ws, int64_t m, int64_t n, int64_t k, void* y,
                                                  int out_f32, void* work, size_t work_bytes, hipStream_t stream)
{
    DqArgs a{static_cast<const uint8_t*>(aq), static_cast<const uint8_t*>(as),
             static_cast<const uint8_t*>(wq), static_cast<const uint8_t*>(ws), y,
             (int)m, (int)n, (int)k, 1.0f};
    if (dq8_decode_first(m, n, k))
        return out_f32 ? launch_dq_decode<DQ_MXFP8, true>(a, stream) : launch_dq_decode<DQ_MXFP8, false>(a, stream);
    if (mxl_mx8_tile_ok(m, n, k)) return mxl_launch_mx8_tile(aq, as, wq, ws, m, n, k, y, out_f32, stream);
    if (dq_decode_ok(DQ_MXFP8, m, n, k))
        return out_f32 ? launch_dq_decode<DQ_MXFP8, true>(a, stream) : launch_dq_decode<DQ_MXFP8, false>(a, stream);
    return dq_run(a, out_f32, work, work_bytes, stream, [&](const DqArgs& x, int f32) {
        if (f32) return launch_dq<DQ_MXFP8, 128, 128, 2, 2, true>(x, stream);
        return launch_dq<DQ_MXFP8, 128, 128, 2, 2, false>(x, stream);
    });
}

// Mixed MX pairs, exact: A codes of a_bits (8: E4M3, 4: E2M1), W codes of
// the other width, each dequantized to bf16 by its own format.
extern "C" hipError_t mxl_launch_mx_mixed_exact_gemm(int a_bits, const void* aq, const void* as, const void* wq,
                                                     const void* ws, int64_t m, int64_t n, int64_t k, void* y,
                                                     int out_f32, void* work, size_t work_bytes, hipStream_t stream)
{
    DqArgs a{static_cast<const uint8_t*>(aq), static_cast<const uint8_t*>(as),
             static_cast<const uint8_t*>(wq), static_cast<const uint8_t*>(ws), y,
             (int)m, (int)n, (int)k, 1.0f};
    return dq_run(a, out_f32, work, work_bytes, stream, [&](const DqArgs& x, int f32) {
        if (a_bits == 8) {   // A MXFP8, W MXFP4
            if (f32) return launch_dq<DQ_MXFP4, 128, 128, 2, 2, true, false, RULE_CEIL, false, DQ_MXFP8>(x, stream);
            return launch_dq<DQ_MXFP4, 128, 128, 2, 2, false, false, RULE_CEIL, false, DQ_MXFP8>(x, stream);
        }
        if (f32) return launch_dq<DQ_MXFP8, 128, 128, 2, 2, true, false, RULE_CEIL, false, DQ_MXFP4>(x, stream);
        return launch_dq<DQ_MXFP8, 128, 128, 2, 2, false, false, RULE_CEIL, false, DQ_MXFP4>(x, stream);
    });
}

extern "C" const char* mxl_mx_mixed_exact_config_name(void)
{
    return "dq_gemm_kernel<mxfp8 x mxfp4 -> exact bf16 per operand, tile 128x128x64, 2x2 waves of 64x64, "
           "bf16 mfma 32x32x16>";
}

template <int RULE>
static hipError_t fused8(const DqArgs& a, int out_f32, hipStream_t stream)
{
    if (out_f32) return launch_dq<DQ_MXFP8, 128, 128, 2, 2, true, true, RULE>(a, stream);
    return launch_dq<DQ_MXFP8, 128, 128, 2, 2, false, true, RULE>(a, stream);
}

extern "C" hipError_t mxl_launch_mxfp8_exact_gemm_fused(int a_rule, const void* a_bf16, const void* wq,
                                                        const void* ws, int64_t m, int64_t n, int64_t k,
                                                        void* y, int out_f32, void* dump_q, void* dump_s,
                                                        hipStream_t stream)
{
    DqArgs a{static_cast<const uint8_t*>(a_bf16), nullptr, static_cast<const uint8_t*>(wq),
             static_cast<const uint8_t*>(ws), y, (int)m, (int)n, (int)k, 1.0f, nullptr, 1, 1 << 30,
             static_cast<uint8_t*>(dump_q), static_cast<uint8_t*>(dump_s)};
    if (a_rule == RULE_CEIL) return fused8<RULE_CEIL>(a, out_f32, stream);
    if (a_rule == RULE_FLOOR) return fused8<RULE_FLOOR>(a, out_f32, stream);
    return fused8<RULE_EVEN>(a, out_f32, stream);
}

// W4A16, any M: bf16 A staged as it is, MXFP4 (w_nv == 0) or NVFP4 (w_nv != 0)
// weights dequantized exactly to bf16; alpha multiplies the result.
extern "C" hipError_t mxl_launch_w4a16_gemm(int w_nv, const void* a_bf16, const void* wq, const void* ws,
                                            int64_t m, int64_t n, int64_t k, float alpha, void* y,
                                            int out_f32, void* work, size_t work_bytes, hipStream_t stream)
{
    DqArgs a{static_cast<const uint8_t*>(a_bf16), nullptr, static_cast<const uint8_t*>(wq),
             static_cast<const uint8_t*>(ws), y, (int)m, (int)n, (int)k, alpha};
    return dq_run(a, out_f32, work, work_bytes, stream, [&](const DqArgs& x, int f32) {
        if (w_nv) {
            if (f32) return launch_dq<DQ_NVFP4, 128, 128, 2, 2, true, false, RULE_CEIL, true>(x, stream);
            return launch_dq<DQ_NVFP4, 128, 128, 2, 2, false, false, RULE_CEIL, true>(x, stream);
        }
        if (f32) return launch_dq<DQ_MXFP4, 128, 128, 2, 2, true, false, RULE_CEIL, true>(x, stream);
        return launch_dq<DQ_MXFP4, 128, 128, 2, 2, false, false, RULE_CEIL, true>(x, stream);
    });
}

// ---- the quantize-once fused MXFP8 GEMM (POOL) ----
// Workspace (256-byte aligned base): A codes [m, k] at 0, E8M0 scales
// [m, k/32] (mx_quantize_act's layout) at the next 256-byte boundary, then at
// the next one the pool counter, a done counter per 128-row block and an
// error word.
static size_t dq_align256(size_t v) { return (v + 255) & ~(size_t)255; }
static size_t dq_pool_scale_offset(int64_t m, int64_t k) { return dq_align256((size_t)m * k); }
static size_t dq_pool_state_offset(int64_t m, int64_t k)
{
    return dq_align256(dq_pool_scale_offset(m, k) + (size_t)m * (k / 32));
}

// Used for k % 128 == 0 and n > 256 (with fewer tile columns the in-tile
// prologue repeats little); 0 otherwise.
extern "C" size_t mxl_dq_pool_workspace(int64_t m, int64_t n, int64_t k)
{
    if (k % 128 != 0 || n <= 256) return 0;
    const int64_t nb = (m + 127) / 128;
    return dq_pool_state_offset(m, k) + (((size_t)(nb + 2) * sizeof(int) + 255) & ~(size_t)255);
}

__global__ void dq_pool_zero_kernel(int* p, int n)
{
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) p[i] = 0;
}

template <int RULE>
static hipError_t pool8(const DqArgs& a, int out_f32, hipStream_t stream)
{
    if (out_f32) return launch_dq_k<DQ_MXFP8, 128, 128, 2, 2, true, false, RULE, false, true, false, true>(a, stream);
    return launch_dq_k<DQ_MXFP8, 128, 128, 2, 2, false, false, RULE, false, true, false, true>(a, stream);
}

// The fused MXFP8 GEMM with A quantized once into `work` (at least
// mxl_dq_pool_workspace bytes, 256-byte aligned; calls sharing it must not
// overlap) by the GEMM's own workgroups.  Y equals mx_quantize_act followed
// by the unsplit mx_gemm.
extern "C" hipError_t mxl_launch_mxfp8_exact_gemm_pool(int a_rule, const void* a_bf16, const void* wq,
                                                       const void* ws, int64_t m, int64_t n, int64_t k, void* y,
                                                       int out_f32, void* work, size_t work_bytes,
                                                       hipStream_t stream)
{
    const size_t need = mxl_dq_pool_workspace(m, n, k);
    if (need == 0 || !work || work_bytes < need || (reinterpret_cast<uintptr_t>(work) & 255))
        return hipErrorInvalidValue;
    uint8_t* w8 = static_cast<uint8_t*>(work);
    const int nb = (int)((m + 127) / 128);
    int* state = reinterpret_cast<int*>(w8 + dq_pool_state_offset(m, k));
    hipLaunchKernelGGL(dq_pool_zero_kernel, dim3((nb + 2 + 255) / 256), dim3(256), 0, stream, state, nb + 2);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    DqArgs a{w8, w8 + dq_pool_scale_offset(m, k), static_cast<const uint8_t*>(wq), static_cast<const uint8_t*>(ws), y,
             (int)m, (int)n, (int)k, 1.0f, nullptr, 1, 1 << 30, nullptr, nullptr,
             static_cast<const uint4*>(a_bf16), state, nb};
    if (a_rule == RULE_CEIL) return pool8<RULE_CEIL>(a, out_f32, stream);
    if (a_rule == RULE_FLOOR) return pool8<RULE_FLOOR>(a, out_f32, stream);
    return pool8<RULE_EVEN>(a, out_f32, stream);
}

extern "C" const char* mxl_w4a16_gemm_config_name(void)
{
    return "dq_gemm_kernel<bf16 A x (mxfp4|nvfp4 -> exact bf16) W, tile 128x128x64, 2x2 waves of 64x64, "
           "bf16 mfma 32x32x16>";
}

extern "C" const char* mxl_nv_gemm_config_name(int64_t m, int64_t n, int64_t k)
{
    if (dq_decode_ok(DQ_NVFP4, m, n, k))
        return "dq_decode_stream_kernel<nvfp4 -> exact f16, 16 W rows per workgroup, each wave streams its own K quarter "
               "through a ring of 3 LDS chunk slots (8 rows x 128 B copies), f16 mfma 16x16x32>, one launch per "
               "16 rows of A";
    if (nv_tile_ok(m, n, k)) return mxl_dq8w_config_name();
    return "dq_gemm_kernel<nvfp4 -> exact f16, tile 128x128x64, 2x2 waves of 64x64, f16 mfma 32x32x16>";
}

extern "C" const char* mxl_mxfp8_exact_config_name(int64_t m, int64_t n, int64_t k)
{
    if (dq8_decode_first(m, n, k) || (!mxl_mx8_tile_ok(m, n, k) && dq_decode_ok(DQ_MXFP8, m, n, k)))
        return "dq_decode_stream_kernel<mxfp8 -> exact bf16, 16 W rows per workgroup, each wave streams its own K "
               "quarter through a ring of 3 LDS chunk slots (8 rows x 128 B copies), bf16 mfma "
               "16x16x32>, one launch per 16 rows of A";
    if (mxl_mx8_tile_ok(m, n, k)) return mxl_mx8_tile_config_name();
    return "dq_gemm_kernel<mxfp8 -> exact bf16, tile 128x128x64, 2x2 waves of 64x64, bf16 mfma 32x32x16>";
}
