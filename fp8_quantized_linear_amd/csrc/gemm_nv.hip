// gemm_nv.hip -- NVFP4 x NVFP4 GEMM for gfx950:
//   Y[m, n] = alpha * sum_k (e2m1_a * s_a) * (e2m1_w * s_w),  alpha = 1/(g_a g_w)
// with E2M1 codes and one E4M3 scale per 16 elements along K.
//
// Operation: the NVFP4 W4A4 serving path of Qwen3.5-27B-NVFP4-GPTQ
// (introduction, "Serving") and Qwen3.5-27B-NVFP4-RTN-weight-only
// (introduction): FP4 elements with per-block scales and per-tensor global
// scales folded into one fp32 factor.
//
// Why f16 matrix cores: the gfx950 scaled matrix-core instructions take only
// power-of-two (E8M0) scales per 32 elements, while NVFP4 scales are E4M3 per
// 16.  An E2M1 value (2 significant bits) times an E4M3 scale (4 significant
// bits, magnitude 2^-9 .. 448) is exact in f16 (11 bits, 2^-24 .. 65504), and
// the product of two such f16 values is exact in fp32.  So each operand is
// dequantized exactly to f16 while it is staged into LDS, and the contraction
// runs on v_mfma_f32_32x32x16_f16 with fp32 accumulation; alpha is applied in
// the epilogue.
//
// f16 matrix-core layout (32x32x16): lane l = r + 32 g holds row/column r and
// the 8 consecutive K elements [8g, 8g + 8) of the 16-wide step.
#include "mx_device.h"

namespace mxl {

constexpr int NV_BK = 64;                 // K elements per LDS stage
constexpr int NV_ROW_BYTES = NV_BK * 2;   // f16 bytes per LDS row per stage (8 chunks)

__device__ __forceinline__ int nv_swz(int row) { return row & 7; }

// E4M3 code -> f16 (exact; NaN codes never occur in valid scales).
__device__ __forceinline__ _Float16 e4m3_to_f16(uint32_t c)
{
    const uint32_t ef = (c >> 3) & 15u, m = c & 7u;
    float v = ef == 0 ? (float)m * 0x1p-9f : __uint_as_float(((ef + 120u) << 23) | (m << 20));
    return (_Float16)((c & 0x80u) ? -v : v);
}

// 8 E2M1 codes (one dword, element 2j in the low nibble of byte j) times a
// scale, as 8 f16 values in a uint4.
__device__ __forceinline__ uint4 dequant8(uint32_t codes, _Float16 s)
{
    const half2_t s2 = {s, s};
    // byte i of `codes` -> 2 f16; the products with the scale are exact
    half2_t h[4];
    h[0] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 0) * s2;
    h[1] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 1) * s2;
    h[2] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 2) * s2;
    h[3] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 3) * s2;
    uint4 out;
    __builtin_memcpy(&out, h, 16);
    return out;
}

struct NvArgs {
    const uint8_t* a_q; const uint8_t* a_s;
    const uint8_t* w_q; const uint8_t* w_s;
    void* y;
    int M, N, K;
    float alpha;
};

template <int BM, int BN, int WM, int WN, bool OUT_F32>
__global__ __launch_bounds__(WM * WN * 64) void nv_gemm_kernel(NvArgs p)
{
    constexpr int NT = WM * WN * 64;
    constexpr int A_TILE = BM * NV_ROW_BYTES, W_TILE = BN * NV_ROW_BYTES;
    constexpr int STAGE = A_TILE + W_TILE;
    constexpr int WTM = BM / WM, WTN = BN / WN, FM = WTM / 32, FN = WTN / 32;
    // a global chunk is 16 B of codes = 32 elements = 2 scale blocks
    constexpr int A_CH = BM * 2, W_CH = BN * 2;
    constexpr int A_PER_T = (A_CH + NT - 1) / NT, W_PER_T = (W_CH + NT - 1) / NT;

    extern __shared__ __align__(16) uint8_t smem[];

    const int tiles_n = (p.N + BN - 1) / BN;
    const int tm = blockIdx.x / tiles_n, tn = blockIdx.x % tiles_n;
    const int m0 = tm * BM, n0 = tn * BN;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave / WN, wn = wave % WN;
    const int K = p.K, KS = K / 16, row_bytes = K / 2;
    const int nk = (K + NV_BK - 1) / NV_BK;

    uint4 ra[A_PER_T], rw[W_PER_T];
    uint32_t sa[A_PER_T], sw[W_PER_T];  // two scale codes (bytes 0, 1)

    auto load_one = [&](const uint8_t* q, const uint8_t* s, int rows_lim, int r0, int qi, int kt,
                        uint4& v, uint32_t& sc) {
        const int row = qi / 2, c = qi % 2;
        const int gr = r0 + row;
        const int kb = kt * (NV_BK / 2) + c * 16;
        v = make_uint4(0, 0, 0, 0);
        sc = 0;
        if (gr < rows_lim && kb < row_bytes) {
            const uint8_t* src = q + (size_t)gr * row_bytes + kb;
            if ((row_bytes & 15) == 0) {
                v = *reinterpret_cast<const uint4*>(src);
            } else {
                // k % 32 == 16: rows are only 8-byte aligned and the last
                // chunk of a row holds a single block of 16 elements
                const uint2 lo = *reinterpret_cast<const uint2*>(src);
                const uint2 hi = kb + 8 < row_bytes ? *reinterpret_cast<const uint2*>(src + 8) : make_uint2(0, 0);
                v = make_uint4(lo.x, lo.y, hi.x, hi.y);
            }
            const int blk = kt * 4 + c * 2;
            sc = (uint32_t)s[(size_t)gr * KS + blk];
            if (blk + 1 < KS) sc |= (uint32_t)s[(size_t)gr * KS + blk + 1] << 8;
        }
    };
    auto load_stage = [&](int kt) {
#pragma unroll
        for (int i = 0; i < A_PER_T; ++i) {
            const int qi = tid + i * NT;
            if (qi < A_CH) load_one(p.a_q, p.a_s, p.M, m0, qi, kt, ra[i], sa[i]);
        }
#pragma unroll
        for (int i = 0; i < W_PER_T; ++i) {
            const int qi = tid + i * NT;
            if (qi < W_CH) load_one(p.w_q, p.w_s, p.N, n0, qi, kt, rw[i], sw[i]);
        }
    };
    auto store_one = [&](uint8_t* tile, int qi, const uint4& v, uint32_t sc) {
        const int row = qi / 2, c = qi % 2;
        const _Float16 s0 = e4m3_to_f16(sc & 0xFFu), s1 = e4m3_to_f16((sc >> 8) & 0xFFu);
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int h = 0; h < 4; ++h) {   // 8 elements per dword -> one 16-B f16 chunk
            const uint4 d = dequant8(w[h], h < 2 ? s0 : s1);
            const int chunk = (c * 4 + h) ^ nv_swz(row);
            *reinterpret_cast<uint4*>(tile + row * NV_ROW_BYTES + chunk * 16) = d;
        }
    };
    auto store_stage = [&](int buf) {
        uint8_t* a_t = smem + buf * STAGE;
        uint8_t* w_t = a_t + A_TILE;
#pragma unroll
        for (int i = 0; i < A_PER_T; ++i) {
            const int qi = tid + i * NT;
            if (qi < A_CH) store_one(a_t, qi, ra[i], sa[i]);
        }
#pragma unroll
        for (int i = 0; i < W_PER_T; ++i) {
            const int qi = tid + i * NT;
            if (qi < W_CH) store_one(w_t, qi, rw[i], sw[i]);
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
        for (int kk = 0; kk < NV_BK / 16; ++kk) {
            half8_t fa[FM], fw[FN];
#pragma unroll
            for (int i = 0; i < FM; ++i) {
                const int row = wm * WTM + i * 32 + r32;
                fa[i] = *reinterpret_cast<const half8_t*>(a_t + row * NV_ROW_BYTES + (((2 * kk + g) ^ nv_swz(row)) * 16));
            }
#pragma unroll
            for (int j = 0; j < FN; ++j) {
                const int row = wn * WTN + j * 32 + r32;
                fw[j] = *reinterpret_cast<const half8_t*>(w_t + row * NV_ROW_BYTES + (((2 * kk + g) ^ nv_swz(row)) * 16));
            }
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(fa[i], fw[j], acc[i][j], 0, 0, 0);
        }
    };

    load_stage(0);
    store_stage(0);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
        const bool more = kt + 1 < nk;
        if (more) load_stage(kt + 1);
        compute_stage(kt & 1);
        if (more) store_stage((kt + 1) & 1);
        __syncthreads();
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
                    const float v = acc[i][j][r] * p.alpha;
                    if (OUT_F32) {
                        reinterpret_cast<float*>(p.y)[(size_t)m * p.N + n] = v;
                    } else {
                        uint32_t u = __float_as_uint(v);
                        u += 0x7FFFu + ((u >> 16) & 1u);
                        reinterpret_cast<uint16_t*>(p.y)[(size_t)m * p.N + n] = (uint16_t)(u >> 16);
                    }
                }
            }
        }
}

template <int BM, int BN, int WM, int WN, bool OUT_F32>
hipError_t launch_nv(const NvArgs& a, hipStream_t stream)
{
    constexpr int LDS = 2 * (BM + BN) * NV_ROW_BYTES;
    auto kern = nv_gemm_kernel<BM, BN, WM, WN, OUT_F32>;
    static bool attr_set = false;
    if (!attr_set) {
        hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, LDS);
        if (e != hipSuccess) return e;
        attr_set = true;
    }
    const int tiles = ((a.M + BM - 1) / BM) * ((a.N + BN - 1) / BN);
    hipLaunchKernelGGL(kern, dim3(tiles), dim3(WM * WN * 64), LDS, stream, a);
    return hipGetLastError();
}

} // namespace mxl

using namespace mxl;

extern "C" hipError_t mxl_launch_nv_gemm(const void* aq, const void* as, const void* wq, const void* ws,
                                         int64_t m, int64_t n, int64_t k, float alpha, void* y,
                                         int out_f32, hipStream_t stream)
{
    NvArgs a{static_cast<const uint8_t*>(aq), static_cast<const uint8_t*>(as),
             static_cast<const uint8_t*>(wq), static_cast<const uint8_t*>(ws), y,
             (int)m, (int)n, (int)k, alpha};
    if (out_f32) return launch_nv<128, 128, 2, 2, true>(a, stream);
    return launch_nv<128, 128, 2, 2, false>(a, stream);
}

extern "C" const char* mxl_nv_gemm_config_name(void)
{
    return "nv_gemm_kernel<tile 128x128x64, 2x2 waves of 64x64, f16 mfma 32x32x16, exact dequant>";
}
