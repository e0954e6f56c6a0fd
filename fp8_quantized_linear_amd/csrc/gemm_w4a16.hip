// gemm_w4a16.hip -- the weight-only (W4A16) linear layer for decode-sized M:
//   Y[m, n] = alpha * sum_k A[m, k] * dq(W)[n, k]
// with bf16 activations used as they are and packed 4-bit weights,
//   MXFP4: dq(w) = e2m1 * 2^(s - 127), E8M0 scale per 32 (alpha normally 1);
//   NVFP4: dq(w) = e2m1 * s_e4m3,      E4M3 scale per 16, alpha = 1 / g_w.
//
// Operation: one packed artifact serves both W4A4 and W4A16 serving
// (Qwen3.5-27B-MXFP4-QAD-W4A4-LR1e-5-s1000, introduction); the NVFP4
// weight-only checkpoint keeps activations in bf16 with weight bytes
// identical to its W4A4 sibling, and its results table quotes this mode's
// generation throughput (Qwen3.5-27B-NVFP4-RTN-weight-only, introduction
// and results).
//
// A weight element times its block scale is exact in bf16 (2 significant
// bits times a power of two, or times 4 significant bits of E4M3), so the
// contraction runs on the bf16 matrix cores (v_mfma_f32_16x16x32_bf16) with
// fp32 accumulation, like the oracle's exact products.  MXFP4 values below
// 2^-126 (blocks whose scale exponent is -127) are flushed, as in the MXFP8
// dequantization.
//
// Design (M <= 16, K % 512 == 0, the W block fits LDS): a stream over W.
//  * One workgroup of 4 waves owns 16 rows of W.  Their contiguous
//    16 x K/2 code block and 16 x K/B scale block (B = 32 or 16) are copied
//    global -> LDS by buffer-to-LDS copies (1 KiB and 256 B each); a copy
//    lane places 16-byte unit u of row r at unit u ^ (r & 15) within aligned
//    groups of 16, so that the step reads below hit distinct banks.
//  * Wave w takes a contiguous quarter of K in groups of 128 (4 steps of
//    the 16x16x32 MFMA).  Lane l = r + 16 g supplies W row r and A row r; in
//    each group it owns 32 consecutive K elements, one 16-byte code unit:
//    one LDS read and one (MXFP4) or two (NVFP4) scale bytes per 4 MFMAs,
//    dequantized to bf16 in registers 8 elements per step.  A and W assign
//    the same K elements to each lane and step, so every step still sums 32
//    distinct k.  The 64 bytes of A per group come straight from global
//    memory (A is at most 16 x K bf16, shared by every workgroup and
//    cache-resident), two groups of loads ahead.  A rows past M read as zero.
//  * The four K quarters are summed through LDS (aliasing the W block).
#include "mx_device.h"

namespace mxl {

typedef __bf16 bf16x8_w __attribute__((ext_vector_type(8)));
typedef float f32x4_w __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2_w __attribute__((ext_vector_type(2)));

struct W4a16Args {
    const uint8_t* a;     // [M, K] bf16
    const uint8_t* w_q;   // [N, K/2] E2M1
    const uint8_t* w_s;   // [N, K/32] E8M0 or [N, K/16] E4M3
    void* y;              // [M, N] bf16 or fp32
    int M, N, K;
    float alpha;
};

// E4M3 code -> fp32 (exact; NaN codes never occur in valid scales)
__device__ __forceinline__ float w4_e4m3_to_f32(uint32_t c)
{
    const uint32_t ef = (c >> 3) & 15u, m = c & 7u;
    const float v = ef == 0 ? (float)m * 0x1p-9f : __uint_as_float(((ef + 120u) << 23) | (m << 20));
    return (c & 0x80u) ? -v : v;
}

// bf16 pairs halved by exponent decrement; results below the normal range
// flush to signed zero
__device__ __forceinline__ uint32_t w4_bf16x2_halve(uint32_t v)
{
    uint32_t out = 0;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        uint32_t h = (v >> (16 * i)) & 0xFFFFu;
        h = ((h >> 7) & 0xFFu) >= 2u ? h - 0x80u : (h & 0x8000u);
        out |= h << (16 * i);
    }
    return out;
}

// 8 E2M1 codes (a dword, element 2j in the low nibble of byte j) dequantized
// to 8 bf16: NVFP4 with the E4M3 scale s, MXFP4 with the exponent e
template <bool NV>
__device__ __forceinline__ bf16x8_w w4_dequant8(uint32_t codes, float s, int e)
{
    uint32_t o[4];
    if (NV) {
        const float2_t f0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, 1.0f, 0);
        const float2_t f1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, 1.0f, 1);
        const float2_t f2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, 1.0f, 2);
        const float2_t f3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, 1.0f, 3);
        o[0] = bf16x2_rne(f0[0] * s, f0[1] * s);
        o[1] = bf16x2_rne(f1[0] * s, f1[1] * s);
        o[2] = bf16x2_rne(f2[0] * s, f2[1] * s);
        o[3] = bf16x2_rne(f3[0] * s, f3[1] * s);
    } else {
        const float p = __uint_as_float((uint32_t)((e < -126 ? -126 : e) + 127) << 23);
        const bf16x2_w h0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, p, 0);
        const bf16x2_w h1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, p, 1);
        const bf16x2_w h2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, p, 2);
        const bf16x2_w h3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, p, 3);
        o[0] = __builtin_bit_cast(uint32_t, h0);
        o[1] = __builtin_bit_cast(uint32_t, h1);
        o[2] = __builtin_bit_cast(uint32_t, h2);
        o[3] = __builtin_bit_cast(uint32_t, h3);
        if (e < -126) {
#pragma unroll
            for (int j = 0; j < 4; ++j) o[j] = w4_bf16x2_halve(o[j]);
        }
    }
    bf16x8_w v;
    __builtin_memcpy(&v, o, 16);
    return v;
}

template <bool NV>
static size_t w4a16_decode_lds_bytes(int K)
{
    const size_t block = (size_t)16 * (K / 2), red = (size_t)4 * 64 * 16;
    return (block > red ? block : red) + (size_t)16 * (K / (NV ? 16 : 32));
}

template <bool NV, bool OUT_F32>
__global__ __launch_bounds__(256) void w4a16_decode_kernel(W4a16Args p)
{
    constexpr int WAVES = 4;
    extern __shared__ __align__(16) uint8_t dsm[];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int r = lane & 15, g = lane >> 4;
    const int n0 = blockIdx.x * 16;
    const int K = p.K, row_bytes = K / 2, KS = K / (NV ? 16 : 32);
    const int units = K / 32;              // 16-byte code units per W row (a multiple of 16)
    const int steps = K / 32;
    const int s0 = wave * steps / WAVES, s1 = (wave + 1) * steps / WAVES;

    // LDS: W codes [16][row_bytes] (later the reduction area), W scales [16][KS]
    constexpr int RED_BYTES = WAVES * 64 * 16;
    uint8_t* w_lds = dsm;
    uint8_t* ws_lds = dsm + (16 * row_bytes > RED_BYTES ? 16 * row_bytes : RED_BYTES);
    const uint32_t lds0 = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)dsm);
    {
        const int4_t rw = make_rsrc(p.w_q, (uint32_t)p.N * row_bytes);
        const int ncopy = 16 * units / 64;
        for (int j = wave; j < ncopy; j += WAVES) {
            const int q = 64 * j + lane, rr = q / units, pu = q - rr * units;
            dma_b128(lds0 + (uint32_t)(64 * j * 16), (n0 + rr) * row_bytes + (pu ^ (rr & 15)) * 16, rw, 0);
        }
        const int4_t rws = make_rsrc(p.w_s, (uint32_t)p.N * KS);
        const uint32_t sbase = lds0 + (uint32_t)(ws_lds - dsm);
        const int sn = 16 * KS / 256;   // K % 512 == 0: whole 256-byte copies
        for (int j = wave; j < sn; j += WAVES) dma_b32(sbase + j * 256, n0 * KS + j * 256 + lane * 4, rws, 0);
    }
    // A rows past M read as zero through the range check.  K is walked in
    // groups of 128 (4 MFMA steps); in group q lane group g owns the 32 K
    // elements [128 q + 32 g, 128 q + 32 g + 32), i.e. code unit 4 q + g of
    // its W row, and feeds their 8-element quarters to the 4 steps (A and W
    // use the same K assignment, so each step still sums 32 distinct k).
    const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc((void*)p.a, (short)0, p.M * K * 2, 0x00020000);
    const int a_off = r * K * 2 + g * 64;   // this lane's A row and K offset within a group
    const int q0 = s0 / 4, q1 = s1 / 4;     // this wave's groups (K % 512 == 0: whole groups)
    constexpr int QR = 2;                   // groups of A loads in flight
    bf16x8_w af[QR][4];
#pragma unroll
    for (int x = 0; x < QR; ++x)
#pragma unroll
        for (int j = 0; j < 4; ++j)
            af[x][j] = __builtin_bit_cast(bf16x8_w,
                                          __builtin_amdgcn_raw_buffer_load_b128(ra, a_off + j * 16, (q0 + x) * 256, 0));
    wait_vmcnt<0>();   // the copies (and the first A groups) have landed
    __syncthreads();

    f32x4_w acc = {0.f, 0.f, 0.f, 0.f};
    const uint8_t* wrow = w_lds + r * row_bytes;
    const uint8_t* srow = ws_lds + r * KS;
    // group q in ring slot x: the A loads of group q + QR go out as group q
    // is computed (past the wave's range they read data that is dropped)
    auto group = [&](int q, int x) __attribute__((always_inline)) {
        const int u = 4 * q + g;
        const uint4 cw = *reinterpret_cast<const uint4*>(wrow + ((u ^ r) * 16));
        float s_lo = 1.0f, s_hi = 1.0f;
        int e = 0;
        if (NV) {
            const uint32_t sp = *reinterpret_cast<const uint16_t*>(srow + 2 * u);
            s_lo = w4_e4m3_to_f32(sp & 0xFFu);
            s_hi = w4_e4m3_to_f32(sp >> 8);
        } else {
            e = (int)srow[u] - 127;
        }
        const uint32_t cws[4] = {cw.x, cw.y, cw.z, cw.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const bf16x8_w b8 = w4_dequant8<NV>(cws[j], j < 2 ? s_lo : s_hi, e);
            const bf16x8_w a8 = af[x][j];
            af[x][j] = __builtin_bit_cast(bf16x8_w,
                                          __builtin_amdgcn_raw_buffer_load_b128(ra, a_off + j * 16, (q + QR) * 256, 0));
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a8, b8, acc, 0, 0, 0);
        }
    };
    int q = q0;
    for (; q + QR <= q1; q += QR) {
#pragma unroll
        for (int x = 0; x < QR; ++x) group(q + x, x);
    }
    if (q < q1) group(q, 0);
    __syncthreads();   // every wave is done with the W block
    f32x4_w* red = reinterpret_cast<f32x4_w*>(w_lds);   // [WAVES][64]
    red[wave * 64 + lane] = acc;
    __syncthreads();
    // lane l of the first wave finishes output rows 4 (l / 16) + i, column n0 + l % 16
    if (tid < 64) {
        f32x4_w v = red[tid];
#pragma unroll
        for (int w = 1; w < WAVES; ++w) {
            const f32x4_w x = red[w * 64 + tid];
            v = f32x4_w{v[0] + x[0], v[1] + x[1], v[2] + x[2], v[3] + x[3]};
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
    wait_vmcnt<0>();   // the trailing A loads have returned
}

template <bool NV, bool OUT_F32>
static hipError_t launch_w4a16_decode(const W4a16Args& a, hipStream_t stream)
{
    hipLaunchKernelGGL((w4a16_decode_kernel<NV, OUT_F32>), dim3((a.N + 15) / 16), dim3(256),
                       w4a16_decode_lds_bytes<NV>(a.K), stream, a);
    return hipGetLastError();
}

} // namespace mxl

using namespace mxl;

// Shapes the decode kernel takes: M <= 16, K % 512 == 0, its LDS block
// within 64 KiB (three workgroups per compute unit).
extern "C" int mxl_w4a16_decode_ok(int w_nv, int64_t m, int64_t k)
{
    if (m > 16 || k % 512 != 0 || k > 65536) return 0;
    return (w_nv ? w4a16_decode_lds_bytes<true>((int)k) : w4a16_decode_lds_bytes<false>((int)k)) <= 65536 ? 1 : 0;
}

extern "C" hipError_t mxl_launch_w4a16_decode(int w_nv, const void* a_bf16, const void* wq, const void* ws,
                                              int64_t m, int64_t n, int64_t k, float alpha, void* y,
                                              int out_f32, hipStream_t stream)
{
    W4a16Args a{static_cast<const uint8_t*>(a_bf16), static_cast<const uint8_t*>(wq),
                static_cast<const uint8_t*>(ws), y, (int)m, (int)n, (int)k, alpha};
    if (w_nv) return out_f32 ? launch_w4a16_decode<true, true>(a, stream) : launch_w4a16_decode<true, false>(a, stream);
    return out_f32 ? launch_w4a16_decode<false, true>(a, stream) : launch_w4a16_decode<false, false>(a, stream);
}

extern "C" const char* mxl_w4a16_decode_config_name(void)
{
    return "w4a16_decode_kernel<16 W rows per workgroup, whole-row copies into swizzled LDS, 4 waves over K "
           "quarters in groups of 128, A two groups ahead, bf16 mfma 16x16x32>";
}
