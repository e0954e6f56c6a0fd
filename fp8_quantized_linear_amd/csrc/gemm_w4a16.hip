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
// fp32 accumulation, like the oracle's exact products.  MXFP4 blocks with
// scale 2^-127 are exact too (as bf16 subnormals).
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

// The two E4M3 codes in bits 0-15 of c as fp32 values, by the hardware
// conversion at scale 1 (exact).  The stream kernel uses it (NVFP4 M = 1:
// 16.2 -> 14.9 us at K = 5120, N = 17408); in the whole-row kernel the bit
// form above measured 1.5% faster.
__device__ __forceinline__ float2_t w4_e4m3x2_to_f32(uint32_t c)
{
    return __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(c, 1.0f, false);
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
        // the conversion reads the scale operand's exponent field as E8M0,
        // field 0 (2^-127) included
        const float p = __uint_as_float((uint32_t)(e + 127) << 23);
        const bf16x2_w h0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, p, 0);
        const bf16x2_w h1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, p, 1);
        const bf16x2_w h2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, p, 2);
        const bf16x2_w h3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, p, 3);
        o[0] = __builtin_bit_cast(uint32_t, h0);
        o[1] = __builtin_bit_cast(uint32_t, h1);
        o[2] = __builtin_bit_cast(uint32_t, h2);
        o[3] = __builtin_bit_cast(uint32_t, h3);
    }
    bf16x8_w v;
    __builtin_memcpy(&v, o, 16);
    return v;
}

// buffer-to-LDS copy of 16 bytes per lane marked non-temporal: W codes are
// read once, streamed past the caches
__device__ __forceinline__ void w4_dma_b128_nt(uint32_t lds, int voff, const int4_t& rsrc, int soff)
{
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, %3 offen nt lds"
                 :: "s"(lds), "v"(voff), "s"(rsrc), "s"(soff) : "memory");
}

// LDS reads at a byte address of the workgroup's LDS
__device__ __forceinline__ uint32_t w4_lds_u32(uint32_t addr)
{
    return *reinterpret_cast<const __attribute__((address_space(3))) uint32_t*>((size_t)addr);
}
__device__ __forceinline__ int4_t w4_lds_v4(uint32_t addr)
{
    return *reinterpret_cast<const __attribute__((address_space(3))) int4_t*>((size_t)addr);
}
// s_waitcnt vmcnt(n) for an n that folds to a constant once loops are
// unrolled (even n <= 14)
__device__ __forceinline__ void w4_wait_vmcnt_n(int n)
{
    switch (n) {
    case 0: wait_vmcnt<0>(); break;
    case 2: wait_vmcnt<2>(); break;
    case 4: wait_vmcnt<4>(); break;
    case 6: wait_vmcnt<6>(); break;
    case 8: wait_vmcnt<8>(); break;
    case 10: wait_vmcnt<10>(); break;
    case 12: wait_vmcnt<12>(); break;
    case 14: wait_vmcnt<14>(); break;
    default: wait_vmcnt<0>(); break;
    }
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

// The same product streamed per wave, for M <= 2 rows of A, K % 1024 == 0
// (QS = K / 512 stages of 128 per wave).  As in mx_decode_stream_kernel, wave
// w owns a contiguous quarter of K: it copies its 16 x K/8 bytes of W codes
// into its own LDS region (8 rows x 128 B non-temporal copies, in stage order),
// and its quarter of each A row next to them, so that it can compute each
// stage as soon as that stage's copies have landed, with an exact vmcnt and
// no wait on the other waves.  The W scale block (16 rows) is copied once by
// all waves together and published by one barrier before the first stage.
//  * LDS: [4 W regions of 16 x K/8 bytes][A: M rows x K bf16][W scales 16 x KS].
//  * Lane (r, g) of stage s (global stage st) holds W row r, K elements
//    [128 st + 32 g, +32) (one 16-byte unit), dequantized 8 elements per
//    MFMA step j, and A row min(r, M - 1), K [128 st + 32 g + 8 j, +8): the
//    rows past M repeat a real row and only feed output rows that are never
//    stored.  The K assignment, the step order and the wave order of the
//    final sum are those of w4a16_decode_kernel, so the results are the same.
template <bool NV, int QS, bool OUT_F32>
__global__ __launch_bounds__(256) void w4a16_decode_stream_kernel(W4a16Args p)
{
    constexpr int WAVES = 4, NC = QS / 2;
    constexpr int K = QS * 512, row_bytes = K / 2, KS = K / (NV ? 16 : 32), QB = row_bytes / WAVES;
    extern __shared__ __align__(16) uint8_t dsm[];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int r = lane & 15, g = lane >> 4;
    const int n0 = blockIdx.x * 16;
    const int st0 = wave * QS;
    const int M = p.M;
    const uint32_t lds0 = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)dsm);
    const uint32_t lds_w = lds0 + (uint32_t)(wave * 16 * QB);
    const uint32_t a_lds = lds0 + (uint32_t)(16 * row_bytes);
    const uint32_t s_lds = a_lds + (uint32_t)(M * K * 2);

    // 1. the W scale block, 256 bytes per copy, spread over the waves
    constexpr int SCOP = 16 * KS / 256;
    {
        const int4_t rws = make_rsrc(p.w_s, (uint32_t)p.N * KS);
#pragma unroll
        for (int j = 0; j < SCOP; ++j)
            if (j % WAVES == wave) dma_b32(s_lds + j * 256, n0 * KS + j * 256 + lane * 4, rws, 0);
    }
    // 2. this wave's quarter of each A row (bf16: K/2 bytes), 256 bytes per copy
    constexpr int ACOP = (K / 2) / 256;   // per A row: a quarter of K in bf16
    {
        const int4_t ra = make_rsrc(p.a, (uint32_t)M * K * 2);
        for (int m = 0; m < M; ++m)
#pragma unroll
            for (int j = 0; j < ACOP; ++j)
                dma_b32(a_lds + (uint32_t)(m * K * 2 + wave * (K / 2) + j * 256), m * K * 2 + wave * (K / 2) + j * 256 + lane * 4,
                        ra, 0);
    }
    // 3. this wave's W codes, in stage order
    {
        const int4_t rw = make_rsrc(p.w_q, (uint32_t)p.N * row_bytes);
        int voffh[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int q = 8 * h + (lane >> 3);
            voffh[h] = (n0 + q) * row_bytes + (((lane & 7) ^ ((q >> 1) & 7)) * 16);
        }
#pragma unroll
        for (int c = 0; c < NC; ++c)
#pragma unroll
            for (int h = 0; h < 2; ++h)
                w4_dma_b128_nt(lds_w + (uint32_t)((2 * c + h) * 1024), voffh[h], rw, wave * QB + c * 128);
    }
    // the scale and A copies have landed once at most the QS W copies are
    // outstanding; the barrier publishes the scale block
    wait_vmcnt<QS>();
    lds_barrier();

    f32x4_w acc = {0.f, 0.f, 0.f, 0.f};
    const uint32_t rd = lds_w + (uint32_t)((r >> 3) * 1024 + (r & 7) * 128);
    const int rsw = (r >> 1) & 7;
    const uint32_t arow = a_lds + (uint32_t)((r < M ? r : M - 1) * K * 2 + st0 * 256 + g * 64);
    const uint32_t srow = s_lds + (uint32_t)(r * KS);
#pragma unroll
    for (int c = 0; c < NC; ++c) {
        w4_wait_vmcnt_n(2 * (NC - 1 - c));
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
            const int u = 2 * c + hf, un = 4 * (st0 + u) + g;   // global 16-byte unit of the W row
            const int4_t cw = w4_lds_v4(rd + (uint32_t)(2 * c * 1024 + (((4 * hf + g) ^ rsw) * 16)));
            float s_lo = 1.0f, s_hi = 1.0f;
            int e = 0;
            if (NV) {
                const float2_t sp = w4_e4m3x2_to_f32(w4_lds_u32(srow + (uint32_t)(2 * un) & ~3u) >> (8 * ((2 * un) & 3)));
                s_lo = sp[0];
                s_hi = sp[1];
            } else {
                e = (int)((w4_lds_u32(srow + (uint32_t)un & ~3u) >> (8 * (un & 3))) & 0xFFu) - 127;
            }
            const uint32_t cws[4] = {(uint32_t)cw[0], (uint32_t)cw[1], (uint32_t)cw[2], (uint32_t)cw[3]};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const bf16x8_w b8 = w4_dequant8<NV>(cws[j], j < 2 ? s_lo : s_hi, e);
                const bf16x8_w a8 = __builtin_bit_cast(bf16x8_w, w4_lds_v4(arow + (uint32_t)(u * 256 + j * 16)));
                acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a8, b8, acc, 0, 0, 0);
            }
        }
    }
    __syncthreads();   // every wave is done with its LDS regions
    f32x4_w* red = reinterpret_cast<f32x4_w*>(dsm);   // [WAVES][64]
    red[wave * 64 + lane] = acc;
    __syncthreads();
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
}

// The same product for M <= 16 rows of A (K % 1024 == 0, QS = K / 512
// stages of 128 per wave) where A does not fit in LDS beside W (above two
// rows, or NVFP4 scales at two rows and K = 5120).  The whole-row kernel
// reads A's full K extent (M x 2K bytes of bf16) from the L2 for every 16
// rows of W, twice the W bytes at M = 8.  Here a workgroup owns two 16-row
// groups of W, so each A fragment serves both, and every wave streams its
// own K quarter of the 32 rows through a ring of RS pair slots, as the W4A4
// decode kernel does above 16 rows of A.
//  * Copy (c, h), h = 0 .. 3, moves rows 8 h .. 8 h + 7 of the 32 x bytes
//    [128 c, 128 c + 128) of the wave's quarter (8 cache lines, 1 KiB) into
//    slot c % RS, with the chunk swizzle of w4a16_decode_stream_kernel.
//  * A comes straight from global memory into a register ring of APR stage
//    pairs (4 x 16 bytes per lane and stage); rows past M read as zero
//    through the buffer range check.  The A loads of pair c + APR go out
//    once pair c has been computed, followed by the W copies of pair c + RS,
//    and the wait before pair c counts exactly the loads and copies issued
//    after both of its own.
//  * Lane (r, g) of stage s holds, for each group rg, W row 16 rg + r, K
//    elements [128 st + 32 g, +32), and A row r, K [128 st + 32 g + 8 j,
//    +8) for MFMA step j: the K assignment, step order and wave order of
//    the whole-row kernel, so the results are bitwise the same.
constexpr int w16_min(int a, int b) { return a < b ? a : b; }
// VMEM operations a wave has issued (after its scale copies) before it
// computes pair c: the prologue's A pairs (8 loads each) and W pairs (cw
// copies each), then per computed pair i the A loads of pair i + APR and the
// W copies of pair i + RSB
constexpr int w16_issued(int c, int nc, int apr, int rsb, int cw)
{
    int n = 8 * w16_min(apr, nc) + cw * w16_min(rsb, nc);
    for (int i = 0; i < c; ++i) n += (i + apr < nc ? 8 : 0) + (i + rsb < nc ? cw : 0);
    return n;
}
// operations issued after the later of pair c's A loads and W copies, at
// the point where pair c is computed: the vmcnt that waits for both
constexpr int w16_wait(int c, int nc, int apr, int rsb, int cw)
{
    const int end_a = c < apr ? 8 * (c + 1) : w16_issued(c - apr, nc, apr, rsb, cw) + 8;
    const int end_w = c < rsb ? 8 * w16_min(apr, nc) + cw * (c + 1)
                              : w16_issued(c - rsb, nc, apr, rsb, cw) + (c - rsb + apr < nc ? 8 : 0) + cw;
    return w16_issued(c, nc, apr, rsb, cw) - (end_a > end_w ? end_a : end_w);
}
// s_waitcnt vmcnt(n) for an n that folds to a constant once loops are
// unrolled (n <= 23)
__device__ __forceinline__ void w16_wait_vmcnt(int n)
{
    switch (n) {
    case 0: wait_vmcnt<0>(); break;   case 1: wait_vmcnt<1>(); break;   case 2: wait_vmcnt<2>(); break;
    case 3: wait_vmcnt<3>(); break;   case 4: wait_vmcnt<4>(); break;   case 5: wait_vmcnt<5>(); break;
    case 6: wait_vmcnt<6>(); break;   case 7: wait_vmcnt<7>(); break;   case 8: wait_vmcnt<8>(); break;
    case 9: wait_vmcnt<9>(); break;   case 10: wait_vmcnt<10>(); break; case 11: wait_vmcnt<11>(); break;
    case 12: wait_vmcnt<12>(); break; case 13: wait_vmcnt<13>(); break; case 14: wait_vmcnt<14>(); break;
    case 15: wait_vmcnt<15>(); break; case 16: wait_vmcnt<16>(); break; case 17: wait_vmcnt<17>(); break;
    case 18: wait_vmcnt<18>(); break; case 19: wait_vmcnt<19>(); break; case 20: wait_vmcnt<20>(); break;
    case 21: wait_vmcnt<21>(); break; case 22: wait_vmcnt<22>(); break; case 23: wait_vmcnt<23>(); break;
    default: wait_vmcnt<0>(); break;
    }
}

template <bool NV, int QS, int RS, bool OUT_F32, int RG = 2, bool PART = false>
__global__ __launch_bounds__(256) void w4a16_decode_stream2_kernel(W4a16Args p)
{
    constexpr int WAVES = 4, NC = QS / 2, RSB = w16_min(RS, NC), APR = w16_min(2, NC);
    constexpr int SLOT = RG * 2048;   // a pair slot: 16 RG rows x 128 B per wave
    static_assert(RG >= 1 && RG <= 5, "row groups per workgroup");
    constexpr int K = QS * 512, row_bytes = K / 2, KS = K / (NV ? 16 : 32), QB = row_bytes / WAVES;
    static_assert(QS % 2 == 0 && QS <= 16, "stream2 shape");
    extern __shared__ __align__(16) uint8_t dsm[];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int r = lane & 15, g = lane >> 4;
    // PART: the grid's workgroups split the ceil(N / 16) row groups evenly,
    // workgroup b taking groups [b G / grid, (b + 1) G / grid), at most RG of
    // them; rows past its last group read as zero and are not stored
    int n0, n_lim;
    if (PART) {
        const int64_t G = (p.N + 15) / 16, b = blockIdx.x, nwg = gridDim.x;
        n0 = (int)(16 * (b * G / nwg));
        n_lim = (int)min((int64_t)p.N, 16 * ((b + 1) * G / nwg));
    } else {
        n0 = blockIdx.x * 16 * RG;
        n_lim = p.N;
    }
    const int st0 = wave * QS;
    const uint32_t lds0 = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)dsm);
    const uint32_t lds_w = lds0 + (uint32_t)(wave * RSB * SLOT);   // this wave's ring
    const uint32_t s_lds = lds0 + (uint32_t)(WAVES * RSB * SLOT);  // W scales [32][KS]

    // 1. the W scale block of the 32 rows, 256 bytes per copy, spread over the waves
    constexpr int SCOP = 16 * RG * KS / 256;
    {
        const int4_t rws = make_rsrc(p.w_s, (uint32_t)n_lim * KS);
#pragma unroll
        for (int j = 0; j < SCOP; ++j)
            if (j % WAVES == wave) dma_b32(s_lds + j * 256, n0 * KS + j * 256 + lane * 4, rws, 0);
    }
    // 2. A fragments of the first APR pairs
    const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc((void*)p.a, (short)0, p.M * K * 2, 0x00020000);
    const int a_off = r * K * 2 + g * 64;
    bf16x8_w af[APR][2][4];
    auto load_a = [&](int c) __attribute__((always_inline)) {
#pragma unroll
        for (int hf = 0; hf < 2; ++hf)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                af[c % APR][hf][j] = __builtin_bit_cast(
                    bf16x8_w, __builtin_amdgcn_raw_buffer_load_b128(ra, a_off + j * 16, (st0 + 2 * c + hf) * 256, 0));
    };
#pragma unroll
    for (int c = 0; c < APR; ++c) load_a(c);
    // 3. the W copies of the first RSB pairs
    const int4_t rw = make_rsrc(p.w_q, (uint32_t)n_lim * row_bytes);
    int voffh[2 * RG];
#pragma unroll
    for (int h = 0; h < 2 * RG; ++h) {
        const int q = 8 * h + (lane >> 3);
        voffh[h] = (n0 + q) * row_bytes + (((lane & 7) ^ ((q >> 1) & 7)) * 16);
    }
    auto copy_pair = [&](int c) __attribute__((always_inline)) {
#pragma unroll
        for (int h = 0; h < 2 * RG; ++h)
            w4_dma_b128_nt(lds_w + (uint32_t)((c % RSB) * SLOT + h * 1024), voffh[h], rw, wave * QB + c * 128);
    };
#pragma unroll
    for (int c = 0; c < RSB; ++c) copy_pair(c);
    // the scale copies have landed once at most the A loads and W copies
    // issued after them are outstanding; the barrier publishes them
    wait_vmcnt<8 * APR + 2 * RG * RSB>();
    lds_barrier();

    f32x4_w acc[RG];
#pragma unroll
    for (int rg = 0; rg < RG; ++rg) acc[rg] = f32x4_w{0.f, 0.f, 0.f, 0.f};
    const uint32_t rd = lds_w + (uint32_t)((r >> 3) * 1024 + (r & 7) * 128);
    const int rsw = (r >> 1) & 7;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
        w16_wait_vmcnt(w16_wait(c, NC, APR, RSB, 2 * RG));
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
            const int un = 4 * (st0 + 2 * c + hf) + g;   // global 16-byte unit of the W row
#pragma unroll
            for (int rg = 0; rg < RG; ++rg) {
                const int4_t cw = w4_lds_v4(rd + (uint32_t)((c % RSB) * SLOT + rg * 2048 + (((4 * hf + g) ^ rsw) * 16)));
                const uint32_t srow = s_lds + (uint32_t)((16 * rg + r) * KS);
                float s_lo = 1.0f, s_hi = 1.0f;
                int e = 0;
                if (NV) {
                    const float2_t sp = w4_e4m3x2_to_f32(w4_lds_u32(srow + (uint32_t)(2 * un) & ~3u) >> (8 * ((2 * un) & 3)));
                    s_lo = sp[0];
                    s_hi = sp[1];
                } else {
                    e = (int)((w4_lds_u32(srow + (uint32_t)un & ~3u) >> (8 * (un & 3))) & 0xFFu) - 127;
                }
                const uint32_t cws[4] = {(uint32_t)cw[0], (uint32_t)cw[1], (uint32_t)cw[2], (uint32_t)cw[3]};
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const bf16x8_w b8 = w4_dequant8<NV>(cws[j], j < 2 ? s_lo : s_hi, e);
                    acc[rg] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[c % APR][hf][j], b8, acc[rg], 0, 0, 0);
                }
            }
        }
        if (c + APR < NC) load_a(c + APR);
        if (c + RSB < NC) {
            // slot c % RSB is free once this pair's LDS reads have returned
            __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
            copy_pair(c + RSB);
        }
    }
    __syncthreads();   // every wave is done with its ring
    f32x4_w* red = reinterpret_cast<f32x4_w*>(dsm);   // [WAVES][RG][64]
#pragma unroll
    for (int rg = 0; rg < RG; ++rg) red[(wave * RG + rg) * 64 + lane] = acc[rg];
    __syncthreads();
    // item e < 64 RG finishes accumulator lane e % 64 of group e / 64: A rows
    // 4 (l / 16) + i, W row n0 + 16 rg + l % 16
    for (int e = tid; e < RG * 64; e += 256) {
        const int l = e & 63, rg = e >> 6;
        f32x4_w v = red[rg * 64 + l];
#pragma unroll
        for (int w = 1; w < WAVES; ++w) {
            const f32x4_w x = red[(w * RG + rg) * 64 + l];
            v = f32x4_w{v[0] + x[0], v[1] + x[1], v[2] + x[2], v[3] + x[3]};
        }
        const int nn = n0 + 16 * rg + (l & 15);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int m = 4 * (l >> 4) + i;
            if (m < p.M && nn < n_lim) {
                const float o = v[i] * p.alpha;
                if (OUT_F32) reinterpret_cast<float*>(p.y)[(size_t)m * p.N + nn] = o;
                else reinterpret_cast<uint16_t*>(p.y)[(size_t)m * p.N + nn] = f32_to_bf16_rne(o);
            }
        }
    }
}

constexpr int W16_SLOTS = 2;   // ring slots (stage pairs) per wave

template <bool NV>
static size_t w4a16_stream2_lds_bytes(int64_t k)
{
    const int nc = (int)(k / 1024), slots = W16_SLOTS < nc ? W16_SLOTS : nc;
    return (size_t)4 * slots * 4096 + (size_t)32 * (k / (NV ? 16 : 32));
}

// whether w4a16_decode_stream2_kernel serves this shape (the dispatch
// prefers w4a16_decode_stream_kernel where that one fits)
static bool w4a16_stream2_ok(int64_t m, int64_t k)
{
    return m >= 1 && m <= 16 && k % 1024 == 0 && k >= 1024 && k <= 8192;
}

// When the 16-row groups of W number 4 to 5 per compute unit (MI355X: 256),
// one workgroup per compute unit takes 4 or 5 of them (the grid splits the
// groups evenly): each CU then loads A once, and none holds a workgroup more
// than the others.  Ring and scale blocks take up to 106 KiB of LDS.  NVFP4
// takes it from 8 rows of A: its dequantization is vector-bound, and below
// that the three workgroups per CU of the 32-row grid issue it faster (N =
// 17408, K = 5120: M = 2 / 4 / 8 / 16 at 16.46 / 17.02 / 18.90 / 24.23 us
// with 32-row workgroups, 17.79 / 17.70 / 18.35 / 20.35 us partitioned;
// MXFP4 at M = 3 / 8 / 16: 14.72 / 17.59 / 22.89 -> 13.25 / 13.97 / 15.36 us).
constexpr int W16_PART_WGS = 256, W16_PART_RG = 5;

static bool w4a16_part_ok(int nv, int64_t m, int64_t n)
{
    const int64_t groups = (n + 15) / 16;
    return (!nv || m >= 8) && groups >= 4 * W16_PART_WGS && groups <= W16_PART_RG * W16_PART_WGS;
}

template <bool NV>
static size_t w4a16_part_lds_bytes(int64_t k)
{
    const int nc = (int)(k / 1024), slots = W16_SLOTS < nc ? W16_SLOTS : nc;
    return (size_t)4 * slots * W16_PART_RG * 2048 + (size_t)16 * W16_PART_RG * (k / (NV ? 16 : 32));
}

template <bool NV, int QS, bool OUT_F32>
static hipError_t launch_w4a16_stream2_qs(const W4a16Args& a, hipStream_t stream)
{
    if (w4a16_part_ok(NV, a.M, a.N)) {
        auto kern = w4a16_decode_stream2_kernel<NV, QS, W16_SLOTS, OUT_F32, W16_PART_RG, true>;
        const size_t lds = w4a16_part_lds_bytes<NV>(QS * 512);
        static bool attr_set = false;  // benign race: setting the same value twice is harmless
        if (!attr_set) {
            const hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize,
                                                     (int)lds);
            if (e != hipSuccess) return e;
            attr_set = true;
        }
        hipLaunchKernelGGL(kern, dim3(W16_PART_WGS), dim3(256), lds, stream, a);
        return hipGetLastError();
    }
    hipLaunchKernelGGL((w4a16_decode_stream2_kernel<NV, QS, W16_SLOTS, OUT_F32>), dim3((a.N + 31) / 32), dim3(256),
                       w4a16_stream2_lds_bytes<NV>(a.K), stream, a);
    return hipGetLastError();
}

template <bool NV, bool OUT_F32>
static hipError_t launch_w4a16_stream2(const W4a16Args& a, hipStream_t stream)
{
    switch (a.K / 512) {
    case 2: return launch_w4a16_stream2_qs<NV, 2, OUT_F32>(a, stream);
    case 4: return launch_w4a16_stream2_qs<NV, 4, OUT_F32>(a, stream);
    case 6: return launch_w4a16_stream2_qs<NV, 6, OUT_F32>(a, stream);
    case 8: return launch_w4a16_stream2_qs<NV, 8, OUT_F32>(a, stream);
    case 10: return launch_w4a16_stream2_qs<NV, 10, OUT_F32>(a, stream);
    case 12: return launch_w4a16_stream2_qs<NV, 12, OUT_F32>(a, stream);
    case 14: return launch_w4a16_stream2_qs<NV, 14, OUT_F32>(a, stream);
    default: return launch_w4a16_stream2_qs<NV, 16, OUT_F32>(a, stream);
    }
}

template <bool NV>
static size_t w4a16_stream_lds_bytes(int64_t m, int64_t k)
{
    return (size_t)(16 * (k / 2) + m * k * 2 + 16 * (k / (NV ? 16 : 32)));
}

// whether w4a16_decode_stream_kernel serves this shape
static bool w4a16_stream_ok(int w_nv, int64_t m, int64_t k)
{
    if (m > 2 || k % 1024 != 0 || k < 1024 || k > 8192) return false;
    return (w_nv ? w4a16_stream_lds_bytes<true>(m, k) : w4a16_stream_lds_bytes<false>(m, k)) <= 65536;
}

template <bool NV, int QS, bool OUT_F32>
static void launch_w4a16_stream_qs(const W4a16Args& a, hipStream_t stream)
{
    hipLaunchKernelGGL((w4a16_decode_stream_kernel<NV, QS, OUT_F32>), dim3((a.N + 15) / 16), dim3(256),
                       w4a16_stream_lds_bytes<NV>(a.M, a.K), stream, a);
}

template <bool NV, bool OUT_F32>
static hipError_t launch_w4a16_stream(const W4a16Args& a, hipStream_t stream)
{
    switch (a.K / 512) {
    case 2: launch_w4a16_stream_qs<NV, 2, OUT_F32>(a, stream); break;
    case 4: launch_w4a16_stream_qs<NV, 4, OUT_F32>(a, stream); break;
    case 6: launch_w4a16_stream_qs<NV, 6, OUT_F32>(a, stream); break;
    case 8: launch_w4a16_stream_qs<NV, 8, OUT_F32>(a, stream); break;
    case 10: launch_w4a16_stream_qs<NV, 10, OUT_F32>(a, stream); break;
    case 12: launch_w4a16_stream_qs<NV, 12, OUT_F32>(a, stream); break;
    case 14: launch_w4a16_stream_qs<NV, 14, OUT_F32>(a, stream); break;
    default: launch_w4a16_stream_qs<NV, 16, OUT_F32>(a, stream); break;
    }
    return hipGetLastError();
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

// Shapes the decode kernels take: M <= 16, K % 512 == 0, and either one of
// the streamed kernels (K % 1024 == 0, K <= 8192) or the whole-row kernel's
// LDS block within 64 KiB (three workgroups per compute unit).
extern "C" int mxl_w4a16_decode_ok(int w_nv, int64_t m, int64_t k)
{
    if (m > 16 || k % 512 != 0 || k > 65536) return 0;
    if (w4a16_stream_ok(w_nv, m, k) || w4a16_stream2_ok(m, k)) return 1;
    return (w_nv ? w4a16_decode_lds_bytes<true>((int)k) : w4a16_decode_lds_bytes<false>((int)k)) <= 65536 ? 1 : 0;
}

extern "C" hipError_t mxl_launch_w4a16_decode(int w_nv, const void* a_bf16, const void* wq, const void* ws,
                                              int64_t m, int64_t n, int64_t k, float alpha, void* y,
                                              int out_f32, hipStream_t stream)
{
    W4a16Args a{static_cast<const uint8_t*>(a_bf16), static_cast<const uint8_t*>(wq),
                static_cast<const uint8_t*>(ws), y, (int)m, (int)n, (int)k, alpha};
    if (w4a16_stream_ok(w_nv, m, k)) {
        if (w_nv) return out_f32 ? launch_w4a16_stream<true, true>(a, stream) : launch_w4a16_stream<true, false>(a, stream);
        return out_f32 ? launch_w4a16_stream<false, true>(a, stream) : launch_w4a16_stream<false, false>(a, stream);
    }
    if (w4a16_stream2_ok(m, k)) {
        if (w_nv) return out_f32 ? launch_w4a16_stream2<true, true>(a, stream) : launch_w4a16_stream2<true, false>(a, stream);
        return out_f32 ? launch_w4a16_stream2<false, true>(a, stream) : launch_w4a16_stream2<false, false>(a, stream);
    }
    if (w_nv) return out_f32 ? launch_w4a16_decode<true, true>(a, stream) : launch_w4a16_decode<true, false>(a, stream);
    return out_f32 ? launch_w4a16_decode<false, true>(a, stream) : launch_w4a16_decode<false, false>(a, stream);
}

extern "C" const char* mxl_w4a16_decode_config_name(int w_nv, int64_t m, int64_t n, int64_t k)
{
    if (w4a16_stream_ok(w_nv, m, k))
        return "w4a16_decode_stream_kernel<16 W rows per workgroup, each wave copies its own K quarter of W and A "
               "into LDS and computes each stage as its copies land, bf16 mfma 16x16x32>";
    if (w4a16_stream2_ok(m, k) && w4a16_part_ok(w_nv, m, n))
        return "w4a16_decode_stream2_kernel<one workgroup per compute unit over 4-5 16-row W groups (each A fragment "
               "serves all of them), each wave streams its own K quarter of W through a ring of 2 LDS pair slots, A "
               "from global memory one pair ahead, bf16 mfma 16x16x32>";
    if (w4a16_stream2_ok(m, k))
        return "w4a16_decode_stream2_kernel<32 W rows per workgroup (each A fragment serves both 16-row groups), each "
               "wave streams its own K quarter of W through a ring of 2 LDS pair slots, A from global memory one pair "
               "ahead, bf16 mfma 16x16x32>";
    return "w4a16_decode_kernel<16 W rows per workgroup, whole-row copies into swizzled LDS, 4 waves over K "
           "quarters in groups of 128, A two groups ahead, bf16 mfma 16x16x32>";
}
