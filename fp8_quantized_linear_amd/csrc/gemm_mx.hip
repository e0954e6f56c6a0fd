// gemm_mx.hip -- block-scaled MX GEMM for gfx950: Y[M, N] = A[M, K] * W[N, K]^T
// with E2M1 (MXFP4) or E4M3 (MXFP8) operands and one E8M0 scale per 32
// elements along K, fp32 accumulation on the scaled matrix cores
// (v_mfma_scale_f32_32x32x64_f8f6f4), bf16 (or fp32) output.
//
// Operation: the W4A4 FP4 GEMM that serves the MXFP4 checkpoints
// (Qwen3.5-9B-MXFP4-QAD-W4A4-LR1e-5-s3000, "Serving"; the block format of
// "How this checkpoint was produced" on Qwen3.5-27B-MXFP4-QAD-W4A4-LR1e-5-s1000)
// and the MXFP8 attention projections of
// Qwen3.8-27B-MXFP8Attn-MXFP4MLP-lmheadMXFP4 (introduction, section 2).  The
// fused variant quantizes bf16 activations per token with the CEIL rule
// inside the GEMM ("Training mode" on the 9B card).
//
// Matrix-core operand layout (32x32x64, established on gfx950 hardware):
//   lane l = r + 32 g holds row (A) / column (B) r of the 32-row fragment.
//   E2M1: its 16 bytes are K elements [32g, 32g + 32) of the 64-wide step.
//   E4M3: bytes 0..15 are K [16g, 16g + 16), bytes 16..31 are K [32 + 16g, ..).
//   Either way lane group g supplies the E8M0 scale of K block g (of 2).
//   Accumulator register i of lane l is C[(i/4)*8 + (l/32)*4 + i%4][l%32].
//
// Tiling: a workgroup of WM x WN waves computes a BM x BN tile of Y; each wave
// a (BM/WM) x (BN/WN) sub-tile of 32x32 matrix-core tiles.  K advances in
// stages of 128 elements staged through LDS (double buffered): per row a
// stage is 64 B (E2M1) or 128 B (E4M3) of codes plus 4 scale bytes.  The
// 16-byte chunks of each LDS row are XOR-swizzled by row so that the 32 lanes
// reading the same chunk of 32 consecutive rows hit distinct banks.
#include "mx_device.h"

namespace mxl {

constexpr int BK = 128;  // K elements per LDS stage

template <int BITS>
struct OpTraits {
    static constexpr int ROW_BYTES = BK * BITS / 8;    // bytes of one row per stage
    static constexpr int CHUNKS = ROW_BYTES / 16;      // 16-byte chunks per row per stage
    __device__ static constexpr int swz(int row) { return BITS == 4 ? ((row >> 1) & 3) : (row & 7); }
};

template <int OPSEL_A, int OPSEL_B, int CBSZ, int BLGP>
__device__ __forceinline__ void mfma_scaled(float16_t& acc, const int8_t_& a, const int8_t_& b, int sa, int sb)
{
    acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, acc, CBSZ, BLGP, OPSEL_A, sa, OPSEL_B, sb);
}

// Load one 32-row matrix-core fragment for K step kk (0 or 1) of the stage
// from an LDS operand tile (rows of ROW_BYTES, swizzled chunks).
template <int BITS>
__device__ __forceinline__ int8_t_ lds_fragment(const uint8_t* tile, int row, int g, int kk)
{
    using T = OpTraits<BITS>;
    int8_t_ f;
    if (BITS == 4) {
        const int c = (2 * kk + g) ^ T::swz(row);
        const int4_t v = *reinterpret_cast<const int4_t*>(tile + row * T::ROW_BYTES + c * 16);
        f[0] = v[0]; f[1] = v[1]; f[2] = v[2]; f[3] = v[3];
        f[4] = 0; f[5] = 0; f[6] = 0; f[7] = 0;
    } else {
        const int c0 = (4 * kk + g) ^ T::swz(row), c1 = (4 * kk + 2 + g) ^ T::swz(row);
        const int4_t v0 = *reinterpret_cast<const int4_t*>(tile + row * T::ROW_BYTES + c0 * 16);
        const int4_t v1 = *reinterpret_cast<const int4_t*>(tile + row * T::ROW_BYTES + c1 * 16);
        f[0] = v0[0]; f[1] = v0[1]; f[2] = v0[2]; f[3] = v0[3];
        f[4] = v1[0]; f[5] = v1[1]; f[6] = v1[2]; f[7] = v1[3];
    }
    return f;
}

struct GemmArgs {
    const uint8_t* a_q;    // [M, K*abits/8] codes (or bf16 A for the fused kernel)
    const uint8_t* a_s;    // [M, K/32] E8M0
    const uint8_t* w_q;    // [N, K*wbits/8]
    const uint8_t* w_s;    // [N, K/32]
    void* y;               // [M, N] bf16 or fp32
    int M, N, K;
};

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f)
{
    uint32_t u = __float_as_uint(f);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

// Tile ordering.  Workgroups are dispatched round-robin over the 8 XCDs
// (workgroup i runs on XCD i % 8), and each XCD has its own L2.  So the
// workgroup id is first remapped so that each XCD receives one contiguous
// range of the tile order, and the tile order itself walks groups of GROUP_N
// tile columns down M (N fastest inside a group): the tiles an XCD runs at
// the same time share a few A row panels and W column panels in its L2.
constexpr int NUM_XCD = 8;

template <int BM, int BN, int GROUP_N>
__device__ __forceinline__ void tile_coords(int M, int N, int& tm, int& tn)
{
    const int tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
    const int total = tiles_m * tiles_n;
    const int id = blockIdx.x;
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

template <int ABITS, int WBITS, int BM, int BN, int WM, int WN, bool FUSED, int A_RULE, bool OUT_F32>
__global__ __launch_bounds__(WM * WN * 64) void mx_gemm_kernel(GemmArgs p)
{
    using TA = OpTraits<ABITS>;
    using TW = OpTraits<WBITS>;
    constexpr int NT = WM * WN * 64;
    constexpr int A_TILE = BM * TA::ROW_BYTES, W_TILE = BN * TW::ROW_BYTES;
    constexpr int STAGE = A_TILE + W_TILE + 4 * (BM + BN);
    constexpr int WTM = BM / WM, WTN = BN / WN;   // wave tile
    constexpr int FM = WTM / 32, FN = WTN / 32;   // 32x32 fragments per wave
    constexpr int CBSZ = ABITS == 4 ? 4 : 0, BLGP = WBITS == 4 ? 4 : 0;
    // global -> LDS work per thread per stage
    constexpr int A_CHUNKS = FUSED ? BM * (BK * 2 / 16) : BM * TA::CHUNKS;  // fused: bf16 chunks of 8
    constexpr int W_CHUNKS = BN * TW::CHUNKS;
    constexpr int A_PER_T = (A_CHUNKS + NT - 1) / NT, W_PER_T = (W_CHUNKS + NT - 1) / NT;
    constexpr int S_ROWS = (FUSED ? 0 : BM) + BN;
    constexpr int S_PER_T = (S_ROWS + NT - 1) / NT;
    static_assert(!FUSED || (A_CHUNKS % NT == 0 && NT % 16 == 0), "fused tile mapping");

    extern __shared__ __align__(16) uint8_t smem[];

    int tm, tn;
    tile_coords<BM, BN, 4>(p.M, p.N, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave / WN, wn = wave % WN;
    const int K = p.K, KB = K / 32;
    const int a_row_bytes = FUSED ? K * 2 : K * ABITS / 8;
    const int w_row_bytes = K * WBITS / 8;
    const int nk = (K + BK - 1) / BK;

    uint4 ra[A_PER_T], rw[W_PER_T];
    uint32_t rs[S_PER_T];

    auto load_stage = [&](int kt) {
#pragma unroll
        for (int i = 0; i < A_PER_T; ++i) {
            const int q = tid + i * NT;
            const int cpr = FUSED ? 16 : TA::CHUNKS;
            const int row = q / cpr, c = q % cpr;
            const int gm = m0 + row;
            const int kb = kt * (FUSED ? BK * 2 : TA::ROW_BYTES) + c * 16;  // byte offset in the row
            ra[i] = make_uint4(0, 0, 0, 0);
            if (q < A_CHUNKS && gm < p.M && kb < a_row_bytes)
                ra[i] = *reinterpret_cast<const uint4*>(p.a_q + (size_t)gm * a_row_bytes + kb);
        }
#pragma unroll
        for (int i = 0; i < W_PER_T; ++i) {
            const int q = tid + i * NT;
            const int row = q / TW::CHUNKS, c = q % TW::CHUNKS;
            const int gn = n0 + row;
            const int kb = kt * TW::ROW_BYTES + c * 16;
            rw[i] = make_uint4(0, 0, 0, 0);
            if (q < W_CHUNKS && gn < p.N && kb < w_row_bytes)
                rw[i] = *reinterpret_cast<const uint4*>(p.w_q + (size_t)gn * w_row_bytes + kb);
        }
#pragma unroll
        for (int i = 0; i < S_PER_T; ++i) {
            const int r = tid + i * NT;
            uint32_t v = 0;
            if (r < S_ROWS) {
                const bool is_a = !FUSED && r < BM;
                const int grow = is_a ? m0 + r : n0 + (r - (FUSED ? 0 : BM));
                const int lim = is_a ? p.M : p.N;
                const uint8_t* sp = is_a ? p.a_s : p.w_s;
                if (grow < lim) {
                    if ((KB & 3) == 0) {
                        // the stage's 4 scale bytes are one aligned dword
                        v = *reinterpret_cast<const uint32_t*>(sp + (size_t)grow * KB + kt * 4);
                    } else {
#pragma unroll
                        for (int b = 0; b < 4; ++b) {
                            const int blk = kt * 4 + b;
                            if (blk < KB) v |= (uint32_t)sp[(size_t)grow * KB + blk] << (8 * b);
                        }
                    }
                }
            }
            rs[i] = v;
        }
    };

    auto store_stage = [&](int buf) {
        uint8_t* st = smem + buf * STAGE;
        uint8_t* a_t = st;
        uint8_t* w_t = st + A_TILE;
        uint32_t* sa_t = reinterpret_cast<uint32_t*>(st + A_TILE + W_TILE);
        uint32_t* sw_t = sa_t + BM;
        if (!FUSED) {
#pragma unroll
            for (int i = 0; i < A_PER_T; ++i) {
                const int q = tid + i * NT;
                if (q < A_CHUNKS) {
                    const int row = q / TA::CHUNKS, c = q % TA::CHUNKS;
                    *reinterpret_cast<uint4*>(a_t + row * TA::ROW_BYTES + ((c ^ TA::swz(row)) * 16)) = ra[i];
                }
            }
        } else {
            // quantize 8 bf16 per lane; 16 consecutive lanes hold one row's
            // 128 elements and each lane quad one block of 32
#pragma unroll
            for (int i = 0; i < A_PER_T; ++i) {
                const int q = tid + i * NT;
                const int row = q / 16, c = q % 16, blk = c / 4, part = c % 4;
                const uint32_t amax = quad_max_u32(amax_bits8(ra[i]));
                const int e = scale_exponent<ABITS == 4 ? ELEM_E2M1 : ELEM_E4M3, A_RULE>(amax);
                if (ABITS == 4) {
                    const uint32_t codes = encode8_e2m1(ra[i], e);
                    const int chunk = blk ^ TA::swz(row);
                    *reinterpret_cast<uint32_t*>(a_t + row * TA::ROW_BYTES + chunk * 16 + part * 4) = codes;
                } else {
                    const uint2 codes = encode8_e4m3(ra[i], e);
                    const int chunk = (2 * blk + part / 2) ^ TA::swz(row);
                    *reinterpret_cast<uint2*>(a_t + row * TA::ROW_BYTES + chunk * 16 + (part % 2) * 8) = codes;
                }
                if (part == 0) (reinterpret_cast<uint8_t*>(sa_t + row))[blk] = (uint8_t)(e + 127);
            }
        }
#pragma unroll
        for (int i = 0; i < W_PER_T; ++i) {
            const int q = tid + i * NT;
            if (q < W_CHUNKS) {
                const int row = q / TW::CHUNKS, c = q % TW::CHUNKS;
                *reinterpret_cast<uint4*>(w_t + row * TW::ROW_BYTES + ((c ^ TW::swz(row)) * 16)) = rw[i];
            }
        }
#pragma unroll
        for (int i = 0; i < S_PER_T; ++i) {
            const int r = tid + i * NT;
            if (r < S_ROWS) {
                if (!FUSED && r < BM) sa_t[r] = rs[i];
                else sw_t[r - (FUSED ? 0 : BM)] = rs[i];
            }
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
        const uint8_t* st = smem + buf * STAGE;
        const uint8_t* a_t = st;
        const uint8_t* w_t = st + A_TILE;
        const uint32_t* sa_t = reinterpret_cast<const uint32_t*>(st + A_TILE + W_TILE);
        const uint32_t* sw_t = sa_t + BM;
        int sa[FM], sw[FN];
#pragma unroll
        for (int i = 0; i < FM; ++i) sa[i] = (int)(sa_t[wm * WTM + i * 32 + r32] >> (8 * g));
#pragma unroll
        for (int j = 0; j < FN; ++j) sw[j] = (int)(sw_t[wn * WTN + j * 32 + r32] >> (8 * g));
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
            int8_t_ fa[FM], fw[FN];
#pragma unroll
            for (int i = 0; i < FM; ++i) fa[i] = lds_fragment<ABITS>(a_t, wm * WTM + i * 32 + r32, g, kk);
#pragma unroll
            for (int j = 0; j < FN; ++j) fw[j] = lds_fragment<WBITS>(w_t, wn * WTN + j * 32 + r32, g, kk);
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j) {
                    if (kk == 0) mfma_scaled<0, 0, CBSZ, BLGP>(acc[i][j], fa[i], fw[j], sa[i], sw[j]);
                    else mfma_scaled<2, 2, CBSZ, BLGP>(acc[i][j], fa[i], fw[j], sa[i], sw[j]);
                }
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

    // epilogue: accumulator (i, j, r) -> Y[m, n]
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) {
            const int n = n0 + wn * WTN + j * 32 + r32;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int m = m0 + wm * WTM + i * 32 + (r / 4) * 8 + g * 4 + (r % 4);
                if (m < p.M && n < p.N) {
                    if (OUT_F32) reinterpret_cast<float*>(p.y)[(size_t)m * p.N + n] = acc[i][j][r];
                    else reinterpret_cast<uint16_t*>(p.y)[(size_t)m * p.N + n] = f32_to_bf16_rne(acc[i][j][r]);
                }
            }
        }
}

template <int ABITS, int WBITS, int BM, int BN, int WM, int WN, bool FUSED, int A_RULE, bool OUT_F32>
hipError_t launch_tile(const GemmArgs& a, hipStream_t stream)
{
    using TA = OpTraits<ABITS>;
    using TW = OpTraits<WBITS>;
    constexpr int STAGE = BM * TA::ROW_BYTES + BN * TW::ROW_BYTES + 4 * (BM + BN);
    constexpr int LDS = 2 * STAGE;
    auto kern = mx_gemm_kernel<ABITS, WBITS, BM, BN, WM, WN, FUSED, A_RULE, OUT_F32>;
    static bool attr_set = false;  // benign race: setting the same value twice is harmless
    if (!attr_set) {
        hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, LDS);
        if (e != hipSuccess) return e;
        attr_set = true;
    }
    const int tiles = ((a.M + BM - 1) / BM) * ((a.N + BN - 1) / BN);
    hipLaunchKernelGGL(kern, dim3(tiles), dim3(WM * WN * 64), LDS, stream, a);
    return hipGetLastError();
}



// ---------------------------------------------------------------- decode (M <= 32)
// Weight streaming for a handful of tokens.  A workgroup owns 16 W rows and
// its 8 waves split the K steps (128 elements each) between them; every wave
// multiplies its K range on the 16x16x128 scaled matrix core (tokens padded
// to 16 rows, MT fragments for up to 16*MT tokens) and the 8 partial tiles
// are summed through LDS.  The W bytes are read exactly once, 64 contiguous
// bytes per row per step; A (at most 32 rows) stays in L2.
//   16x16x128 layout: lane l = r + 16 g holds row/column r and K block g of
//   the step (16 bytes of E2M1); the output register i of lane l is
//   C[(l/16)*4 + i][l%16].
typedef float float4_t_ __attribute__((ext_vector_type(4)));

template <int MT, bool OUT_F32>
__global__ __launch_bounds__(512) void mx_decode_kernel(GemmArgs p)
{
    constexpr int WAVES = 8, UNROLL = 4;
    __shared__ float red[WAVES][MT][64][4];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int r = lane & 15, g = lane >> 4;
    const int n0 = blockIdx.x * 16, n = n0 + r;
    const int K = p.K, KB = K / 32, row_bytes = K / 2;
    const int steps = (K + 127) / 128;
    const int s0 = wave * steps / WAVES, s1 = (wave + 1) * steps / WAVES;

    float4_t_ acc[MT];
#pragma unroll
    for (int t = 0; t < MT; ++t) acc[t] = float4_t_{0.f, 0.f, 0.f, 0.f};

    for (int sb = s0; sb < s1; sb += UNROLL) {
        int4_t wf[UNROLL], af[UNROLL][MT];
        int ws[UNROLL], as[UNROLL][MT];
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) {
            const int blk = 4 * (sb + u) + g;
            const bool ok = sb + u < s1 && blk < KB;
            wf[u] = int4_t{0, 0, 0, 0};
            ws[u] = 0;
            if (ok && n < p.N) {
                wf[u] = *reinterpret_cast<const int4_t*>(p.w_q + (size_t)n * row_bytes + blk * 16);
                ws[u] = p.w_s[(size_t)n * KB + blk];
            }
#pragma unroll
            for (int t = 0; t < MT; ++t) {
                const int m = t * 16 + r;
                af[u][t] = int4_t{0, 0, 0, 0};
                as[u][t] = 0;
                if (ok && m < p.M) {
                    af[u][t] = *reinterpret_cast<const int4_t*>(p.a_q + (size_t)m * row_bytes + blk * 16);
                    as[u][t] = p.a_s[(size_t)m * KB + blk];
                }
            }
        }
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) {
            const int8_t_ b8 = int8_t_{wf[u][0], wf[u][1], wf[u][2], wf[u][3], 0, 0, 0, 0};
#pragma unroll
            for (int t = 0; t < MT; ++t) {
                const int8_t_ a8 = int8_t_{af[u][t][0], af[u][t][1], af[u][t][2], af[u][t][3], 0, 0, 0, 0};
                acc[t] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a8, b8, acc[t], 4, 4, 0, as[u][t], 0, ws[u]);
            }
        }
    }
#pragma unroll
    for (int t = 0; t < MT; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) red[wave][t][lane][i] = acc[t][i];
    __syncthreads();
    // one output element per thread: (t, lane, i) -> m = 16 t + (lane/16)*4 + i, n = n0 + lane%16
    for (int e = tid; e < MT * 64 * 4; e += WAVES * 64) {
        const int t = e / 256, l = (e / 4) % 64, i = e % 4;
        float v = 0.f;
#pragma unroll
        for (int w = 0; w < WAVES; ++w) v += red[w][t][l][i];
        const int m = t * 16 + (l / 16) * 4 + i, nn = n0 + l % 16;
        if (m < p.M && nn < p.N) {
            if (OUT_F32) reinterpret_cast<float*>(p.y)[(size_t)m * p.N + nn] = v;
            else reinterpret_cast<uint16_t*>(p.y)[(size_t)m * p.N + nn] = f32_to_bf16_rne(v);
        }
    }
}

template <int MT, bool OUT_F32>
hipError_t launch_decode(const GemmArgs& a, hipStream_t stream)
{
    hipLaunchKernelGGL((mx_decode_kernel<MT, OUT_F32>), dim3((a.N + 15) / 16), dim3(512), 0, stream, a);
    return hipGetLastError();
}

} // namespace mxl

using namespace mxl;

// ---------------------------------------------------------------- dispatch
// Shape classes (MXFP4 and fast-path MXFP8):
//   decode  : M <= 32 (MXFP4)                     -> mx_decode_kernel
//   large   : MXFP4, M >= 1024 and N >= 1024       -> 256x256 tiles, 2x2 waves of 128x128
//             (the E4M3 fragments are twice as wide and would spill there)
//   default : everything else                      -> 128x128 tiles, 2x2 waves of 64x64
enum ShapeClass { SC_DECODE, SC_LARGE, SC_DEFAULT };

static ShapeClass classify(int a_bits, int64_t m, int64_t n, bool fused)
{
    if (!fused && a_bits == 4 && m <= 32) return SC_DECODE;
    if (a_bits == 4 && m >= 1024 && n >= 1024) return SC_LARGE;
    return SC_DEFAULT;
}

template <int AB, int WB, bool FUSED, int RULE, bool F32>
static hipError_t dispatch_tile(const GemmArgs& a, ShapeClass sc, hipStream_t s)
{
    if (AB == 4 && sc == SC_LARGE) return launch_tile<AB, WB, 256, 256, 2, 2, FUSED, RULE, F32>(a, s);
    return launch_tile<AB, WB, 128, 128, 2, 2, FUSED, RULE, F32>(a, s);
}

template <int AB, int WB, bool FUSED, int RULE>
static hipError_t dispatch_out(const GemmArgs& a, ShapeClass sc, bool f32, hipStream_t s)
{
    if (f32) return dispatch_tile<AB, WB, FUSED, RULE, true>(a, sc, s);
    return dispatch_tile<AB, WB, FUSED, RULE, false>(a, sc, s);
}

extern "C" hipError_t mxl_launch_mx_gemm(int a_bits, int w_bits, const void* aq, const void* as,
                                         const void* wq, const void* ws, int64_t m, int64_t n,
                                         int64_t k, void* y, int out_f32, hipStream_t stream)
{
    GemmArgs a{static_cast<const uint8_t*>(aq), static_cast<const uint8_t*>(as),
               static_cast<const uint8_t*>(wq), static_cast<const uint8_t*>(ws), y, (int)m, (int)n, (int)k};
    const ShapeClass sc = classify(a_bits, m, n, false);
    if (sc == SC_DECODE) {
        if (m <= 16) return out_f32 ? launch_decode<1, true>(a, stream) : launch_decode<1, false>(a, stream);
        return out_f32 ? launch_decode<2, true>(a, stream) : launch_decode<2, false>(a, stream);
    }
    if (a_bits == 4 && w_bits == 4) return dispatch_out<4, 4, false, RULE_CEIL>(a, sc, out_f32, stream);
    if (a_bits == 8 && w_bits == 8) return dispatch_out<8, 8, false, RULE_CEIL>(a, sc, out_f32, stream);
    return hipErrorInvalidValue;
}

extern "C" hipError_t mxl_launch_mx_gemm_fused(int a_bits, int a_rule, const void* a_bf16, int w_bits,
                                               const void* wq, const void* ws, int64_t m, int64_t n,
                                               int64_t k, void* y, int out_f32, hipStream_t stream)
{
    GemmArgs a{static_cast<const uint8_t*>(a_bf16), nullptr, static_cast<const uint8_t*>(wq),
               static_cast<const uint8_t*>(ws), y, (int)m, (int)n, (int)k};
    const ShapeClass sc = classify(a_bits, m, n, true);
    if (a_bits == 4 && w_bits == 4) {
        if (a_rule == RULE_CEIL) return dispatch_out<4, 4, true, RULE_CEIL>(a, sc, out_f32, stream);
        if (a_rule == RULE_FLOOR) return dispatch_out<4, 4, true, RULE_FLOOR>(a, sc, out_f32, stream);
        return dispatch_out<4, 4, true, RULE_EVEN>(a, sc, out_f32, stream);
    }
    if (a_bits == 8 && w_bits == 8) {
        if (a_rule == RULE_CEIL) return dispatch_out<8, 8, true, RULE_CEIL>(a, sc, out_f32, stream);
        if (a_rule == RULE_FLOOR) return dispatch_out<8, 8, true, RULE_FLOOR>(a, sc, out_f32, stream);
        return dispatch_out<8, 8, true, RULE_EVEN>(a, sc, out_f32, stream);
    }
    return hipErrorInvalidValue;
}

extern "C" const char* mxl_mx_gemm_config_name(int a_bits, int64_t m, int64_t n, int fused)
{
    switch (classify(a_bits, m, n, fused != 0)) {
    case SC_DECODE:
        return "mx_decode_kernel<16 W rows per workgroup, 8-wave split-K, scaled mfma 16x16x128>";
    case SC_LARGE:
        return "mx_gemm_kernel<tile 256x256x128, 2x2 waves of 128x128, scaled mfma 32x32x64>";
    default:
        return "mx_gemm_kernel<tile 128x128x128, 2x2 waves of 64x64, scaled mfma 32x32x64>";
    }
}
