// gemm_prefill.hip -- the large-shape MXFP4 GEMM for gfx950:
//   Y[M, N] = A[M, K] * W[N, K]^T, E2M1 codes with an E8M0 scale per 32 along
//   K, fp32 accumulation on v_mfma_scale_f32_32x32x64_f8f6f4, bf16/fp32 output.
//
// Operation: the W4A4 FP4 GEMM that serves the MXFP4 checkpoints
// (Qwen3.5-9B-MXFP4-QAD-W4A4-LR1e-5-s3000, "Serving"), for prefill-sized M.
//
// Design (one 256x256 output tile per workgroup of 4 waves, each wave a
// 128x128 sub-tile of 4x4 matrix-core fragments held in 256 AGPRs):
//  * K advances in stages of 128 elements.  A stage is 16 KiB of A codes,
//    16 KiB of W codes and 2 x 1 KiB of scales, and lives in one slot of a
//    4-slot LDS ring (136 KiB), three stages ahead of the one being computed.
//  * Stages are copied global -> LDS by the buffer-load-to-LDS path (each
//    instruction writes 64 lanes x 16 B contiguously at the address in M0).
//    No registers are spent on staging and no LDS write instructions are
//    issued.  The swizzled LDS layout is obtained by choosing, per lane, which
//    global 16-byte chunk lands at that lane's LDS position.  Rows past the
//    end of A or W read as zero (buffer range check).
//  * These copies are issued from inline assembly, so the compiler does not
//    track them; every wave waits for its own copies of stage kt with an
//    explicit vmcnt before the workgroup barrier that publishes the stage.
//    Each wave issues exactly 10 copies per stage, so the count of copies
//    still allowed in flight is 10 per later stage.
//  * W is the matrix core's first operand, A the second, so each lane's
//    accumulator holds 4 consecutive output columns; the epilogue stages each
//    32-row band of a wave's tile through LDS and writes whole 256-byte row
//    segments to Y.
//  * Matrix-core layout (32x32x64, E2M1): lane l = r + 32 g holds row r of a
//    fragment and K elements [32 g, 32 g + 32) of the 64-wide step; lane
//    group g supplies the E8M0 scale of K block g.  Accumulator register i of
//    lane l is C[(i/4)*8 + g*4 + i%4][r] with C = W_frag x A_frag^T.
//  * Tile order: XCD-aware grouped order (tile_coords in mx_device.h).
// Requires K % 128 == 0 (whole stages, aligned scale dwords); other shapes
// use the general tile kernel.
#include "mx_device.h"

namespace mxl {

constexpr int PF_BM = 256, PF_BN = 256, PF_BK = 128, PF_NS = 4;
constexpr int PF_ROWB = PF_BK / 2;                 // E2M1 bytes of a row per stage
constexpr int PF_TILE = PF_BM * PF_ROWB;           // 16 KiB per operand per stage
constexpr int PF_SCALE = PF_BM * 4;                // 1 KiB of scales per operand per stage
constexpr int PF_SLOT = 2 * PF_TILE + 2 * PF_SCALE;
constexpr int PF_LDS = PF_NS * PF_SLOT;            // 139264 bytes
constexpr int PF_COPIES = 10;                      // copies per wave per stage

struct PrefillArgs {
    const uint8_t* a_q; const uint8_t* a_s;
    const uint8_t* w_q; const uint8_t* w_s;
    void* y;
    int M, N, K;
};

// 16-byte chunk swizzle of the 64-byte LDS rows: the 32 lanes reading the
// same logical chunk of 32 consecutive rows touch distinct banks.
__device__ __forceinline__ int pf_swz(int row) { return (row >> 1) & 3; }

__device__ __forceinline__ void dma_b128(uint32_t lds, int voff, const int4_t& rsrc, int soff)
{
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
                 :: "s"(lds), "v"(voff), "s"(rsrc), "s"(soff) : "memory");
}
__device__ __forceinline__ void dma_b32(uint32_t lds, int voff, const int4_t& rsrc, int soff)
{
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dword %1, %2, %3 offen lds"
                 :: "s"(lds), "v"(voff), "s"(rsrc), "s"(soff) : "memory");
}
template <int N>
__device__ __forceinline__ void wait_vmcnt()
{
    static_assert(N >= 0 && N <= 63, "vmcnt range");
    asm volatile("s_waitcnt vmcnt(%0)" :: "n"(N) : "memory");
}

__device__ __forceinline__ int4_t make_rsrc(const void* base, uint32_t bytes)
{
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, (int)bytes, 0x00020000);
    int4_t v;
    __builtin_memcpy(&v, &r, 16);
    // uniform by construction; make that explicit so it lives in SGPRs
    v[0] = __builtin_amdgcn_readfirstlane(v[0]);
    v[1] = __builtin_amdgcn_readfirstlane(v[1]);
    v[2] = __builtin_amdgcn_readfirstlane(v[2]);
    v[3] = __builtin_amdgcn_readfirstlane(v[3]);
    return v;
}

template <bool OUT_F32>
__global__ __launch_bounds__(256, 1) void mx_gemm_prefill_kernel(PrefillArgs p)
{
    extern __shared__ __align__(16) uint8_t smem[];

    int tm, tn;
    tile_coords<PF_BM, PF_BN, 4>(p.M, p.N, tm, tn);
    const int m0 = tm * PF_BM, n0 = tn * PF_BN;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: feeds M0
    const int wm = wave >> 1, wn = wave & 1;
    const int r32 = lane & 31, g = lane >> 5;
    const int K = p.K, KB = K / 32, row_bytes = K / 2;
    const int nk = K / PF_BK;

    const int4_t rsrc_a = make_rsrc(p.a_q, (uint32_t)p.M * row_bytes);
    const int4_t rsrc_w = make_rsrc(p.w_q, (uint32_t)p.N * row_bytes);
    const int4_t rsrc_as = make_rsrc(p.a_s, (uint32_t)p.M * KB);
    const int4_t rsrc_ws = make_rsrc(p.w_s, (uint32_t)p.N * KB);
    const uint32_t lds0 = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)smem);

    // Per-lane source offsets.  Wave w copies code segments 4w .. 4w+3 of each
    // operand (a segment is 16 rows x 64 B = 1 KiB of LDS); LDS position L of
    // a segment is row 16*seg + L/4, physical chunk L%4, which holds logical
    // chunk (L%4) ^ swz(row).  Scale segment w holds dwords 64w .. 64w+63 of
    // the stage's scale area, ordered (row group of 128, r, fragment i): dword
    // p is tile row (p/128)*128 + (p%4)*32 + (p/4)%32.
    int a_voff[4], w_voff[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        const int row = 16 * (4 * wave + s) + lane / 4;
        const int c = (lane & 3) ^ pf_swz(row);
        a_voff[s] = (m0 + row) * row_bytes + c * 16;
        w_voff[s] = (n0 + row) * row_bytes + c * 16;
    }
    int as_voff, ws_voff;
    {
        const int pidx = 64 * wave + lane;
        const int row = (pidx / 128) * 128 + (pidx % 4) * 32 + (pidx / 4) % 32;
        as_voff = (m0 + row) * KB;
        ws_voff = (n0 + row) * KB;
    }

    auto issue_stage = [&](int kt) {
        const uint32_t slot = lds0 + (uint32_t)((kt % PF_NS) * PF_SLOT);
        const int soff_codes = kt * PF_ROWB, soff_scales = kt * 4;
#pragma unroll
        for (int s = 0; s < 4; ++s) dma_b128(slot + (4 * wave + s) * 1024, a_voff[s], rsrc_a, soff_codes);
#pragma unroll
        for (int s = 0; s < 4; ++s) dma_b128(slot + PF_TILE + (4 * wave + s) * 1024, w_voff[s], rsrc_w, soff_codes);
        dma_b32(slot + 2 * PF_TILE + wave * 256, as_voff, rsrc_as, soff_scales);
        dma_b32(slot + 2 * PF_TILE + PF_SCALE + wave * 256, ws_voff, rsrc_ws, soff_scales);
    };

    float16_t acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    auto compute_stage = [&](int kt) {
        const uint8_t* slot = smem + (kt % PF_NS) * PF_SLOT;
        const uint8_t* a_t = slot;
        const uint8_t* w_t = slot + PF_TILE;
        // this lane's 4 scale dwords per operand (fragments i = 0..3), shifted so
        // that byte 2*kk selects K block 2*kk + g
        const int4_t sa4 = *reinterpret_cast<const int4_t*>(slot + 2 * PF_TILE + (wm * 128 + r32 * 4) * 4);
        const int4_t sw4 = *reinterpret_cast<const int4_t*>(slot + 2 * PF_TILE + PF_SCALE + (wn * 128 + r32 * 4) * 4);
        int sa[4], sw[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            sa[i] = (int)((uint32_t)sa4[i] >> (8 * g));
            sw[i] = (int)((uint32_t)sw4[i] >> (8 * g));
        }
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
            int4_t fa[4], fw[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int row = wm * 128 + i * 32 + r32;
                fa[i] = *reinterpret_cast<const int4_t*>(a_t + row * PF_ROWB + (((2 * kk + g) ^ pf_swz(row)) * 16));
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int row = wn * 128 + j * 32 + r32;
                fw[j] = *reinterpret_cast<const int4_t*>(w_t + row * PF_ROWB + (((2 * kk + g) ^ pf_swz(row)) * 16));
            }
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int8_t_ b8 = int8_t_{fw[j][0], fw[j][1], fw[j][2], fw[j][3], 0, 0, 0, 0};
                    const int8_t_ a8 = int8_t_{fa[i][0], fa[i][1], fa[i][2], fa[i][3], 0, 0, 0, 0};
                    if (kk == 0)
                        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(b8, a8, acc[i][j], 4, 4, 0, sw[j], 0, sa[i]);
                    else
                        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(b8, a8, acc[i][j], 4, 4, 2, sw[j], 2, sa[i]);
                }
        }
    };

    // prologue: three stages in flight
#pragma unroll
    for (int s = 0; s < PF_NS - 1; ++s)
        if (s < nk) issue_stage(s);

    for (int kt = 0; kt < nk; ++kt) {
        // wait for this wave's copies of stage kt (later stages may stay in flight)
        const int later = nk - 1 - kt;
        if (later >= 2) wait_vmcnt<2 * PF_COPIES>();
        else if (later == 1) wait_vmcnt<PF_COPIES>();
        else wait_vmcnt<0>();
        lds_barrier();  // stage kt is in LDS for every wave; slot of stage kt-1 is free
        if (kt + PF_NS - 1 < nk) issue_stage(kt + PF_NS - 1);
        compute_stage(kt);
    }
    lds_barrier();  // all waves are done reading the ring

    // Epilogue, one 32-row band (fragment row i) at a time through this
    // wave's private LDS region: write the band row-major, read it back as
    // whole row segments and store them with 16-byte stores.
    constexpr int ESZ = OUT_F32 ? 4 : 2;
    constexpr int ROWB = 128 * ESZ + 16;                 // padded LDS row
    uint8_t* region = smem + wave * (32 * ROWB);
    const bool vec_ok = (p.N % (16 / ESZ)) == 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int col = j * 32 + q * 8 + g * 4;
                uint8_t* dst = region + r32 * ROWB + col * ESZ;
                if (OUT_F32) {
                    *reinterpret_cast<float4_t*>(dst) =
                        float4_t{acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]};
                } else {
                    const uint32_t lo = (uint32_t)f32_to_bf16_rne(acc[i][j][4 * q]) |
                                        ((uint32_t)f32_to_bf16_rne(acc[i][j][4 * q + 1]) << 16);
                    const uint32_t hi = (uint32_t)f32_to_bf16_rne(acc[i][j][4 * q + 2]) |
                                        ((uint32_t)f32_to_bf16_rne(acc[i][j][4 * q + 3]) << 16);
                    *reinterpret_cast<uint2*>(dst) = make_uint2(lo, hi);
                }
            }
        constexpr int LPR = 128 * ESZ / 16;               // lanes per 16-byte-chunked row
        constexpr int RPI = 64 / LPR;                      // rows per read instruction
#pragma unroll
        for (int t = 0; t < 32 / RPI; ++t) {
            const int row = t * RPI + lane / LPR, c16 = lane % LPR;
            const uint4 v = *reinterpret_cast<const uint4*>(region + row * ROWB + c16 * 16);
            const int m = m0 + wm * 128 + i * 32 + row;
            const int n = n0 + wn * 128 + c16 * (16 / ESZ);
            if (m < p.M) {
                uint8_t* yrow = reinterpret_cast<uint8_t*>(p.y) + ((size_t)m * p.N) * ESZ;
                if (vec_ok && n + 16 / ESZ <= p.N) {
                    const int4_t iv = int4_t{(int)v.x, (int)v.y, (int)v.z, (int)v.w};
                    __builtin_nontemporal_store(iv, reinterpret_cast<int4_t*>(yrow + (size_t)n * ESZ));
                } else {
                    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
                    for (int e = 0; e < 16 / ESZ; ++e) {
                        if (n + e < p.N) {
                            if (OUT_F32) reinterpret_cast<uint32_t*>(yrow)[n + e] = w[e];
                            else reinterpret_cast<uint16_t*>(yrow)[n + e] = (uint16_t)(w[e / 2] >> (16 * (e % 2)));
                        }
                    }
                }
            }
        }
    }
}

template <bool OUT_F32>
hipError_t launch_prefill(const PrefillArgs& a, hipStream_t stream)
{
    auto kern = mx_gemm_prefill_kernel<OUT_F32>;
    static bool attr_set = false;
    if (!attr_set) {
        hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, PF_LDS);
        if (e != hipSuccess) return e;
        attr_set = true;
    }
    const int tiles = ((a.M + PF_BM - 1) / PF_BM) * ((a.N + PF_BN - 1) / PF_BN);
    hipLaunchKernelGGL(kern, dim3(tiles), dim3(256), PF_LDS, stream, a);
    return hipGetLastError();
}

} // namespace mxl

using namespace mxl;

// Shapes this kernel accepts: K % 128 == 0 and every operand below 2 GiB
// (32-bit buffer offsets).  The caller checks them (mxl_prefill_ok).
extern "C" int mxl_prefill_ok(int64_t m, int64_t n, int64_t k)
{
    if (k % PF_BK != 0) return 0;
    const int64_t lim = ((int64_t)1 << 31) - (int64_t)PF_BM * (k / 2) - 1024;
    return (m + PF_BM) * (k / 2) < lim && (n + PF_BN) * (k / 2) < lim ? 1 : 0;
}

extern "C" hipError_t mxl_launch_mx_prefill(const void* aq, const void* as, const void* wq, const void* ws,
                                            int64_t m, int64_t n, int64_t k, void* y, int out_f32,
                                            hipStream_t stream)
{
    PrefillArgs a{static_cast<const uint8_t*>(aq), static_cast<const uint8_t*>(as),
                  static_cast<const uint8_t*>(wq), static_cast<const uint8_t*>(ws), y, (int)m, (int)n, (int)k};
    return out_f32 ? launch_prefill<true>(a, stream) : launch_prefill<false>(a, stream);
}
