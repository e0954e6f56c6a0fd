// gemm_prefill.hip -- the large-shape MXFP4 GEMM for gfx950:
//   Y[M, N] = A[M, K] * W[N, K]^T, E2M1 codes with an E8M0 scale per 32 along
//   K, fp32 accumulation on v_mfma_scale_f32_32x32x64_f8f6f4, bf16/fp32 output.
//
// Operation: the W4A4 FP4 GEMM that serves the MXFP4 checkpoints
// (Qwen3.5-9B-MXFP4-QAD-W4A4-LR1e-5-s3000, "Serving"), for prefill-sized M.
//
// Design (one 256x256 output tile per workgroup of 4 waves, each wave a
// 128x128 sub-tile of 4x4 matrix-core fragments held in 256 AGPRs):
//  * K advances in stages of 128 elements.  A stage's codes (16 KiB of A, 16
//    KiB of W) live in one slot of a 3-slot LDS ring.  The E8M0 scales travel
//    separately, in windows of 8 stages (32 bytes per row per operand, 16 KiB
//    per window) held in a 3-window LDS ring: fetching 4 scale bytes per row
//    per stage would cost one 64-row gather per 256 bytes, which measured as
//    the dominant cost of the loop; a window fetch moves 32 contiguous bytes
//    per row.
//  * Everything is copied global -> LDS by the buffer-load-to-LDS path (each
//    instruction writes 64 lanes x its width contiguously at the address in
//    M0), so no registers are spent on staging.  The swizzled code layout is
//    obtained by choosing, per lane, which global 16-byte chunk lands at that
//    lane's LDS position.  Rows past the end of A or W read as zero (buffer
//    range check); copies past the last stage use a zero-sized buffer and
//    fill a free slot with zeros, which keeps the loop free of branches and
//    the outstanding-copy count the same every stage.
//  * Each wave issues 10 copies per stage: 2 scale pieces (8 rows x 32 B each)
//    of the window after next, then 8 code copies (16 rows x 64 B each) of
//    the stage three ahead.  A wave waits for its own copies with an explicit
//    vmcnt (the copies come from inline assembly the compiler does not
//    track), then a workgroup barrier publishes them.
//  * The fragments of stage s+1 (16 code reads, 8 scale reads per lane) are
//    read from LDS while the 32 matrix-core instructions of stage s run, into
//    a second register set, so no LDS latency is exposed; the loop is
//    unrolled by two to alternate the sets without copies.  Reads, copies and
//    matrix-core instructions are pinned in place with scheduling barriers.
//  * W is the matrix core's first operand, A the second, so each lane's
//    accumulator holds 4 consecutive output columns; the epilogue stages each
//    32-row band of a wave's tile through LDS and writes whole 256-byte row
//    segments to Y.
//  * Matrix-core layout (32x32x64, E2M1): lane l = r + 32 g holds row r of a
//    fragment and K elements [32 g, 32 g + 32) of the 64-wide step; lane
//    group g supplies the E8M0 scale of K block g.  Accumulator register i of
//    lane l is C[(i/4)*8 + g*4 + i%4][r] with C = W_frag x A_frag^T.
//  * Tile order: XCD-aware grouped order (tile_coords in mx_device.h).
// Requires K % 128 == 0 (whole stages); other shapes use the general tile
// kernel.
#include "mx_device.h"

namespace mxl {

constexpr int PF_BM = 256, PF_BN = 256, PF_BK = 128;
constexpr int PF_ROWB = PF_BK / 2;                 // E2M1 bytes of a row per stage
constexpr int PF_TILE = PF_BM * PF_ROWB;           // 16 KiB per operand per stage
constexpr int PF_NS = 3;                           // code slots; copies run PF_NS stages ahead
constexpr int PF_SLOT = 2 * PF_TILE;               // A codes, then W codes
constexpr int PF_SWS = 8;                          // stages per scale window
constexpr int PF_SWB = PF_SWS * 4;                 // scale bytes per row per window
constexpr int PF_WIN = 2 * PF_BM * PF_SWB;         // A scales [256][32 B], then W scales
constexpr int PF_NWIN = 3;
constexpr int PF_SC0 = PF_NS * PF_SLOT;            // the scale windows follow the code ring
constexpr int PF_LDS = PF_SC0 + PF_NWIN * PF_WIN;  // 147456 bytes
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

// one stage's operands in registers: code fragments per 64-wide step kk, and
// the raw scale dwords (4 blocks of the stage) of this lane's fragment rows
struct PfFrags {
    int4_t a[2][4], w[2][4];
    int sa[4], sw[4];
};

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

    // Code copies: wave w copies segments 4w .. 4w+3 (16 rows x 64 B = 1 KiB
    // of LDS each) of each operand.  LDS position L of a segment is row
    // 16*seg + L/4, physical chunk L%4, which holds logical chunk
    // (L%4) ^ swz(row).
    int a_voff[4], w_voff[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        const int row = 16 * (4 * wave + s) + lane / 4;
        const int c = (lane & 3) ^ pf_swz(row);
        a_voff[s] = (m0 + row) * row_bytes + c * 16;
        w_voff[s] = (n0 + row) * row_bytes + c * 16;
    }
    // Scale pieces: piece j (0..7) of a window is copy t = 4 j + wave of each
    // operand, rows 8t .. 8t+7 of the tile, 32 bytes each ([row][32 B] in LDS).
    // The window offset is part of the per-lane offset so that the buffer
    // range check covers it (a partial last window may run past a row).
    const int srow = lane >> 3, sdw = lane & 7;
    auto sc_voff = [&](int base, int j, int win) {
        return (base + 8 * (4 * j + wave) + srow) * KB + win * PF_SWB + sdw * 4;
    };

    // Copy c (0..9) of virtual stage y: c = 0, 1 are the A and W pieces
    // (y + 4) % 8 of scale window (y + 4) / 8 + 1; c = 2..9 are the code
    // copies of stage y + PF_NS.  Stage y + PF_NS goes to the slot of stage y,
    // whose fragments were read during stage y - 1.  A window's pieces are
    // issued during the 8 stages that end four stages before its first stage
    // is read, into the buffer of the window three back.
    auto copy = [&](int y, int c) {
        if (c < 2) {
            const int win = ((y + 4) >> 3) + 1, j = (y + 4) & 7;
            const int live = __builtin_amdgcn_readfirstlane(win * PF_SWS < nk ? 1 : 0);
            int4_t r = c == 0 ? rsrc_as : rsrc_ws;
            r[2] = live ? r[2] : 0;
            const uint32_t dst = lds0 + PF_SC0 + (uint32_t)((win % PF_NWIN) * PF_WIN) + (4 * j + wave) * 256 +
                                 c * PF_BM * PF_SWB;
            dma_b32(dst, sc_voff(c == 0 ? m0 : n0, j, win), r, 0);
        } else {
            const int ks = y + PF_NS;
            const int live = __builtin_amdgcn_readfirstlane(ks < nk ? 1 : 0);
            const int s = (c - 2) & 3;
            int4_t r = c < 6 ? rsrc_a : rsrc_w;
            r[2] = live ? r[2] : 0;
            const uint32_t dst = lds0 + (uint32_t)((ks % PF_NS) * PF_SLOT) + (c < 6 ? 0 : PF_TILE) + (4 * wave + s) * 1024;
            dma_b128(dst, c < 6 ? a_voff[s] : w_voff[s], r, ks * PF_ROWB);
        }
    };

    // LDS read q (0..23) of stage s: 16 code fragments, then 8 scale dwords
    auto read_piece = [&](int s, int q, PfFrags& f) {
        if (q < 16) {
            const uint8_t* slot = smem + (s % PF_NS) * PF_SLOT;
            const int kk = q >> 3, x = q & 7;
            if (x < 4) {
                const int row = wm * 128 + x * 32 + r32;
                f.a[kk][x] = *reinterpret_cast<const int4_t*>(slot + row * PF_ROWB + (((2 * kk + g) ^ pf_swz(row)) * 16));
            } else {
                const int row = wn * 128 + (x - 4) * 32 + r32;
                f.w[kk][x - 4] =
                    *reinterpret_cast<const int4_t*>(slot + PF_TILE + row * PF_ROWB + (((2 * kk + g) ^ pf_swz(row)) * 16));
            }
        } else {
            const uint8_t* win = smem + PF_SC0 + ((s / PF_SWS) % PF_NWIN) * PF_WIN + (s % PF_SWS) * 4;
            const int x = q - 16;
            if (x < 4) {
                const int row = wm * 128 + x * 32 + r32;
                f.sa[x] = (int)*reinterpret_cast<const uint32_t*>(win + row * PF_SWB);
            } else {
                const int row = wn * 128 + (x - 4) * 32 + r32;
                f.sw[x - 4] = (int)*reinterpret_cast<const uint32_t*>(win + PF_BM * PF_SWB + row * PF_SWB);
            }
        }
    };

    float16_t acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    // matrix-core instruction q (0..31) of a stage: step kk = q / 16, fragment (i, j)
    auto mfma = [&](int q, const PfFrags& f, const int* sa, const int* sw) {
        const int kk = q >> 4, i = (q >> 2) & 3, j = q & 3;
        const int8_t_ b8 = int8_t_{f.w[kk][j][0], f.w[kk][j][1], f.w[kk][j][2], f.w[kk][j][3], 0, 0, 0, 0};
        const int8_t_ a8 = int8_t_{f.a[kk][i][0], f.a[kk][i][1], f.a[kk][i][2], f.a[kk][i][3], 0, 0, 0, 0};
        if (kk == 0)
            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(b8, a8, acc[i][j], 4, 4, 0, sw[j], 0, sa[i]);
        else
            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(b8, a8, acc[i][j], 4, 4, 2, sw[j], 2, sa[i]);
    };

    // Stage s: computed from `cur`; stage s + 1 is read into `nxt`; virtual
    // stage s issues its copies.
    auto stage = [&](int s, const PfFrags& cur, PfFrags& nxt) {
        // The copies of stage s + 1 were issued two stages ago; only the 10 of
        // the previous stage may still be in flight.
        wait_vmcnt<PF_COPIES>();
        lds_barrier();
        // byte 2 kk + g of a scale dword is this lane's block; after the shift
        // it sits at byte 2 kk, which the instruction's op_sel picks
        int sa[4], sw[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            sa[i] = (int)((uint32_t)cur.sa[i] >> (8 * g));
            sw[i] = (int)((uint32_t)cur.sw[i] >> (8 * g));
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int q = 0; q < 32; ++q) {
            mfma(q, cur, sa, sw);
            if (q < 24) {
                __builtin_amdgcn_sched_barrier(0);
                read_piece(s + 1, q, nxt);
                __builtin_amdgcn_sched_barrier(0);
            }
            if ((q % 3) == 1 && q / 3 < PF_COPIES) {
                __builtin_amdgcn_sched_barrier(0);
                copy(s, q / 3);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        __builtin_amdgcn_sched_barrier(0);
    };

    // Prologue: all of window 0, then virtual stages -4 .. -1 (window 1's
    // pieces 0..3 and the codes of stages 0..2).
#pragma unroll
    for (int j = 0; j < PF_SWS; ++j) {
        const uint32_t dst = lds0 + PF_SC0 + (4 * j + wave) * 256;
        dma_b32(dst, sc_voff(m0, j, 0), rsrc_as, 0);
        dma_b32(dst + PF_BM * PF_SWB, sc_voff(n0, j, 0), rsrc_ws, 0);
    }
    copy(-4, 0);
    copy(-4, 1);
    for (int y = -3; y < 0; ++y)
#pragma unroll
        for (int c = 0; c < PF_COPIES; ++c) copy(y, c);
    wait_vmcnt<2 * PF_COPIES>();  // window 0 and stage 0 have landed
    lds_barrier();
    PfFrags X, Y;
#pragma unroll
    for (int q = 0; q < 24; ++q) read_piece(0, q, X);

    int s = 0;
    for (; s + 1 < nk; s += 2) {
        stage(s, X, Y);
        stage(s + 1, Y, X);
    }
    if (s < nk) stage(s, X, Y);
    wait_vmcnt<0>();   // the trailing zero-fill copies have landed
    lds_barrier();     // every wave is done with the rings

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
                    const uint32_t lo = bf16x2_rne(acc[i][j][4 * q], acc[i][j][4 * q + 1]);
                    const uint32_t hi = bf16x2_rne(acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]);
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
#pragma unroll
                    for (int e = 0; e < 16 / ESZ; ++e) {
                        const int wi = OUT_F32 ? e : e / 2;
                        const uint32_t word = wi == 0 ? v.x : wi == 1 ? v.y : wi == 2 ? v.z : v.w;
                        if (n + e < p.N) {
                            if (OUT_F32) reinterpret_cast<uint32_t*>(yrow)[n + e] = word;
                            else reinterpret_cast<uint16_t*>(yrow)[n + e] = (uint16_t)(word >> (16 * (e % 2)));
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
