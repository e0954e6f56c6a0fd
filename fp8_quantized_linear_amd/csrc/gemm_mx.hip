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
//   Accumulator register i of lane l is C[(i/4)*8 + (l/32)*4 + i%4][l%32]
//   (C = first operand x second operand^T; the tile kernel passes W first).
//
// Tiling: a workgroup of WM x WN waves computes a BM x BN tile of Y; each wave
// a (BM/WM) x (BN/WN) sub-tile of 32x32 matrix-core tiles.  K advances in
// stages of 128 elements staged through LDS (double buffered): per row a
// stage is 64 B (E2M1) or 128 B (E4M3) of codes plus 4 scale bytes.  The
// 16-byte chunks of each LDS row are XOR-swizzled by row so that the 32 lanes
// reading the same chunk of 32 consecutive rows hit distinct banks.
#include "mx_device.h"

#include <cstdio>
#include <type_traits>

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

// Scaled MFMA with byte selectors chosen at run time; after unrolling the
// selectors are constants and the branches fold away.
template <int CBSZ, int BLGP>
__device__ __forceinline__ void mfma_scaled_sel(float16_t& acc, const int8_t_& a, const int8_t_& b, int sa,
                                                int sb, int pa, int pb)
{
#define MXL_MF(OA, OB) acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, acc, CBSZ, BLGP, OA, sa, OB, sb)
#define MXL_ROW(OA)                  \
    if (pb == 0) MXL_MF(OA, 0);      \
    else if (pb == 1) MXL_MF(OA, 1); \
    else if (pb == 2) MXL_MF(OA, 2); \
    else MXL_MF(OA, 3);
    if (pa == 0) { MXL_ROW(0) }
    else if (pa == 1) { MXL_ROW(1) }
    else if (pa == 2) { MXL_ROW(2) }
    else { MXL_ROW(3) }
#undef MXL_ROW
#undef MXL_MF
}

// LDS layout of a stage's E8M0 scales.  Lane (r, g) of a wave needs, for
// fragment i of its wave tile and K step kk, the byte of K block 2*kk + g of
// its row.  Each tile row therefore stores two 16-bit entries,
//   entry g = byte g | byte (g + 2) << 8,
// placed so that one lane's entries for its F = WT/32 fragments are adjacent:
// entry index ((wave_row_group * 32 + r) * 2 + g) * F + i.  One 4-byte (F = 2)
// or 8-byte (F = 4) LDS read then gives a lane all its scales for the stage,
// and the scale operand's byte selector picks 2 * (i % 2) + kk.
template <int WT>
__device__ __forceinline__ int scale_entry(int r, int g)
{
    constexpr int F = WT / 32;
    return (((r / WT) * 32 + (r % 32)) * 2 + g) * F + (r % WT) / 32;
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
    // split-K: workgroup b computes K stages [s * chunk, (s + 1) * chunk) of
    // tile b % tiles for s = b / tiles; with splits > 1 it writes its fp32
    // partial tile to part + s * M * N and splitk_reduce_kernel sums them
    float* part;
    int splits, chunk;
    // fused kernel only, optional: the prologue's A codes [M, K*abits/8] and
    // E8M0 scales [M, K/32], written by the tiles of the first tile column
    uint8_t* dump_q;
    uint8_t* dump_s;
};


// PREFETCH = 2 keeps two K stages in flight in registers (the loop is
// unrolled by two so that the register sets swap roles statically and the
// compiler waits only for the stage being written to LDS); 1 keeps one.
template <int ABITS, int WBITS, int BM, int BN, int WM, int WN, bool FUSED, int A_RULE, bool OUT_F32,
          int PREFETCH = 1, bool SCALE_DWORD = false>
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
    static_assert(!FUSED || (A_CHUNKS % NT == 0 && NT % 16 == 0), "fused tile mapping");

    extern __shared__ __align__(16) uint8_t smem[];

    const int tiles = ((p.M + BM - 1) / BM) * ((p.N + BN - 1) / BN);
    const int split = blockIdx.x / tiles;
    int tm, tn;
    tile_coords<BM, BN, 4>(p.M, p.N, blockIdx.x - split * tiles, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave / WN, wn = wave % WN;
    const int K = p.K, KB = K / 32;
    const int a_row_bytes = FUSED ? K * 2 : K * ABITS / 8;
    const int w_row_bytes = K * WBITS / 8;
    const int kt0 = split * p.chunk;                                  // this split's first stage
    const int nk = min(p.chunk, (K + BK - 1) / BK - kt0);            // and its stage count

    constexpr int SA_PER_T = FUSED ? 1 : (BM + NT - 1) / NT;   // A scale rows per thread
    constexpr int SW_PER_T = (BN + NT - 1) / NT;                 // W scale rows per thread
    struct Stage {
        uint4 ra[A_PER_T], rw[W_PER_T];
        uint32_t rsa[SA_PER_T], rsw[SW_PER_T];
        int kt;   // global stage index
    };

    // Buffer resources: 32-bit per-lane offsets, the stage offset in a scalar
    // register, and rows past the end of a tensor read as zero in hardware.
    // (The host splits launches so that every tensor stays below 2 GiB.)
    const __amdgpu_buffer_rsrc_t rsrc_a =
        __builtin_amdgcn_make_buffer_rsrc((void*)p.a_q, (short)0, p.M * a_row_bytes, 0x00020000);
    const __amdgpu_buffer_rsrc_t rsrc_w =
        __builtin_amdgcn_make_buffer_rsrc((void*)p.w_q, (short)0, p.N * w_row_bytes, 0x00020000);
    const __amdgpu_buffer_rsrc_t rsrc_as =
        __builtin_amdgcn_make_buffer_rsrc((void*)p.a_s, (short)0, FUSED ? 0 : p.M * KB, 0x00020000);
    const __amdgpu_buffer_rsrc_t rsrc_ws =
        __builtin_amdgcn_make_buffer_rsrc((void*)p.w_s, (short)0, p.N * KB, 0x00020000);
    constexpr int A_CPR = FUSED ? 16 : TA::CHUNKS;          // 16-byte chunks per row per stage
    constexpr int A_STAGE_BYTES = FUSED ? BK * 2 : TA::ROW_BYTES;
    const int a_c = tid % A_CPR, w_c = tid % TW::CHUNKS;      // chunk column: same for all i
    const int a_voff0 = (m0 + tid / A_CPR) * a_row_bytes + a_c * 16;
    const int w_voff0 = (n0 + tid / TW::CHUNKS) * w_row_bytes + w_c * 16;
    static_assert(NT % A_CPR == 0 && NT % TW::CHUNKS == 0, "chunk column must be loop invariant");

    static_assert(A_CHUNKS % NT == 0 && W_CHUNKS % NT == 0, "even work split");

    // Branch-free stage loads with uniform buffer descriptors.  Rows past the
    // end of a tensor read as zero (buffer range check).  When K is a multiple
    // of the stage (SCALE_DWORD), no stage has a K tail; otherwise the tail
    // chunks are zeroed by a select.
    auto scale_dword = [&](const __amdgpu_buffer_rsrc_t& rs, const uint8_t* sp, int grow, int lim, int kt) -> uint32_t {
        if (SCALE_DWORD) return (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(rs, grow * KB, kt * 4, 0);
        uint32_t v = 0;
        if (grow < lim) {
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                const int blk = kt * 4 + b;
                if (blk < KB) v |= (uint32_t)sp[(size_t)grow * KB + blk] << (8 * b);
            }
        }
        return v;
    };
    auto load_stage = [&](int kl, Stage& st) {
        const int kt = kt0 + kl;   // global stage index
        st.kt = kt;
        const bool a_in_k = SCALE_DWORD || kt * A_STAGE_BYTES + a_c * 16 < a_row_bytes;
        const bool w_in_k = SCALE_DWORD || kt * TW::ROW_BYTES + w_c * 16 < w_row_bytes;
#pragma unroll
        for (int i = 0; i < A_PER_T; ++i) {
            const int voff = a_voff0 + i * (NT / A_CPR) * a_row_bytes;
            const int4_t v = __builtin_amdgcn_raw_buffer_load_b128(rsrc_a, voff, kt * A_STAGE_BYTES, 0);
            st.ra[i] = make_uint4((uint32_t)v[0], (uint32_t)v[1], (uint32_t)v[2], (uint32_t)v[3]);
            if (!a_in_k) st.ra[i] = make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < W_PER_T; ++i) {
            const int voff = w_voff0 + i * (NT / TW::CHUNKS) * w_row_bytes;
            const int4_t v = __builtin_amdgcn_raw_buffer_load_b128(rsrc_w, voff, kt * TW::ROW_BYTES, 0);
            st.rw[i] = make_uint4((uint32_t)v[0], (uint32_t)v[1], (uint32_t)v[2], (uint32_t)v[3]);
            if (!w_in_k) st.rw[i] = make_uint4(0, 0, 0, 0);
        }
        // scale rows: threads beyond the tile's rows load a neighbouring row
        // (or zero) and never store it
        if (!FUSED) {
#pragma unroll
            for (int i = 0; i < SA_PER_T; ++i) st.rsa[i] = scale_dword(rsrc_as, p.a_s, m0 + tid + i * NT, p.M, kt);
        }
#pragma unroll
        for (int i = 0; i < SW_PER_T; ++i) st.rsw[i] = scale_dword(rsrc_ws, p.w_s, n0 + tid + i * NT, p.N, kt);
    };

    auto store_stage = [&](const Stage& sg, int buf) {
        const uint4* ra = sg.ra;
        const uint4* rw = sg.rw;
        uint8_t* st = smem + buf * STAGE;
        uint8_t* a_t = st;
        uint8_t* w_t = st + A_TILE;
        uint16_t* sa16 = reinterpret_cast<uint16_t*>(st + A_TILE + W_TILE);
        uint16_t* sw16 = sa16 + 2 * BM;
        if (!FUSED) {
#pragma unroll
            for (int i = 0; i < A_PER_T; ++i) {
                const int q = tid + i * NT;
                const int row = q / TA::CHUNKS, c = q % TA::CHUNKS;
                *reinterpret_cast<uint4*>(a_t + row * TA::ROW_BYTES + ((c ^ TA::swz(row)) * 16)) = ra[i];
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
                // debug dump of the prologue's codes (first tile column only)
                const int grow = m0 + row, kel = sg.kt * BK + c * 8;
                const bool dump = BM == 128 && p.dump_q != nullptr && tn == 0 && grow < p.M && kel < p.K;
                if (ABITS == 4) {
                    const uint32_t codes = encode8_e2m1(ra[i], e);
                    const int chunk = blk ^ TA::swz(row);
                    *reinterpret_cast<uint32_t*>(a_t + row * TA::ROW_BYTES + chunk * 16 + part * 4) = codes;
                    if (dump) *reinterpret_cast<uint32_t*>(p.dump_q + (size_t)grow * (p.K / 2) + kel / 2) = codes;
                } else {
                    const uint2 codes = encode8_e4m3(ra[i], e);
                    const int chunk = (2 * blk + part / 2) ^ TA::swz(row);
                    *reinterpret_cast<uint2*>(a_t + row * TA::ROW_BYTES + chunk * 16 + (part % 2) * 8) = codes;
                    if (dump) *reinterpret_cast<uint2*>(p.dump_q + (size_t)grow * p.K + kel) = codes;
                }
                if (dump && part == 0) p.dump_s[(size_t)grow * (p.K / 32) + kel / 32] = (uint8_t)(e + 127);
                if (part == 0)
                    reinterpret_cast<uint8_t*>(sa16)[scale_entry<WTM>(row, blk % 2) * 2 + blk / 2] = (uint8_t)(e + 127);
            }
        }
#pragma unroll
        for (int i = 0; i < W_PER_T; ++i) {
            const int q = tid + i * NT;
            const int row = q / TW::CHUNKS, c = q % TW::CHUNKS;
            *reinterpret_cast<uint4*>(w_t + row * TW::ROW_BYTES + ((c ^ TW::swz(row)) * 16)) = rw[i];
        }
        auto put_scales = [&](uint16_t* base, int r, uint32_t v, auto wt) {
            constexpr int WT = decltype(wt)::value;
            base[scale_entry<WT>(r, 0)] = (uint16_t)((v & 0xFFu) | ((v >> 8) & 0xFF00u));
            base[scale_entry<WT>(r, 1)] = (uint16_t)(((v >> 8) & 0xFFu) | ((v >> 16) & 0xFF00u));
        };
        if (!FUSED) {
#pragma unroll
            for (int i = 0; i < SA_PER_T; ++i)
                if (BM % NT == 0 || tid + i * NT < BM)
                    put_scales(sa16, tid + i * NT, sg.rsa[i], std::integral_constant<int, WTM>{});
        }
#pragma unroll
        for (int i = 0; i < SW_PER_T; ++i)
            if (BN % NT == 0 || tid + i * NT < BN)
                put_scales(sw16, tid + i * NT, sg.rsw[i], std::integral_constant<int, WTN>{});
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
        const uint16_t* sa16 = reinterpret_cast<const uint16_t*>(st + A_TILE + W_TILE);
        const uint16_t* sw16 = sa16 + 2 * BM;
        static_assert(FM % 2 == 0 && FN % 2 == 0, "scale entries come in pairs");
        int sa[FM / 2], sw[FN / 2];
        {
            const uint32_t* pa = reinterpret_cast<const uint32_t*>(sa16 + scale_entry<WTM>(wm * WTM + r32, g));
            const uint32_t* pw = reinterpret_cast<const uint32_t*>(sw16 + scale_entry<WTN>(wn * WTN + r32, g));
#pragma unroll
            for (int i = 0; i < FM / 2; ++i) sa[i] = (int)pa[i];
#pragma unroll
            for (int j = 0; j < FN / 2; ++j) sw[j] = (int)pw[j];
        }
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
                    // W is the matrix core's A operand and A its B operand, so the
                    // accumulator holds Y^T: each lane ends up with 4 consecutive
                    // output columns (see the epilogue)
                    mfma_scaled_sel<BLGP, CBSZ>(acc[i][j], fw[j], fa[i], sw[j / 2], sa[i / 2],
                                                 2 * (j % 2) + kk, 2 * (i % 2) + kk);
                }
        }
    };

    Stage s0, s1;
    load_stage(0, s0);
    if (PREFETCH >= 2 && nk > 1) load_stage(1, s1);
    store_stage(s0, 0);
    lds_barrier();
    if (PREFETCH == 3) {
        // As PREFETCH == 2, but each half first writes the stage that has been
        // in flight for a whole compute period to the free LDS buffer, and only
        // then issues the next stage's loads (a scheduling fence keeps that
        // order), so no wait ever covers the loads just issued.
        int kt = 0;
        for (; kt + 1 < nk; kt += 2) {
            store_stage(s1, 1);                      // stage kt + 1 -> buffer 1
            __builtin_amdgcn_sched_barrier(0);
            if (kt + 2 < nk) load_stage(kt + 2, s0);
            compute_stage(0);                        // stage kt from buffer 0
            lds_barrier();
            if (kt + 2 < nk) store_stage(s0, 0);     // stage kt + 2 -> buffer 0
            __builtin_amdgcn_sched_barrier(0);
            if (kt + 3 < nk) load_stage(kt + 3, s1);
            compute_stage(1);                        // stage kt + 1 from buffer 1
            lds_barrier();
        }
        if (kt < nk) compute_stage(0);
    } else if (PREFETCH == 2) {
        int kt = 0;
        for (; kt + 1 < nk; kt += 2) {
            // LDS buffer 0 holds stage kt; s1 holds stage kt + 1 (in flight)
            if (kt + 2 < nk) load_stage(kt + 2, s0);
            compute_stage(0);
            store_stage(s1, 1);
            lds_barrier();
            // LDS buffer 1 holds stage kt + 1; s0 holds stage kt + 2 (in flight)
            if (kt + 3 < nk) load_stage(kt + 3, s1);
            compute_stage(1);
            if (kt + 2 < nk) store_stage(s0, 0);
            lds_barrier();
        }
        if (kt < nk) compute_stage(0);  // odd stage count: the last stage is in buffer 0
    } else {
        for (int kt = 0; kt < nk; ++kt) {
            const bool more = kt + 1 < nk;
            if (more) load_stage(kt + 1, s1);
            compute_stage(kt & 1);
            if (more) store_stage(s1, (kt + 1) & 1);
            lds_barrier();
        }
    }

    // fp32 partial tile of this split (same layout as an fp32 Y); only the
    // 128 x 128 unfused kernel is ever launched with splits
    if constexpr (!FUSED && BM == 128) if (p.splits > 1) {
        float* part = p.part + (size_t)split * p.M * p.N;
        const bool vec = (p.N & 3) == 0;
#pragma unroll
        for (int i = 0; i < FM; ++i) {
            const int m = m0 + wm * WTM + i * 32 + r32;
#pragma unroll
            for (int j = 0; j < FN; ++j)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    // registers 4q .. 4q+3: 4 consecutive columns of row m
                    const int n = n0 + wn * WTN + j * 32 + q * 8 + g * 4;
                    if (m >= p.M) continue;
                    if (vec && n + 3 < p.N) {
                        *reinterpret_cast<float4_t*>(part + (size_t)m * p.N + n) =
                            float4_t{acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]};
                    } else {
#pragma unroll
                        for (int t = 0; t < 4; ++t)
                            if (n + t < p.N) part[(size_t)m * p.N + n + t] = acc[i][j][4 * q + t];
                    }
                }
        }
        return;
    }

    // epilogue: accumulator (i, j) register r holds Y[m][n] with
    //   m = tile row of fragment i + lane % 32,
    //   n = tile column of fragment j + (r / 4) * 8 + (lane / 32) * 4 + r % 4,
    // so registers 4q .. 4q+3 are 4 consecutive columns of one row: one 8-byte
    // (bf16) or 16-byte (fp32) store when the row is aligned and in range.
    const bool vec_ok = (p.N & 3) == 0;
#pragma unroll
    for (int i = 0; i < FM; ++i) {
        const int m = m0 + wm * WTM + i * 32 + r32;
#pragma unroll
        for (int j = 0; j < FN; ++j) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int n = n0 + wn * WTN + j * 32 + q * 8 + g * 4;
                const float v0 = acc[i][j][4 * q], v1 = acc[i][j][4 * q + 1];
                const float v2 = acc[i][j][4 * q + 2], v3 = acc[i][j][4 * q + 3];
                if (m < p.M && vec_ok && n + 3 < p.N) {
                    if (OUT_F32) {
                        *reinterpret_cast<float4_t*>(reinterpret_cast<float*>(p.y) + (size_t)m * p.N + n) =
                            float4_t{v0, v1, v2, v3};
                    } else {
                        const uint32_t lo = bf16x2_rne(v0, v1);
                        const uint32_t hi = bf16x2_rne(v2, v3);
                        *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(p.y) + (size_t)m * p.N + n) =
                            make_uint2(lo, hi);
                    }
                } else if (m < p.M) {
                    const float vv[4] = {v0, v1, v2, v3};
#pragma unroll
                    for (int t = 0; t < 4; ++t) {
                        if (n + t < p.N) {
                            if (OUT_F32) reinterpret_cast<float*>(p.y)[(size_t)m * p.N + n + t] = vv[t];
                            else reinterpret_cast<uint16_t*>(p.y)[(size_t)m * p.N + n + t] = f32_to_bf16_rne(vv[t]);
                        }
                    }
                }
            }
        }
    }
}

template <int ABITS, int WBITS, int BM, int BN, int WM, int WN, bool FUSED, int A_RULE, bool OUT_F32,
          int PREFETCH = 1, bool SCALE_DWORD = false>
hipError_t launch_tile(const GemmArgs& a, hipStream_t stream)
{
    using TA = OpTraits<ABITS>;
    using TW = OpTraits<WBITS>;
    constexpr int STAGE = BM * TA::ROW_BYTES + BN * TW::ROW_BYTES + 4 * (BM + BN);
    constexpr int LDS = 2 * STAGE;
    auto kern = mx_gemm_kernel<ABITS, WBITS, BM, BN, WM, WN, FUSED, A_RULE, OUT_F32, PREFETCH, SCALE_DWORD>;
    static bool attr_set = false;  // benign race: setting the same value twice is harmless
    if (!attr_set) {
        hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, LDS);
        if (e != hipSuccess) return e;
        attr_set = true;
    }
    const int tiles = ((a.M + BM - 1) / BM) * ((a.N + BN - 1) / BN);
    hipLaunchKernelGGL(kern, dim3(tiles * a.splits), dim3(WM * WN * 64), LDS, stream, a);
    return hipGetLastError();
}

// ---------------------------------------------------------------- split-K
// Y = alpha * sum over s of part[s] (fp32 partial products [M, N] each),
// summed in split order, so the result does not depend on scheduling; 4
// elements per lane (any M*N: the tail lanes take single elements).
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float* __restrict__ part, int splits,
                                                            int64_t mn, float alpha, void* __restrict__ y,
                                                            int out_f32)
{
    const int64_t i4 = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
    if (i4 >= mn) return;
    if (i4 + 4 <= mn && (mn & 3) == 0) {
        float4_t acc = *reinterpret_cast<const float4_t*>(part + i4);
        for (int s = 1; s < splits; ++s) acc += *reinterpret_cast<const float4_t*>(part + (size_t)s * mn + i4);
        acc *= alpha;
        if (out_f32) *reinterpret_cast<float4_t*>(reinterpret_cast<float*>(y) + i4) = acc;
        else *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(y) + i4) =
                 make_uint2(bf16x2_rne(acc[0], acc[1]), bf16x2_rne(acc[2], acc[3]));
        return;
    }
    for (int64_t i = i4; i < i4 + 4 && i < mn; ++i) {
        float v = part[i];
        for (int s = 1; s < splits; ++s) v += part[(size_t)s * mn + i];
        v *= alpha;
        if (out_f32) reinterpret_cast<float*>(y)[i] = v;
        else reinterpret_cast<uint16_t*>(y)[i] = f32_to_bf16_rne(v);
    }
}

// K splits for a launch of `tiles` tiles over nk stages: up to 128 tiles, as
// many splits as still fit one workgroup per compute unit (256), so that all
// of them run in one round; from 129 to two_max tiles (0: none), two splits,
// one round at two workgroups per CU; every split at least min_stages long,
// and (even) a whole number of stage pairs per split.  Returns the split
// count and sets the stages per split.
extern "C" int mxl_choose_splits(int64_t tiles, int nk, int min_stages, int even, int two_max, int* chunk)
{
    int s = 1;
    if (tiles <= 128) {
        s = (int)(256 / tiles);
    } else if (tiles <= two_max) {
        s = 2;
    }
    const int cap = nk / min_stages;
    if (s > cap) s = cap;
    if (s < 1) s = 1;
    int c = (nk + s - 1) / s;
    if (even && (c & 1)) ++c;
    *chunk = c;
    return (nk + c - 1) / c;
}

extern "C" hipError_t mxl_launch_splitk_reduce(const float* part, int splits, int64_t mn, float alpha, void* y,
                                               int out_f32, hipStream_t stream)
{
    const int64_t blocks = (mn + 1023) / 1024;
    hipLaunchKernelGGL(splitk_reduce_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, part, splits, mn, alpha,
                       y, out_f32);
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
__global__ __launch_bounds__(512) void mx_decode_generic_kernel(GemmArgs p)
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

// Decode-shaped MXFP4 GEMM for K too large for mx_decode_kernel's LDS block
// (M <= 32, K % 128 == 0).  Its cost is the number of vector-memory
// instructions per CU as much as bytes.
//  * One workgroup of 4 waves owns 32 rows of W (two groups of 16); wave w
//    owns a contiguous quarter of K and walks it in chunks of CH stages of
//    128, issuing every load of a chunk before its matrix-core work.
//  * Operands follow the lane layout of v_mfma_scale_f32_16x16x128_f8f6f4
//    (lane r + 16 g: row r, K elements [32 g, 32 g + 32) of the stage), so
//    each 16-byte load is a fragment: one instruction reads 16 rows x 64
//    contiguous bytes.  An A fragment (MT groups of 16 rows; rows past M
//    read as zero through the buffer range check) serves both W groups.
//  * The scales of the workgroup's W rows and of A are contiguous in memory;
//    they are staged once into LDS with 16-byte loads (a few instructions per
//    workgroup instead of one per stage) and read from there per stage.
//  * The four K quarters are summed through LDS at the end.
template <int MT, int CH, bool OUT_F32>
__global__ __launch_bounds__(256) void mx_decode_direct_kernel(GemmArgs p)
{
    constexpr int WAVES = 4, RG = 2;   // waves, W row groups of 16
    extern __shared__ __align__(16) uint8_t dsm[];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: the step offsets go in SGPRs
    const int r = lane & 15, g = lane >> 4;
    const int n0 = blockIdx.x * 16 * RG;
    const int K = p.K, KB = K / 32, row_bytes = K / 2;
    const int steps = K / 128;
    const int s0 = wave * steps / WAVES, s1 = (wave + 1) * steps / WAVES;

    const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc((void*)p.w_q, (short)0, p.N * row_bytes, 0x00020000);
    const __amdgpu_buffer_rsrc_t rws = __builtin_amdgcn_make_buffer_rsrc((void*)p.w_s, (short)0, p.N * KB, 0x00020000);
    const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc((void*)p.a_q, (short)0, p.M * row_bytes, 0x00020000);
    const __amdgpu_buffer_rsrc_t ras = __builtin_amdgcn_make_buffer_rsrc((void*)p.a_s, (short)0, p.M * KB, 0x00020000);

    // LDS: W scales [16 RG rows][KB], A scales [16 MT rows][KB], then the reduction area
    uint8_t* sw_lds = dsm;
    uint8_t* sa_lds = dsm + 16 * RG * KB;
    float4_t_* red = reinterpret_cast<float4_t_*>(dsm + 16 * (RG + MT) * KB);   // [WAVES][RG][MT][64]

    // stage the scales: 16-byte pieces of the two contiguous byte ranges
    {
        const int wn = 16 * RG * KB / 16, an = 16 * MT * KB / 16;
        for (int i = tid; i < wn + an; i += 256) {
            const int4_t v = i < wn ? __builtin_amdgcn_raw_buffer_load_b128(rws, n0 * KB + i * 16, 0, 0)
                                    : __builtin_amdgcn_raw_buffer_load_b128(ras, (i - wn) * 16, 0, 0);
            *reinterpret_cast<int4_t*>(dsm + i * 16) = v;
        }
    }

    int w_voff[RG], a_voff[MT];
#pragma unroll
    for (int h = 0; h < RG; ++h) w_voff[h] = (n0 + 16 * h + r) * row_bytes + g * 16;
#pragma unroll
    for (int t = 0; t < MT; ++t) a_voff[t] = (16 * t + r) * row_bytes + g * 16;

    float4_t_ acc[RG][MT];
#pragma unroll
    for (int h = 0; h < RG; ++h)
#pragma unroll
        for (int t = 0; t < MT; ++t) acc[h][t] = float4_t_{0.f, 0.f, 0.f, 0.f};

    __syncthreads();   // scales are in LDS

    // `cnt` stages from stage sb (cnt == CH: straight-line code)
    auto chunk = [&](int sb, int cnt) {
        int4_t wf[CH][RG], af[CH][MT];
#pragma unroll
        for (int u = 0; u < CH; ++u)
            if (u < cnt) {
#pragma unroll
                for (int h = 0; h < RG; ++h) wf[u][h] = __builtin_amdgcn_raw_buffer_load_b128(rw, w_voff[h], (sb + u) * 64, 0);
#pragma unroll
                for (int t = 0; t < MT; ++t) af[u][t] = __builtin_amdgcn_raw_buffer_load_b128(ra, a_voff[t], (sb + u) * 64, 0);
            }
#pragma unroll
        for (int u = 0; u < CH; ++u)
            if (u < cnt) {
                const int st = sb + u;
                int wsb[RG], asb[MT];
                // the dword of a row's scales for stage st holds blocks 4 st .. 4 st + 3; lane group g takes byte g
#pragma unroll
                for (int h = 0; h < RG; ++h)
                    wsb[h] = (int)(*reinterpret_cast<const uint32_t*>(sw_lds + (16 * h + r) * KB + 4 * st) >> (8 * g));
#pragma unroll
                for (int t = 0; t < MT; ++t)
                    asb[t] = (int)(*reinterpret_cast<const uint32_t*>(sa_lds + (16 * t + r) * KB + 4 * st) >> (8 * g));
#pragma unroll
                for (int h = 0; h < RG; ++h) {
                    const int8_t_ b8 = int8_t_{wf[u][h][0], wf[u][h][1], wf[u][h][2], wf[u][h][3], 0, 0, 0, 0};
#pragma unroll
                    for (int t = 0; t < MT; ++t) {
                        const int8_t_ a8 = int8_t_{af[u][t][0], af[u][t][1], af[u][t][2], af[u][t][3], 0, 0, 0, 0};
                        acc[h][t] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a8, b8, acc[h][t], 4, 4, 0, asb[t], 0, wsb[h]);
                    }
                }
            }
    };
    int sb = s0;
    for (; sb + CH <= s1; sb += CH) chunk(sb, CH);
    if (sb < s1) chunk(sb, s1 - sb);

#pragma unroll
    for (int h = 0; h < RG; ++h)
#pragma unroll
        for (int t = 0; t < MT; ++t) red[((wave * RG + h) * MT + t) * 64 + lane] = acc[h][t];
    __syncthreads();
    // thread e < RG * MT * 64 finishes accumulator lane e % 64 of (row group h, A tile t):
    // A rows 16 t + 4 (l / 16) + i, W row n0 + 16 h + l % 16
    if (tid < RG * MT * 64) {
        const int l = tid & 63, ht = tid >> 6, h = ht / MT, t = ht % MT;
        float4_t_ v = red[(h * MT + t) * 64 + l];
#pragma unroll
        for (int w = 1; w < WAVES; ++w) {
            const float4_t_ x = red[((w * RG + h) * MT + t) * 64 + l];
            v = float4_t_{v[0] + x[0], v[1] + x[1], v[2] + x[2], v[3] + x[3]};
        }
        const int nn = n0 + 16 * h + (l & 15);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int m = 16 * t + 4 * (l >> 4) + i;
            if (m < p.M && nn < p.N) {
                if (OUT_F32) reinterpret_cast<float*>(p.y)[(size_t)m * p.N + nn] = v[i];
                else reinterpret_cast<uint16_t*>(p.y)[(size_t)m * p.N + nn] = f32_to_bf16_rne(v[i]);
            }
        }
    }
}

template <int MT>
static size_t decode_direct_lds_bytes(int K)
{
    return (size_t)16 * (2 + MT) * (K / 32) + (size_t)4 * 2 * MT * 64 * 16;
}

// Decode-shaped MXFP4 GEMM (M <= 32, K % 512 == 0, K up to 8192):
// a stream over W.  One workgroup of 4 waves owns 16 rows of W.
//  * W streams as whole rows: the 16 x K/2 byte block is contiguous, and each
//    buffer-to-LDS copy moves 1 KiB of it (8 full cache lines; the pattern
//    that streams fastest).  A copy lane places its 16-byte unit u of row r at
//    unit u ^ (r & 15) of the LDS row (within aligned groups of 16 units), so
//    the fragment reads below hit 16 distinct banks.
//  * Scales of the W rows and of A (contiguous byte ranges) are copied into
//    LDS the same way, 256 bytes per copy, so one wait covers everything.
//  * After one barrier, wave w takes a contiguous quarter of K and runs
//    v_mfma_scale_f32_16x16x128_f8f6f4 per stage (lane r + 16 g: row r, K
//    elements [32 g, 32 g + 32) of the stage): W fragments from LDS, A
//    fragments (MT groups of 16 rows; rows past M read as zero) loaded
//    directly; they are the same for every workgroup and stay in the caches.
//  * The four K quarters are summed through LDS (aliasing the W block).
template <int MT, bool OUT_F32>
__global__ __launch_bounds__(256) void mx_decode_kernel(GemmArgs p)
{
    constexpr int WAVES = 4;
    extern __shared__ __align__(16) uint8_t dsm[];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: the step offsets go in SGPRs
    const int r = lane & 15, g = lane >> 4;
    const int n0 = blockIdx.x * 16;
    const int K = p.K, KB = K / 32, row_bytes = K / 2;
    const int steps = K / 128;
    const int s0 = wave * steps / WAVES, s1 = (wave + 1) * steps / WAVES;
    const int units = KB;                  // 16-byte units per W row
    const int swz_units = units & ~15;     // units inside whole groups of 16 get swizzled

    // LDS: W block [16][row_bytes] (later the reduction area, so at least its size), W scales [16][KB],
    // A scales [16 MT][KB]
    constexpr int RED_BYTES = WAVES * MT * 64 * 16;
    uint8_t* w_lds = dsm;
    uint8_t* sw_lds = dsm + (16 * row_bytes > RED_BYTES ? 16 * row_bytes : RED_BYTES);
    uint8_t* sa_lds = sw_lds + 16 * KB;
    const uint32_t lds0 = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)dsm);

    // W block copies: copy j moves block units [64 j, 64 j + 64)
    {
        const int4_t rsrc = make_rsrc(p.w_q, (uint32_t)p.N * row_bytes);
        const int ncopy = 16 * units / 64;
        for (int j = wave; j < ncopy; j += WAVES) {
            const int q = 64 * j + lane, rr = q / units, pu = q - rr * units;
            const int u = pu < swz_units ? pu ^ (rr & 15) : pu;
            dma_b128(lds0 + (uint32_t)(64 * j * 16), (n0 + rr) * row_bytes + u * 16, rsrc, 0);
        }
    }
    // scale copies, 256 bytes each: the W rows' scales (16 KB bytes, contiguous) and A's (16 MT KB bytes)
    {
        const int4_t rws = make_rsrc(p.w_s, (uint32_t)p.N * KB);
        const int4_t ras = make_rsrc(p.a_s, (uint32_t)p.M * KB);
        const uint32_t sbase = lds0 + (uint32_t)(sw_lds - dsm);
        const int wn = 16 * KB / 256, an = 16 * MT * KB / 256;   // KB % 16 == 0 here
        for (int j = wave; j < wn + an; j += WAVES) {
            if (j < wn) dma_b32(sbase + j * 256, n0 * KB + j * 256 + lane * 4, rws, 0);
            else dma_b32(sbase + j * 256, (j - wn) * 256 + lane * 4, ras, 0);
        }
    }
    const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc((void*)p.a_q, (short)0, p.M * row_bytes, 0x00020000);
    // this wave's A fragments, issued before waiting on anything
    constexpr int SMAX = 16;   // stages per wave held in registers (K <= 8192)
    int4_t af[SMAX][MT];
#pragma unroll
    for (int u = 0; u < SMAX; ++u)
        if (s0 + u < s1)
#pragma unroll
            for (int t = 0; t < MT; ++t)
                af[u][t] = __builtin_amdgcn_raw_buffer_load_b128(ra, (16 * t + r) * row_bytes + g * 16, (s0 + u) * 64, 0);

    wait_vmcnt<0>();
    __syncthreads();

    float4_t_ acc[MT];
#pragma unroll
    for (int t = 0; t < MT; ++t) acc[t] = float4_t_{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int u = 0; u < SMAX; ++u) {
        const int st = s0 + u;
        if (st < s1) {
            const int un = 4 * st + g;
            const int pu = un < swz_units ? un ^ r : un;
            const int4_t wv = *reinterpret_cast<const int4_t*>(w_lds + r * row_bytes + pu * 16);
            const int8_t_ b8 = int8_t_{wv[0], wv[1], wv[2], wv[3], 0, 0, 0, 0};
            // the dword of a row's scales for stage st holds blocks 4 st .. 4 st + 3; lane group g takes byte g
            const int wsb = (int)(*reinterpret_cast<const uint32_t*>(sw_lds + r * KB + 4 * st) >> (8 * g));
#pragma unroll
            for (int t = 0; t < MT; ++t) {
                const int asb = (int)(*reinterpret_cast<const uint32_t*>(sa_lds + (16 * t + r) * KB + 4 * st) >> (8 * g));
                const int8_t_ a8 = int8_t_{af[u][t][0], af[u][t][1], af[u][t][2], af[u][t][3], 0, 0, 0, 0};
                acc[t] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a8, b8, acc[t], 4, 4, 0, asb, 0, wsb);
            }
        }
    }
    __syncthreads();   // every wave is done with the W block
    float4_t_* red = reinterpret_cast<float4_t_*>(w_lds);   // [WAVES][MT][64]
#pragma unroll
    for (int t = 0; t < MT; ++t) red[(wave * MT + t) * 64 + lane] = acc[t];
    __syncthreads();
    // thread e < MT * 64 finishes accumulator lane e % 64 of A tile t:
    // A rows 16 t + 4 (l / 16) + i, W row n0 + l % 16
    if (tid < MT * 64) {
        const int l = tid & 63, t = tid >> 6;
        float4_t_ v = red[t * 64 + l];
#pragma unroll
        for (int w = 1; w < WAVES; ++w) {
            const float4_t_ x = red[(w * MT + t) * 64 + l];
            v = float4_t_{v[0] + x[0], v[1] + x[1], v[2] + x[2], v[3] + x[3]};
        }
        const int nn = n0 + (l & 15);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int m = 16 * t + 4 * (l >> 4) + i;
            if (m < p.M && nn < p.N) {
                if (OUT_F32) reinterpret_cast<float*>(p.y)[(size_t)m * p.N + nn] = v[i];
                else reinterpret_cast<uint16_t*>(p.y)[(size_t)m * p.N + nn] = f32_to_bf16_rne(v[i]);
            }
        }
    }
}

// Decode-shaped MXFP4 GEMM streamed per wave (M <= 16 MT, MT <= 2, K =
// 1024 QS / 2 with QS stages of 128 per wave, K <= 8192).  One workgroup of
// 4 waves owns RG groups of 16 W rows (RG consecutive groups, or with PART
// an even share of them per compute unit) and wave w a contiguous quarter
// of K.  Each wave copies its own 16 RG x K/8-byte part of W into its own
// LDS region and consumes it stage by stage as the copies land, so no wave
// waits for another one (or for the whole block) before its matrix-core
// work; the four partial sums meet once, at the end.  Each A fragment a
// wave loads serves all RG groups.
//  * Copy (c, h) moves rows 8 h .. 8 h + 7 x bytes [128 c, 128 c + 128) of
//    the wave's quarter: 8 full cache lines, 1 KiB.  The copies go out in c
//    order, and stages 2 c and 2 c + 1 wait for copies (c, 0) and (c, 1)
//    only, with an exact vmcnt.
//  * Inside the 1 KiB of copy (c, h), row q of the group (8 h <= q < 8 h +
//    8) holds its 16-byte chunk L at 128 (q % 8) + 16 (L ^ ((q >> 1) & 7)):
//    the 16 rows of one lane group, reading the same chunk, cover all 64
//    banks.  The swizzle is chosen by which chunk each copy lane fetches.
//  * The A fragments of all the wave's stages (MT groups of 16 rows; rows
//    past M read as zero through the buffer range check) and the scale
//    dwords of its stages (a row's dword 4 s .. 4 s + 3 holds stage s's 4
//    blocks) are loaded into registers before the W copies (after those of
//    the first stage pair with one row group per workgroup), so the copies'
//    waits cover them as well.
//  * Operands follow v_mfma_scale_f32_16x16x128_f8f6f4 (lane r + 16 g: row
//    r, K elements [32 g, 32 g + 32) of the stage), as in mx_decode_kernel,
//    and the partial sums are added in the same wave order.
// s_waitcnt vmcnt(n) for an n that folds to a constant once loops are
// unrolled (n <= 14 here)
__device__ __forceinline__ void wait_vmcnt_n(int n)
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

// buffer-to-LDS copy of 16 bytes per lane marked non-temporal: data read
// once, streamed past the caches
__device__ __forceinline__ void dma_b128_nt(uint32_t lds, int voff, const int4_t& rsrc, int soff)
{
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, %3 offen nt lds"
                 :: "s"(lds), "v"(voff), "s"(rsrc), "s"(soff) : "memory");
}

__device__ __forceinline__ uint32_t lds_read_u32(uint32_t addr)
{
    return *reinterpret_cast<const __attribute__((address_space(3))) uint32_t*>((size_t)addr);
}

__device__ __forceinline__ int4_t lds_read_v4(uint32_t addr)
{
    return *reinterpret_cast<const __attribute__((address_space(3))) int4_t*>((size_t)addr);
}

template <int MT, int QS, int RS, int RG, bool OUT_F32, bool PART = false>
__global__ __launch_bounds__(256) void mx_decode_stream_kernel(GemmArgs p)
{
    constexpr int WAVES = 4, NC = QS / 2, RSB = RS < NC ? RS : NC;
    constexpr int SLOT = RG * 2048;       // a pair slot: RG groups of 16 rows x 128 B per wave
    static_assert(QS % 2 == 0 && QS <= 16 && MT <= 2 && RSB >= 1 && RG >= 1 && RG <= 5, "decode stream shape");
    extern __shared__ __align__(16) uint8_t dsm[];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: the copy offsets go in SGPRs
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
    const int K = QS * 512, KB = K / 32, row_bytes = K / 2;
    const int QB = row_bytes / WAVES;     // W bytes per row per wave (64 QS)
    const int st0 = wave * QS;            // this wave's first stage

    const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc((void*)p.a_q, (short)0, p.M * row_bytes, 0x00020000);
    const int4_t rw = make_rsrc(p.w_q, (uint32_t)n_lim * row_bytes);
    const uint32_t lds0 = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)dsm);
    const uint32_t lds_w = lds0 + (uint32_t)(wave * RSB * SLOT);   // this wave's ring of RSB pair slots

    // The scale blocks of the workgroup's 16 RG W rows and of A's 16 MT rows
    // (contiguous [rows][K/32] byte ranges) go to LDS first, 256 bytes per
    // copy, spread over the waves; one barrier publishes them.
    constexpr int SCOP = (RG + MT) * QS;   // 16 KB / 256 bytes per 16 rows
    const uint32_t sw_lds = lds0 + (uint32_t)(WAVES * RSB * SLOT), sa_lds = sw_lds + (uint32_t)(16 * RG * KB);
    {
        const int4_t rws4 = make_rsrc(p.w_s, (uint32_t)n_lim * KB);
        const int4_t ras4 = make_rsrc(p.a_s, (uint32_t)p.M * KB);
#pragma unroll
        for (int j = 0; j < SCOP; ++j)
            if (j % WAVES == wave) {
                if (j < RG * QS) dma_b32(sw_lds + j * 256, n0 * KB + j * 256 + lane * 4, rws4, 0);
                else dma_b32(sw_lds + j * 256, (j - RG * QS) * 256 + lane * 4, ras4, 0);
            }
    }
    // the wave's W copies, in stage order: pair c (copies (c, 0) and (c, 1))
    // goes to ring slot c % RSB; the first RSB pairs now, each later one
    // once the pair before it in its slot has been computed
    // (copy h of a pair: rows 8 h .. 8 h + 7 of the workgroup's 16 RG rows)
    int voffh[2 * RG];
#pragma unroll
    for (int h = 0; h < 2 * RG; ++h) {
        const int q = 8 * h + (lane >> 3);
        voffh[h] = (n0 + q) * row_bytes + (((lane & 7) ^ ((q >> 1) & 7)) * 16);
    }
    auto copy_pair = [&](int c) __attribute__((always_inline)) {
#pragma unroll
        for (int h = 0; h < 2 * RG; ++h)
            dma_b128_nt(lds_w + (uint32_t)((c % RSB) * SLOT + h * 1024), voffh[h], rw, wave * QB + c * 128);
    };
    // with one row group per workgroup, pair 0 goes out before the A loads,
    // so that its trip to HBM overlaps their issue (M = 8: 12.06 -> 11.75 us;
    // the per-CU grid measured 2% slower with it and issues it after them).
    // Pair 0 is needed together with every A fragment anyway, and the later
    // pairs follow the A loads, so the waits below count only W copies.
    if (!PART) copy_pair(0);
    // A fragments of every stage of the wave
    int4_t af[QS][MT];
#pragma unroll
    for (int u = 0; u < QS; ++u)
#pragma unroll
        for (int t = 0; t < MT; ++t)
            af[u][t] = __builtin_amdgcn_raw_buffer_load_b128(ra, (16 * t + r) * row_bytes + g * 16, (st0 + u) * 64, 0);
#pragma unroll
    for (int c = PART ? 0 : 1; c < RSB; ++c) copy_pair(c);

    // the scale copies have landed once at most the A loads and W copies
    // issued after them are outstanding
    wait_vmcnt<QS * MT + 2 * RG * RSB>();
    lds_barrier();

    float4_t_ acc[RG][MT];
#pragma unroll
    for (int rg = 0; rg < RG; ++rg)
#pragma unroll
        for (int t = 0; t < MT; ++t) acc[rg][t] = float4_t_{0.f, 0.f, 0.f, 0.f};
    const uint32_t rd = lds_w + (uint32_t)((r >> 3) * 1024 + (r & 7) * 128);
    const int rsw = (r >> 1) & 7;
    const uint32_t rsw_l = sw_lds + (uint32_t)(r * KB + 4 * st0), rsa_l = sa_lds + (uint32_t)(r * KB + 4 * st0);
#pragma unroll
    for (int c = 0; c < NC; ++c) {
        // pairs 0 .. min(c - 1 + RSB, NC - 1) have been issued: pair c's
        // copies have landed once at most the copies of the later ones are
        // outstanding
        {
            const int last = c - 1 + RSB < NC - 1 ? c - 1 + RSB : NC - 1;
            wait_vmcnt_n(2 * RG * (last - c));
        }
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
            const int u = 2 * c + hf;
#pragma unroll
            for (int rg = 0; rg < RG; ++rg) {
                const int4_t wv = lds_read_v4(rd + (uint32_t)((c % RSB) * SLOT + rg * 2048 + (((4 * hf + g) ^ rsw) * 16)));
                const int8_t_ b8 = int8_t_{wv[0], wv[1], wv[2], wv[3], 0, 0, 0, 0};
                // a row's scale dword for stage s holds blocks 4 s .. 4 s + 3; lane group g takes byte g
                const int wsb = (int)(lds_read_u32(rsw_l + (uint32_t)(16 * rg * KB + 4 * u)) >> (8 * g));
#pragma unroll
                for (int t = 0; t < MT; ++t) {
                    const int asb = (int)(lds_read_u32(rsa_l + (uint32_t)(16 * t * KB + 4 * u)) >> (8 * g));
                    const int8_t_ a8 = int8_t_{af[u][t][0], af[u][t][1], af[u][t][2], af[u][t][3], 0, 0, 0, 0};
                    acc[rg][t] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a8, b8, acc[rg][t], 4, 4, 0, asb, 0, wsb);
                }
            }
        }
        if (c + RSB < NC) {
            // slot c % RSB is free once this pair's LDS reads have returned
            __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
            copy_pair(c + RSB);
        }
    }
    __syncthreads();   // every wave is done with its LDS region
    float4_t_* red = reinterpret_cast<float4_t_*>(dsm);   // [WAVES][RG][MT][64]
#pragma unroll
    for (int rg = 0; rg < RG; ++rg)
#pragma unroll
        for (int t = 0; t < MT; ++t) red[((wave * RG + rg) * MT + t) * 64 + lane] = acc[rg][t];
    __syncthreads();
    // item e < RG * MT * 64 finishes accumulator lane e % 64 of (W group rg,
    // A tile t): A rows 16 t + 4 (l / 16) + i, W row n0 + 16 rg + l % 16
    for (int e = tid; e < RG * MT * 64; e += 256) {
        const int l = e & 63, rt = e >> 6, rg = rt / MT, t = rt % MT;
        float4_t_ v = red[(rg * MT + t) * 64 + l];
#pragma unroll
        for (int w = 1; w < WAVES; ++w) {
            const float4_t_ x = red[((w * RG + rg) * MT + t) * 64 + l];
            v = float4_t_{v[0] + x[0], v[1] + x[1], v[2] + x[2], v[3] + x[3]};
        }
        const int nn = n0 + 16 * rg + (l & 15);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int m = 16 * t + 4 * (l >> 4) + i;
            if (m < p.M && nn < n_lim) {
                if (OUT_F32) reinterpret_cast<float*>(p.y)[(size_t)m * p.N + nn] = v[i];
                else reinterpret_cast<uint16_t*>(p.y)[(size_t)m * p.N + nn] = f32_to_bf16_rne(v[i]);
            }
        }
    }
}

// The streamed decode kernel keeps either every stage pair of a wave's
// quarter in flight (K / 1024 slots) or a ring of a few slots (2 KiB per 16
// rows each per wave), refilled as pairs are computed.  The ring lets more
// workgroups share a CU: it measured faster from M = 16 up (more A fragment
// loads in flight) and slightly slower below, and it is the only form whose
// LDS fits at K = 8192.  Above M = 16 a workgroup owns two 16-row groups of
// W, so that each A fragment it loads from the L2 serves both.
struct DecodeStreamCfg {
    int rg;      // 16-row W groups per workgroup
    int slots;   // ring slots (stage pairs) per wave; K / 1024 = every pair
};

static DecodeStreamCfg decode_stream_cfg(int64_t m, int64_t k)
{
    if (m > 16) return {2, 2};
    const int all = (int)(k / 1024);
    const size_t whole = (size_t)4 * all * 2048 + (size_t)16 * 2 * (k / 32);
    if (m <= 8 && whole <= 65536) return {1, all};
    return {1, 3};
}

static size_t decode_stream_lds_bytes(int mt, int k, DecodeStreamCfg c)
{
    const int nc = k / 1024, slots = c.slots < nc ? c.slots : nc;
    return (size_t)4 * slots * c.rg * 2048 + (size_t)16 * (c.rg + mt) * (k / 32);
}

static bool decode_stream_ring(int64_t m, int64_t k) { return decode_stream_cfg(m, k).slots < k / 1024; }

// whether mx_decode_stream_kernel serves M rows of A at this K
static bool decode_stream_ok(int64_t m, int64_t k)
{
    return m <= 32 && k % 1024 == 0 && k >= 1024 && k <= 8192 &&
           decode_stream_lds_bytes(m > 16 ? 2 : 1, (int)k, decode_stream_cfg(m, k)) <= 65536;
}

// Above 8 rows of A, when the 16-row groups of W number 4 to 5 per compute
// unit (MI355X: 256), one workgroup per compute unit takes 4 or 5 of them
// (the grid splits the groups evenly), so each CU loads the A fragments
// once instead of once per one or two groups, and no CU holds one workgroup
// more than others.  Its ring (2 pair slots of 5 groups per wave, 80 KiB)
// and scale blocks take up to 108 KiB of LDS.  (N = 17408, K = 5120: M = 32
// 17.83 -> 14.07 us, M = 16 13.87 -> 12.45 us; at M = 8 and below it measured
// equal or slower.)
constexpr int DEC_PART_WGS = 256, DEC_PART_RG = 5;

static bool decode_part_ok(int64_t m, int64_t n)
{
    const int64_t groups = (n + 15) / 16;
    return m > 8 && groups >= 4 * DEC_PART_WGS && groups <= DEC_PART_RG * DEC_PART_WGS;
}

template <int MT, int QS, bool OUT_F32>
static hipError_t launch_decode_stream_qs(const GemmArgs& a, hipStream_t stream)
{
    const DecodeStreamCfg c = decode_stream_cfg(a.M, a.K);
    const dim3 block(256);
    if constexpr (MT <= 2) {
        if (decode_part_ok(a.M, a.N)) {
            auto kern = mx_decode_stream_kernel<MT, QS, 2, DEC_PART_RG, OUT_F32, true>;
            const size_t lds_p = decode_stream_lds_bytes(MT, QS * 512, DecodeStreamCfg{DEC_PART_RG, 2});
            static bool attr_set = false;  // benign race: setting the same value twice is harmless
            if (!attr_set) {
                const hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize,
                                                         (int)lds_p);
                if (e != hipSuccess) return e;
                attr_set = true;
            }
            hipLaunchKernelGGL(kern, dim3(DEC_PART_WGS), block, lds_p, stream, a);
            return hipGetLastError();
        }
    }
    const size_t lds = decode_stream_lds_bytes(MT, a.K, c);
    if (MT == 2 && c.rg == 2)
        hipLaunchKernelGGL((mx_decode_stream_kernel<MT, QS, 2, 2, OUT_F32>), dim3((a.N + 31) / 32), block, lds, stream, a);
    else if (c.slots == 3)
        hipLaunchKernelGGL((mx_decode_stream_kernel<MT, QS, 3, 1, OUT_F32>), dim3((a.N + 15) / 16), block, lds, stream, a);
    else
        hipLaunchKernelGGL((mx_decode_stream_kernel<MT, QS, QS / 2, 1, OUT_F32>), dim3((a.N + 15) / 16), block, lds, stream, a);
    return hipGetLastError();
}

template <int MT, bool OUT_F32>
static hipError_t launch_decode_stream(const GemmArgs& a, hipStream_t stream)
{
    switch (a.K / 512) {
    case 2: return launch_decode_stream_qs<MT, 2, OUT_F32>(a, stream);
    case 4: return launch_decode_stream_qs<MT, 4, OUT_F32>(a, stream);
    case 6: return launch_decode_stream_qs<MT, 6, OUT_F32>(a, stream);
    case 8: return launch_decode_stream_qs<MT, 8, OUT_F32>(a, stream);
    case 10: return launch_decode_stream_qs<MT, 10, OUT_F32>(a, stream);
    case 12: return launch_decode_stream_qs<MT, 12, OUT_F32>(a, stream);
    case 14: return launch_decode_stream_qs<MT, 14, OUT_F32>(a, stream);
    default: return launch_decode_stream_qs<MT, 16, OUT_F32>(a, stream);
    }
}

template <int MT>
static size_t decode_lds_bytes(int K)
{
    const size_t block = (size_t)16 * (K / 2), red = (size_t)4 * MT * 64 * 16;
    return (block > red ? block : red) + (size_t)16 * (1 + MT) * (K / 32);
}

// which decode kernel runs with MT 16-row A fragments: 2 = LDS block,
// 1 = direct loads (MT <= 2), 0 = generic
template <int MT>
static int decode_kind_mt(int64_t k)
{
    if (k % 128 != 0) return 0;
    if (k % 512 == 0 && k <= 8192 && decode_lds_bytes<MT>((int)k) <= 65536) return 2;
    if (MT <= 2 && decode_direct_lds_bytes<MT <= 2 ? MT : 2>((int)k) <= 65536) return 1;
    return 0;
}

static int decode_kind(int64_t m, int64_t k)
{
    if (m <= 16) return decode_kind_mt<1>(k);
    if (m <= 32) return decode_kind_mt<2>(k);
    return decode_kind_mt<3>(k);
}

template <int MT, bool OUT_F32>
hipError_t launch_decode(const GemmArgs& a, hipStream_t stream)
{
    if constexpr (MT <= 2) {
        if (decode_stream_ok(a.M, a.K)) return launch_decode_stream<MT, OUT_F32>(a, stream);
    }
    const int kind = decode_kind_mt<MT>(a.K);
    if (kind == 2)
        hipLaunchKernelGGL((mx_decode_kernel<MT, OUT_F32>), dim3((a.N + 15) / 16), dim3(256), decode_lds_bytes<MT>(a.K),
                           stream, a);
    else if (kind == 1 && MT <= 2)
        hipLaunchKernelGGL((mx_decode_direct_kernel<MT <= 2 ? MT : 2, MT == 1 ? 10 : 5, OUT_F32>), dim3((a.N + 31) / 32),
                           dim3(256), decode_direct_lds_bytes<MT <= 2 ? MT : 2>(a.K), stream, a);
    else
        hipLaunchKernelGGL((mx_decode_generic_kernel<MT, OUT_F32>), dim3((a.N + 15) / 16), dim3(512), 0, stream, a);
    return hipGetLastError();
}

} // namespace mxl

using namespace mxl;

// ---------------------------------------------------------------- dispatch
// Shape classes (MXFP4 and fast-path MXFP8):
//   decode  : M <= 48 (MXFP4)                     -> mx_decode_kernel
//   large   : MXFP4, M, N >= 1024, K % 128 == 0    -> 256x256 tiles, 2x2 waves of 128x128
//             (the E4M3 fragments are twice as wide and would spill there)
//   default : everything else                      -> 128x128 tiles, 2x2 waves of 64x64
enum ShapeClass { SC_DECODE, SC_LARGE, SC_DEFAULT };

static ShapeClass classify(int a_bits, int w_bits, int64_t m, int64_t n, int64_t k, bool fused)
{
    if (a_bits != 4 || w_bits != 4) return SC_DEFAULT;   // MXFP8 and mixed pairs: the 128 x 128 tile kernel
    // up to three 16-row A fragments: with a fourth the LDS-block kernel
    // needs 296 VGPRs (one wave per SIMD) and loses to the tile kernel
    if (!fused && a_bits == 4 && m <= 48) return SC_DECODE;
    if (a_bits == 4 && m >= 1024 && n >= 1024 && k % 128 == 0) return SC_LARGE;
    return SC_DEFAULT;
}

template <int AB, int WB, bool FUSED, int RULE, bool F32>
static hipError_t dispatch_tile(const GemmArgs& a, ShapeClass sc, hipStream_t s)
{
    if constexpr (AB == 4 && WB == 4) if (sc == SC_LARGE)
        return launch_tile<AB, WB, 256, 256, 2, 2, FUSED, RULE, F32, FUSED ? 1 : 3, true>(a, s);
    if constexpr (!FUSED) if (a.K % BK == 0)   // whole stages: dword scale loads, two stages in flight
        return launch_tile<AB, WB, 128, 128, 2, 2, FUSED, RULE, F32, 3, true>(a, s);
    return launch_tile<AB, WB, 128, 128, 2, 2, FUSED, RULE, F32>(a, s);
}

// Split-K plan of the 128 x 128 tile kernel (the default class): splits and
// stages per split; 1 split when the tiles already fill the machine.
static int default_splits(int64_t m, int64_t n, int64_t k, int* chunk)
{
    const int64_t tiles = ((m + 127) / 128) * ((n + 127) / 128);
    return mxl_choose_splits(tiles, (int)((k + BK - 1) / BK), 4, 0, 0, chunk);
}

template <int AB, int WB, bool FUSED, int RULE>
static hipError_t dispatch_out(const GemmArgs& a, ShapeClass sc, bool f32, hipStream_t s)
{
    if (f32) return dispatch_tile<AB, WB, FUSED, RULE, true>(a, sc, s);
    return dispatch_tile<AB, WB, FUSED, RULE, false>(a, sc, s);
}

extern "C" int mxl_prefill_ok(int64_t m, int64_t n, int64_t k);
extern "C" hipError_t mxl_launch_mx_prefill(const void* aq, const void* as, const void* wq, const void* ws,
                                            int64_t m, int64_t n, int64_t k, void* y, int out_f32,
                                            hipStream_t stream);

// Workspace bytes mx_gemm can use for split-K on this shape (0: none).
extern "C" size_t mxl_mx_gemm_workspace(int a_bits, int w_bits, int64_t m, int64_t n, int64_t k)
{
    if (classify(a_bits, w_bits, m, n, k, false) != SC_DEFAULT) return 0;
    int chunk;
    const int s = default_splits(m, n, k, &chunk);
    return s > 1 ? (size_t)s * m * n * sizeof(float) : 0;
}

extern "C" hipError_t mxl_launch_mx_gemm(int a_bits, int w_bits, const void* aq, const void* as,
                                         const void* wq, const void* ws, int64_t m, int64_t n,
                                         int64_t k, void* y, int out_f32, void* work, size_t work_bytes,
                                         hipStream_t stream)
{
    GemmArgs a{static_cast<const uint8_t*>(aq), static_cast<const uint8_t*>(as),
               static_cast<const uint8_t*>(wq), static_cast<const uint8_t*>(ws), y, (int)m, (int)n, (int)k,
               nullptr, 1, 1 << 30, nullptr, nullptr};
    const ShapeClass sc = classify(a_bits, w_bits, m, n, k, false);
    if (sc == SC_DEFAULT && work) {
        int chunk;
        const int splits = default_splits(m, n, k, &chunk);
        if (splits > 1 && work_bytes >= (size_t)splits * m * n * sizeof(float)) {
            a.part = static_cast<float*>(work);
            a.splits = splits;
            a.chunk = chunk;
            hipError_t e = hipErrorInvalidValue;
            if (a_bits == 4 && w_bits == 4) e = dispatch_out<4, 4, false, RULE_CEIL>(a, sc, true, stream);
            else if (a_bits == 8 && w_bits == 8) e = dispatch_out<8, 8, false, RULE_CEIL>(a, sc, true, stream);
            else if (a_bits == 8 && w_bits == 4) e = dispatch_out<8, 4, false, RULE_CEIL>(a, sc, true, stream);
            else if (a_bits == 4 && w_bits == 8) e = dispatch_out<4, 8, false, RULE_CEIL>(a, sc, true, stream);
            if (e != hipSuccess) return e;
            return mxl_launch_splitk_reduce(a.part, splits, m * n, 1.0f, y, out_f32, stream);
        }
    }
    if (sc == SC_LARGE && mxl_prefill_ok(m, n, k))
        return mxl_launch_mx_prefill(aq, as, wq, ws, m, n, k, y, out_f32, stream);
    if (sc == SC_DECODE) {
        if (m <= 16) return out_f32 ? launch_decode<1, true>(a, stream) : launch_decode<1, false>(a, stream);
        if (m <= 32) return out_f32 ? launch_decode<2, true>(a, stream) : launch_decode<2, false>(a, stream);
        return out_f32 ? launch_decode<3, true>(a, stream) : launch_decode<3, false>(a, stream);
    }
    if (a_bits == 4 && w_bits == 4) return dispatch_out<4, 4, false, RULE_CEIL>(a, sc, out_f32, stream);
    if (a_bits == 8 && w_bits == 8) return dispatch_out<8, 8, false, RULE_CEIL>(a, sc, out_f32, stream);
    if (a_bits == 8 && w_bits == 4) return dispatch_out<8, 4, false, RULE_CEIL>(a, sc, out_f32, stream);
    if (a_bits == 4 && w_bits == 8) return dispatch_out<4, 8, false, RULE_CEIL>(a, sc, out_f32, stream);
    return hipErrorInvalidValue;
}

// Whether the kernel that mx_gemm (fused_in_tile: mx_gemm_fused with the
// in-tile prologue) selects for this shape can address its operands.  The
// prefill kernel checks its own limits (mxl_prefill_ok); the tile and decode
// kernels take 32-bit byte offsets and buffer sizes, so their operands (plus
// one tile of overrun rows) must stay below 2 GiB.
extern "C" int mxl_mx_gemm_fits(int a_bits, int w_bits, int64_t m, int64_t n, int64_t k, int fused_in_tile)
{
    const ShapeClass sc = classify(a_bits, w_bits, m, n, k, fused_in_tile != 0);
    if (!fused_in_tile && sc == SC_LARGE && mxl_prefill_ok(m, n, k)) return 1;
    const int64_t lim = (int64_t)1 << 31;
    const int64_t a_row = fused_in_tile ? 2 * k : k * a_bits / 8, w_row = k * w_bits / 8;
    return (m + 256) * a_row < lim && (n + 256) * w_row < lim ? 1 : 0;
}

extern "C" size_t mxl_prefill_fq_workspace(int64_t m, int64_t k);
extern "C" hipError_t mxl_launch_mx_prefill_fq(int a_rule, const void* a_bf16, const void* wq, const void* ws,
                                               int64_t m, int64_t n, int64_t k, void* y, int out_f32, void* work,
                                               size_t work_bytes, hipStream_t stream);

// Workspace bytes mx_gemm_fused can use on this shape: the quantize-once
// launch for large MXFP4 shapes (0: none).
extern "C" size_t mxl_mx_gemm_fused_workspace(int a_bits, int64_t m, int64_t n, int64_t k)
{
    if (a_bits == 4 && classify(4, 4, m, n, k, true) == SC_LARGE && mxl_prefill_ok(m, n, k))
        return mxl_prefill_fq_workspace(m, k);
    return 0;
}

extern "C" hipError_t mxl_launch_mx_gemm_fused(int a_bits, int a_rule, const void* a_bf16, int w_bits,
                                               const void* wq, const void* ws, int64_t m, int64_t n,
                                               int64_t k, void* y, int out_f32, void* dump_q, void* dump_s,
                                               void* work, size_t work_bytes, hipStream_t stream)
{
    // large MXFP4 shapes with a workspace: quantize A once, in the same launch
    if (!dump_q && a_bits == 4 && w_bits == 4 && work) {
        const size_t need = mxl_mx_gemm_fused_workspace(a_bits, m, n, k);
        if (need > 0 && work_bytes >= need) {
            const hipError_t e = mxl_launch_mx_prefill_fq(a_rule, a_bf16, wq, ws, m, n, k, y, out_f32, work,
                                                          work_bytes, stream);
            return e;
        }
    }
    GemmArgs a{static_cast<const uint8_t*>(a_bf16), nullptr, static_cast<const uint8_t*>(wq),
               static_cast<const uint8_t*>(ws), y, (int)m, (int)n, (int)k, nullptr, 1, 1 << 30,
               static_cast<uint8_t*>(dump_q), static_cast<uint8_t*>(dump_s)};
    // the dump is built into the 128 x 128 fused kernel only (the 256 x 256
    // one has no registers to spare); both accumulate alike
    const ShapeClass sc = dump_q ? SC_DEFAULT : classify(a_bits, w_bits, m, n, k, true);
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

extern "C" const char* mxl_mx_gemm_config_name(int a_bits, int w_bits, int64_t m, int64_t n, int64_t k, int fused)
{
    switch (classify(a_bits, w_bits, m, n, k, fused != 0)) {
    case SC_DECODE:
        if (decode_stream_ok(m, k) && decode_part_ok(m, n))
            return "mx_decode_stream_kernel<one workgroup per compute unit over 4-5 16-row W groups (each A fragment "
                   "serves all of them), each wave streams its own K quarter through a ring of 2 LDS pair slots (8 rows "
                   "x 128 B non-temporal copies) and computes each stage as its copies land, scaled mfma 16x16x128>";
        if (decode_stream_ok(m, k))
            return m > 16 ? "mx_decode_stream_kernel<32 W rows per workgroup (each A fragment serves both 16-row groups), "
                            "each wave streams its own K quarter through a ring of 2 LDS pair slots (8 rows x 128 B "
                            "non-temporal copies) and computes each stage as its copies land, scaled mfma 16x16x128>"
                   : decode_stream_ring(m, k)
                       ? "mx_decode_stream_kernel<16 W rows per workgroup, each wave streams its own K quarter through a "
                         "ring of 3 LDS pair slots (8 rows x 128 B non-temporal copies) and computes each stage as its "
                         "copies land, scaled mfma 16x16x128>"
                       : "mx_decode_stream_kernel<16 W rows per workgroup, each wave copies its whole K quarter into LDS "
                         "(8 rows x 128 B non-temporal copies) and computes each stage as its copies land, scaled mfma "
                         "16x16x128>";
        switch (decode_kind(m, k)) {
        case 2: return "mx_decode_kernel<16 W rows per workgroup, whole-row copies into swizzled LDS, 4 waves over K "
                       "quarters, scaled mfma 16x16x128>";
        case 1: return "mx_decode_direct_kernel<32 W rows per workgroup, 4 waves over K quarters, scales staged in LDS, "
                       "scaled mfma 16x16x128>";
        default: return "mx_decode_generic_kernel<16 W rows per workgroup, 8-wave split-K, scaled mfma 16x16x128>";
        }
    case SC_LARGE:
        if (!fused && mxl_prefill_ok(m, n, k))
            return "mx_gemm_prefill_kernel<tile 256x256x128, 2x2 waves of 128x128, two 256-K pair slots + "
                   "4-pair scale windows fed by buffer-to-LDS copies, stage-ahead fragments, scaled mfma 32x32x64; "
                   "a last round of tiles at most half full runs as 256x128 halves>";
        if (fused && a_bits == 4 && mxl_prefill_ok(m, n, k))
            return "mx_gemm_prefill_fq_kernel<A quantized once into the workspace from a pool of 32-row chunks, "
                   "then the prefill tiles> with a workspace, else mx_gemm_kernel<tile 256x256x128, 2x2 waves of "
                   "128x128, scaled mfma 32x32x64, A quantized in each tile>";
        return "mx_gemm_kernel<tile 256x256x128, 2x2 waves of 128x128, scaled mfma 32x32x64>";
    default:
        if (!fused) {
            int chunk;
            const int s = default_splits(m, n, k, &chunk);
            if (s > 1) {
                static thread_local char buf[192];
                std::snprintf(buf, sizeof buf,
                              "mx_gemm_kernel<tile 128x128x128, 2x2 waves of 64x64, scaled mfma 32x32x64>, "
                              "split-K %d x %d stages with a workspace, else one split", s, chunk);
                return buf;
            }
        }
        return "mx_gemm_kernel<tile 128x128x128, 2x2 waves of 64x64, scaled mfma 32x32x64>";
    }
}
