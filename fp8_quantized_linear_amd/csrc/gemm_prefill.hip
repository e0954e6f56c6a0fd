// gemm_prefill.hip -- the large-shape MXFP4 GEMM for gfx950:
//   Y[M, N] = A[M, K] * W[N, K]^T, E2M1 codes with an E8M0 scale per 32 along
//   K, fp32 accumulation on v_mfma_scale_f32_32x32x64_f8f6f4, bf16/fp32 output.
//
// Operation: the W4A4 FP4 GEMM that serves the MXFP4 checkpoints
// (Qwen3.5-9B-MXFP4-QAD-W4A4-LR1e-5-s3000, "Serving"), for prefill-sized M.
//
// Design (one 256 x BN output tile per workgroup of 4 waves, 2 x 2 waves, each
// wave a 128 x BN/2 sub-tile of 32x32 matrix-core fragments held in AGPRs;
// BN = 256 for the bulk of the tiles, 128 for the tail, see below):
//  * K advances in pairs of 256 elements, each computed as two sub-stages of
//    128.  A pair's codes (32 KiB of A, BN * 128 bytes of W) live in one of
//    two LDS slots, 128 bytes per row, so that every copy moves 8 rows x 128
//    contiguous bytes (whole cache lines).  The E8M0 scales travel
//    separately, in windows of 4 pairs (32 bytes per row per operand) held in
//    two LDS buffers: fetching the 8 scale bytes of a row per pair would cost
//    one 64-row gather per 512 bytes, which measured as the dominant cost of
//    the loop; a window moves 32 contiguous bytes per row.  For BN = 256 the
//    slots and windows fill the 160 KiB of LDS exactly.
//  * Everything is copied global -> LDS by the buffer-load-to-LDS path (each
//    instruction writes 64 lanes x its width contiguously at the address in
//    M0), so no registers are spent on staging.  The swizzled code layout is
//    obtained by choosing, per lane, which global 16-byte chunk lands at that
//    lane's LDS position.  All offsets are per-lane, so the buffer range
//    check turns anything past the end of A or W into zeros (rows past M or
//    N, the half pair when K % 256 == 128); copies past the last pair use a
//    zero-sized buffer and fill a free slot with zeros, which keeps the loop
//    free of branches and the outstanding-copy count the same every pair.
//  * During the second sub-stage of pair p every wave issues the same number
//    of copies: 2 A and 2 W scale copies (8 rows x 32 B each) of a window,
//    then 8 A and BN/32 W code copies of pair p + 2 into the slot of pair p,
//    whose fragments were all read by then.  With BN = 128 a window piece
//    has only 4 W copies, so two waves copy from a zero-sized buffer into a
//    dummy area to keep the count uniform.  The copies come from inline
//    assembly the compiler does not track: at the start of each second
//    sub-stage every wave waits for all of its copies (vmcnt(0); they were
//    issued two sub-stages earlier) and a workgroup barrier publishes them.
//    That is the loop's only barrier.
//  * The fragments of sub-stage s+1 are read from LDS while the
//    matrix-core instructions of sub-stage s run, into a second register set,
//    so no LDS latency is exposed; the loop is unrolled by two to alternate
//    the sets without copies.  Reads, copies and matrix-core instructions are
//    spread evenly and pinned in place with scheduling barriers.
//  * W is the matrix core's first operand, A the second, so each lane's
//    accumulator holds 4 consecutive output columns; the epilogue stages each
//    32-row band of a wave's tile through LDS and writes whole row segments
//    to Y.
//  * Matrix-core layout (32x32x64, E2M1): lane l = r + 32 g holds row r of a
//    fragment and K elements [32 g, 32 g + 32) of the 64-wide step; lane
//    group g supplies the E8M0 scale of K block g.  Accumulator register i of
//    lane l is C[(i/4)*8 + g*4 + i%4][r] with C = W_frag x A_frag^T.
//  * Tile order: workgroup ids are first mapped XCD-aware (dispatch is
//    round-robin over the 8 XCDs, each with its own L2: each XCD gets a
//    contiguous range of the order), then walk groups of 4 tile columns down
//    M (N fastest inside a group).
//  * Tail: with C compute units, T tiles take ceil(T / C) rounds.  When the
//    last round is at most half full (0 < T mod C <= C/2), the T mod C tiles
//    at the end of the order are computed by a second launch as 256 x 128
//    halves, so that round costs about half a tile instead of a full one.
//    Every output element accumulates the same sub-stages in the same order
//    in both kernels, so the split does not change any result.
// Requires K % 128 == 0; other shapes use the general tile kernel.
#include "mx_device.h"

#include <type_traits>

namespace mxl {

constexpr int PF_BM = 256, PF_BK = 128;            // tile rows of A; K per sub-stage
constexpr int PF_PK = 256;                         // K per pair
constexpr int PF_PROWB = PF_PK / 2;                // 128 code bytes of a row per pair
constexpr int PF_ATILE = PF_BM * PF_PROWB;         // 32 KiB of A codes per pair
constexpr int PF_NSL = 2;                          // pair slots
constexpr int PF_WPAIRS = 4;                       // pairs per scale window
constexpr int PF_SWB = PF_WPAIRS * 8;              // 32 scale bytes per row per window
constexpr int PF_NWIN = 2;                         // scale window buffers
constexpr int PF_GROUP_N = 4;                      // tile columns per group of the tile order

// LDS layout for tile width BN: A code slots [2][32 KiB], W code slots
// [2][BN x 128 B], scale windows [2][A 256 x 32 B | W BN x 32 B], then (BN =
// 128) 1 KiB that absorbs the scale copies of waves with none to make.  Both
// slots of an operand lie within 64 KiB of its first, so a per-lane base
// register reaches every fragment of either slot through the read's 16-bit
// immediate offset.
template <int BN>
struct PfLayout {
    static constexpr int W_TILE = BN * PF_PROWB;
    static constexpr int W0 = PF_NSL * PF_ATILE;   // W code slots
    static constexpr int WIN = (PF_BM + BN) * PF_SWB;
    static constexpr int SC0 = W0 + PF_NSL * W_TILE;
    static constexpr int DUMMY = SC0 + PF_NWIN * WIN;
    static constexpr int LDS = DUMMY + (BN == 256 ? 0 : 1024);   // 163840 bytes for BN = 256
    static constexpr int WFR = BN / 64;            // W fragments per wave (a wave covers BN/2 W rows)
    static constexpr int ACOP = PF_ATILE / 1024 / 4;        // 8 A code copies per wave per pair
    static constexpr int WCOP = BN * PF_PROWB / 1024 / 4;   // BN/32 W code copies per wave per pair
    static constexpr int SCOP = 4;                 // scale copies per wave per pair (2 A, 2 W)
    static constexpr int COPIES = SCOP + ACOP + WCOP;
    static constexpr int READS = 8 + 2 * WFR + 4 + WFR;     // LDS reads per lane per sub-stage
    static constexpr int MFMAS = 8 * WFR;          // matrix-core instructions per wave per sub-stage
    static constexpr int READ_SPAN = MFMAS * 3 / 4;  // reads go out during the first 3/4 of a
                                                     // sub-stage, leaving the rest to cover them
    static_assert(LDS <= 163840, "LDS");
    static_assert((PF_NSL - 1) * PF_ATILE + 3 * 32 * PF_PROWB < 65536 &&
                      (PF_NSL - 1) * W_TILE + (WFR - 1) * 32 * PF_PROWB < 65536,
                  "fragment offsets fit the read's immediate");
};

struct PrefillArgs {
    const uint8_t* a_q; const uint8_t* a_s;
    const uint8_t* w_q; const uint8_t* w_s;
    void* y;
    uint8_t* h_q; uint8_t* h_s;   // SwiGLU epilogue: MXFP4 codes and scales of h
    int M, N, K;
    int tile_base;   // first tile (in the tile order) of this launch
    int count;       // workgroups of this launch
    float alpha;     // NVFP4: Y = alpha * accumulator
};

// 16-byte chunk swizzle of the 128-byte LDS rows: the lanes reading the same
// logical chunk of 16 consecutive rows touch distinct banks.
__device__ __forceinline__ int pf_swz(int row) { return (row >> 1) & 7; }

// This workgroup's index in [0, count): workgroup b runs on XCD b % 8, and
// each XCD receives one contiguous range.
__device__ __forceinline__ int pf_xcd_order(int count)
{
    const int id = blockIdx.x;
    const int xcd = id % NUM_XCD, j = id / NUM_XCD;
    const int q = count / NUM_XCD, r = count % NUM_XCD;
    return xcd * q + (xcd < r ? xcd : r) + j;
}

// Tile t of the grouped order over the 256 x 256 tile grid.
__device__ __forceinline__ void pf_tile(int t, int M, int N, int& tm, int& tn)
{
    const int tiles_m = (M + PF_BM - 1) / PF_BM, tiles_n = (N + 255) / 256;
    const int group_size = PF_GROUP_N * tiles_m;
    const int first_n = (t / group_size) * PF_GROUP_N;
    const int gn = (tiles_n - first_n) < PF_GROUP_N ? (tiles_n - first_n) : PF_GROUP_N;
    const int in = t % group_size;
    tm = in / gn;
    tn = first_n + in % gn;
}

// LDS reads at a byte address of the workgroup's LDS
__device__ __forceinline__ int4_t lds_read_b128(uint32_t addr)
{
    return *reinterpret_cast<const __attribute__((address_space(3))) int4_t*>((size_t)addr);
}
__device__ __forceinline__ uint32_t lds_read_b32(uint32_t addr)
{
    return *reinterpret_cast<const __attribute__((address_space(3))) uint32_t*>((size_t)addr);
}

// one sub-stage's operands in registers: code fragments per 64-wide step kk,
// and the raw scale dwords (4 blocks of the sub-stage) of this lane's rows
template <int WFR>
struct PfFrags {
    int4_t a[2][4], w[2][WFR];
    int sa[4], sw[WFR];
};

// The uniform part of the copies issued during one pair: buffer descriptors
// (zero-sized once past the last pair or window), the K offset and LDS slot
// of the code copies, and the LDS bases and buffer offsets of the
// scale-window piece.
struct PfPairCopies {
    int4_t ra, rw, ras, rws;
    int coff, asoff, wsoff;
    uint32_t adst, wdst, asdst, wsdst;
};

// EPI selects the epilogue: PF_EPI_Y stores Y; PF_EPI_SWIGLU applies SwiGLU
// to gate/up column pairs and stores h quantized to MXFP4 (CEIL rule).
constexpr int PF_EPI_Y = 0, PF_EPI_SWIGLU = 1;

template <bool OUT_F32, int BN, int EPI>
__global__ __launch_bounds__(256, 1) void mx_gemm_prefill_kernel(PrefillArgs p)
{
    extern __shared__ __align__(16) uint8_t smem[];
#define PF_TILE_T pf_xcd_order(p.count)
#include "gemm_prefill_tile.inc"
#undef PF_TILE_T
}

// The large-shape exact MXFP8 GEMM: E4M3 codes with E8M0 scales per 32,
// converted exactly to bf16 in registers and contracted on the bf16 matrix
// cores, in the FP4 kernel's tile structure (gemm_tile8.inc).  The MXFP8 W8A8
// attention projections of Qwen3.8-27B-MXFP8Attn-MXFP4MLP-lmheadMXFP4
// (introduction, section 2).  Requires K % 128 == 0.
template <bool OUT_F32, int BN>
__global__ __launch_bounds__(256, 1) void mx8_gemm_tile_kernel(PrefillArgs p)
{
    extern __shared__ __align__(16) uint8_t smem[];
#define PF_TILE_T pf_xcd_order(p.count)
#include "gemm_tile8.inc"
#undef PF_TILE_T
}

// The large-shape exact NVFP4 GEMM on 8 waves (two per SIMD), in the tile
// structure of the kernels above (gemm_tile_dq8w.inc): the codes are
// converted to f16 and multiplied by their E4M3 block scales in registers, 6
// vector instructions per matrix-core instruction, more than one wave per
// SIMD can issue beside the matrix cores.  Requires K % 256 == 0.  The body
// also holds the MXFP8 variant; MXFP8 runs on the 4-wave kernel instead,
// which converts each code twice per tile rather than up to four times and
// measured as fast (226.9 against 232.9 us on 4096 x 6144 x 5120, bitwise
// equal): the bf16 matrix cores run at a power-limited clock, and the extra
// conversions cost as much as the extra issue slots gain.
constexpr int DQ8W_MXFP8 = 1, DQ8W_NVFP4 = 2;
template <int FMT, bool OUT_F32, int BN>
__global__ __launch_bounds__(512, 1) void dq8w_gemm_tile_kernel(PrefillArgs p)
{
    extern __shared__ __align__(16) uint8_t smem[];
#define PF_TILE_T pf_xcd_order(p.count)
#include "gemm_tile_dq8w.inc"
#undef PF_TILE_T
}

// ---------------------------------------------------------------------------
// Fused activation quantization for the large shapes, quantizing A once.
// A prologue inside each tile (mx_gemm_kernel<FUSED>) redoes the quantization
// of its A block for every tile column: 68 times for the 8192 x 5120 x 17408
// projection.  Here the workgroups quantize each 256-row block of A once,
// into a workspace, exactly as mx_quantize_act does (the same device
// functions, the same layout), and the tiles read the codes from there.
//
// Before its tile, a workgroup claims 32-row chunks of A (of any block) from
// a pool counter and quantizes them until the pool is empty, then waits until
// its own block's done counter shows every chunk of the block.  It only ever
// waits for chunks that running workgroups have claimed and finish without
// waiting, so the scheme needs no co-residency and runs as ordinary launches
// (the same two as mx_gemm: 256 x 256 tiles, then the 256 x 128 halves of a
// last round at most half full).  The first round of workgroups quantizes
// all of A together; later ones find the pool empty and their block done.
//
// Visibility: a chunk's writer waits for its stores (acknowledged by the L2)
// and, from one thread, releases (one write-back of its XCD's L2) before
// counting the chunk done.  A reader polls the done counter with device-scope
// atomic loads and needs no invalidation: the codes are read only after their
// block is done, no L2 holds lines of the block from before (the launch
// starts with the caches' acquire, the region is written only here, and
// blocks start on cache-line boundaries: the workspace is 256-byte aligned,
// the scale plane starts at the next 256-byte boundary after the codes, and a
// block holds 256 rows of k/2 code bytes and of k/32 scale bytes, k % 128 ==
// 0, so no cache line holds bytes of two blocks).  Every poll is bounded
// (about 0.5 s); a tile that gives up sets the error word and fills its part
// of Y with NaN, so that no mistake can hang the GPU or pass for a result.
// ---------------------------------------------------------------------------
constexpr int PF_FQ_CHUNK_ROWS = 32;
constexpr int PF_FQ_SPINS = 1 << 21;           // x s_sleep(4): about 0.5 s

// mx_quantize_act (MXFP4, rule RULE) of rows [r0, r1) of A (bf16, k per row):
// the per-group work of mx_quantize_kernel; consecutive threads take
// consecutive 8-element groups, so lane quads hold the blocks of 32.  Each
// thread loads 16 groups before it encodes any (one workgroup per CU streams
// the chunk; 32 measured the same), and a lane quad is always wholly inside
// or wholly past r1 (k / 8 is a multiple of 16 groups).
template <int RULE>
__device__ __forceinline__ void pf_quantize_rows(const uint4* __restrict__ x, int k, int r0, int r1,
                                                 uint8_t* __restrict__ q, uint8_t* __restrict__ s)
{
    constexpr int G = 16;
    const int lane = threadIdx.x & 63;
    const int64_t g_end = (int64_t)r1 * (k / 8);
    for (int64_t g0 = (int64_t)r0 * (k / 8) + threadIdx.x; g0 < g_end; g0 += G * 256) {
        uint4 v[G];
#pragma unroll
        for (int j = 0; j < G; ++j) {
            const int64_t g = g0 + 256 * j;
            v[j] = x[g < g_end ? g : g0];
        }
#pragma unroll
        for (int j = 0; j < G; ++j) {
            const int64_t g = g0 + 256 * j;
            const int e = scale_exponent<ELEM_E2M1, RULE>(quad_max_u32(amax_bits8(v[j])));
            const uint32_t c = encode8_e2m1(v[j], e);
            if (g < g_end) {
                reinterpret_cast<uint32_t*>(q)[g] = c;
                if ((lane & 3) == 0) s[g >> 2] = (uint8_t)(e + 127);
            }
        }
    }
}

// Makes sure A block tm (rows [256 tm, 256 tm + 256) clipped to M) is
// quantized into p.a_q / p.a_s.  Before that, the workgroup takes chunks from
// the pool of all blocks' chunks (chunk c: block c / 8, rows 32 (c % 8) ..
// of it) until the pool is empty, so the first round of workgroups quantizes
// all of A together.  state: the pool counter, done counters [nb] (8 chunks
// each, empty chunks past M included), the error word.  Returns false if the
// poll gave up.
template <int RULE>
__device__ __forceinline__ bool pf_ensure_block(const PrefillArgs& p, const uint4* a_bf16, int* state, int nb,
                                                int tm, uint8_t* smem)
{
    constexpr int CPB = PF_BM / PF_FQ_CHUNK_ROWS;    // chunks per block
    int* pool = state;
    int* done = state + 1;
    int* word = reinterpret_cast<int*>(smem);
    while (true) {
        __syncthreads();
        if (threadIdx.x == 0) *word = __hip_atomic_fetch_add(pool, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __syncthreads();
        const int c = *word;
        if (c >= nb * CPB) break;
        const int b = c / CPB, r0 = b * PF_BM + (c % CPB) * PF_FQ_CHUNK_ROWS;
        const int r1 = min(r0 + PF_FQ_CHUNK_ROWS, p.M);
        if (r0 < r1)
            pf_quantize_rows<RULE>(a_bf16, p.K, r0, r1, const_cast<uint8_t*>(p.a_q), const_cast<uint8_t*>(p.a_s));
        wait_vmcnt<0>();
        __syncthreads();
        if (threadIdx.x == 0) __hip_atomic_fetch_add(done + b, 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        int v = 0;
        for (int spin = 0; spin < PF_FQ_SPINS; ++spin) {
            v = __hip_atomic_load(done + tm, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            if (v >= CPB) break;
            __builtin_amdgcn_s_sleep(4);
        }
        if (v < CPB) __hip_atomic_store(state + 1 + nb, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        *word = v >= CPB ? 1 : 0;
    }
    __syncthreads();
    const bool ok = *word != 0;
    __syncthreads();   // the tile reuses this LDS word
    return ok;
}

// The prefill kernel with the quantize-once prologue: p.a_q / p.a_s point at
// the workspace's codes and scales, a_bf16 is A; state as above, zeroed
// before the first of the call's launches.
template <bool OUT_F32, int BN, int RULE>
__global__ __launch_bounds__(256, 1) void mx_gemm_prefill_fq_kernel(PrefillArgs p, const uint4* a_bf16, int* state,
                                                                    int nb)
{
    constexpr int EPI = PF_EPI_Y;
    extern __shared__ __align__(16) uint8_t smem[];
    const int tile_t = pf_xcd_order(p.count);
    int tm, tn;
    pf_tile(p.tile_base + (BN == 256 ? tile_t : tile_t / 2), p.M, p.N, tm, tn);
    if (!pf_ensure_block<RULE>(p, a_bf16, state, nb, tm, smem)) {
        fill_tile_nan(p.y, p.M, p.N, tm * PF_BM, tn * 256 + (BN == 256 ? 0 : (tile_t % 2) * 128), PF_BM, BN,
                      OUT_F32);
        return;
    }
#define PF_TILE_T tile_t
#include "gemm_prefill_tile.inc"
#undef PF_TILE_T
}

template <bool OUT_F32, int BN, int EPI>
hipError_t launch_prefill_part(PrefillArgs a, int tile_base, int count, hipStream_t stream)
{
    auto kern = mx_gemm_prefill_kernel<OUT_F32, BN, EPI>;
    static bool attr_set = false;
    if (!attr_set) {
        hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize,
                                           PfLayout<BN>::LDS);
        if (e != hipSuccess) return e;
        attr_set = true;
    }
    a.tile_base = tile_base;
    a.count = count;
    hipLaunchKernelGGL(kern, dim3(count), dim3(256), PfLayout<BN>::LDS, stream, a);
    return hipGetLastError();
}

// Compute units of the current device (cached per device).
static int prefill_cu_count()
{
    static int cached[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    if (cached[dev] == 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
        cached[dev] = n;
    }
    return cached[dev];
}

// Tiles of the tail launch (0: none) for T tiles on C compute units.
static int prefill_tail_tiles(int T, int C)
{
    const int rem = T % C;
    return (rem > 0 && 2 * rem <= C) ? rem : 0;
}

template <bool OUT_F32, int EPI = PF_EPI_Y>
hipError_t launch_prefill(const PrefillArgs& a, hipStream_t stream)
{
    const int T = ((a.M + PF_BM - 1) / PF_BM) * ((a.N + 255) / 256);
    const int tail = prefill_tail_tiles(T, prefill_cu_count());
    if (T - tail > 0) {
        const hipError_t e = launch_prefill_part<OUT_F32, 256, EPI>(a, 0, T - tail, stream);
        if (e != hipSuccess) return e;
    }
    if (tail > 0) return launch_prefill_part<OUT_F32, 128, EPI>(a, T - tail, 2 * tail, stream);
    return hipSuccess;
}

template <bool OUT_F32, int BN>
static hipError_t launch_mx8_part(PrefillArgs a, int tile_base, int count, hipStream_t stream)
{
    auto kern = mx8_gemm_tile_kernel<OUT_F32, BN>;
    static bool attr_set = false;
    if (!attr_set) {
        hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize,
                                           PfLayout<BN>::LDS);
        if (e != hipSuccess) return e;
        attr_set = true;
    }
    a.tile_base = tile_base;
    a.count = count;
    hipLaunchKernelGGL(kern, dim3(count), dim3(256), PfLayout<BN>::LDS, stream, a);
    return hipGetLastError();
}

template <bool OUT_F32>
static hipError_t launch_mx8(const PrefillArgs& a, hipStream_t stream)
{
    const int T = ((a.M + PF_BM - 1) / PF_BM) * ((a.N + 255) / 256);
    const int tail = prefill_tail_tiles(T, prefill_cu_count());
    if (T - tail > 0) {
        const hipError_t e = launch_mx8_part<OUT_F32, 256>(a, 0, T - tail, stream);
        if (e != hipSuccess) return e;
    }
    if (tail > 0) return launch_mx8_part<OUT_F32, 128>(a, T - tail, 2 * tail, stream);
    return hipSuccess;
}

template <int FMT, bool OUT_F32, int BN>
static hipError_t launch_dq8w_part(PrefillArgs a, int tile_base, int count, hipStream_t stream)
{
    auto kern = dq8w_gemm_tile_kernel<FMT, OUT_F32, BN>;
    static bool attr_set = false;
    if (!attr_set) {
        hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize,
                                           PfLayout<BN>::LDS);
        if (e != hipSuccess) return e;
        attr_set = true;
    }
    a.tile_base = tile_base;
    a.count = count;
    hipLaunchKernelGGL(kern, dim3(count), dim3(512), PfLayout<BN>::LDS, stream, a);
    return hipGetLastError();
}

template <int FMT, bool OUT_F32>
static hipError_t launch_dq8w(const PrefillArgs& a, hipStream_t stream)
{
    const int T = ((a.M + PF_BM - 1) / PF_BM) * ((a.N + 255) / 256);
    const int tail = prefill_tail_tiles(T, prefill_cu_count());
    if (T - tail > 0) {
        const hipError_t e = launch_dq8w_part<FMT, OUT_F32, 256>(a, 0, T - tail, stream);
        if (e != hipSuccess) return e;
    }
    if (tail > 0) return launch_dq8w_part<FMT, OUT_F32, 128>(a, T - tail, 2 * tail, stream);
    return hipSuccess;
}

// Clears the quantize-once state (pool and done counters, error word).
__global__ void pf_zero_kernel(int* p, int n)
{
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) p[i] = 0;
}

// Workspace layout of the quantize-once launches (256-byte aligned base): A
// codes [m, k/2] at 0, E8M0 scales [m, k/32] (mx_quantize_act's layout) at
// the next 256-byte boundary, then at the next one the state: the chunk pool
// counter, a done counter per 256-row block, and an error word.
static size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }
static size_t prefill_fq_scale_offset(int64_t m, int64_t k) { return align256((size_t)m * (k / 2)); }
static size_t prefill_fq_state_offset(int64_t m, int64_t k)
{
    return align256(prefill_fq_scale_offset(m, k) + (size_t)m * (k / 32));
}

template <bool OUT_F32, int BN, int RULE>
static hipError_t launch_prefill_fq_part(PrefillArgs a, int tile_base, int count, const uint4* x, int* state,
                                         int nb, hipStream_t stream)
{
    auto kern = mx_gemm_prefill_fq_kernel<OUT_F32, BN, RULE>;
    static bool attr_set = false;
    if (!attr_set) {
        hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize,
                                           PfLayout<BN>::LDS);
        if (e != hipSuccess) return e;
        attr_set = true;
    }
    a.tile_base = tile_base;
    a.count = count;
    hipLaunchKernelGGL(kern, dim3(count), dim3(256), PfLayout<BN>::LDS, stream, a, x, state, nb);
    return hipGetLastError();
}

template <bool OUT_F32, int RULE>
static hipError_t launch_prefill_fq(PrefillArgs a, const void* a_bf16, int* state, hipStream_t stream)
{
    const int nb = (a.M + PF_BM - 1) / PF_BM;
    hipLaunchKernelGGL(pf_zero_kernel, dim3((nb + 2 + 255) / 256), dim3(256), 0, stream, state, nb + 2);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const uint4* x = static_cast<const uint4*>(a_bf16);
    const int T = ((a.M + PF_BM - 1) / PF_BM) * ((a.N + 255) / 256);
    const int tail = prefill_tail_tiles(T, prefill_cu_count());
    if (T - tail > 0) {
        e = launch_prefill_fq_part<OUT_F32, 256, RULE>(a, 0, T - tail, x, state, nb, stream);
        if (e != hipSuccess) return e;
    }
    if (tail > 0) return launch_prefill_fq_part<OUT_F32, 128, RULE>(a, T - tail, 2 * tail, x, state, nb, stream);
    return hipSuccess;
}

} // namespace mxl

using namespace mxl;

// Workspace bytes of the quantize-once fused launches (mxl_prefill_ok shapes).
extern "C" size_t mxl_prefill_fq_workspace(int64_t m, int64_t k)
{
    const int64_t nb = (m + PF_BM - 1) / PF_BM;
    return prefill_fq_state_offset(m, k) + (((size_t)(nb + 2) * sizeof(int) + 255) & ~(size_t)255);
}

// The quantize-once fused GEMM: A bf16 [m, k] quantized with rule a_rule
// (MXFP4) into `work` (at least mxl_prefill_fq_workspace bytes, 256-byte
// aligned; calls sharing it must not overlap), and Y = A W^T.
extern "C" hipError_t mxl_launch_mx_prefill_fq(int a_rule, const void* a_bf16, const void* wq, const void* ws,
                                               int64_t m, int64_t n, int64_t k, void* y, int out_f32, void* work,
                                               size_t work_bytes, hipStream_t stream)
{
    if (!work || work_bytes < mxl_prefill_fq_workspace(m, k) || (reinterpret_cast<uintptr_t>(work) & 255))
        return hipErrorInvalidValue;
    uint8_t* w8 = static_cast<uint8_t*>(work);
    PrefillArgs a{w8, w8 + prefill_fq_scale_offset(m, k), static_cast<const uint8_t*>(wq),
                  static_cast<const uint8_t*>(ws),
                  y, nullptr, nullptr, (int)m, (int)n, (int)k, 0, 0};
    int* state = reinterpret_cast<int*>(w8 + prefill_fq_state_offset(m, k));
    if (a_rule == RULE_CEIL)
        return out_f32 ? launch_prefill_fq<true, RULE_CEIL>(a, a_bf16, state, stream)
                       : launch_prefill_fq<false, RULE_CEIL>(a, a_bf16, state, stream);
    if (a_rule == RULE_FLOOR)
        return out_f32 ? launch_prefill_fq<true, RULE_FLOOR>(a, a_bf16, state, stream)
                       : launch_prefill_fq<false, RULE_FLOOR>(a, a_bf16, state, stream);
    return out_f32 ? launch_prefill_fq<true, RULE_EVEN>(a, a_bf16, state, stream)
                   : launch_prefill_fq<false, RULE_EVEN>(a, a_bf16, state, stream);
}

// Shapes this kernel accepts: K % 128 == 0 and every operand below 2 GiB
// (32-bit buffer offsets).  The caller checks them (mxl_prefill_ok).
extern "C" int mxl_prefill_ok(int64_t m, int64_t n, int64_t k)
{
    if (k % PF_BK != 0) return 0;
    const int64_t lim = ((int64_t)1 << 31) - (int64_t)PF_BM * (k / 2) - 1024;
    return (m + PF_BM) * (k / 2) < lim && (n + 256) * (k / 2) < lim ? 1 : 0;
}

extern "C" hipError_t mxl_launch_mx_prefill(const void* aq, const void* as, const void* wq, const void* ws,
                                            int64_t m, int64_t n, int64_t k, void* y, int out_f32,
                                            hipStream_t stream)
{
    PrefillArgs a{static_cast<const uint8_t*>(aq), static_cast<const uint8_t*>(as),
                  static_cast<const uint8_t*>(wq), static_cast<const uint8_t*>(ws), y, nullptr, nullptr,
                  (int)m, (int)n, (int)k, 0, 0};
    return out_f32 ? launch_prefill<true>(a, stream) : launch_prefill<false>(a, stream);
}

// The gate_up projection with the SwiGLU + MXFP4 epilogue: W is [n, k] with
// rows alternating 32 gate and 32 up rows (n % 64 == 0); h_q [m, n/4] and
// h_s [m, n/64].  Same shape limits as the plain kernel.
extern "C" hipError_t mxl_launch_mx_prefill_swiglu(const void* aq, const void* as, const void* wq,
                                                   const void* ws, int64_t m, int64_t n, int64_t k, void* h_q,
                                                   void* h_s, hipStream_t stream)
{
    PrefillArgs a{static_cast<const uint8_t*>(aq), static_cast<const uint8_t*>(as),
                  static_cast<const uint8_t*>(wq), static_cast<const uint8_t*>(ws), nullptr,
                  static_cast<uint8_t*>(h_q), static_cast<uint8_t*>(h_s), (int)m, (int)n, (int)k, 0, 0};
    return launch_prefill<false, PF_EPI_SWIGLU>(a, stream);
}

extern "C" const char* mxl_prefill_swiglu_config_name(void)
{
    return "mx_gemm_prefill_kernel<swiglu epilogue> 256x256 tiles (4 waves of 128x128, 32x32x64 mxfp4 mfma), "
           "gate/up rows interleaved by 32, h quantized to mxfp4 (ceil) in registers";
}

// Shapes the large-tile exact MXFP8 kernel takes: K % 128 == 0, at least
// 256 tiles of 256 x 256 (one per compute unit; fewer tiles run the 128 x
// 128 kernel, with split-K), and every operand below 2 GiB (32-bit buffer
// offsets, one byte per code).
extern "C" int mxl_mx8_tile_ok(int64_t m, int64_t n, int64_t k)
{
    if (k % 128 != 0 || ((m + 255) / 256) * ((n + 255) / 256) < 256) return 0;
    const int64_t lim = ((int64_t)1 << 31) - (int64_t)PF_BM * k - 1024;
    return (m + PF_BM) * k < lim && (n + 256) * k < lim ? 1 : 0;
}

extern "C" hipError_t mxl_launch_mx8_tile(const void* aq, const void* as, const void* wq, const void* ws, int64_t m,
                                          int64_t n, int64_t k, void* y, int out_f32, hipStream_t stream)
{
    PrefillArgs a{static_cast<const uint8_t*>(aq), static_cast<const uint8_t*>(as),
                  static_cast<const uint8_t*>(wq), static_cast<const uint8_t*>(ws), y, nullptr, nullptr,
                  (int)m, (int)n, (int)k, 0, 0};
    return out_f32 ? launch_mx8<true>(a, stream) : launch_mx8<false>(a, stream);
}

extern "C" const char* mxl_mx8_tile_config_name(void)
{
    return "mx8_gemm_tile_kernel<mxfp8 -> exact bf16 in registers, tile 256x256, 2x2 waves of 128x128, two 128-K "
           "pair slots + 8-pair scale windows fed by buffer-to-LDS copies, bf16 mfma 32x32x16; a last round at "
           "most half full runs as 256x128 halves>";
}

// Whether the 8-wave exact GEMM takes this shape: fmt 2 NVFP4 (K % 256 ==
// 0; fmt 1, MXFP8, is not launched); at least 256 tiles of 256 x 256 (fewer
// leave compute units idle, and the 128 x 128 kernel with split-K serves
// them); code bytes plus one tile of overrun rows within 32-bit buffer
// offsets.
extern "C" int mxl_dq8w_ok(int fmt, int64_t m, int64_t n, int64_t k)
{
    if (fmt != DQ8W_NVFP4) return 0;
    if (k % (fmt == DQ8W_NVFP4 ? 256 : 128) != 0 || ((m + 255) / 256) * ((n + 255) / 256) < 256) return 0;
    const int64_t rb = fmt == DQ8W_NVFP4 ? k / 2 : k;
    const int64_t lim = ((int64_t)1 << 31) - (int64_t)PF_BM * rb - 1024;
    return (m + PF_BM) * rb < lim && (n + 256) * rb < lim ? 1 : 0;
}

extern "C" hipError_t mxl_launch_dq8w(int fmt, const void* aq, const void* as, const void* wq, const void* ws,
                                      int64_t m, int64_t n, int64_t k, float alpha, void* y, int out_f32,
                                      hipStream_t stream)
{
    PrefillArgs a{static_cast<const uint8_t*>(aq), static_cast<const uint8_t*>(as),
                  static_cast<const uint8_t*>(wq), static_cast<const uint8_t*>(ws), y, nullptr, nullptr,
                  (int)m, (int)n, (int)k, 0, 0, alpha};
    if (fmt != DQ8W_NVFP4) return hipErrorInvalidValue;
    return out_f32 ? launch_dq8w<DQ8W_NVFP4, true>(a, stream) : launch_dq8w<DQ8W_NVFP4, false>(a, stream);
}

extern "C" const char* mxl_dq8w_config_name(void)
{
    return "dq8w_gemm_tile_kernel<nvfp4 -> exact f16 in registers, tile 256x256, 8 waves (2 per SIMD) as 2x4 of "
           "128x64, two 256-K pair slots + 2-pair scale windows fed by buffer-to-LDS copies, f16 mfma 32x32x16; a "
           "last round at most half full runs as 256x128 halves>";
}
