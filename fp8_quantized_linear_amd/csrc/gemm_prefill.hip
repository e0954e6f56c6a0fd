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
    using L = PfLayout<BN>;
    constexpr int WFR = L::WFR;
    extern __shared__ __align__(16) uint8_t smem[];

    int m0, n0;
    {
        const int t = pf_xcd_order(p.count);
        int tm, tn;
        if (BN == 256) {
            pf_tile(p.tile_base + t, p.M, p.N, tm, tn);
            n0 = tn * 256;
        } else {   // halves of the tail tiles; both halves of a tile on one XCD
            pf_tile(p.tile_base + t / 2, p.M, p.N, tm, tn);
            n0 = tn * 256 + (t % 2) * 128;
        }
        m0 = tm * PF_BM;
    }
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: feeds M0
    const int wm = wave >> 1, wn = wave & 1;
    const int r32 = lane & 31, g = lane >> 5;
    const int K = p.K, KB = K / 32, row_bytes = K / 2;
    const int nk = K / PF_BK;          // sub-stages
    const int np = (nk + 1) / 2;       // pairs (the last is half when K % 256 == 128)

    const int4_t rsrc_a = make_rsrc(p.a_q, (uint32_t)p.M * row_bytes);
    const int4_t rsrc_w = make_rsrc(p.w_q, (uint32_t)p.N * row_bytes);
    const int4_t rsrc_as = make_rsrc(p.a_s, (uint32_t)p.M * KB);
    const int4_t rsrc_ws = make_rsrc(p.w_s, (uint32_t)p.N * KB);
    const uint32_t lds0 = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)smem);

    // Code copies, 8 rows x 128 B = 1 KiB of LDS each: wave w copies A rows
    // [64 w, 64 w + 64) and W rows [8 WCOP w, 8 WCOP (w + 1)).  LDS position L
    // of a copy is row 8*copy + L/8, physical chunk L%8, which holds logical
    // chunk (L%8) ^ swz(row).  Per-lane offsets of pair 0; pair kp adds kp*128.
    int a_voff[L::ACOP], w_voff[L::WCOP];
#pragma unroll
    for (int s = 0; s < L::ACOP; ++s) {
        const int row = 8 * (L::ACOP * wave + s) + lane / 8;
        a_voff[s] = (m0 + row) * row_bytes + ((lane & 7) ^ pf_swz(row)) * 16;
    }
#pragma unroll
    for (int s = 0; s < L::WCOP; ++s) {
        const int row = 8 * (L::WCOP * wave + s) + lane / 8;
        w_voff[s] = (n0 + row) * row_bytes + ((lane & 7) ^ pf_swz(row)) * 16;
    }
    const uint32_t a_dst = lds0 + (uint32_t)(L::ACOP * wave * 1024);           // in A slot 0
    const uint32_t w_dst = lds0 + L::W0 + (uint32_t)(L::WCOP * wave * 1024);   // in W slot 0

    // Scale copies move 8 rows x 32 B ([row][32 B] in LDS).  A window is
    // issued as 4 pieces; piece j holds A copies t = 8 j + (0 .. 7) and W
    // copies t = (WSC/4) j + (0 .. WSC/4 - 1), copy t covering rows
    // [8 t, 8 t + 8) of the window.  Wave w makes copies 2 w and 2 w + 1 of
    // each piece; with BN = 128 waves 2 and 3 have no W copy and fill the
    // spare area from a zero-sized buffer instead.
    constexpr int WSC = BN / 8;
    const bool ws_real = 2 * wave + 1 < WSC / 4;
    const int srow = lane >> 3, sdw = lane & 7;
    int as_v[2], ws_v[2];
#pragma unroll
    for (int c = 0; c < 2; ++c) {
        as_v[c] = (m0 + 8 * (2 * wave + c) + srow) * KB + sdw * 4;
        ws_v[c] = (n0 + 8 * (2 * wave + c) + srow) * KB + sdw * 4;
    }

    // Copies issued during pair y: piece (y + 5) % 4 of scale window
    // (y + 5) / 4, and the codes of pair y + 2 (into the slot of pair y).
    // Window w is issued during pairs 4w-5 .. 4w-2, after every read of
    // window w-2 (same buffer), and has landed by the barrier that precedes
    // its first read in pair 4w-1.
    auto pair_copies = [&](int y) __attribute__((always_inline)) {
        PfPairCopies cp;
        const int kp = y + 2;
        const bool livec = kp < np;
        cp.ra = rsrc_a;
        cp.ra[2] = livec ? cp.ra[2] : 0;
        cp.rw = rsrc_w;
        cp.rw[2] = livec ? cp.rw[2] : 0;
        cp.coff = kp * PF_PROWB;
        cp.adst = a_dst + (uint32_t)((kp & (PF_NSL - 1)) * PF_ATILE);
        cp.wdst = w_dst + (uint32_t)((kp & (PF_NSL - 1)) * L::W_TILE);
        const int win = (y + 5) >> 2, j = (y + 5) & 3;
        const bool lives = win * PF_WPAIRS < np;
        const uint32_t wbuf = lds0 + L::SC0 + (uint32_t)((win & (PF_NWIN - 1)) * L::WIN);
        cp.ras = rsrc_as;
        cp.ras[2] = lives ? cp.ras[2] : 0;
        cp.rws = rsrc_ws;
        cp.rws[2] = (lives && ws_real) ? cp.rws[2] : 0;
        cp.asdst = wbuf + (uint32_t)((8 * j + 2 * wave) * 256);
        cp.wsdst = ws_real ? wbuf + PF_BM * PF_SWB + (uint32_t)(((WSC / 4) * j + 2 * wave) * 256)
                           : lds0 + L::DUMMY + (uint32_t)((wave & 1) * 512);
        cp.asoff = 64 * j * KB + win * PF_SWB;
        cp.wsoff = 8 * (WSC / 4) * j * KB + win * PF_SWB;
        return cp;
    };
    // copy c (0 .. COPIES-1) of a pair: 2 A and 2 W scale copies, then the A
    // and W code copies
    auto copy = [&](int c, const PfPairCopies& cp) __attribute__((always_inline)) {
        if (c < 2) {
            dma_b32_at(cp.asdst, c * 256, as_v[c], cp.asoff, cp.ras);
        } else if (c < 4) {
            dma_b32_at(cp.wsdst, (c - 2) * 256, ws_v[c - 2], cp.wsoff, cp.rws);
        } else if (c - 4 < L::ACOP) {
            const int cc = c - 4;
            dma_b128_at(cp.adst, cc * 1024, a_voff[cc], cp.coff, cp.ra);
        } else {
            const int s = c - 4 - L::ACOP;
            dma_b128_at(cp.wdst, s * 1024, w_voff[s], cp.coff, cp.rw);
        }
    };

    // LDS read addresses.  Fragment rows of one lane differ by multiples of
    // 32, so they share the chunk swizzle (r32 >> 1) & 7: a fragment's
    // address is a per-(half, step) base plus 4096 bytes per 32 rows, which
    // the read takes as an immediate.  During pair pr the half-1 bases point
    // into slot pr % 2 (read by its first sub-stage) and the half-0 bases
    // into slot (pr + 1) % 2 (read by its second, for the next pair); after
    // the pair both move to the other slot.
    const int swl = pf_swz(r32);
    uint32_t abase[2][2], wbase[2][2];   // LDS byte addresses
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
            const int ch = ((4 * h + 2 * kk + g) ^ swl) * 16;
            abase[h][kk] = lds0 + (wm * 128 + r32) * PF_PROWB + ch;
            wbase[h][kk] = lds0 + L::W0 + (wn * (BN / 2) + r32) * PF_PROWB + ch;
        }
    const uint32_t sa_lane = lds0 + L::SC0 + (wm * 128 + r32) * PF_SWB;
    const uint32_t sw_lane = lds0 + L::SC0 + PF_BM * PF_SWB + (wn * (BN / 2) + r32) * PF_SWB;
    // scale-read bases of pair pr: one add per pair, kept opaque so that the
    // per-read part stays an immediate
    auto scale_base = [&](int pr, uint32_t& sa, uint32_t& sw) __attribute__((always_inline)) {
        const uint32_t off = (uint32_t)(((pr / PF_WPAIRS) & (PF_NWIN - 1)) * L::WIN + (pr % PF_WPAIRS) * 8);
        sa = sa_lane + off;
        sw = sw_lane + off;
        asm volatile("" : "+v"(sa), "+v"(sw));
    };

    // LDS read q (0 .. READS-1) of half h (code bases abase/wbase[h], scale
    // bases sa/sw): code fragments (A of both steps, then W of both steps),
    // then the scale dwords (A, then W)
    auto read_piece = [&](int q, PfFrags<WFR>& f, int h, uint32_t sa, uint32_t sw) __attribute__((always_inline)) {
        if (q < 8) {
            const int kk = q >> 2, x = q & 3;
            f.a[kk][x] = lds_read_b128(abase[h][kk] + x * 32 * PF_PROWB);
        } else if (q < 8 + 2 * WFR) {
            const int kk = (q - 8) / WFR, x = (q - 8) % WFR;
            f.w[kk][x] = lds_read_b128(wbase[h][kk] + x * 32 * PF_PROWB);
        } else if (q < 12 + 2 * WFR) {
            const int x = q - 8 - 2 * WFR;
            f.sa[x] = (int)lds_read_b32(sa + h * 4 + x * 32 * PF_SWB);
        } else {
            const int x = q - 12 - 2 * WFR;
            f.sw[x] = (int)lds_read_b32(sw + h * 4 + x * 32 * PF_SWB);
        }
    };

    float16_t acc[4][WFR];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < WFR; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    // matrix-core instruction q of a sub-stage: step kk = q / (4 WFR), fragment (i, j)
    auto mfma = [&](int q, const PfFrags<WFR>& f, const int* sa, const int* sw) __attribute__((always_inline)) {
        const int kk = q / (4 * WFR), i = (q / WFR) % 4, j = q % WFR;
        const int8_t_ b8 = int8_t_{f.w[kk][j][0], f.w[kk][j][1], f.w[kk][j][2], f.w[kk][j][3], 0, 0, 0, 0};
        const int8_t_ a8 = int8_t_{f.a[kk][i][0], f.a[kk][i][1], f.a[kk][i][2], f.a[kk][i][3], 0, 0, 0, 0};
        if (kk == 0)
            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(b8, a8, acc[i][j], 4, 4, 0, sw[j], 0, sa[i]);
        else
            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(b8, a8, acc[i][j], 4, 4, 2, sw[j], 2, sa[i]);
    };

    // One sub-stage: computed from `cur` while the next sub-stage (half nh,
    // scale bases nsa/nsw) is read into `nxt`.  The second sub-stage of a
    // pair first waits for all copies issued so far (the next pair) and then
    // issues the pair's copies; the first computes their uniform part in its
    // read-free tail.
    auto sub = [&](const PfFrags<WFR>& cur, PfFrags<WFR>& nxt, bool second, int nh, uint32_t nsa, uint32_t nsw,
                   int pr, PfPairCopies& cp) __attribute__((always_inline)) {
        if (second) {
            wait_vmcnt<0>();
            lds_barrier();
        }
        // byte 2 kk + g of a scale dword is this lane's block; after the shift
        // it sits at byte 2 kk, which the instruction's op_sel picks
        int sa[4], sw[WFR];
#pragma unroll
        for (int i = 0; i < 4; ++i) sa[i] = (int)((uint32_t)cur.sa[i] >> (8 * g));
#pragma unroll
        for (int j = 0; j < WFR; ++j) sw[j] = (int)((uint32_t)cur.sw[j] >> (8 * g));
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int q = 0; q < L::MFMAS; ++q) {
            mfma(q, cur, sa, sw);
#pragma unroll
            for (int x = q * L::READS / L::READ_SPAN; x < (q + 1) * L::READS / L::READ_SPAN && x < L::READS; ++x) {
                __builtin_amdgcn_sched_barrier(0);
                read_piece(x, nxt, nh, nsa, nsw);
                __builtin_amdgcn_sched_barrier(0);
            }
            if (!second && q == L::READ_SPAN) {
                __builtin_amdgcn_sched_barrier(0);
                cp = pair_copies(pr);
                __builtin_amdgcn_sched_barrier(0);
            }
            if (second) {
#pragma unroll
                for (int c = q * L::COPIES / L::MFMAS; c < (q + 1) * L::COPIES / L::MFMAS; ++c) {
                    __builtin_amdgcn_sched_barrier(0);
                    copy(c, cp);
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
        }
        __builtin_amdgcn_sched_barrier(0);
    };

    // Prologue: the copy slots of virtual pairs -5 .. -1, with code copies
    // only where they name pairs 0 and 1: windows 0 and (piece 0 of) 1, pairs
    // 0 and 1.
    for (int y = -5; y < 0; ++y) {
        const PfPairCopies cp = pair_copies(y);
#pragma unroll
        for (int c = 0; c < 4; ++c) copy(c, cp);
        if (y >= -2) {
#pragma unroll
            for (int c = 4; c < L::COPIES; ++c) copy(c, cp);
        }
    }
    // sub-stage 0 needs window 0 and pair 0; the copies of virtual pair -1
    // (pair 1, piece 0 of window 1) may still be in flight, and the first
    // second sub-stage waits for them
    wait_vmcnt<L::COPIES>();
    lds_barrier();
    PfFrags<WFR> X, Y;
    uint32_t sa_c, sw_c;   // scale-read bases of the current pair
    scale_base(0, sa_c, sw_c);
#pragma unroll
    for (int q = 0; q < L::READS; ++q) read_piece(q, X, 0, sa_c, sw_c);   // half 0 of pair 0, slot 0
    // the half-0 bases move to slot 1 for the second sub-stage of pair 0
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
        abase[0][kk] += PF_ATILE;
        wbase[0][kk] += L::W_TILE;
    }

    int da = PF_ATILE, dw = L::W_TILE;   // slot step of the half-1 bases (the half-0 bases step by minus it)
    int pr = 0;
    for (; 2 * pr + 1 < nk; ++pr) {
        uint32_t sa_n, sw_n;
        scale_base(pr + 1, sa_n, sw_n);
        PfPairCopies cp;
        sub(X, Y, false, 1, sa_c, sw_c, pr, cp);
        sub(Y, X, true, 0, sa_n, sw_n, pr, cp);
        sa_c = sa_n;
        sw_c = sw_n;
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
            abase[1][kk] += da;
            abase[0][kk] -= da;
            wbase[1][kk] += dw;
            wbase[0][kk] -= dw;
        }
        da = -da;
        dw = -dw;
    }
    if (2 * pr < nk) {   // the half pair when K % 256 == 128
        PfPairCopies cp;
        sub(X, Y, false, 1, sa_c, sw_c, pr, cp);
    }
    wait_vmcnt<0>();   // the trailing zero-fill copies have landed
    lds_barrier();     // every wave is done with the slots

    if constexpr (EPI == PF_EPI_SWIGLU) {
        // W's rows alternate 32 gate rows and 32 up rows, so W fragment 2jj
        // of a wave holds the gate and fragment 2jj + 1 the up values of the
        // same 32 h columns, in the same registers of the same lanes.  Each
        // value is rounded to bf16 as a stored Y would be, h = SwiGLU(gate,
        // up) is rounded to bf16, and one fragment row of h (32 columns) is
        // one MXFP4 block: lane (r, g) holds 16 of its values, the lane
        // (r, 1 - g) the other 16.  h is [M, N/2]: codes [M, N/4] bytes,
        // scales [M, N/64] bytes.
        const int I = p.N / 2, hrow_b = I / 2, hblocks = I / 32;
        const int hb0 = (n0 + wn * (BN / 2)) / 64;    // first h block of this wave
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int m = m0 + wm * 128 + i * 32 + r32;
#pragma unroll
            for (int jj = 0; jj < WFR / 2; ++jj) {
                uint32_t hv[8];
                uint32_t amax = 0;
#pragma unroll
                for (int t = 0; t < 8; ++t) {
                    const uint32_t gb = bf16x2_rne(acc[i][2 * jj][2 * t], acc[i][2 * jj][2 * t + 1]);
                    const uint32_t ub = bf16x2_rne(acc[i][2 * jj + 1][2 * t], acc[i][2 * jj + 1][2 * t + 1]);
                    const float h0 = swiglu_f32(__uint_as_float(gb << 16), __uint_as_float(ub << 16));
                    const float h1 = swiglu_f32(__uint_as_float(gb & 0xFFFF0000u), __uint_as_float(ub & 0xFFFF0000u));
                    hv[t] = bf16x2_rne(h0, h1);
                    const uint32_t lo = hv[t] & 0x7FFFu, hi = (hv[t] >> 16) & 0x7FFFu;
                    amax = amax > lo ? amax : lo;
                    amax = amax > hi ? amax : hi;
                }
                const auto am = __builtin_amdgcn_permlane32_swap(amax, amax, false, false);
                amax = am[0] > am[1] ? am[0] : am[1];
                const int e = scale_exponent<ELEM_E2M1, RULE_CEIL>(amax);
                // codes of register groups 0,1 and 2,3: group q covers columns
                // 8q + 4g .. +3 of the block, 2 bytes
                const uint32_t c01 = encode8_e2m1(make_uint4(hv[0], hv[1], hv[2], hv[3]), e);
                const uint32_t c23 = encode8_e2m1(make_uint4(hv[4], hv[5], hv[6], hv[7]), e);
                // lane g = 0 receives groups 0, 1 of both lane halves (bytes
                // 0..7 of the block's 16), lane g = 1 groups 2, 3 (bytes 8..15)
                const auto sw = __builtin_amdgcn_permlane32_swap(c01, c23, false, false);
                const uint32_t d0 = (sw[0] & 0xFFFFu) | (sw[1] << 16);
                const uint32_t d1 = (sw[0] >> 16) | (sw[1] & 0xFFFF0000u);
                const int hb = hb0 + jj;
                if (m < p.M && hb < hblocks) {
                    uint8_t* dst = p.h_q + (size_t)m * hrow_b + hb * 16 + g * 8;
                    *reinterpret_cast<uint2*>(dst) = make_uint2(d0, d1);
                    if (g == 0) p.h_s[(size_t)m * hblocks + hb] = (uint8_t)(e + 127);
                }
            }
        }
        return;
    }

    // Epilogue, one 32-row band (fragment row i) at a time through two
    // band buffers in this wave's private LDS region: band i + 1 is written
    // row-major while band i is read back as whole row segments and stored
    // with 16-byte stores.  A wave's LDS operations execute in order, so the
    // reads see the writes issued before them and the writes of band i + 2
    // come after the reads of band i in the same buffer.
    constexpr int ESZ = OUT_F32 ? 4 : 2;
    constexpr int WCOLS = BN / 2;                        // output columns of a wave
    constexpr int ROWB = WCOLS * ESZ + 16;               // padded LDS row
    constexpr int BAND = 32 * ROWB;
    static_assert(8 * BAND <= L::LDS, "epilogue buffers");
    uint8_t* region = smem + wave * (2 * BAND);
    constexpr int LPR = WCOLS * ESZ / 16;                // lanes per 16-byte-chunked row
    constexpr int RPI = 64 / LPR;                        // rows per read instruction
    const int lrow = lane / LPR, c16 = lane % LPR;
    // full tiles with rows of whole 16-byte chunks store without checks, at
    // a uniform band base plus a 32-bit per-lane offset
    const bool full = m0 + PF_BM <= p.M && n0 + BN <= p.N && (p.N % (16 / ESZ)) == 0;
    uint8_t* ywave = reinterpret_cast<uint8_t*>(p.y) + ((size_t)(m0 + wm * 128) * p.N + n0 + wn * WCOLS) * ESZ;
    const uint32_t lane_off = (uint32_t)(lrow * p.N * ESZ + c16 * 16);

    auto write_band = [&](int i) __attribute__((always_inline)) {
        uint8_t* buf = region + (i & 1) * BAND;
#pragma unroll
        for (int j = 0; j < WFR; ++j)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                if (OUT_F32) {
                    uint8_t* dst = buf + r32 * ROWB + (j * 32 + q * 8 + g * 4) * ESZ;
                    *reinterpret_cast<float4_t*>(dst) =
                        float4_t{acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]};
                } else if (q % 2 == 0) {
                    // bf16: register groups q and q + 1 hold columns 8q + 4g .. +3 and
                    // 8(q+1) + 4g .. +3.  Swapping the upper lane half of group q
                    // with the lower half of group q + 1 leaves lane (r, g) with the
                    // 8 consecutive columns 8(q + g) .. +7 of row r: one 16-byte
                    // write, which the padded rows keep free of bank conflicts.
                    const uint32_t a0 = bf16x2_rne(acc[i][j][4 * q], acc[i][j][4 * q + 1]);
                    const uint32_t a1 = bf16x2_rne(acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]);
                    const uint32_t b0 = bf16x2_rne(acc[i][j][4 * q + 4], acc[i][j][4 * q + 5]);
                    const uint32_t b1 = bf16x2_rne(acc[i][j][4 * q + 6], acc[i][j][4 * q + 7]);
                    const auto s0 = __builtin_amdgcn_permlane32_swap(a0, b0, false, false);
                    const auto s1 = __builtin_amdgcn_permlane32_swap(a1, b1, false, false);
                    uint8_t* dst = buf + r32 * ROWB + (j * 32 + (q + g) * 8) * ESZ;
                    *reinterpret_cast<int4_t*>(dst) = int4_t{(int)s0[0], (int)s1[0], (int)s0[1], (int)s1[1]};
                }
            }
    };
    write_band(0);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        if (i + 1 < 4) write_band(i + 1);
        const uint8_t* buf = region + (i & 1) * BAND;
        int4_t v[32 / RPI];
#pragma unroll
        for (int t = 0; t < 32 / RPI; ++t) v[t] = *reinterpret_cast<const int4_t*>(buf + (t * RPI + lrow) * ROWB + c16 * 16);
        if (full) {
#pragma unroll
            for (int t = 0; t < 32 / RPI; ++t) {
                uint8_t* yb = ywave + (size_t)(i * 32 + t * RPI) * p.N * ESZ;
                __builtin_nontemporal_store(v[t], reinterpret_cast<int4_t*>(yb + lane_off));
            }
            continue;
        }
#pragma unroll
        for (int t = 0; t < 32 / RPI; ++t) {
            const int row = t * RPI + lrow;
            const int m = m0 + wm * 128 + i * 32 + row;
            const int n = n0 + wn * WCOLS + c16 * (16 / ESZ);
            if (m >= p.M) continue;
            uint8_t* yrow = reinterpret_cast<uint8_t*>(p.y) + ((size_t)m * p.N) * ESZ;
            if ((p.N % (16 / ESZ)) == 0 && n + 16 / ESZ <= p.N) {
                __builtin_nontemporal_store(v[t], reinterpret_cast<int4_t*>(yrow + (size_t)n * ESZ));
            } else {
#pragma unroll
                for (int e = 0; e < 16 / ESZ; ++e) {
                    const int wi = OUT_F32 ? e : e / 2;
                    const uint32_t word = (uint32_t)v[t][wi];
                    if (n + e < p.N) {
                        if (OUT_F32) reinterpret_cast<uint32_t*>(yrow)[n + e] = word;
                        else reinterpret_cast<uint16_t*>(yrow)[n + e] = (uint16_t)(word >> (16 * (e % 2)));
                    }
                }
            }
        }
    }
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

} // namespace mxl

using namespace mxl;

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
