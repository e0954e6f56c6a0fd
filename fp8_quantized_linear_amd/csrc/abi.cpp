// abi.cpp -- the C ABI of libmxlinear.so (declared in include/mxlinear.h):
// argument validation (done before any HIP call), device check, dispatch to
// the gfx950 kernel launchers, status strings and host helpers.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cfloat>
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>

#include "mxlinear.h"

extern "C" {
hipError_t mxl_launch_mx_quantize(int elem, int rule, const void* x, int64_t total, void* q, void* s,
                                  hipStream_t stream);
hipError_t mxl_launch_nv_quantize(const void* x, int64_t total, float g, void* q, void* s,
                                  hipStream_t stream);
hipError_t mxl_launch_mx_fake_quant(int elem, int rule, const void* x, int64_t total, void* y,
                                   hipStream_t stream);
hipError_t mxl_launch_nv_fake_quant(const void* x, int64_t total, float g, void* y, hipStream_t stream);
hipError_t mxl_launch_swiglu_quant(const void* x, int64_t rows, int64_t inter, void* q, void* s,
                                  hipStream_t stream);
hipError_t mxl_launch_mx_prefill_swiglu(const void* aq, const void* as, const void* wq, const void* ws, int64_t m,
                                        int64_t n, int64_t k, void* h_q, void* h_s, hipStream_t stream);
int mxl_prefill_ok(int64_t m, int64_t n, int64_t k);
const char* mxl_prefill_swiglu_config_name(void);
hipError_t mxl_launch_amax(const void* x, int64_t count, float* out, hipStream_t stream);
hipError_t mxl_launch_mx_gemm(int a_bits, int w_bits, const void* aq, const void* as, const void* wq,
                              const void* ws, int64_t m, int64_t n, int64_t k, void* y, int out_f32,
                              void* work, size_t work_bytes, hipStream_t stream);
size_t mxl_mx_gemm_workspace(int a_bits, int w_bits, int64_t m, int64_t n, int64_t k);
int mxl_mx_gemm_fits(int a_bits, int w_bits, int64_t m, int64_t n, int64_t k, int fused_in_tile);
hipError_t mxl_launch_mx_mixed_exact_gemm(int a_bits, const void* aq, const void* as, const void* wq,
                                          const void* ws, int64_t m, int64_t n, int64_t k, void* y, int out_f32,
                                          void* work, size_t work_bytes, hipStream_t stream);
const char* mxl_mx_mixed_exact_config_name(void);
int mxl_mx8_tile_ok(int64_t m, int64_t n, int64_t k);
size_t mxl_dq_workspace(int64_t m, int64_t n, int64_t k);
int mxl_dq_splits(int64_t m, int64_t n, int64_t k);
int mxl_dq_decode_ok(int nv, int64_t m, int64_t n, int64_t k);
hipError_t mxl_launch_mx_gemm_fused(int a_bits, int a_rule, const void* a_bf16, int w_bits,
                                    const void* wq, const void* ws, int64_t m, int64_t n, int64_t k,
                                    void* y, int out_f32, void* dump_q, void* dump_s, void* work,
                                    size_t work_bytes, hipStream_t stream);
size_t mxl_mx_gemm_fused_workspace(int a_bits, int64_t m, int64_t n, int64_t k);
size_t mxl_dq_pool_workspace(int64_t m, int64_t n, int64_t k);
hipError_t mxl_launch_mxfp8_exact_gemm_pool(int a_rule, const void* a_bf16, const void* wq, const void* ws, int64_t m,
                                            int64_t n, int64_t k, void* y, int out_f32, void* work, size_t work_bytes,
                                            hipStream_t stream);
hipError_t mxl_launch_nv_gemm(const void* aq, const void* as, const void* wq, const void* ws, int64_t m,
                              int64_t n, int64_t k, float alpha, void* y, int out_f32, void* work,
                              size_t work_bytes, hipStream_t stream);
hipError_t mxl_launch_mxfp8_exact_gemm(const void* aq, const void* as, const void* wq, const void* ws,
                                       int64_t m, int64_t n, int64_t k, void* y, int out_f32, void* work,
                                       size_t work_bytes, hipStream_t stream);
hipError_t mxl_launch_mxfp8_exact_gemm_fused(int a_rule, const void* a_bf16, const void* wq, const void* ws,
                                             int64_t m, int64_t n, int64_t k, void* y, int out_f32, void* dump_q,
                                             void* dump_s, hipStream_t stream);
hipError_t mxl_launch_w4a16_gemm(int w_nv, const void* a_bf16, const void* wq, const void* ws, int64_t m,
                                 int64_t n, int64_t k, float alpha, void* y, int out_f32, void* work,
                                 size_t work_bytes, hipStream_t stream);
hipError_t mxl_launch_w4a16_decode(int w_nv, const void* a_bf16, const void* wq, const void* ws, int64_t m,
                                   int64_t n, int64_t k, float alpha, void* y, int out_f32, hipStream_t stream);
int mxl_w4a16_decode_ok(int w_nv, int64_t m, int64_t k);
const char* mxl_w4a16_gemm_config_name(void);
const char* mxl_w4a16_decode_config_name(int w_nv, int64_t m, int64_t n, int64_t k);
const char* mxl_mx_gemm_config_name(int a_bits, int w_bits, int64_t m, int64_t n, int64_t k, int fused);
const char* mxl_nv_gemm_config_name(int64_t m, int64_t n, int64_t k);
const char* mxl_mxfp8_exact_config_name(int64_t m, int64_t n, int64_t k);
}

namespace {

constexpr int64_t kMaxDim = (int64_t)1 << 30;  // kernels index rows/columns with 32-bit ints

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool valid_fmt(int f) { return f == MX_FMT_MXFP4 || f == MX_FMT_MXFP8 || f == MX_FMT_NVFP4; }
bool valid_rule(int r) { return r == MX_RULE_FLOOR || r == MX_RULE_CEIL || r == MX_RULE_EVEN; }

bool log_enabled()
{
    static int v = -1;
    if (v < 0) {
        const char* e = std::getenv("MXL_LOG");
        v = (e && e[0] && e[0] != '0') ? 1 : 0;
    }
    return v == 1;
}

// gfx950 check, cached per device ordinal.
std::atomic<int> g_dev_ok[64];

mx_status check_device()
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return MX_ERR_HIP;
    if (dev < 0 || dev >= 64) return MX_ERR_UNSUPPORTED;
    int st = g_dev_ok[dev].load(std::memory_order_relaxed);
    if (st == 0) {
        hipDeviceProp_t prop;
        if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return MX_ERR_HIP;
        st = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
        g_dev_ok[dev].store(st, std::memory_order_relaxed);
    }
    return st == 1 ? MX_OK : MX_ERR_UNSUPPORTED;
}

mx_status from_hip(hipError_t e) { return e == hipSuccess ? MX_OK : MX_ERR_HIP; }

// Split-K scratch of mx_gemm_noalloc: a file-scope device array that every
// GPU the library runs on holds for the life of the process.  Host code never
// passes the array's name to a kernel (on the host it is only a stand-in):
// the device address comes from hipGetSymbolAddress, once per device, with
// that device current, and is kept per device.
constexpr size_t kNoallocScratchBytes = (size_t)MX_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) uint8_t scratch[kNoallocScratchBytes];
std::once_flag g_scratch_once[64];
void* g_scratch_ptr[64];

// The current device's address of `scratch` (nullptr if the runtime refused).
void* scratch_address(int dev)
{
    std::call_once(g_scratch_once[dev], [dev]() {
        void* ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess) ptr = nullptr;
        g_scratch_ptr[dev] = ptr;
    });
    return g_scratch_ptr[dev];
}

mx_status check_quant_args(mx_format fmt, mx_scale_rule rule, const void* x, int64_t rows, int64_t k,
                           float gscale, const void* q, const void* s)
{
    if (!valid_fmt(fmt) || (fmt != MX_FMT_NVFP4 && !valid_rule(rule))) return MX_ERR_INVALID_ARG;
    if (!x || !q || !s) return MX_ERR_INVALID_ARG;
    if (rows < 1 || k < 1 || rows > kMaxDim || k > kMaxDim) return MX_ERR_SHAPE;
    if (k % (fmt == MX_FMT_NVFP4 ? 16 : 32) != 0) return MX_ERR_SHAPE;
    if (fmt == MX_FMT_NVFP4 && !(std::isfinite(gscale) && gscale > 0.0f)) return MX_ERR_INVALID_ARG;
    if (!aligned16(x) || !aligned16(q) || !aligned16(s)) return MX_ERR_ALIGN;
    return MX_OK;
}

mx_status quantize(mx_format fmt, mx_scale_rule rule, const void* x, int64_t rows, int64_t k, float g,
                   void* q, void* s, mx_stream_t stream)
{
    mx_status st = check_quant_args(fmt, rule, x, rows, k, g, q, s);
    if (st != MX_OK) return st;
    if ((st = check_device()) != MX_OK) return st;
    const int64_t total = rows * k;
    hipStream_t hs = static_cast<hipStream_t>(stream);
    if (fmt == MX_FMT_NVFP4) return from_hip(mxl_launch_nv_quantize(x, total, g, q, s, hs));
    return from_hip(mxl_launch_mx_quantize(fmt == MX_FMT_MXFP4 ? 0 : 1, (int)rule, x, total, q, s, hs));
}

mx_status check_gemm_shape(int64_t m, int64_t n, int64_t k, int block)
{
    if (m < 1 || n < 1 || k < 1 || m > kMaxDim || n > kMaxDim || k > kMaxDim) return MX_ERR_SHAPE;
    if (k % block != 0) return MX_ERR_SHAPE;
    return MX_OK;
}

int bits_of(mx_format f) { return f == MX_FMT_MXFP8 ? 8 : 4; }

// Kernel family of mx_gemm for an MX pair: the block-scaled matrix cores
// (MXFP4 x MXFP4; pairs with an MXFP8 operand under MX_FP8_FAST), or exact
// dequantization to bf16 (MXFP8 x MXFP8 and mixed pairs by default).
enum MxPath { PATH_SCALED, PATH_EXACT8, PATH_MIXED_EXACT };

MxPath mx_path(mx_format a, mx_format w, unsigned flags)
{
    if ((a == MX_FMT_MXFP4 && w == MX_FMT_MXFP4) || (flags & MX_FP8_FAST)) return PATH_SCALED;
    return a == w ? PATH_EXACT8 : PATH_MIXED_EXACT;
}

// Split-K workspace mx_gemm uses for this pair and shape (0: none).
size_t gemm_workspace_need(mx_format a, mx_format w, int64_t m, int64_t n, int64_t k, unsigned flags)
{
    const MxPath path = mx_path(a, w, flags);
    if (path == PATH_SCALED) return mxl_mx_gemm_workspace(bits_of(a), bits_of(w), m, n, k);
    if (path == PATH_EXACT8 && mxl_dq_decode_ok(0, m, n, k)) return 0;   // the decode kernel does not split
    return mxl_dq_workspace(m, n, k);
}

bool aligned256(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 255u) == 0; }

// Workspace bytes of the quantize-once launches (A quantized inside the
// GEMM's own workgroups), 0 where the shape has none: large MXFP4 shapes on
// the prefill kernel, exact MXFP8 on the 128 x 128 kernel.
size_t fused_pool_need(mx_format a, mx_format w, int64_t m, int64_t n, int64_t k, unsigned flags)
{
    if (a != w) return 0;
    if (a == MX_FMT_MXFP8) return (flags & MX_FP8_FAST) ? 0 : mxl_dq_pool_workspace(m, n, k);
    return mxl_mx_gemm_fused_workspace(bits_of(a), m, n, k);
}

// Whether mx_gemm_fused requires the quantizer path (A quantized into the
// workspace by the standalone quantizer, then mx_gemm's kernel): mixed
// pairs, and exact MXFP8 on the shapes of the large-tile kernel (so the
// result stays bitwise that of mx_quantize_act followed by mx_gemm).
bool fused_requires_quantizer(mx_format a, mx_format w, int64_t m, int64_t n, int64_t k, unsigned flags)
{
    if (a != w) return true;
    return a == MX_FMT_MXFP8 && !(flags & MX_FP8_FAST) && mxl_mx8_tile_ok(m, n, k);
}

// Whether a call that brings a workspace takes the quantizer path: where it
// is required, and on the quantize-once shapes unless MX_FUSED_IN_GEMM asks
// for the one-launch variant (the separate full-occupancy quantizer launch
// plus the GEMM measured faster: 414 / 437 us against 451 / 450 us on the
// 8192 x 5120 x 17408 and 8192 x 17408 x 5120 MXFP4 projections).
bool fused_via_quantizer(mx_format a, mx_format w, int64_t m, int64_t n, int64_t k, unsigned flags)
{
    if (flags & MX_DEBUG_DUMP_AQ) return false;
    if (fused_requires_quantizer(a, w, m, n, k, flags)) return true;
    return !(flags & MX_FUSED_IN_GEMM) && fused_pool_need(a, w, m, n, k, flags) > 0;
}

// Workspace mx_gemm_fused uses: A's codes and scales (dump, quantizer
// path), the quantize-once codes, scales and state (MX_FUSED_IN_GEMM), or
// none (the in-tile prologue).
size_t fused_workspace_need(mx_format a, mx_format w, int64_t m, int64_t n, int64_t k, unsigned flags)
{
    if (fused_via_quantizer(a, w, m, n, k, flags) || (flags & MX_DEBUG_DUMP_AQ))
        return (size_t)m * k * bits_of(a) / 8 + (size_t)m * (k / 32);
    return fused_pool_need(a, w, m, n, k, flags);
}

// W4A16: the decode kernel takes M <= 16 with K % 512 == 0 when its W block
// fits LDS and W's bytes stay within 32-bit buffer offsets
bool w4a16_use_decode(bool nv, int64_t m, int64_t n, int64_t k)
{
    // the decode kernels form 32-bit W offsets up to the last row of their
    // last workgroup (32 rows)
    return mxl_w4a16_decode_ok(nv ? 1 : 0, m, k) && (n + 32) * (k / 2) < ((int64_t)1 << 31);
}

} // namespace

extern "C" {

int mx_abi_version(void) { return MXLINEAR_ABI_VERSION; }

const char* mx_status_string(mx_status s)
{
    switch (s) {
    case MX_OK: return "ok";
    case MX_ERR_INVALID_ARG: return "invalid argument (null pointer, unknown enum or bad format/rule pair)";
    case MX_ERR_SHAPE: return "invalid shape (m, n, k must be >= 1 and k a multiple of the block size)";
    case MX_ERR_ALIGN: return "misaligned pointer (all tensors must be 16-byte aligned)";
    case MX_ERR_WORKSPACE: return "workspace too small";
    case MX_ERR_UNSUPPORTED: return "unsupported (device is not gfx950, or format pair not implemented)";
    case MX_ERR_HIP: return "HIP runtime error";
    }
    return "unknown status";
}

mx_status mx_quantize_act(mx_format fmt, mx_scale_rule rule, const void* a_bf16, int64_t m, int64_t k,
                          float global_scale, void* a_q, void* a_s, mx_stream_t stream)
{
    return quantize(fmt, rule, a_bf16, m, k, global_scale, a_q, a_s, stream);
}

mx_status mx_pack_weights(mx_format fmt, mx_scale_rule rule, const void* w_bf16, int64_t n, int64_t k,
                          float global_scale, void* w_q, void* w_s, mx_stream_t stream)
{
    return quantize(fmt, rule, w_bf16, n, k, global_scale, w_q, w_s, stream);
}

mx_status mx_gemm(mx_format a_fmt, mx_format w_fmt, const void* a_q, const void* a_s, const void* w_q,
                  const void* w_s, int64_t m, int64_t n, int64_t k, void* y, void* workspace, size_t ws_bytes,
                  unsigned flags, mx_stream_t stream)
{
    if (!valid_fmt(a_fmt) || !valid_fmt(w_fmt) || a_fmt == MX_FMT_NVFP4 || w_fmt == MX_FMT_NVFP4)
        return MX_ERR_INVALID_ARG;
    if (!a_q || !a_s || !w_q || !w_s || !y) return MX_ERR_INVALID_ARG;
    if (flags & ~(MX_OUT_F32 | MX_FP8_FAST)) return MX_ERR_INVALID_ARG;
    mx_status st = check_gemm_shape(m, n, k, 32);
    if (st != MX_OK) return st;
    if (!aligned16(a_q) || !aligned16(a_s) || !aligned16(w_q) || !aligned16(w_s) || !aligned16(y) ||
        (workspace && !aligned16(workspace)))
        return MX_ERR_ALIGN;
    const size_t need = gemm_workspace_need(a_fmt, w_fmt, m, n, k, flags);
    if (workspace && need > 0 && ws_bytes < need) return MX_ERR_WORKSPACE;
    const MxPath path = mx_path(a_fmt, w_fmt, flags);
    const int ab = bits_of(a_fmt), wb = bits_of(w_fmt);
    if (path == PATH_SCALED && !mxl_mx_gemm_fits(ab, wb, m, n, k, 0)) return MX_ERR_UNSUPPORTED;
    if ((st = check_device()) != MX_OK) return st;
    const int f32 = (flags & MX_OUT_F32) ? 1 : 0;
    if (log_enabled())
        std::fprintf(stderr, "[mxlinear] mx_gemm m=%lld n=%lld k=%lld -> %s\n", (long long)m, (long long)n,
                     (long long)k,
                     path == PATH_EXACT8 ? mxl_mxfp8_exact_config_name(m, n, k)
                     : path == PATH_MIXED_EXACT ? mxl_mx_mixed_exact_config_name()
                                                : mxl_mx_gemm_config_name(ab, wb, m, n, k, 0));
    hipStream_t hs = static_cast<hipStream_t>(stream);
    if (path == PATH_EXACT8)
        return from_hip(mxl_launch_mxfp8_exact_gemm(a_q, a_s, w_q, w_s, m, n, k, y, f32, workspace, ws_bytes, hs));
    if (path == PATH_MIXED_EXACT)
        return from_hip(mxl_launch_mx_mixed_exact_gemm(ab, a_q, a_s, w_q, w_s, m, n, k, y, f32, workspace,
                                                       ws_bytes, hs));
    return from_hip(mxl_launch_mx_gemm(ab, wb, a_q, a_s, w_q, w_s, m, n, k, y, f32, workspace, ws_bytes, hs));
}

mx_status mx_gemm_noalloc(mx_format a_fmt, mx_format w_fmt, const void* a_q, const void* a_s, const void* w_q,
                          const void* w_s, int64_t m, int64_t n, int64_t k, void* y, unsigned flags,
                          mx_stream_t stream)
{
    if (!valid_fmt(a_fmt) || !valid_fmt(w_fmt) || a_fmt == MX_FMT_NVFP4 || w_fmt == MX_FMT_NVFP4)
        return MX_ERR_INVALID_ARG;
    if (flags & ~(MX_OUT_F32 | MX_FP8_FAST)) return MX_ERR_INVALID_ARG;
    mx_status st = check_gemm_shape(m, n, k, 32);
    if (st != MX_OK) return st;
    const size_t need = gemm_workspace_need(a_fmt, w_fmt, m, n, k, flags);
    if (need > kNoallocScratchBytes) return MX_ERR_WORKSPACE;
    void* ws = nullptr;
    if (need > 0) {
        // the remaining argument checks run in mx_gemm; the scratch address
        // needs the current device, so check it first
        if (!a_q || !a_s || !w_q || !w_s || !y) return MX_ERR_INVALID_ARG;
        if ((st = check_device()) != MX_OK) return st;
        int dev = 0;
        if (hipGetDevice(&dev) != hipSuccess) return MX_ERR_HIP;
        ws = scratch_address(dev);
        if (!ws) return MX_ERR_HIP;
    }
    return mx_gemm(a_fmt, w_fmt, a_q, a_s, w_q, w_s, m, n, k, y, ws, ws ? kNoallocScratchBytes : 0, flags, stream);
}

mx_status mx_gemm_fused(mx_format a_fmt, mx_format w_fmt, const void* a_bf16, mx_scale_rule a_rule,
                        const void* w_q, const void* w_s, int64_t m, int64_t n, int64_t k, void* y,
                        void* workspace, size_t ws_bytes, unsigned flags, mx_stream_t stream)
{
    if (!valid_fmt(a_fmt) || !valid_fmt(w_fmt) || a_fmt == MX_FMT_NVFP4 || w_fmt == MX_FMT_NVFP4 ||
        !valid_rule(a_rule))
        return MX_ERR_INVALID_ARG;
    if (!a_bf16 || !w_q || !w_s || !y) return MX_ERR_INVALID_ARG;
    if (flags & ~(MX_OUT_F32 | MX_FP8_FAST | MX_DEBUG_DUMP_AQ | MX_FUSED_IN_GEMM)) return MX_ERR_INVALID_ARG;
    mx_status st = check_gemm_shape(m, n, k, 32);
    if (st != MX_OK) return st;
    if (!aligned16(a_bf16) || !aligned16(w_q) || !aligned16(w_s) || !aligned16(y) ||
        (workspace && !aligned16(workspace)))
        return MX_ERR_ALIGN;
    const int ab = bits_of(a_fmt), wb = bits_of(w_fmt);
    const int f32 = (flags & MX_OUT_F32) ? 1 : 0;
    const size_t need = fused_workspace_need(a_fmt, w_fmt, m, n, k, flags);
    const size_t qb = (size_t)m * k * ab / 8;
    hipStream_t hs = static_cast<hipStream_t>(stream);

    if (fused_via_quantizer(a_fmt, w_fmt, m, n, k, flags) &&
        (workspace || fused_requires_quantizer(a_fmt, w_fmt, m, n, k, flags))) {
        // quantize A into the workspace (mx_quantize_act's layout, which is
        // also the dump's), then mx_gemm's kernel reads it there
        if (!workspace || ws_bytes < need) return MX_ERR_WORKSPACE;
        const MxPath path = mx_path(a_fmt, w_fmt, flags);
        if (path == PATH_SCALED && !mxl_mx_gemm_fits(ab, wb, m, n, k, 0)) return MX_ERR_UNSUPPORTED;
        if ((st = check_device()) != MX_OK) return st;
        void* aq = workspace;
        void* as = static_cast<uint8_t*>(workspace) + qb;
        hipError_t e = mxl_launch_mx_quantize(a_fmt == MX_FMT_MXFP4 ? 0 : 1, (int)a_rule, a_bf16, m * k, aq, as, hs);
        if (e != hipSuccess) return MX_ERR_HIP;
        if (path == PATH_EXACT8)   // unsplit: the kernel mx_gemm picks without a workspace
            return from_hip(mxl_launch_mxfp8_exact_gemm(aq, as, w_q, w_s, m, n, k, y, f32, nullptr, 0, hs));
        if (path == PATH_MIXED_EXACT)
            return from_hip(mxl_launch_mx_mixed_exact_gemm(ab, aq, as, w_q, w_s, m, n, k, y, f32, nullptr, 0, hs));
        return from_hip(mxl_launch_mx_gemm(ab, wb, aq, as, w_q, w_s, m, n, k, y, f32, nullptr, 0, hs));
    }

    // debug dump of the prologue's codes and scales into the workspace
    void *dump_q = nullptr, *dump_s = nullptr;
    bool use_ws = false;
    if (flags & MX_DEBUG_DUMP_AQ) {
        if (!workspace || ws_bytes < need) return MX_ERR_WORKSPACE;
        dump_q = workspace;
        dump_s = static_cast<uint8_t*>(workspace) + qb;
    } else if (workspace && need > 0) {   // MX_FUSED_IN_GEMM on a quantize-once shape
        if (ws_bytes < need) return MX_ERR_WORKSPACE;
        if (!aligned256(workspace)) return MX_ERR_ALIGN;
        use_ws = true;
    }
    const bool exact8 = a_fmt == MX_FMT_MXFP8 && !(flags & MX_FP8_FAST);
    // without the quantize-once workspace the in-tile prologue kernels run;
    // the MX ones address operands with 32-bit offsets
    if (!exact8 && !use_ws && !mxl_mx_gemm_fits(ab, wb, m, n, k, 1)) return MX_ERR_UNSUPPORTED;
    if ((st = check_device()) != MX_OK) return st;
    if (exact8) {
        if (use_ws)
            return from_hip(mxl_launch_mxfp8_exact_gemm_pool((int)a_rule, a_bf16, w_q, w_s, m, n, k, y, f32,
                                                             workspace, ws_bytes, hs));
        return from_hip(mxl_launch_mxfp8_exact_gemm_fused((int)a_rule, a_bf16, w_q, w_s, m, n, k, y, f32, dump_q,
                                                          dump_s, hs));
    }
    return from_hip(mxl_launch_mx_gemm_fused(ab, (int)a_rule, a_bf16, wb, w_q, w_s, m, n, k, y, f32, dump_q, dump_s,
                                             use_ws ? workspace : nullptr, use_ws ? ws_bytes : 0, hs));
}

mx_status mx_gemm_fused_workspace_size(mx_format a_fmt, mx_format w_fmt, int64_t m, int64_t n, int64_t k,
                                       unsigned flags, size_t* bytes)
{
    if (!valid_fmt(a_fmt) || !valid_fmt(w_fmt) || a_fmt == MX_FMT_NVFP4 || w_fmt == MX_FMT_NVFP4 || !bytes)
        return MX_ERR_INVALID_ARG;
    if (flags & ~(MX_OUT_F32 | MX_FP8_FAST | MX_DEBUG_DUMP_AQ | MX_FUSED_IN_GEMM)) return MX_ERR_INVALID_ARG;
    mx_status st = check_gemm_shape(m, n, k, 32);
    if (st != MX_OK) return st;
    *bytes = fused_workspace_need(a_fmt, w_fmt, m, n, k, flags);
    return MX_OK;
}

mx_status nv_gemm(const void* a_q, const void* a_s, const void* w_q, const void* w_s, int64_t m, int64_t n,
                  int64_t k, float alpha, void* y, void* workspace, size_t ws_bytes, unsigned flags,
                  mx_stream_t stream)
{
    if (!a_q || !a_s || !w_q || !w_s || !y) return MX_ERR_INVALID_ARG;
    if (flags & ~MX_OUT_F32) return MX_ERR_INVALID_ARG;
    if (!std::isfinite(alpha)) return MX_ERR_INVALID_ARG;
    mx_status st = check_gemm_shape(m, n, k, 16);
    if (st != MX_OK) return st;
    if (!aligned16(a_q) || !aligned16(a_s) || !aligned16(w_q) || !aligned16(w_s) || !aligned16(y) ||
        (workspace && !aligned16(workspace)))
        return MX_ERR_ALIGN;
    const size_t need = mxl_dq_decode_ok(1, m, n, k) ? 0 : mxl_dq_workspace(m, n, k);
    if (workspace && need > 0 && ws_bytes < need) return MX_ERR_WORKSPACE;
    if ((st = check_device()) != MX_OK) return st;
    return from_hip(mxl_launch_nv_gemm(a_q, a_s, w_q, w_s, m, n, k, alpha, y, (flags & MX_OUT_F32) ? 1 : 0,
                                       workspace, ws_bytes, static_cast<hipStream_t>(stream)));
}

mx_status mx_gemm_w4a16(mx_format w_fmt, const void* a_bf16, const void* w_q, const void* w_s, int64_t m,
                        int64_t n, int64_t k, float alpha, void* y, void* workspace, size_t ws_bytes,
                        unsigned flags, mx_stream_t stream)
{
    if (!valid_fmt(w_fmt)) return MX_ERR_INVALID_ARG;
    if (w_fmt == MX_FMT_MXFP8) return MX_ERR_UNSUPPORTED;
    if (!a_bf16 || !w_q || !w_s || !y) return MX_ERR_INVALID_ARG;
    if (workspace && !aligned16(workspace)) return MX_ERR_ALIGN;
    if (flags & ~MX_OUT_F32) return MX_ERR_INVALID_ARG;
    if (!std::isfinite(alpha)) return MX_ERR_INVALID_ARG;
    const bool nv = w_fmt == MX_FMT_NVFP4;
    mx_status st = check_gemm_shape(m, n, k, nv ? 16 : 32);
    if (st != MX_OK) return st;
    if (!aligned16(a_bf16) || !aligned16(w_q) || !aligned16(w_s) || !aligned16(y)) return MX_ERR_ALIGN;
    const size_t need = w4a16_use_decode(nv, m, n, k) ? 0 : mxl_dq_workspace(m, n, k);
    if (workspace && need > 0 && ws_bytes < need) return MX_ERR_WORKSPACE;
    if ((st = check_device()) != MX_OK) return st;
    const int f32 = (flags & MX_OUT_F32) ? 1 : 0;
    hipStream_t hs = static_cast<hipStream_t>(stream);
    if (w4a16_use_decode(nv, m, n, k))
        return from_hip(mxl_launch_w4a16_decode(nv ? 1 : 0, a_bf16, w_q, w_s, m, n, k, alpha, y, f32, hs));
    return from_hip(mxl_launch_w4a16_gemm(nv ? 1 : 0, a_bf16, w_q, w_s, m, n, k, alpha, y, f32, workspace,
                                          ws_bytes, hs));
}

mx_status mx_gemm_workspace_size(mx_format a_fmt, mx_format w_fmt, int64_t m, int64_t n, int64_t k,
                                 unsigned flags, size_t* bytes)
{
    if (!valid_fmt(a_fmt) || !valid_fmt(w_fmt) || !bytes) return MX_ERR_INVALID_ARG;
    const bool nv = a_fmt == MX_FMT_NVFP4;
    if (nv != (w_fmt == MX_FMT_NVFP4)) return MX_ERR_INVALID_ARG;
    mx_status st = check_gemm_shape(m, n, k, nv ? 16 : 32);
    if (st != MX_OK) return st;
    *bytes = nv ? (mxl_dq_decode_ok(1, m, n, k) ? 0 : mxl_dq_workspace(m, n, k))
                : gemm_workspace_need(a_fmt, w_fmt, m, n, k, flags);
    return MX_OK;
}

mx_status mx_gemm_w4a16_workspace_size(mx_format w_fmt, int64_t m, int64_t n, int64_t k, size_t* bytes)
{
    if (!valid_fmt(w_fmt) || !bytes) return MX_ERR_INVALID_ARG;
    if (w_fmt == MX_FMT_MXFP8) return MX_ERR_UNSUPPORTED;
    const bool nv = w_fmt == MX_FMT_NVFP4;
    mx_status st = check_gemm_shape(m, n, k, nv ? 16 : 32);
    if (st != MX_OK) return st;
    *bytes = w4a16_use_decode(nv, m, n, k) ? 0 : mxl_dq_workspace(m, n, k);
    return MX_OK;
}

mx_status mx_gemm_w4a16_plan(mx_format w_fmt, int64_t m, int64_t n, int64_t k, char* name, size_t len)
{
    if (!valid_fmt(w_fmt) || !name || len == 0) return MX_ERR_INVALID_ARG;
    if (w_fmt == MX_FMT_MXFP8) return MX_ERR_UNSUPPORTED;
    const bool nv = w_fmt == MX_FMT_NVFP4;
    mx_status st = check_gemm_shape(m, n, k, nv ? 16 : 32);
    if (st != MX_OK) return st;
    const bool dec = w4a16_use_decode(nv, m, n, k);
    const int splits = dec ? 1 : mxl_dq_splits(m, n, k);
    std::snprintf(name, len, "w4a16 %s %s%s", nv ? "nvfp4" : "mxfp4",
                  dec ? mxl_w4a16_decode_config_name(nv ? 1 : 0, m, n, k) : mxl_w4a16_gemm_config_name(),
                  splits > 1 ? ", split-K with a workspace, else one split" : "");
    return MX_OK;
}

mx_status mx_fake_quant(mx_format fmt, mx_scale_rule rule, const void* x_bf16, int64_t rows, int64_t k,
                        float global_scale, void* y_bf16, mx_stream_t stream)
{
    mx_status st = check_quant_args(fmt, rule, x_bf16, rows, k, global_scale, y_bf16, y_bf16);
    if (st != MX_OK) return st;
    const int64_t total = rows * k;
    const uintptr_t xa = reinterpret_cast<uintptr_t>(x_bf16), ya = reinterpret_cast<uintptr_t>(y_bf16);
    const uintptr_t bytes = (uintptr_t)total * 2u;
    if (xa < ya + bytes && ya < xa + bytes) return MX_ERR_INVALID_ARG;  // overlapping x and y
    if ((st = check_device()) != MX_OK) return st;
    hipStream_t hs = static_cast<hipStream_t>(stream);
    if (fmt == MX_FMT_NVFP4) return from_hip(mxl_launch_nv_fake_quant(x_bf16, total, global_scale, y_bf16, hs));
    return from_hip(mxl_launch_mx_fake_quant(fmt == MX_FMT_MXFP4 ? 0 : 1, (int)rule, x_bf16, total, y_bf16, hs));
}

mx_status mx_swiglu_quant(const void* x_bf16, int64_t m, int64_t inter, void* h_q, void* h_s, mx_stream_t stream)
{
    if (!x_bf16 || !h_q || !h_s) return MX_ERR_INVALID_ARG;
    if (m < 1 || m > kMaxDim || inter < 32 || inter % 32 != 0 || inter > kMaxDim / 2) return MX_ERR_SHAPE;
    if (!aligned16(x_bf16) || !aligned16(h_q) || !aligned16(h_s)) return MX_ERR_ALIGN;
    mx_status st = check_device();
    if (st != MX_OK) return st;
    return from_hip(mxl_launch_swiglu_quant(x_bf16, m, inter, h_q, h_s, static_cast<hipStream_t>(stream)));
}

mx_status mx_gemm_swiglu_quant(const void* a_q, const void* a_s, const void* w_q, const void* w_s, int64_t m,
                               int64_t inter, int64_t k, void* h_q, void* h_s, mx_stream_t stream)
{
    if (!a_q || !a_s || !w_q || !w_s || !h_q || !h_s) return MX_ERR_INVALID_ARG;
    if (inter < 32 || inter % 32 != 0 || inter > kMaxDim / 2) return MX_ERR_SHAPE;
    mx_status st = check_gemm_shape(m, 2 * inter, k, 32);
    if (st != MX_OK) return st;
    if (!mxl_prefill_ok(m, 2 * inter, k)) return MX_ERR_UNSUPPORTED;
    if (!aligned16(a_q) || !aligned16(a_s) || !aligned16(w_q) || !aligned16(w_s) || !aligned16(h_q) ||
        !aligned16(h_s))
        return MX_ERR_ALIGN;
    if ((st = check_device()) != MX_OK) return st;
    if (log_enabled())
        std::fprintf(stderr, "[mxlinear] mx_gemm_swiglu_quant m=%lld inter=%lld k=%lld -> %s\n", (long long)m,
                     (long long)inter, (long long)k, mxl_prefill_swiglu_config_name());
    return from_hip(mxl_launch_mx_prefill_swiglu(a_q, a_s, w_q, w_s, m, 2 * inter, k, h_q, h_s,
                                                 static_cast<hipStream_t>(stream)));
}

mx_status mx_gemm_swiglu_quant_plan(int64_t m, int64_t inter, int64_t k, char* name, size_t len)
{
    if (!name || len == 0) return MX_ERR_INVALID_ARG;
    if (inter < 32 || inter % 32 != 0 || inter > kMaxDim / 2) return MX_ERR_SHAPE;
    mx_status st = check_gemm_shape(m, 2 * inter, k, 32);
    if (st != MX_OK) return st;
    if (!mxl_prefill_ok(m, 2 * inter, k)) return MX_ERR_UNSUPPORTED;
    std::snprintf(name, len, "mxfp4 %s", mxl_prefill_swiglu_config_name());
    return MX_OK;
}

mx_status mx_tensor_amax(const void* x_bf16, int64_t count, float* amax_dev, mx_stream_t stream)
{
    if (!x_bf16 || !amax_dev) return MX_ERR_INVALID_ARG;
    if (count < 1) return MX_ERR_SHAPE;
    if (!aligned16(x_bf16) || (reinterpret_cast<uintptr_t>(amax_dev) & 3u)) return MX_ERR_ALIGN;
    mx_status st = check_device();
    if (st != MX_OK) return st;
    return from_hip(mxl_launch_amax(x_bf16, count, amax_dev, static_cast<hipStream_t>(stream)));
}

// g = RNE_fp32(2688 / amax).  The double quotient is within one fp32 ulp of
// the exact one; the float candidates around it are compared by their exact
// distance |c * amax - 2688| (c * amax is exact in a double), ties to the
// even significand.
float mx_nv_global_scale(float amax)
{
    if (!(amax > 0.0f) || !std::isfinite(amax)) return 1.0f;
    const double a = (double)amax;
    const double q = 2688.0 / a;
    if (q > (double)FLT_MAX) return FLT_MAX;
    float c = (float)q;
    float best = c;
    double bestd = std::fabs((double)c * a - 2688.0);
    float lo = c, hi = c;
    for (int i = 0; i < 2; ++i) {
        lo = std::nextafter(lo, 0.0f);
        hi = std::nextafter(hi, FLT_MAX);
        const float cand[2] = {lo, hi};
        for (float v : cand) {
            const double d = std::fabs((double)v * a - 2688.0);
            uint32_t vb, bb;
            std::memcpy(&vb, &v, 4);
            std::memcpy(&bb, &best, 4);
            if (d < bestd || (d == bestd && (vb & 1u) == 0 && (bb & 1u) == 1)) {
                best = v;
                bestd = d;
            }
        }
    }
    return best;
}

mx_status mx_gemm_plan(mx_format a_fmt, mx_format w_fmt, int64_t m, int64_t n, int64_t k, int fused,
                       unsigned flags, char* name, size_t len)
{
    if (!valid_fmt(a_fmt) || !valid_fmt(w_fmt) || !name || len == 0) return MX_ERR_INVALID_ARG;
    const bool nv = a_fmt == MX_FMT_NVFP4;
    if (nv != (w_fmt == MX_FMT_NVFP4)) return MX_ERR_INVALID_ARG;
    mx_status st = check_gemm_shape(m, n, k, nv ? 16 : 32);
    if (st != MX_OK) return st;
    static const char* names[3] = {"mxfp4", "mxfp8", "nvfp4"};
    char fmt[16];
    if (a_fmt == w_fmt) std::snprintf(fmt, sizeof fmt, "%s", names[a_fmt]);
    else std::snprintf(fmt, sizeof fmt, "%sx%s", names[a_fmt], names[w_fmt]);
    const MxPath path = nv ? PATH_EXACT8 : mx_path(a_fmt, w_fmt, flags);
    const bool via_q = fused && !nv && fused_via_quantizer(a_fmt, w_fmt, m, n, k, flags);
    const char* cfg = nv ? mxl_nv_gemm_config_name(m, n, k)
                    : path == PATH_EXACT8 ? mxl_mxfp8_exact_config_name(m, n, k)
                    : path == PATH_MIXED_EXACT ? mxl_mx_mixed_exact_config_name()
                                               : mxl_mx_gemm_config_name(bits_of(a_fmt), bits_of(w_fmt), m, n, k,
                                                                         fused && a_fmt == w_fmt && !via_q);
    const bool dq_decode = (nv || path == PATH_EXACT8) && mxl_dq_decode_ok(nv ? 1 : 0, m, n, k);
    const int splits = (nv || path != PATH_SCALED) && !fused && !dq_decode ? mxl_dq_splits(m, n, k) : 1;
    const char* pre = !fused || nv ? ""
                      : !via_q ? "fused-quant "
                      : fused_requires_quantizer(a_fmt, w_fmt, m, n, k, flags)
                          ? "fused-quant (mx_quantize_act into the workspace, then) "
                          : "fused-quant (with a workspace: mx_quantize_act into it, then; without: the in-tile "
                            "prologue) ";
    if (splits > 1)
        std::snprintf(name, len, "%s%s %s, split-K %d with a workspace, else one split", pre, fmt, cfg, splits);
    else
        std::snprintf(name, len, "%s%s %s", pre, fmt, cfg);
    return MX_OK;
}

} // extern "C"
