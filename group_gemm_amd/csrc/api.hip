// api.hip -- the C ABI: argument validation, workspace layout, grid sizing and launches.
// Host code only; it never reads group_sizes or any other device data (except in
// gg_read_device_status, which exists for tests), never synchronises and never allocates,
// so every call can be captured in a HIP graph.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "groupgemm.h"
#include "launch.hpp"

// Scratch of ragged_dot_m_noalloc: the per-call state that the workspace holds for the other
// calls (status word at offset 0, the 8 tile-queue counters at offset 64), kept in a
// file-scope device array for callers that cannot allocate.  Each GPU holds its own copy
// for the life of the process; every no-allocation call on a GPU shares it.
constexpr size_t kScratchBytes = 256;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

namespace {

constexpr size_t kHeader = 256;   // workspace bytes before any padded buffer (status word first)
constexpr int64_t kMaxCopies = int64_t(1) << 30;   // moe_permute: tokens * top_k
constexpr size_t kQueueOffset = 64;                 // workspace header bytes before the 8 tile queues

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

size_t elem_bytes(gg_dtype d) { return d == GG_DT_F32 ? 4 : d == GG_DT_BF16 ? 2 : 1; }

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

int64_t cdiv64(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Compute units of the current device, cached per device.
int device_cus(int* cus) {
    static int cache[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return -1;
    if (dev >= 0 && dev < 64 && cache[dev] > 0) { *cus = cache[dev]; return 0; }
    int v = 0;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0) return -1;
    if (dev >= 0 && dev < 64) cache[dev] = v;
    *cus = v;
    return 0;
}

// Persistent grid: one workgroup per CU (the big-tile kernels hold 128+ KiB of LDS),
// never more than there are tiles, at least 1 so the status word is always written.
int persistent_grid(int64_t tile_bound, int per_cu, int cus) {
    int64_t g = (int64_t)cus * per_cu;
    if (tile_bound < g) g = tile_bound;
    if (g < 1) g = 1;
    return (int)g;
}

bool fits_i32(int64_t x) { return x >= 0 && x <= INT32_MAX; }

// Shape and group-size checks shared by every entry point.
gg_status check_shape(int64_t m, int64_t k, int64_t n, int32_t g, const int32_t* gs) {
    if (!gs) return GG_ERR_NULL_PTR;
    if (m < 0 || k < 0 || n < 0 || g < 1 || g > GG_MAX_GROUPS) return GG_ERR_BAD_SHAPE;
    if (!fits_i32(m) || !fits_i32(k) || !fits_i32(n)) return GG_ERR_BAD_SHAPE;
    if (!aligned(gs, 4)) return GG_ERR_MISALIGNED;
    return GG_OK;
}

gg_status check_common(int64_t m, int64_t k, int64_t n, int32_t g, const int32_t* gs, void* ws, size_t ws_bytes,
                       size_t need) {
    if (!gs || !ws) return GG_ERR_NULL_PTR;
    gg_status st = check_shape(m, k, n, g, gs);
    if (st != GG_OK) return st;
    if (!aligned(ws, 16)) return GG_ERR_MISALIGNED;
    if (ws_bytes < need) return GG_ERR_WORKSPACE_TOO_SMALL;
    return GG_OK;
}

// ragged_dot_m body, shared with the batched stage of padded_dot (uniform_rows > 0).
// Epilogue of the ring kernels: out = alpha * acc + bias[h] + beta * out.  `on` false: plain
// store (every kernel family); true: only the ring kernels implement it.
struct EpiArgs {
    bool on = false;
    const float* bias = nullptr;
    int64_t bias_stride = 0;
    float alpha = 1.f, beta = 0.f;
};

// `status` may be NULL (the padded form's batched stage leaves the word to the scatter);
// `ws` is the caller's workspace, whose header also holds the bf16 kernel's tile queues.
gg_status run_m(const void* lhs, const void* rhs, const int32_t* gs, void* out, int64_t m, int64_t k, int64_t n,
                int32_t g, gg_dtype in, gg_dtype outd, const uint8_t* ls, const uint8_t* rs, uint32_t* status,
                void* ws, int uniform_rows, hipStream_t s, bool rhs_nk = false, const EpiArgs& ep = EpiArgs()) {
    int cus;
    if (device_cus(&cus) != 0) return GG_ERR_HIP;
    gg::MParams p{};
    p.lhs = lhs; p.rhs = rhs; p.lhs_scale = ls; p.rhs_scale = rs; p.group_sizes = gs; p.out = out; p.status = status;
    p.m = (int)m; p.k = (int)k; p.n = (int)n; p.g = g; p.uniform_rows = uniform_rows;
    p.out_f32 = outd == GG_DT_F32;
    p.rhs_nk = rhs_nk ? 1 : 0;
    p.epi = ep.on ? 1 : 0; p.bias = ep.bias; p.bias_stride = ep.bias_stride; p.alpha = ep.alpha; p.beta = ep.beta;
    p.tile_queue = (int*)((char*)ws + kQueueOffset);
    hipError_t e;
    if (rhs_nk) {   // [g,n,k] weights: the bf16 ring kernel only
        const bool vec = aligned(lhs, 16) && aligned(rhs, 16) && aligned(out, 16) && k % 8 == 0 && n % 8 == 0;
        if (in != GG_DT_BF16 || !vec || !gg::ragged_m_bf16_fast_ok(p)) return GG_ERR_UNSUPPORTED;
        int64_t bound = (cdiv64(m, gg::ragged_m_bf16_fast_bm(p)) + g + 1) * cdiv64(n, 256);
        if (!fits_i32(bound)) return GG_ERR_BAD_SHAPE;
        e = gg::launch_ragged_m_bf16_fast(p, persistent_grid(bound, 1, cus), s);
    } else if (in == GG_DT_F32) {
        if (ep.on) return GG_ERR_UNSUPPORTED;
        gg::TileShape ts = gg::tiles_m_f32();
        int64_t bound = (cdiv64(m, ts.bm) + g + 1) * cdiv64(n, ts.bn);
        if (!fits_i32(bound)) return GG_ERR_BAD_SHAPE;
        e = gg::launch_ragged_m_f32(p, persistent_grid(bound, 4, cus), s);
    } else if (in == GG_DT_BF16) {
        const bool vec = aligned(lhs, 16) && aligned(rhs, 16) && aligned(out, 16) && k % 8 == 0 && n % 8 == 0;
        const bool fast = vec && gg::ragged_m_bf16_fast_ok(p);
        gg::TileShape ts = gg::tiles_m_bf16();
        if (fast) ts = {gg::ragged_m_bf16_fast_bm(p), 256};
        int64_t bound = (cdiv64(m, ts.bm) + g + 1) * cdiv64(n, ts.bn);
        if (!fits_i32(bound)) return GG_ERR_BAD_SHAPE;
        if (ep.on && !fast) return GG_ERR_UNSUPPORTED;
        if (fast) e = gg::launch_ragged_m_bf16_fast(p, persistent_grid(bound, 1, cus), s);
        else e = gg::launch_ragged_m_bf16(p, persistent_grid(bound, 1, cus), vec, s);
    } else {
        const bool fast = aligned(lhs, 16) && aligned(rhs, 16) && aligned(out, 16) && aligned(ls, 4) && aligned(rs, 4) &&
                          gg::ragged_m_mx_fast_ok(p);
        gg::TileShape ts = gg::tiles_m_e4m3();
        if (fast) ts = {256, 256};
        int64_t bound = (cdiv64(m, ts.bm) + g + 1) * cdiv64(n, ts.bn);
        if (!fits_i32(bound)) return GG_ERR_BAD_SHAPE;
        if (ep.on && !fast) return GG_ERR_UNSUPPORTED;
        if (fast) e = gg::launch_ragged_m_mx_fast(p, persistent_grid(bound, 1, cus), s);
        else e = gg::launch_ragged_m_e4m3(p, persistent_grid(bound, 1, cus), s);
    }
    return e == hipSuccess ? GG_OK : GG_ERR_HIP;
}

gg_status run_k(const void* lhs, const void* dout, const int32_t* gs, void* out, int64_t m, int64_t k, int64_t n,
                int32_t g, gg_dtype in, gg_dtype outd, uint32_t* status, int uniform_rows, hipStream_t s,
                const EpiArgs& ep = EpiArgs()) {
    int cus;
    if (device_cus(&cus) != 0) return GG_ERR_HIP;
    gg::KParams p{};
    p.lhs = lhs; p.dout = dout; p.group_sizes = gs; p.out = out; p.status = status;
    p.m = (int)m; p.k = (int)k; p.n = (int)n; p.g = g; p.uniform_rows = uniform_rows;
    p.out_f32 = outd == GG_DT_F32;
    p.epi = ep.on ? 1 : 0; p.alpha = ep.alpha; p.beta = ep.beta;
    hipError_t e;
    if (in == GG_DT_F32) {
        if (ep.on) return GG_ERR_UNSUPPORTED;
        gg::TileShape ts = gg::tiles_k_f32();
        int64_t bound = (int64_t)g * cdiv64(k, ts.bm) * cdiv64(n, ts.bn);
        if (!fits_i32(bound)) return GG_ERR_BAD_SHAPE;
        e = gg::launch_ragged_k_f32(p, persistent_grid(bound, 4, cus), s);
    } else {
        gg::TileShape ts = gg::tiles_k_bf16();
        int64_t bound = (int64_t)g * cdiv64(k, ts.bm) * cdiv64(n, ts.bn);
        if (!fits_i32(bound)) return GG_ERR_BAD_SHAPE;
        const bool vec = aligned(lhs, 16) && aligned(dout, 16) && k % 8 == 0 && n % 8 == 0;
        const bool fast = vec && aligned(out, 16) && gg::ragged_k_bf16_fast_ok(p);
        if (ep.on && !fast) return GG_ERR_UNSUPPORTED;
        if (fast) e = gg::launch_ragged_k_bf16_fast(p, persistent_grid(bound, 1, cus), s);
        else e = gg::launch_ragged_k_bf16(p, persistent_grid(bound, 1, cus), vec, s);
    }
    return e == hipSuccess ? GG_OK : GG_ERR_HIP;
}

// Device address of `scratch` on the current device, resolved once per device with that
// device current (host code must never pass the array's own name: that is a host-side
// stand-in, not a device address).  NULL if the lookup fails.
void* scratch_address() {
    static std::mutex mu;
    static void* addr[64] = {nullptr};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
    std::lock_guard<std::mutex> lock(mu);
    if (!addr[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
        addr[dev] = p;
    }
    return addr[dev];
}

bool m_dtypes_ok(gg_dtype in, gg_dtype out) {
    if (in == GG_DT_F32) return out == GG_DT_F32;
    if (in == GG_DT_BF16 || in == GG_DT_E4M3) return out == GG_DT_BF16 || out == GG_DT_F32;
    return false;
}
bool k_dtypes_ok(gg_dtype in, gg_dtype out) {
    if (in == GG_DT_F32) return out == GG_DT_F32;
    if (in == GG_DT_BF16) return out == GG_DT_F32 || out == GG_DT_BF16;
    return false;
}

}  // namespace

extern "C" {

int gg_abi_version(void) { return GG_ABI_VERSION; }

const char* gg_status_string(gg_status s) {
    switch (s) {
        case GG_OK: return "ok";
        case GG_ERR_NULL_PTR: return "a required pointer is NULL";
        case GG_ERR_BAD_SHAPE: return "bad shape (negative size, g outside [1, GG_MAX_GROUPS], or too large)";
        case GG_ERR_BAD_DTYPE: return "unsupported element type combination";
        case GG_ERR_MISALIGNED: return "misaligned pointer";
        case GG_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
        case GG_ERR_UNSUPPORTED: return "unsupported argument combination";
        case GG_ERR_HIP: return "HIP runtime error";
        default: break;
    }
    return "unknown status";
}

size_t gg_workspace_bytes(gg_op op, int64_t m, int64_t k, int64_t n, int32_t g, int64_t capacity, gg_dtype in) {
    if (m < 0 || k < 0 || n < 0 || g < 1 || g > GG_MAX_GROUPS) return 0;
    if (in != GG_DT_F32 && in != GG_DT_BF16 && in != GG_DT_E4M3) return 0;
    switch (op) {
        case GG_OP_RAGGED_M:
        case GG_OP_RAGGED_K: return kHeader;
        case GG_OP_PADDED_M: {
            if (capacity < 1) return 0;
            const size_t rows = (size_t)g * (size_t)capacity;
            size_t b = kHeader;
            b += align_up(rows * (size_t)k * elem_bytes(in), 256);    // padded lhs
            b += align_up(rows * (size_t)n * 4, 256);                 // padded result (room for fp32)
            if (in == GG_DT_E4M3) b += align_up(rows * (size_t)(k / 32), 256);   // padded lhs scales
            return b;
        }
        case GG_OP_PADDED_K: {
            if (capacity < 1) return 0;
            const size_t rows = (size_t)g * (size_t)capacity;
            return kHeader + align_up(rows * (size_t)k * elem_bytes(in), 256) + align_up(rows * (size_t)n * elem_bytes(in), 256);
        }
        case GG_OP_PERMUTE: {
            if (m > kMaxCopies) return 0;
            const gg::PermuteGeometry pg = gg::permute_geometry(m);
            return kHeader + align_up((size_t)pg.nblk * (size_t)g * 4, 256) + align_up((size_t)pg.nblk * 4, 256);
        }
        default: break;
    }
    return 0;
}

gg_status ragged_dot_m(const void* lhs, const void* rhs, const int32_t* group_sizes, void* out, int64_t m, int64_t k,
                       int64_t n, int32_t g, gg_dtype in_dtype, gg_dtype out_dtype, const uint8_t* lhs_scale,
                       const uint8_t* rhs_scale, void* workspace, size_t workspace_bytes, void* stream) {
    gg_status st = check_common(m, k, n, g, group_sizes, workspace, workspace_bytes, kHeader);
    if (st != GG_OK) return st;
    if (!m_dtypes_ok(in_dtype, out_dtype)) return GG_ERR_BAD_DTYPE;
    if ((m * k > 0 && !lhs) || (k * n > 0 && !rhs) || (m * n > 0 && !out)) return GG_ERR_NULL_PTR;
    const size_t es = elem_bytes(in_dtype);
    if (!aligned(lhs, es) || !aligned(rhs, es) || !aligned(out, elem_bytes(out_dtype))) return GG_ERR_MISALIGNED;
    if (in_dtype == GG_DT_E4M3) {
        if (k % 32 != 0) return GG_ERR_UNSUPPORTED;
        if ((m * k > 0 && !lhs_scale) || (k * n > 0 && !rhs_scale)) return GG_ERR_NULL_PTR;
        if (!aligned(lhs, 16) || !aligned(rhs, 16)) return GG_ERR_MISALIGNED;
    }
    return run_m(lhs, rhs, group_sizes, out, m, k, n, g, in_dtype, out_dtype, lhs_scale, rhs_scale, (uint32_t*)workspace, workspace,
                 0, (hipStream_t)stream);
}

gg_status ragged_dot_m_noalloc(const void* lhs, const void* rhs, const int32_t* group_sizes, void* out, int64_t m,
                               int64_t k, int64_t n, int32_t g, gg_dtype in_dtype, gg_dtype out_dtype,
                               const uint8_t* lhs_scale, const uint8_t* rhs_scale, uint32_t* status, void* stream) {
    // the scratch must hold what the workspace of ragged_dot_m would (the same for any shape)
    const size_t need = gg_workspace_bytes(GG_OP_RAGGED_M, m, k, n, g, 0, in_dtype);
    if (need > kScratchBytes) return GG_ERR_WORKSPACE_TOO_SMALL;
    if (!aligned(status, 4)) return GG_ERR_MISALIGNED;
    gg_status st = check_shape(m, k, n, g, group_sizes);
    if (st != GG_OK) return st;
    if (!m_dtypes_ok(in_dtype, out_dtype)) return GG_ERR_BAD_DTYPE;
    if ((m * k > 0 && !lhs) || (k * n > 0 && !rhs) || (m * n > 0 && !out)) return GG_ERR_NULL_PTR;
    const size_t es = elem_bytes(in_dtype);
    if (!aligned(lhs, es) || !aligned(rhs, es) || !aligned(out, elem_bytes(out_dtype))) return GG_ERR_MISALIGNED;
    if (in_dtype == GG_DT_E4M3) {
        if (k % 32 != 0) return GG_ERR_UNSUPPORTED;
        if ((m * k > 0 && !lhs_scale) || (k * n > 0 && !rhs_scale)) return GG_ERR_NULL_PTR;
        if (!aligned(lhs, 16) || !aligned(rhs, 16)) return GG_ERR_MISALIGNED;
    }
    void* ws = scratch_address();   // looked up only once every argument has passed its check
    if (!ws) return GG_ERR_HIP;
    return run_m(lhs, rhs, group_sizes, out, m, k, n, g, in_dtype, out_dtype, lhs_scale, rhs_scale,
                 status ? status : (uint32_t*)ws, ws, 0, (hipStream_t)stream);
}

gg_status ragged_dot_m_nk(const void* lhs, const void* rhs_nk, const int32_t* group_sizes, void* out, int64_t m,
                          int64_t k, int64_t n, int32_t g, gg_dtype in_dtype, gg_dtype out_dtype, void* workspace,
                          size_t workspace_bytes, void* stream) {
    gg_status st = check_common(m, k, n, g, group_sizes, workspace, workspace_bytes, kHeader);
    if (st != GG_OK) return st;
    if (in_dtype != GG_DT_BF16) return GG_ERR_UNSUPPORTED;
    if (!m_dtypes_ok(in_dtype, out_dtype)) return GG_ERR_BAD_DTYPE;
    if ((m * k > 0 && !lhs) || (k * n > 0 && !rhs_nk) || (m * n > 0 && !out)) return GG_ERR_NULL_PTR;
    if (!aligned(lhs, 16) || !aligned(rhs_nk, 16) || !aligned(out, 16)) return GG_ERR_MISALIGNED;
    if (k % 8 != 0 || n % 8 != 0) return GG_ERR_UNSUPPORTED;
    return run_m(lhs, rhs_nk, group_sizes, out, m, k, n, g, in_dtype, out_dtype, nullptr, nullptr, (uint32_t*)workspace, workspace,
                 0, (hipStream_t)stream, true);
}

gg_status ragged_dot_m_epilogue(const void* lhs, const void* rhs, const int32_t* group_sizes, void* out, int64_t m,
                                int64_t k, int64_t n, int32_t g, gg_dtype in_dtype, gg_dtype out_dtype,
                                const uint8_t* lhs_scale, const uint8_t* rhs_scale, const float* bias, int64_t bias_stride,
                                float alpha, float beta, void* workspace, size_t workspace_bytes, void* stream) {
    if (bias && (bias_stride < n || !aligned(bias, 4))) return bias_stride < n ? GG_ERR_BAD_SHAPE : GG_ERR_MISALIGNED;
    EpiArgs ep;
    ep.on = bias != nullptr || alpha != 1.f || beta != 0.f;
    ep.bias = bias; ep.bias_stride = bias_stride; ep.alpha = alpha; ep.beta = beta;
    gg_status st = check_common(m, k, n, g, group_sizes, workspace, workspace_bytes, kHeader);
    if (st != GG_OK) return st;
    if (!m_dtypes_ok(in_dtype, out_dtype)) return GG_ERR_BAD_DTYPE;
    if ((m * k > 0 && !lhs) || (k * n > 0 && !rhs) || (m * n > 0 && !out)) return GG_ERR_NULL_PTR;
    const size_t es = elem_bytes(in_dtype);
    if (!aligned(lhs, es) || !aligned(rhs, es) || !aligned(out, elem_bytes(out_dtype))) return GG_ERR_MISALIGNED;
    if (in_dtype == GG_DT_E4M3) {
        if (k % 32 != 0) return GG_ERR_UNSUPPORTED;
        if ((m * k > 0 && !lhs_scale) || (k * n > 0 && !rhs_scale)) return GG_ERR_NULL_PTR;
        if (!aligned(lhs, 16) || !aligned(rhs, 16)) return GG_ERR_MISALIGNED;
    }
    return run_m(lhs, rhs, group_sizes, out, m, k, n, g, in_dtype, out_dtype, lhs_scale, rhs_scale, (uint32_t*)workspace, workspace,
                 0, (hipStream_t)stream, false, ep);
}

gg_status ragged_dot_k_epilogue(const void* lhs, const void* dout, const int32_t* group_sizes, void* out, int64_t m,
                                int64_t k, int64_t n, int32_t g, gg_dtype in_dtype, gg_dtype out_dtype, float alpha,
                                float beta, void* workspace, size_t workspace_bytes, void* stream) {
    EpiArgs ep;
    ep.on = alpha != 1.f || beta != 0.f;
    ep.alpha = alpha; ep.beta = beta;
    gg_status st = check_common(m, k, n, g, group_sizes, workspace, workspace_bytes, kHeader);
    if (st != GG_OK) return st;
    if (!k_dtypes_ok(in_dtype, out_dtype)) return GG_ERR_BAD_DTYPE;
    if ((m * k > 0 && !lhs) || (m * n > 0 && !dout) || (k * n > 0 && !out)) return GG_ERR_NULL_PTR;
    const size_t es = elem_bytes(in_dtype);
    if (!aligned(lhs, es) || !aligned(dout, es) || !aligned(out, elem_bytes(out_dtype))) return GG_ERR_MISALIGNED;
    return run_k(lhs, dout, group_sizes, out, m, k, n, g, in_dtype, out_dtype, (uint32_t*)workspace, 0,
                 (hipStream_t)stream, ep);
}

gg_status ragged_dot_m_gated(const void* lhs, const void* w0, const void* w1, const int32_t* group_sizes, void* out,
                             int64_t m, int64_t k, int64_t n, int32_t g, gg_dtype in_dtype, gg_dtype out_dtype,
                             gg_activation act, const float* bias0, const float* bias1, int64_t bias_stride,
                             void* workspace, size_t workspace_bytes, void* stream) {
    gg_status st = check_common(m, k, n, g, group_sizes, workspace, workspace_bytes, kHeader);
    if (st != GG_OK) return st;
    if (in_dtype != GG_DT_BF16) return GG_ERR_UNSUPPORTED;
    if (!m_dtypes_ok(in_dtype, out_dtype)) return GG_ERR_BAD_DTYPE;
    if (act != GG_ACT_SILU && act != GG_ACT_GELU_TANH) return GG_ERR_UNSUPPORTED;
    if ((m * k > 0 && !lhs) || (k * n > 0 && (!w0 || !w1)) || (m * n > 0 && !out)) return GG_ERR_NULL_PTR;
    if ((bias0 || bias1) && bias_stride < n) return GG_ERR_BAD_SHAPE;
    if (!aligned(bias0, 4) || !aligned(bias1, 4)) return GG_ERR_MISALIGNED;
    if (!aligned(lhs, 16) || !aligned(w0, 16) || !aligned(w1, 16) || !aligned(out, 16)) return GG_ERR_MISALIGNED;
    if (k % 8 != 0 || n % 8 != 0) return GG_ERR_UNSUPPORTED;
    int cus;
    if (device_cus(&cus) != 0) return GG_ERR_HIP;
    gg::GParams p{};
    p.lhs = lhs; p.w0 = w0; p.w1 = w1; p.group_sizes = group_sizes; p.out = out; p.status = (uint32_t*)workspace;
    p.bias0 = bias0; p.bias1 = bias1; p.bias_stride = bias_stride;
    p.m = (int)m; p.k = (int)k; p.n = (int)n; p.g = g; p.out_f32 = out_dtype == GG_DT_F32; p.act = (int)act;
    if (!gg::ragged_m_gated_ok(p)) return GG_ERR_UNSUPPORTED;
    const int64_t bound = (cdiv64(m, 256) + g + 1) * cdiv64(n, 128);
    if (!fits_i32(bound)) return GG_ERR_BAD_SHAPE;
    return gg::launch_ragged_m_gated(p, persistent_grid(bound, 1, cus), (hipStream_t)stream) == hipSuccess ? GG_OK
                                                                                                           : GG_ERR_HIP;
}

gg_status ragged_dot_k(const void* lhs, const void* dout, const int32_t* group_sizes, void* out, int64_t m, int64_t k,
                       int64_t n, int32_t g, gg_dtype in_dtype, gg_dtype out_dtype, void* workspace,
                       size_t workspace_bytes, void* stream) {
    gg_status st = check_common(m, k, n, g, group_sizes, workspace, workspace_bytes, kHeader);
    if (st != GG_OK) return st;
    if (!k_dtypes_ok(in_dtype, out_dtype)) return GG_ERR_BAD_DTYPE;
    if ((m * k > 0 && !lhs) || (m * n > 0 && !dout) || (k * n > 0 && !out)) return GG_ERR_NULL_PTR;
    const size_t es = elem_bytes(in_dtype);
    if (!aligned(lhs, es) || !aligned(dout, es) || !aligned(out, elem_bytes(out_dtype))) return GG_ERR_MISALIGNED;
    return run_k(lhs, dout, group_sizes, out, m, k, n, g, in_dtype, out_dtype, (uint32_t*)workspace, 0,
                 (hipStream_t)stream);
}

gg_status padded_dot(gg_op mode, const void* a, const void* b, const int32_t* group_sizes, void* out, int64_t m,
                     int64_t k, int64_t n, int32_t g, int64_t capacity, gg_dtype in_dtype, gg_dtype out_dtype,
                     const uint8_t* a_scale, const uint8_t* b_scale, void* workspace, size_t workspace_bytes,
                     void* stream) {
    if (mode != GG_OP_PADDED_M && mode != GG_OP_PADDED_K) return GG_ERR_UNSUPPORTED;
    if (capacity < 1 || !fits_i32(capacity) || !fits_i32((int64_t)g * capacity)) return GG_ERR_BAD_SHAPE;
    const size_t need = gg_workspace_bytes(mode, m, k, n, g, capacity, in_dtype);
    gg_status st = check_common(m, k, n, g, group_sizes, workspace, workspace_bytes, need ? need : kHeader);
    if (st != GG_OK) return st;
    const bool is_m = mode == GG_OP_PADDED_M;
    if (is_m ? !m_dtypes_ok(in_dtype, out_dtype) : !k_dtypes_ok(in_dtype, out_dtype)) return GG_ERR_BAD_DTYPE;
    if (need == 0) return GG_ERR_BAD_SHAPE;
    const size_t es = elem_bytes(in_dtype), os = elem_bytes(out_dtype);
    if (!a || !b || !out) return GG_ERR_NULL_PTR;
    if (!aligned(a, es) || !aligned(b, es) || !aligned(out, os)) return GG_ERR_MISALIGNED;
    if (in_dtype == GG_DT_E4M3) {
        if (!is_m) return GG_ERR_BAD_DTYPE;
        if (k % 32 != 0) return GG_ERR_UNSUPPORTED;
        if (!a_scale || !b_scale) return GG_ERR_NULL_PTR;
        if (!aligned(a, 16) || !aligned(b, 16)) return GG_ERR_MISALIGNED;
    }
    hipStream_t s = (hipStream_t)stream;
    uint32_t* status = (uint32_t*)workspace;
    uint8_t* base = (uint8_t*)workspace + kHeader;
    const int64_t rows = (int64_t)g * capacity;
    uint8_t* pa = base;
    uint8_t* pb = pa + align_up((size_t)rows * (size_t)k * es, 256);
    hipError_t e;
    if (is_m) {
        // 1. expand: lhs rows -> [g, C, k] (+ their scales)
        e = gg::launch_pad_scatter(a, pa, group_sizes, (int)m, g, (int)capacity, (long long)k * (long long)es, status, s);
        if (e != hipSuccess) return GG_ERR_HIP;
        uint8_t* psc = pb + align_up((size_t)rows * (size_t)n * 4, 256);
        if (in_dtype == GG_DT_E4M3) {
            e = gg::launch_pad_scatter(a_scale, psc, group_sizes, (int)m, g, (int)capacity, (long long)(k / 32), nullptr, s);
            if (e != hipSuccess) return GG_ERR_HIP;
        }
        // 2. one uniform batched GEMM [g, C, k] x [g, k, n] -> [g, C, n]
        st = run_m(pa, b, group_sizes, pb, rows, k, n, g, in_dtype, out_dtype, psc, b_scale, nullptr, workspace, (int)capacity, s);
        if (st != GG_OK) return st;
        // 3. compact: [g, C, n] -> [m, n]
        e = gg::launch_pad_gather(pb, out, group_sizes, (int)m, g, (int)capacity, (long long)n * (long long)os, s);
        return e == hipSuccess ? GG_OK : GG_ERR_HIP;
    }
    // contracting form: expand both operands, then one uniform batched contraction
    e = gg::launch_pad_scatter(a, pa, group_sizes, (int)m, g, (int)capacity, (long long)k * (long long)es, status, s);
    if (e != hipSuccess) return GG_ERR_HIP;
    e = gg::launch_pad_scatter(b, pb, group_sizes, (int)m, g, (int)capacity, (long long)n * (long long)es, nullptr, s);
    if (e != hipSuccess) return GG_ERR_HIP;
    return run_k(pa, pb, group_sizes, out, rows, k, n, g, in_dtype, out_dtype, nullptr, (int)capacity, s);
}

gg_status moe_permute(const void* x, const uint8_t* x_scale, const int32_t* experts, void* sorted_x,
                      uint8_t* sorted_scale, int32_t* group_sizes, int32_t* sorted_to_copy, int32_t* copy_to_sorted,
                      int64_t tokens, int32_t top_k, int64_t k, int32_t g, gg_dtype dtype, void* workspace,
                      size_t workspace_bytes, void* stream) {
    if (!group_sizes || !workspace) return GG_ERR_NULL_PTR;
    if (tokens < 0 || top_k < 1 || k < 0 || g < 1 || g > GG_MAX_GROUPS || !fits_i32(k)) return GG_ERR_BAD_SHAPE;
    if (tokens > kMaxCopies / top_k) return GG_ERR_BAD_SHAPE;
    if (dtype != GG_DT_F32 && dtype != GG_DT_BF16 && dtype != GG_DT_E4M3) return GG_ERR_BAD_DTYPE;
    const int64_t M = tokens * top_k;
    if (M > 0 && (!experts || !sorted_to_copy || !copy_to_sorted)) return GG_ERR_NULL_PTR;
    if (tokens * k > 0 && (!x || !sorted_x)) return GG_ERR_NULL_PTR;
    const bool mx = dtype == GG_DT_E4M3;
    if (mx && k % 32 != 0) return GG_ERR_UNSUPPORTED;
    if (mx && tokens * k > 0 && (!x_scale || !sorted_scale)) return GG_ERR_NULL_PTR;
    if (!mx && (x_scale || sorted_scale)) return GG_ERR_BAD_DTYPE;
    const size_t es = elem_bytes(dtype);
    if (!aligned(x, es) || !aligned(sorted_x, es) || !aligned(experts, 4) || !aligned(group_sizes, 4) ||
        !aligned(sorted_to_copy, 4) || !aligned(copy_to_sorted, 4) || !aligned(workspace, 16))
        return GG_ERR_MISALIGNED;
    if (workspace_bytes < gg_workspace_bytes(GG_OP_PERMUTE, M, k, 0, g, 0, dtype)) return GG_ERR_WORKSPACE_TOO_SMALL;
    const gg::PermuteGeometry pg = gg::permute_geometry(M);
    uint8_t* ws = (uint8_t*)workspace;
    gg::PermuteArgs a{};
    a.x = x; a.x_scale = mx ? x_scale : nullptr; a.experts = experts;
    a.sorted_x = sorted_x; a.sorted_scale = mx ? sorted_scale : nullptr;
    a.group_sizes = group_sizes; a.sorted_to_copy = sorted_to_copy; a.copy_to_sorted = copy_to_sorted;
    a.status = (uint32_t*)ws;
    a.total_routed = (int*)(ws + 4);
    a.counts = (int*)(ws + kHeader);
    a.bad = (int*)(ws + kHeader + align_up((size_t)pg.nblk * (size_t)g * 4, 256));
    a.tokens = (int)tokens; a.top_k = top_k; a.g = g;
    a.row_bytes = k * (int64_t)es;
    a.scale_row_bytes = mx ? k / 32 : 0;
    return gg::launch_permute(a, (hipStream_t)stream) == hipSuccess ? GG_OK : GG_ERR_HIP;
}

gg_status moe_unpermute(const void* y, const int32_t* copy_to_sorted, const float* weights, void* out, int64_t tokens,
                        int32_t top_k, int64_t n, gg_dtype in_dtype, gg_dtype out_dtype, void* stream) {
    if (tokens < 0 || top_k < 1 || n < 0 || !fits_i32(n)) return GG_ERR_BAD_SHAPE;
    if (tokens > 0 && (!copy_to_sorted || !weights)) return GG_ERR_NULL_PTR;
    if (tokens > kMaxCopies / top_k) return GG_ERR_BAD_SHAPE;
    if ((in_dtype != GG_DT_F32 && in_dtype != GG_DT_BF16) || (out_dtype != GG_DT_F32 && out_dtype != GG_DT_BF16))
        return GG_ERR_BAD_DTYPE;
    if (tokens * n > 0 && (!y || !out)) return GG_ERR_NULL_PTR;
    if (!aligned(y, elem_bytes(in_dtype)) || !aligned(out, elem_bytes(out_dtype)) || !aligned(copy_to_sorted, 4) ||
        !aligned(weights, 4))
        return GG_ERR_MISALIGNED;
    return gg::launch_combine(y, in_dtype == GG_DT_BF16, (int)(tokens * top_k), copy_to_sorted, weights, (int)tokens,
                              top_k, (int)n, out, out_dtype == GG_DT_BF16, (hipStream_t)stream) == hipSuccess
               ? GG_OK
               : GG_ERR_HIP;
}

gg_status gg_schedule(const int32_t* group_sizes, int64_t m, int64_t n, int32_t g, int32_t block_m, int32_t block_n,
                      int32_t* row_off, int32_t* tile_off, uint32_t* status, void* stream) {
    if (!group_sizes || !row_off || !tile_off || !status) return GG_ERR_NULL_PTR;
    if (m < 0 || n < 0 || g < 1 || g > GG_MAX_GROUPS || !fits_i32(m) || !fits_i32(n)) return GG_ERR_BAD_SHAPE;
    if (block_m < 1 || block_m > 4096 || block_n < 1 || block_n > 4096) return GG_ERR_BAD_SHAPE;
    if (!aligned(group_sizes, 4) || !aligned(row_off, 4) || !aligned(tile_off, 4) || !aligned(status, 4))
        return GG_ERR_MISALIGNED;
    hipError_t e = gg::launch_schedule(group_sizes, (int)m, (int)n, g, block_m, block_n, row_off, tile_off, status,
                                       (hipStream_t)stream);
    return e == hipSuccess ? GG_OK : GG_ERR_HIP;
}

gg_status gg_read_device_status(const void* workspace, uint32_t* flags, void* stream) {
    if (!workspace || !flags) return GG_ERR_NULL_PTR;
    hipStream_t s = (hipStream_t)stream;
    if (hipStreamSynchronize(s) != hipSuccess) return GG_ERR_HIP;
    if (hipMemcpy(flags, workspace, sizeof(uint32_t), hipMemcpyDeviceToHost) != hipSuccess) return GG_ERR_HIP;
    return GG_OK;
}

}  // extern "C"
