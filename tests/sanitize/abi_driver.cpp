// abi_driver.cpp -- the C ABI's host-side argument checks under AddressSanitizer and
// UndefinedBehaviorSanitizer (api.hip built with host instrumentation, linked with the kernel
// objects).  Every entry point is called with arguments its validation must refuse -- null,
// misaligned and fake addresses, negative and oversized shapes, unknown element types, short
// workspaces -- and with a deterministic stream of random arguments.  Runs only where no GPU is
// visible: a call that passed validation then fails at its first runtime call and returns
// GG_ERR_HIP, so no fake address ever reaches a kernel.  Exit status 0 on success.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdio.h>

#include "groupgemm.h"

static int failures = 0;
#define EXPECT(call, code)                                                                    \
    do {                                                                                      \
        const int got_ = (int)(call);                                                         \
        if (got_ != (code)) {                                                                 \
            fprintf(stderr, "line %d: %s returned %d, expected %d\n", __LINE__, #call, got_, (code)); \
            ++failures;                                                                       \
        }                                                                                     \
    } while (0)

static uint64_t rng = 0x9E3779B97F4A7C15ull;
static uint64_t next_u64() {   // splitmix64
    uint64_t z = (rng += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}
static int64_t pick_dim() {
    static const int64_t v[] = {-1, 0, 1, 7, 8, 31, 32, 64, 96, 4096, 14336, (int64_t)1 << 31, -((int64_t)1 << 40)};
    return v[next_u64() % (sizeof v / sizeof v[0])];
}
static void* pick_ptr() {
    static void* const v[] = {nullptr, (void*)0x10000, (void*)0x10001, (void*)0x10002, (void*)0x10008, (void*)0x10010};
    return v[next_u64() % (sizeof v / sizeof v[0])];
}
static int pick_code(int lo, int hi) { return lo + (int)(next_u64() % (uint64_t)(hi - lo + 1)); }

int main() {
    int devices = 0;
    if (hipGetDeviceCount(&devices) == hipSuccess && devices > 0) {
        printf("a GPU is visible: skipped (this driver passes fake addresses)\n");
        return 77;
    }
    void* P = (void*)0x10000;                   // aligned, never dereferenced
    const int32_t* GS = (const int32_t*)P;
    const gg_dtype BF = GG_DT_BF16, F32 = GG_DT_F32, E4 = GG_DT_E4M3;

    // ragged_dot_m
    EXPECT(ragged_dot_m(P, P, nullptr, P, 64, 64, 64, 4, BF, BF, nullptr, nullptr, P, 4096, nullptr), GG_ERR_NULL_PTR);
    EXPECT(ragged_dot_m(P, P, GS, P, 64, 64, 64, 0, BF, BF, nullptr, nullptr, P, 4096, nullptr), GG_ERR_BAD_SHAPE);
    EXPECT(ragged_dot_m(P, P, GS, P, 64, 64, 64, 1025, BF, BF, nullptr, nullptr, P, 4096, nullptr), GG_ERR_BAD_SHAPE);
    EXPECT(ragged_dot_m(P, P, GS, P, -1, 64, 64, 4, BF, BF, nullptr, nullptr, P, 4096, nullptr), GG_ERR_BAD_SHAPE);
    EXPECT(ragged_dot_m(P, P, GS, P, 64, (int64_t)1 << 31, 64, 4, BF, BF, nullptr, nullptr, P, 4096, nullptr), GG_ERR_BAD_SHAPE);
    EXPECT(ragged_dot_m(P, P, GS, P, 64, 64, 64, 4, F32, BF, nullptr, nullptr, P, 4096, nullptr), GG_ERR_BAD_DTYPE);
    EXPECT(ragged_dot_m(P, P, GS, P, 64, 64, 64, 4, (gg_dtype)7, BF, nullptr, nullptr, P, 4096, nullptr), GG_ERR_BAD_DTYPE);
    EXPECT(ragged_dot_m(P, P, GS, P, 64, 64, 64, 4, BF, BF, nullptr, nullptr, (void*)0x10004, 4096, nullptr), GG_ERR_MISALIGNED);
    EXPECT(ragged_dot_m((void*)0x10001, P, GS, P, 64, 64, 64, 4, BF, BF, nullptr, nullptr, P, 4096, nullptr), GG_ERR_MISALIGNED);
    EXPECT(ragged_dot_m(P, P, GS, P, 64, 64, 64, 4, BF, BF, nullptr, nullptr, P, 8, nullptr), GG_ERR_WORKSPACE_TOO_SMALL);
    EXPECT(ragged_dot_m(P, P, GS, P, 64, 48, 64, 4, E4, BF, (const uint8_t*)P, (const uint8_t*)P, P, 4096, nullptr), GG_ERR_UNSUPPORTED);
    EXPECT(ragged_dot_m(P, P, GS, P, 64, 64, 64, 4, E4, BF, nullptr, (const uint8_t*)P, P, 4096, nullptr), GG_ERR_NULL_PTR);
    // the no-allocation form
    EXPECT(ragged_dot_m_noalloc(P, P, nullptr, P, 64, 64, 64, 4, BF, BF, nullptr, nullptr, nullptr, nullptr), GG_ERR_NULL_PTR);
    EXPECT(ragged_dot_m_noalloc(P, P, GS, P, 64, 64, 64, 4, BF, BF, nullptr, nullptr, (uint32_t*)0x10002, nullptr), GG_ERR_MISALIGNED);
    // ragged_dot_m_nk, epilogues, gated
    EXPECT(ragged_dot_m_nk(P, P, GS, P, 64, 64, 64, 4, F32, F32, P, 4096, nullptr), GG_ERR_UNSUPPORTED);
    EXPECT(ragged_dot_m_nk(P, (void*)0x10008, GS, P, 64, 64, 64, 4, BF, BF, P, 4096, nullptr), GG_ERR_MISALIGNED);
    EXPECT(ragged_dot_m_nk(P, P, GS, P, 64, 60, 64, 4, BF, BF, P, 4096, nullptr), GG_ERR_UNSUPPORTED);
    EXPECT(ragged_dot_m_epilogue(P, P, GS, P, 64, 64, 64, 4, BF, BF, nullptr, nullptr, (const float*)P, 32, 1.f, 0.f, P, 4096,
                                 nullptr), GG_ERR_BAD_SHAPE);
    EXPECT(ragged_dot_m_epilogue(P, P, GS, P, 64, 64, 64, 4, BF, BF, nullptr, nullptr, (const float*)0x10002, 64, 1.f, 0.f, P,
                                 4096, nullptr), GG_ERR_MISALIGNED);
    EXPECT(ragged_dot_k_epilogue(P, P, GS, P, 64, 64, 64, 4, E4, F32, 1.f, 1.f, P, 4096, nullptr), GG_ERR_BAD_DTYPE);
    EXPECT(ragged_dot_m_gated(P, P, P, GS, P, 64, 64, 64, 4, BF, BF, (gg_activation)9, nullptr, nullptr, 0, P, 4096, nullptr),
           GG_ERR_UNSUPPORTED);
    EXPECT(ragged_dot_m_gated(P, P, nullptr, GS, P, 64, 64, 64, 4, BF, BF, GG_ACT_SILU, nullptr, nullptr, 0, P, 4096, nullptr),
           GG_ERR_NULL_PTR);
    // ragged_dot_k, padded_dot
    EXPECT(ragged_dot_k(P, P, GS, P, 64, 64, 64, 4, BF, F32, P, 8, nullptr), GG_ERR_WORKSPACE_TOO_SMALL);
    EXPECT(ragged_dot_k(P, P, GS, P, 64, 64, 64, 4, E4, F32, P, 4096, nullptr), GG_ERR_BAD_DTYPE);
    EXPECT(padded_dot(GG_OP_RAGGED_M, P, P, GS, P, 64, 64, 64, 4, 16, BF, BF, nullptr, nullptr, P, 1 << 30, nullptr),
           GG_ERR_UNSUPPORTED);
    EXPECT(padded_dot(GG_OP_PADDED_M, P, P, GS, P, 64, 64, 64, 4, 0, BF, BF, nullptr, nullptr, P, 1 << 30, nullptr),
           GG_ERR_BAD_SHAPE);
    EXPECT(padded_dot(GG_OP_PADDED_M, P, P, GS, P, 64, 64, 64, 4, (int64_t)1 << 40, BF, BF, nullptr, nullptr, P, 1 << 30,
                      nullptr), GG_ERR_BAD_SHAPE);
    const size_t need = gg_workspace_bytes(GG_OP_PADDED_M, 64, 64, 64, 4, 16, BF);
    EXPECT(need > 256, 1);
    EXPECT(padded_dot(GG_OP_PADDED_M, P, P, GS, P, 64, 64, 64, 4, 16, BF, BF, nullptr, nullptr, P, need - 1, nullptr),
           GG_ERR_WORKSPACE_TOO_SMALL);
    // permute / un-permute, schedule, status
    const size_t pneed = gg_workspace_bytes(GG_OP_PERMUTE, 128, 64, 0, 8, 0, BF);
    EXPECT(moe_permute(P, nullptr, nullptr, P, nullptr, (int32_t*)P, (int32_t*)P, (int32_t*)P, 64, 2, 64, 8, BF, P, pneed,
                       nullptr), GG_ERR_NULL_PTR);
    EXPECT(moe_permute(P, nullptr, GS, P, nullptr, (int32_t*)P, (int32_t*)P, (int32_t*)P, (int64_t)1 << 29, 4, 64, 8, BF, P,
                       pneed, nullptr), GG_ERR_BAD_SHAPE);
    EXPECT(moe_permute(P, nullptr, GS, P, nullptr, (int32_t*)P, (int32_t*)P, (int32_t*)P, 64, 2, 64, 8, BF, P, pneed - 1,
                       nullptr), GG_ERR_WORKSPACE_TOO_SMALL);
    EXPECT(moe_unpermute(P, GS, (const float*)P, P, -1, 2, 64, BF, BF, nullptr), GG_ERR_BAD_SHAPE);
    EXPECT(moe_unpermute(P, GS, (const float*)0x10002, P, 64, 2, 64, BF, BF, nullptr), GG_ERR_MISALIGNED);
    EXPECT(gg_schedule(GS, 9, 1, 3, 0, 1, (int32_t*)P, (int32_t*)P, (uint32_t*)P, nullptr), GG_ERR_BAD_SHAPE);
    EXPECT(gg_read_device_status(nullptr, nullptr, nullptr), GG_ERR_NULL_PTR);
    EXPECT(gg_workspace_bytes(GG_OP_PERMUTE, ((int64_t)1 << 30) + 1, 16, 0, 8, 0, BF), 0);
    EXPECT(gg_workspace_bytes((gg_op)17, 64, 64, 64, 4, 0, BF), 0);
    for (int c = -3; c < 12; ++c)
        if (!gg_status_string((gg_status)c)) ++failures;

    // random arguments: every call returns a status code and touches no memory it was handed
    for (int it = 0; it < 200000; ++it) {
        const int64_t m = pick_dim(), k = pick_dim(), n = pick_dim();
        const int32_t g = (int32_t)pick_code(-2, 1100);
        const gg_dtype in = (gg_dtype)pick_code(-1, 3), out = (gg_dtype)pick_code(-1, 3);
        void *a = pick_ptr(), *b = pick_ptr(), *o = pick_ptr(), *ws = pick_ptr();
        const size_t wsb = (size_t)pick_code(0, 1 << 20);
        const int32_t* gs = (const int32_t*)pick_ptr();
        int rc;
        switch (it % 9) {
            case 0: rc = ragged_dot_m(a, b, gs, o, m, k, n, g, in, out, (const uint8_t*)pick_ptr(), (const uint8_t*)pick_ptr(),
                                      ws, wsb, nullptr); break;
            case 1: rc = ragged_dot_k(a, b, gs, o, m, k, n, g, in, out, ws, wsb, nullptr); break;
            case 2: rc = ragged_dot_m_nk(a, b, gs, o, m, k, n, g, in, out, ws, wsb, nullptr); break;
            case 3: rc = padded_dot((gg_op)pick_code(-1, 5), a, b, gs, o, m, k, n, g, pick_dim(), in, out, nullptr, nullptr, ws,
                                    wsb, nullptr); break;
            case 4: rc = ragged_dot_m_epilogue(a, b, gs, o, m, k, n, g, in, out, nullptr, nullptr, (const float*)pick_ptr(),
                                               pick_dim(), 2.f, 1.f, ws, wsb, nullptr); break;
            case 5: rc = ragged_dot_m_gated(a, b, b, gs, o, m, k, n, g, in, out, (gg_activation)pick_code(-1, 3), nullptr, nullptr,
                                            0, ws, wsb, nullptr); break;
            case 6: rc = moe_permute(a, nullptr, gs, b, nullptr, (int32_t*)o, (int32_t*)o, (int32_t*)o, m, (int32_t)pick_code(-1, 9),
                                     k, g, in, ws, wsb, nullptr); break;
            case 7: rc = moe_unpermute(a, gs, (const float*)b, o, m, (int32_t)pick_code(-1, 9), n, in, out, nullptr); break;
            default: rc = ragged_dot_m_noalloc(a, b, gs, o, m, k, n, g, in, out, nullptr, nullptr, (uint32_t*)pick_ptr(), nullptr);
        }
        if (rc < 0 || rc > 7) { fprintf(stderr, "iteration %d: status %d out of range\n", it, rc); ++failures; }
        (void)gg_workspace_bytes((gg_op)pick_code(-1, 5), m, k, n, g, pick_dim(), in);
    }
    printf("abi driver: %d failures\n", failures);
    return failures ? 2 : 0;
}
