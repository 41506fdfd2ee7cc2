// padded.hip -- the pre- and post-processing of the padded-dot baseline, and the
// scan-only kernel behind gg_schedule.
//
// "Group-GEMM in XLA: Making Mixture-of-Experts Fast and Memory-Efficient" (AMD ROCm blog),
// Part 1 "The Naive Support, and Why It Hurts: Padded-Dot": pick a capacity C, pad every
// group's rows to C, run one batched GEMM over g x [C, k] x [k, n], and compact the output
// again; Part 4 describes the baseline as expanding the ragged input into g padded
// matrices with pre- and post-processing of inputs and outputs.
#include "common.hpp"
#include "launch.hpp"

namespace gg {

namespace pad {
constexpr int NT = 256;
constexpr int ROWS_PER_WG = 16;

__device__ inline void copy_row(const uint8_t* __restrict__ src, uint8_t* __restrict__ dst, long long bytes, bool zero) {
    const bool vec = ((((uintptr_t)src) | ((uintptr_t)dst) | (uintptr_t)bytes) & 15) == 0;
    if (vec) {
        const long long n16 = bytes >> 4;
        for (long long i = threadIdx.x; i < n16; i += NT)
            ((uint4*)dst)[i] = zero ? make_uint4(0, 0, 0, 0) : ((const uint4*)src)[i];
    } else {
        for (long long i = threadIdx.x; i < bytes; i += NT) dst[i] = zero ? (uint8_t)0 : src[i];
    }
}

// dst[h, c, :] = src[row_off[h] + c, :] for c < min(size_h, cap); zeros for the rest.
__global__ __launch_bounds__(NT) void scatter(const uint8_t* __restrict__ src, uint8_t* __restrict__ dst,
                                              const int32_t* __restrict__ gs, int m, int g, int cap,
                                              long long row_bytes, uint32_t* status) {
    __shared__ Tables tab;
    int tiles, covered;
    build_tables<NT>(gs, g, m, 1, 0, tab, &tiles, &covered);
    if (blockIdx.x == 0) {
        int over = 0;
        for (int h = threadIdx.x; h < g; h += NT) over |= tab.row_off[h + 1] - tab.row_off[h] > cap;
        over = __syncthreads_or(over);
        if (threadIdx.x == 0 && status) *status = tab.flags | (over ? GG_DEV_OVER_CAPACITY : 0u);
    }
    const long long total = (long long)g * cap;
    for (long long row = (long long)blockIdx.x * ROWS_PER_WG; row < total; row += (long long)gridDim.x * ROWS_PER_WG) {
        for (int i = 0; i < ROWS_PER_WG && row + i < total; ++i) {
            const long long pr = row + i;
            const int h = (int)(pr / cap), c = (int)(pr % cap);
            const int size = tab.row_off[h + 1] - tab.row_off[h];
            const bool live = c < size;
            copy_row(src + (live ? (size_t)(tab.row_off[h] + c) * row_bytes : 0), dst + (size_t)pr * row_bytes, row_bytes,
                     !live);
        }
    }
}

// dst[r, :] = src[h, r - row_off[h], :] for covered rows within capacity; zeros elsewhere.
__global__ __launch_bounds__(NT) void gather(const uint8_t* __restrict__ src, uint8_t* __restrict__ dst,
                                             const int32_t* __restrict__ gs, int m, int g, int cap, long long row_bytes) {
    __shared__ Tables tab;
    int tiles, covered;
    build_tables<NT>(gs, g, m, 1, 0, tab, &tiles, &covered);
    for (long long row = (long long)blockIdx.x * ROWS_PER_WG; row < m; row += (long long)gridDim.x * ROWS_PER_WG) {
        for (int i = 0; i < ROWS_PER_WG && row + i < m; ++i) {
            const int r = (int)(row + i);
            bool live = r < covered;
            int h = 0, c = 0;
            if (live) {
                int lo = 0, hi = g;   // largest h with row_off[h] <= r
                while (hi - lo > 1) {
                    const int mid = (lo + hi) >> 1;
                    if (tab.row_off[mid] <= r) lo = mid; else hi = mid;
                }
                h = lo;
                c = r - tab.row_off[h];
                live = c < cap;
            }
            copy_row(src + (live ? ((size_t)h * cap + c) * row_bytes : 0), dst + (size_t)r * row_bytes, row_bytes, !live);
        }
    }
}

__global__ __launch_bounds__(512) void schedule(const int32_t* __restrict__ gs, int m, int n, int g, int bm, int bn,
                                                int32_t* row_off, int32_t* tile_off, uint32_t* status) {
    __shared__ Tables tab;
    int tiles, covered;
    build_tables<512>(gs, g, m, bm, (n + bn - 1) / bn, tab, &tiles, &covered);
    for (int h = threadIdx.x; h <= g; h += 512) {
        row_off[h] = tab.row_off[h];
        tile_off[h] = tab.tile_off[h];
    }
    if (threadIdx.x == 0) *status = tab.flags;
}
}  // namespace pad

static int pad_grid(long long rows) {
    long long b = (rows + pad::ROWS_PER_WG - 1) / pad::ROWS_PER_WG;
    if (b < 1) b = 1;
    if (b > 4096) b = 4096;
    return (int)b;
}

hipError_t launch_pad_scatter(const void* src, void* dst, const int32_t* gs, int m, int g, int cap, long long row_bytes,
                              uint32_t* status, hipStream_t s) {
    hipLaunchKernelGGL(pad::scatter, dim3(pad_grid((long long)g * cap)), dim3(pad::NT), 0, s, (const uint8_t*)src,
                       (uint8_t*)dst, gs, m, g, cap, row_bytes, status);
    return hipGetLastError();
}

hipError_t launch_pad_gather(const void* src, void* dst, const int32_t* gs, int m, int g, int cap, long long row_bytes,
                             hipStream_t s) {
    hipLaunchKernelGGL(pad::gather, dim3(pad_grid(m)), dim3(pad::NT), 0, s, (const uint8_t*)src, (uint8_t*)dst, gs, m,
                       g, cap, row_bytes);
    return hipGetLastError();
}

hipError_t launch_schedule(const int32_t* gs, int m, int n, int g, int bm, int bn, int32_t* row_off, int32_t* tile_off,
                           uint32_t* status, hipStream_t s) {
    hipLaunchKernelGGL(pad::schedule, dim3(1), dim3(512), 0, s, gs, m, n, g, bm, bn, row_off, tile_off, status);
    return hipGetLastError();
}

}  // namespace gg
