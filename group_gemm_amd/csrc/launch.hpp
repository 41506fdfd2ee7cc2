// launch.hpp -- parameter blocks and host-side launchers of the gfx950 kernels (internal).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "groupgemm.h"

namespace gg {

// Non-contracting ragged dot: out[m,n] = per-group lhs[m,k] . rhs[g,k,n].
struct MParams {
    const void* lhs;            // [m,k]
    const void* rhs;            // [g,k,n]
    const uint8_t* lhs_scale;   // [m,k/32]   (e4m3 only)
    const uint8_t* rhs_scale;   // [g,k/32,n] (e4m3 only)
    const int32_t* group_sizes; // [g] device, or NULL when uniform_rows > 0
    void* out;                  // [m,n]
    uint32_t* status;           // device status word, written by workgroup 0
    int m, k, n, g;
    int uniform_rows;           // > 0: every group has exactly this many rows (batched form)
    int out_f32;                // 1: fp32 output, 0: bf16 output
    int rhs_nk;                 // 1: rhs is [g,n,k] (k contiguous; the dgrad classes), 0: [g,k,n]
    // epilogue (epi != 0): out = alpha * acc + bias[h, :] + beta * out, in place
    int epi;
    const float* bias;          // [g, bias_stride] fp32 rows, or NULL
    int64_t bias_stride;
    float alpha, beta;
    // 8 device ints the launcher zeroes: one tile queue per XCD (the bf16 ring kernel's walk,
    // ring.hpp), or NULL for the static walk; the other kernels walk statically
    int* tile_queue;
};

// Contracting ragged dot: out[g,k,n] = per-group lhs[rows,k]^T . dout[rows,n].
struct KParams {
    const void* lhs;            // [m,k]
    const void* dout;           // [m,n]
    const int32_t* group_sizes;
    void* out;                  // [g,k,n]
    uint32_t* status;
    int m, k, n, g;
    int uniform_rows;
    int out_f32;
    // epilogue (epi != 0): out[h] = alpha * acc + beta * out[h], in place
    int epi;
    float alpha, beta;
};

// Fused gate/up projection: out[m,n] = act(lhs . w0[h] + b0[h]) * (lhs . w1[h] + b1[h]).
struct GParams {
    const void* lhs;            // [m,k]
    const void* w0;             // [g,k,n] gate weights
    const void* w1;             // [g,k,n] up weights
    const int32_t* group_sizes;
    void* out;                  // [m,n]
    uint32_t* status;
    const float* bias0;         // [g, bias_stride] or NULL
    const float* bias1;
    int64_t bias_stride;
    int m, k, n, g;
    int out_f32;
    int act;                    // gg_activation
};
bool ragged_m_gated_ok(const GParams& p);
hipError_t launch_ragged_m_gated(const GParams& p, int grid, hipStream_t s);

// Zeroes the 8 tile-queue counters of a ring kernel (a one-block kernel, so the call can be
// captured in a graph).
hipError_t launch_clear_queues(int* queues, hipStream_t s);

// Kernel families.  Each launcher returns the hipError_t of its launch.
hipError_t launch_ragged_m_bf16(const MParams& p, int grid, bool vec, hipStream_t s);
// vectorised bf16 kernel (16-byte aligned operands, k % 8 == 0, n % 8 == 0)
bool ragged_m_bf16_fast_ok(const MParams& p);
int ragged_m_bf16_fast_bm(const MParams& p);   // tile rows the vectorised kernel picks (n tiles are 256 wide)
hipError_t launch_ragged_m_bf16_fast(const MParams& p, int grid, hipStream_t s);
hipError_t launch_ragged_m_f32(const MParams& p, int grid, hipStream_t s);
hipError_t launch_ragged_m_e4m3(const MParams& p, int grid, hipStream_t s);
// MXFP8 ring kernel (16-byte aligned operands and output, 4-byte aligned scales,
// k % 128 == 0, n % 16 == 0); 256 x 256 tiles
bool ragged_m_mx_fast_ok(const MParams& p);
hipError_t launch_ragged_m_mx_fast(const MParams& p, int grid, hipStream_t s);
hipError_t launch_ragged_k_bf16(const KParams& p, int grid, bool vec, hipStream_t s);
// contracting ring kernel (16-byte aligned operands and output, k % 8 == 0, n % 8 == 0)
bool ragged_k_bf16_fast_ok(const KParams& p);
hipError_t launch_ragged_k_bf16_fast(const KParams& p, int grid, hipStream_t s);
hipError_t launch_ragged_k_f32(const KParams& p, int grid, hipStream_t s);

// MoE permute / un-permute.
constexpr int kMaxChunks = 64;   // upper bound on the permute's histogram / rank workgroups
struct PermuteGeometry { int chunk, nblk; };   // copies per chunk, number of chunks
PermuteGeometry permute_geometry(int64_t copies);
struct PermuteArgs {
    const void* x;                 // [tokens, row_bytes]
    const void* x_scale;           // [tokens, scale_row_bytes] or NULL
    const int32_t* experts;        // [tokens * top_k]
    void* sorted_x;                // [tokens * top_k, row_bytes]
    void* sorted_scale;            // [tokens * top_k, scale_row_bytes] or NULL
    int32_t* group_sizes;          // [g]
    int32_t* sorted_to_copy;       // [tokens * top_k]
    int32_t* copy_to_sorted;       // [tokens * top_k]
    int* counts;                   // workspace [nblk, g]
    int* bad;                      // workspace [nblk]
    int* total_routed;             // workspace [1]
    uint32_t* status;
    int tokens, top_k, g;
    int64_t row_bytes, scale_row_bytes;
};
hipError_t launch_permute(const PermuteArgs& a, hipStream_t s);
hipError_t launch_combine(const void* y, bool y_bf16, int rows, const int32_t* copy_to_sorted, const float* w,
                          int tokens, int top_k, int n, void* out, bool out_bf16, hipStream_t s);

// Static tile geometry of each family (host-side grid sizing).
struct TileShape { int bm, bn; };
TileShape tiles_m_bf16();
TileShape tiles_m_f32();
TileShape tiles_m_e4m3();
TileShape tiles_k_bf16();   // bm along k (output rows), bn along n
TileShape tiles_k_f32();

// padded_dot helpers: scatter rows of `src` [m, row_elems] into `dst` [g, cap, row_elems]
// (zero-filling the padding), and gather rows back.  elem_bytes in {1, 2, 4}.
hipError_t launch_pad_scatter(const void* src, void* dst, const int32_t* group_sizes, int m, int g,
                              int cap, long long row_bytes, uint32_t* status, hipStream_t s);
hipError_t launch_pad_gather(const void* src, void* dst, const int32_t* group_sizes, int m, int g,
                             int cap, long long row_bytes, hipStream_t s);

// Scan-only kernel behind gg_schedule.
hipError_t launch_schedule(const int32_t* group_sizes, int m, int n, int g, int bm, int bn,
                           int32_t* row_off, int32_t* tile_off, uint32_t* status, hipStream_t s);

}  // namespace gg
