// common.hpp -- device-side building blocks shared by the gfx950 ragged-dot kernels:
// vector types, the group_sizes -> offsets block scan, the persistent tile walk and the
// lane layouts of the MFMA and LDS-transpose instructions used by the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "groupgemm.h"

namespace gg {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

#define GG_LDS(T, p) ((__attribute__((address_space(3))) T*)(p))

constexpr int kWave = 64;

// ---------------------------------------------------------------------------------------
// Lane layouts (gfx950), as used below.
//
// v_mfma_f32_32x32x16_bf16: lane l holds A[row l%32][8 k-values] and B[8 k-values][col l%32];
//   lanes with the same l/32 must hold the same 8 k indices (here k = 8*(l/32) + 0..7 of a
//   16-wide k slice).  Result element e of lane l is C[8*(e/4) + 4*(l/32) + e%4][l%32].
// v_mfma_f32_16x16x4_f32: lane l holds A[l%16][l/16] and B[l/16][l%16];
//   result element e is C[4*(l/16) + e][l%16].
// v_mfma_scale_f32_32x32x64_f8f6f4 (e4m3 operands): lane l = r + 32h holds, for row (A) or
//   column (B) r, the 16 k-values 16h..16h+15 followed by 32+16h..32+16h+15 of a 64-wide k
//   slice.  Its E8M0 scale register holds the scale of row/column r for the 32-wide k block
//   h.  Result layout as for the 32x32 bf16 instruction.
// ds_read_b64_tr_b16: in every group of 16 lanes, lane j receives element j%4 of the 8 bytes
//   addressed by lane 4r + j/4 of the group, for r = 0..3.  So if lane 4r + c of a group
//   addresses row r, columns 4c..4c+3 of a 4 x 16 block of 16-bit values, lane j receives
//   column j (rows 0..3).
// ds_read_b64_tr_b8: in every group of 16 lanes, lane j receives byte j%8 of the 8 bytes
//   addressed by lane 2r + j/8, for r = 0..7: lane 2r + c addressing row r, bytes 8c..8c+7
//   of an 8 x 16 byte block gives lane j column j (rows 0..7).
// ---------------------------------------------------------------------------------------

__device__ inline i16x4 lds_read_tr16(const void* lds_ptr) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16(GG_LDS(i16x4, lds_ptr));
}
__device__ inline i32x2 lds_read_tr8(const void* lds_ptr) {
    return __builtin_amdgcn_ds_read_tr8_b64_v2i32(GG_LDS(i32x2, lds_ptr));
}

// round-to-nearest-even fp32 -> bf16 bits (finite inputs; NaN stays NaN)
__device__ inline uint16_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7f800000u) == 0x7f800000u) return (uint16_t)((u >> 16) | ((u & 0xffffu) ? 0x40u : 0u));
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

__device__ inline int cdiv(int a, int b) { return (a + b - 1) / b; }

// ---------------------------------------------------------------------------------------
// group_sizes -> offsets.  Every workgroup of a launch recomputes the (tiny) tables into
// LDS, the way the blog's descriptor-update kernels do a block scan over the group sizes
// ("Group-GEMM in XLA", Part 2 "The Compile-Time vs. Runtime Problem").
//
// Clamping: s_h = max(size_h, 0); p_h = sum_{j<h} s_j; group h owns rows
// [min(p_h, m), min(p_h + s_h, m)).  row_off[h] = min(p_h, m); row_off[g] = rows covered.

struct Tables {
    int row_off[GG_MAX_GROUPS + 1];
    int tile_off[GG_MAX_GROUPS + 1];
    long long wave_tmp[16];
    int flags;
};

// inclusive scan of v over the 64 lanes of a wave
__device__ inline long long wave_inclusive_scan(long long v) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        long long u = __shfl_up(v, d, 64);
        if (lane >= d) v += u;
    }
    return v;
}

// Exclusive block scan of per-thread totals; returns this thread's exclusive prefix and
// writes the block total to *total.  All NT threads must call it.
template <int NT>
__device__ long long block_exclusive_scan(long long v, Tables& T, long long* total) {
    static_assert(NT % 64 == 0 && NT / 64 <= 16, "block size");
    const int wave = threadIdx.x / 64, lane = threadIdx.x & 63;
    long long inc = wave_inclusive_scan(v);
    __syncthreads();
    if (lane == 63) T.wave_tmp[wave] = inc;
    __syncthreads();
    long long before = 0, all = 0;
#pragma unroll
    for (int w = 0; w < NT / 64; ++w) {
        long long x = T.wave_tmp[w];
        if (w < wave) before += x;
        all += x;
    }
    *total = all;
    return before + inc - v;
}

// Builds row_off / tile_off for `g` groups into T, where a group of s rows contributes
// ceil(s / block_m) * tiles_per_mtile tiles (tiles_per_mtile may be 0 for "rows only").
// Returns (via refs) the number of GEMM tiles and the rows covered; T.flags gets GG_DEV_*.
// (Forced inline: the larger ring kernels otherwise call it out of line.)
template <int NT>
__device__ __attribute__((always_inline)) inline void build_tables(const int32_t* __restrict__ group_sizes, int g, long long m,
                             int block_m, int tiles_per_mtile, Tables& T, int* n_tiles,
                             int* covered) {
    constexpr int PER = (GG_MAX_GROUPS + NT - 1) / NT;
    const int t0 = threadIdx.x * PER;
    long long s[PER];
    int neg = 0;
    long long local = 0;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        int h = t0 + i;
        int v = h < g ? group_sizes[h] : 0;
        neg |= v < 0;
        s[i] = v < 0 ? 0 : v;
        local += s[i];
    }
    long long total;
    long long p = block_exclusive_scan<NT>(local, T, &total);
    int mt[PER];
    long long tiles_local = 0;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        int h = t0 + i;
        long long st = p < m ? p : m;
        long long en = p + s[i] < m ? p + s[i] : m;
        if (h < g) T.row_off[h] = (int)st;
        mt[i] = h < g ? (int)((en - st + block_m - 1) / block_m) * tiles_per_mtile : 0;
        tiles_local += mt[i];
        p += s[i];
    }
    long long tiles_total;
    long long tp = block_exclusive_scan<NT>(tiles_local, T, &tiles_total);
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        int h = t0 + i;
        if (h < g) T.tile_off[h] = (int)tp;
        tp += mt[i];
    }
    const int any_neg = __syncthreads_or(neg);
    if (threadIdx.x == 0) {
        long long cov = total < m ? total : m;
        T.row_off[g] = (int)cov;
        T.tile_off[g] = (int)tiles_total;
        T.flags = (any_neg ? GG_DEV_NEGATIVE_SIZE : 0u) | (total > m ? GG_DEV_SUM_EXCEEDS_M : 0u);
    }
    __syncthreads();
    *n_tiles = T.tile_off[g];
    *covered = T.row_off[g];
}

// Group of GEMM tile t: the largest h with tile_off[h] <= t ("the largest g such that
// prefix_exclusive[g] <= row_start", "Group-GEMM in XLA", Part 3 "Non-Contracting"); empty
// groups repeat the previous offset and are skipped by taking the largest such h.
__device__ inline int find_group(const int* tile_off, int g, int t) {
    int lo = 0, hi = g;   // tile_off[lo] <= t < tile_off[hi]
    while (hi - lo > 1) {
        int mid = (lo + hi) >> 1;
        if (tile_off[mid] <= t) lo = mid; else hi = mid;
    }
    return lo;
}

// Workgroups are handed to the 8 XCDs round-robin by id.  Renumber them so that
// consecutive virtual ids run on the same XCD (and share its L2); grid must be a
// multiple of 8.
__device__ inline int xcd_virtual_id(int wg, int grid) {
    if ((grid & 7) != 0) return wg;
    return (wg & 7) * (grid >> 3) + (wg >> 3);
}

}  // namespace gg
