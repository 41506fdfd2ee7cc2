// ragged_k.hip -- contracting ragged dot (the weight-gradient case) on gfx950:
//   out[h] = lhs[rows of h, :]^T . dout[rows of h, :]    -> out [g, k, n]
//
// "Group-GEMM in XLA: Making Mixture-of-Experts Fast and Memory-Efficient" (AMD ROCm blog),
// Part 3 "Contracting": the group index is an output dimension, so groups are a parallel
// launch axis, and each group reduces only over its own slice [start, end) of the
// contracted axis, read from the prefix table; Part 4 Table 7, class wgrad_wi.
//
// Both operands have the contracted (row) axis as their slow axis, so both tiles are
// staged in LDS row-major and read with ds_read_b64_tr_b16 into k-consecutive MFMA
// fragments.  Tiles are (group, k-tile, n-tile); a persistent workgroup walks them with
// the groups in decreasing size order (longest first) so the work per round is even.
// An empty group still owns its tiles, which write exact zeros.
#include "common.hpp"
#include "launch.hpp"

namespace gg {

namespace kbf16 {
constexpr int BM = 256, BN = 256, BR = 64, NT = 512;   // BM along k (output rows), BN along n
constexpr int LPT_MAX_G = 64;                           // longest-first order up to this many groups

struct Smem {
    uint16_t a[2][BR * BM];
    uint16_t b[2][BR * BN];
    Tables tab;
    int order[LPT_MAX_G];
};

// same layout as the rhs tile of the non-contracting kernel: row-major [BR][256] with
// 16-byte chunks XOR-swizzled in 64-byte units
__device__ inline int swz(int kr) { return ((kr & 3) | (((kr >> 3) & 1) << 2)) << 2; }
__device__ inline int off(int kr, int nn) { return kr * 256 + ((((nn >> 3) ^ swz(kr))) << 3) + (nn & 7); }

struct Regs { uint4 a[4]; uint4 b[4]; };

template <bool VEC>
__device__ inline void load_rows(uint4 (&v)[4], const uint16_t* __restrict__ src, int ld, int row_base, int rows_left,
                                 int col0, int cols) {
    const int t = threadIdx.x;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int r = (t >> 5) + 16 * i;
        const int c = col0 + ((t & 31) << 3);
        uint4 x = make_uint4(0, 0, 0, 0);
        if (r < rows_left) {
            const uint16_t* p = src + (size_t)(row_base + r) * (size_t)ld + c;
            if (VEC) {
                if (c < cols) x = *(const uint4*)p;
            } else {
                uint16_t e[8];
#pragma unroll
                for (int q = 0; q < 8; ++q) e[q] = (c + q < cols) ? p[q] : (uint16_t)0;
                x = make_uint4(e[0] | (e[1] << 16), e[2] | (e[3] << 16), e[4] | (e[5] << 16), e[6] | (e[7] << 16));
            }
        }
        v[i] = x;
    }
}

__device__ inline void store_rows(const uint4 (&v)[4], uint16_t* dst) {
    const int t = threadIdx.x;
#pragma unroll
    for (int i = 0; i < 4; ++i) *(uint4*)(dst + off((t >> 5) + 16 * i, (t & 31) << 3)) = v[i];
}

// 8 k-consecutive (row-consecutive) bf16 values of column (base + l%32) via two
// transpose reads; rows 16 s + 8 (l/32) + 0..7.
__device__ inline bf16x8 frag(const uint16_t* tile, int s, int colbase) {
    const int l = threadIdx.x & 63;
    const int q = l >> 4, rr = (l >> 2) & 3, c = l & 3;
    const int nn = colbase + 16 * (q & 1) + 4 * c;
    const int kr0 = 16 * s + 8 * (q >> 1) + rr;
    const i16x4 lo = lds_read_tr16(tile + off(kr0, nn));
    const i16x4 hi = lds_read_tr16(tile + off(kr0 + 4, nn));
    typedef short i16x8 __attribute__((ext_vector_type(8)));
    const i16x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    return __builtin_bit_cast(bf16x8, v);
}

template <bool VEC, typename OutT>
__global__ __launch_bounds__(NT, 1) void kernel(KParams p) {
    __shared__ Smem sm;
    const uint16_t* __restrict__ lhs = (const uint16_t*)p.lhs;
    const uint16_t* __restrict__ dout = (const uint16_t*)p.dout;
    OutT* __restrict__ out = (OutT*)p.out;
    const int nti = cdiv(p.k, BM), ntj = cdiv(p.n, BN);
    const int per = nti * ntj;
    const int total = p.g * per;
    const bool lpt = p.uniform_rows == 0 && p.g <= LPT_MAX_G;
    if (p.uniform_rows == 0) {
        int gemm_tiles, covered;
        build_tables<NT>(p.group_sizes, p.g, p.m, 1, 0, sm.tab, &gemm_tiles, &covered);
        if (blockIdx.x == 0 && threadIdx.x == 0 && p.status) *p.status = sm.tab.flags;
        if (lpt) {   // rank of every group by (size desc, index asc)
            const int h = threadIdx.x;
            if (h < p.g) {
                const int sh = sm.tab.row_off[h + 1] - sm.tab.row_off[h];
                int rank = 0;
                for (int j = 0; j < p.g; ++j) {
                    const int sj = sm.tab.row_off[j + 1] - sm.tab.row_off[j];
                    rank += (sj > sh) || (sj == sh && j < h);
                }
                sm.order[rank] = h;
            }
            __syncthreads();
        }
    }
    const int wave = threadIdx.x >> 6, wm = wave >> 2, wn = wave & 3;
    const int l = threadIdx.x & 63;

    for (int t = xcd_virtual_id(blockIdx.x, gridDim.x); t < total; t += gridDim.x) {
        const int pg = t / per, local = t - pg * per;
        const int grp = lpt ? sm.order[pg] : pg;
        int row_base, size;
        if (p.uniform_rows > 0) { row_base = grp * p.uniform_rows; size = p.uniform_rows; }
        else { row_base = sm.tab.row_off[grp]; size = sm.tab.row_off[grp + 1] - row_base; }
        const int it = local % nti, jt = local / nti;
        const int i0 = it * BM, j0 = jt * BN;

        f32x16 acc[4][2];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

        const int nr = cdiv(size, BR);
        Regs R;
        if (nr > 0) {
            load_rows<VEC>(R.a, lhs, p.k, row_base, size, i0, p.k);
            load_rows<VEC>(R.b, dout, p.n, row_base, size, j0, p.n);
            store_rows(R.a, sm.a[0]);
            store_rows(R.b, sm.b[0]);
            __syncthreads();
        }
        for (int rt = 0; rt < nr; ++rt) {
            const int cur = rt & 1;
            if (rt + 1 < nr) {
                const int rb = row_base + (rt + 1) * BR, left = size - (rt + 1) * BR;
                load_rows<VEC>(R.a, lhs, p.k, rb, left, i0, p.k);
                load_rows<VEC>(R.b, dout, p.n, rb, left, j0, p.n);
            }
#pragma unroll
            for (int s = 0; s < BR / 16; ++s) {
                bf16x8 af[4], bfr[2];
#pragma unroll
                for (int i = 0; i < 4; ++i) af[i] = frag(sm.a[cur], s, 128 * wm + 32 * i);
#pragma unroll
                for (int j = 0; j < 2; ++j) bfr[j] = frag(sm.b[cur], s, 64 * wn + 32 * j);
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                    for (int j = 0; j < 2; ++j)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
            }
            if (rt + 1 < nr) {
                store_rows(R.a, sm.a[cur ^ 1]);
                store_rows(R.b, sm.b[cur ^ 1]);
            }
            __syncthreads();
        }
        OutT* og = out + (size_t)grp * (size_t)p.k * (size_t)p.n;
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const int col = j0 + 64 * wn + 32 * j + (l & 31);
                if (col >= p.n) continue;
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const int r = i0 + 128 * wm + 32 * i + 8 * (e >> 2) + 4 * (l >> 5) + (e & 3);
                    if (r < p.k) {
                        OutT* dst = og + (size_t)r * (size_t)p.n + col;
                        if constexpr (sizeof(OutT) == 2) *dst = f32_to_bf16(acc[i][j][e]);
                        else *dst = acc[i][j][e];
                    }
                }
            }
    }
}
}  // namespace kbf16

TileShape tiles_k_bf16() { return {kbf16::BM, kbf16::BN}; }

hipError_t launch_ragged_k_bf16(const KParams& p, int grid, bool vec, hipStream_t s) {
    if (p.out_f32) {
        if (vec) hipLaunchKernelGGL((kbf16::kernel<true, float>), dim3(grid), dim3(kbf16::NT), 0, s, p);
        else hipLaunchKernelGGL((kbf16::kernel<false, float>), dim3(grid), dim3(kbf16::NT), 0, s, p);
    } else {
        if (vec) hipLaunchKernelGGL((kbf16::kernel<true, uint16_t>), dim3(grid), dim3(kbf16::NT), 0, s, p);
        else hipLaunchKernelGGL((kbf16::kernel<false, uint16_t>), dim3(grid), dim3(kbf16::NT), 0, s, p);
    }
    return hipGetLastError();
}

// ---------------------------------------------------------------------------------------
// fp32 inputs: 64 x 64 output tile, 16 contracted rows per step, v_mfma_f32_16x16x4_f32.
namespace kf32 {
constexpr int BM = 64, BN = 64, BR = 16, NT = 256;

struct Smem {
    float a[BR][BM + 1];   // lhs rows x k-cols
    float b[BR][BN + 1];   // dout rows x n-cols
    Tables tab;
};

__global__ __launch_bounds__(NT) void kernel(KParams p) {
    __shared__ Smem sm;
    const float* __restrict__ lhs = (const float*)p.lhs;
    const float* __restrict__ dout = (const float*)p.dout;
    float* __restrict__ out = (float*)p.out;
    const int nti = cdiv(p.k, BM), ntj = cdiv(p.n, BN);
    const int per = nti * ntj, total = p.g * per;
    if (p.uniform_rows == 0) {
        int gemm_tiles, covered;
        build_tables<NT>(p.group_sizes, p.g, p.m, 1, 0, sm.tab, &gemm_tiles, &covered);
        if (blockIdx.x == 0 && threadIdx.x == 0 && p.status) *p.status = sm.tab.flags;
    }
    const int l = threadIdx.x & 63, wave = threadIdx.x >> 6, wm = wave >> 1, wn = wave & 1;
    for (int t = xcd_virtual_id(blockIdx.x, gridDim.x); t < total; t += gridDim.x) {
        const int grp = t / per, local = t - grp * per;
        int row_base, size;
        if (p.uniform_rows > 0) { row_base = grp * p.uniform_rows; size = p.uniform_rows; }
        else { row_base = sm.tab.row_off[grp]; size = sm.tab.row_off[grp + 1] - row_base; }
        const int i0 = (local % nti) * BM, j0 = (local / nti) * BN;
        f32x4 acc[2][2];
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
        for (int r0 = 0; r0 < size; r0 += BR) {
            for (int idx = threadIdx.x; idx < BR * BM; idx += NT) {
                const int r = idx / BM, c = idx % BM;
                sm.a[r][c] = (r0 + r < size && i0 + c < p.k) ? lhs[(size_t)(row_base + r0 + r) * p.k + i0 + c] : 0.f;
            }
            for (int idx = threadIdx.x; idx < BR * BN; idx += NT) {
                const int r = idx / BN, c = idx % BN;
                sm.b[r][c] = (r0 + r < size && j0 + c < p.n) ? dout[(size_t)(row_base + r0 + r) * p.n + j0 + c] : 0.f;
            }
            __syncthreads();
#pragma unroll
            for (int s = 0; s < BR / 4; ++s)
#pragma unroll
                for (int i = 0; i < 2; ++i)
#pragma unroll
                    for (int j = 0; j < 2; ++j) {
                        const float av = sm.a[4 * s + (l >> 4)][32 * wm + 16 * i + (l & 15)];
                        const float bv = sm.b[4 * s + (l >> 4)][32 * wn + 16 * j + (l & 15)];
                        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(av, bv, acc[i][j], 0, 0, 0);
                    }
            __syncthreads();
        }
        float* og = out + (size_t)grp * (size_t)p.k * (size_t)p.n;
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const int col = j0 + 32 * wn + 16 * j + (l & 15);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int r = i0 + 32 * wm + 16 * i + 4 * (l >> 4) + e;
                    if (r < p.k && col < p.n) og[(size_t)r * p.n + col] = acc[i][j][e];
                }
            }
    }
}
}  // namespace kf32

TileShape tiles_k_f32() { return {kf32::BM, kf32::BN}; }

hipError_t launch_ragged_k_f32(const KParams& p, int grid, hipStream_t s) {
    hipLaunchKernelGGL(kf32::kernel, dim3(grid), dim3(kf32::NT), 0, s, p);
    return hipGetLastError();
}

}  // namespace gg
