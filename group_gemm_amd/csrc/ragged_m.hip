// ragged_m.hip -- non-contracting ragged dot (the MoE forward case) as one persistent
// Group-GEMM launch on gfx950.
//
// "Group-GEMM in XLA: Making Mixture-of-Experts Fast and Memory-Efficient" (AMD ROCm blog):
//   Part 1 "The Ragged-Dot Operation" -- lhs [m,k] rows stacked in group order, rhs [g,k,n],
//   group_sizes [g] known only at run time; Part 3 "Non-Contracting (the MoE Case)" -- per
//   tile: find the group, select rhs[g], accumulate a tiled dot over k, masked store.
//
// Differences from the blog's kernels, for gfx950:
//   * tiles are group-aligned: group h gets ceil(m_h / BM) m-tiles of its own, so no tile
//     straddles a group boundary and no row is dropped (the blog's Table 2 example masks a
//     row of a straddling tile that no other tile computes);
//   * one persistent launch: every workgroup rebuilds the group tables in LDS, then walks
//     tiles wg, wg + grid, ... up to the runtime tile count (a static upper bound sizes
//     the grid, as the aiter PR's cdiv(tokens, BM) + E bound does);
//   * within a group the raster is chosen per group at run time: m-tiles fastest when the
//     group's lhs rows are smaller than its weight matrix (m_h <= n), else n-tiles fastest
//     (the blog's M/N swap, decided on the true size instead of the M/G average);
//   * rows past sum(group_sizes) are written as zeros by extra tiles (aiter PR: a
//     zero-filled output keeps stale NaN out of downstream masks).
#include "common.hpp"
#include "launch.hpp"

namespace gg {

// =======================================================================================
// bf16 inputs: 256 x 256 output tile, k step 64, 8 waves (2 x 4), each wave 128 x 64 built
// from 4 x 2 v_mfma_f32_32x32x16_bf16 blocks.
// LDS: A [256][64] and B [64][256] bf16, double buffered (128 KiB) + group tables.
// A rows are k-contiguous and feed the MFMA directly (ds_read_b128).  B rows are
// n-contiguous (rhs as given, no per-call relayout); ds_read_b64_tr_b16 turns them into
// k-consecutive fragments.
// =======================================================================================
namespace mbf16 {
constexpr int BM = 256, BN = 256, BK = 64, NT = 512;

struct Smem {
    uint16_t a[2][BM * BK];
    uint16_t b[2][BK * BN];
    Tables tab;
};

// A element (r, kk): 16-byte chunk kk/8 of row r, chunks XOR-swizzled by (r >> 1) & 7 so
// that 16 consecutive rows read at one chunk hit distinct banks.
__device__ inline int a_off(int r, int chunk) { return r * BK + ((chunk ^ ((r >> 1) & 7)) << 3); }
// B element (kr, nn): 16-byte chunk nn/8 of row kr, XOR-swizzled in 64-byte units by a
// 3-bit function of the row so the 8 rows one transpose read touches land in distinct units.
__device__ inline int b_swz(int kr) { return ((kr & 3) | (((kr >> 3) & 1) << 2)) << 2; }
__device__ inline int b_off(int kr, int nn) { return kr * BN + ((((nn >> 3) ^ b_swz(kr))) << 3) + (nn & 7); }

struct Regs { uint4 a[4]; uint4 b[4]; };

template <bool VEC>
__device__ inline void load_tiles(Regs& R, const uint16_t* __restrict__ lhs, const uint16_t* __restrict__ rhs_g,
                                  int row0, int rows_valid, int col0, int kk, int k, int n) {
    const int t = threadIdx.x;
    // A: thread t -> chunk t&7 of rows (t>>3) + 64 i
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int r = (t >> 3) + 64 * i;
        const int kc = kk + ((t & 7) << 3);
        uint4 v = make_uint4(0, 0, 0, 0);
        if (r < rows_valid) {
            const uint16_t* src = lhs + (size_t)(row0 + r) * (size_t)k + kc;
            if (VEC) {
                if (kc < k) v = *(const uint4*)src;
            } else {
                uint16_t e[8];
#pragma unroll
                for (int q = 0; q < 8; ++q) e[q] = (kc + q < k) ? src[q] : (uint16_t)0;
                v = make_uint4(e[0] | (e[1] << 16), e[2] | (e[3] << 16), e[4] | (e[5] << 16), e[6] | (e[7] << 16));
            }
        }
        R.a[i] = v;
    }
    // B: thread t -> chunk t&31 of rows (t>>5) + 16 i
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int kr = kk + (t >> 5) + 16 * i;
        const int nc = col0 + ((t & 31) << 3);
        uint4 v = make_uint4(0, 0, 0, 0);
        if (kr < k) {
            const uint16_t* src = rhs_g + (size_t)kr * (size_t)n + nc;
            if (VEC) {
                if (nc < n) v = *(const uint4*)src;
            } else {
                uint16_t e[8];
#pragma unroll
                for (int q = 0; q < 8; ++q) e[q] = (nc + q < n) ? src[q] : (uint16_t)0;
                v = make_uint4(e[0] | (e[1] << 16), e[2] | (e[3] << 16), e[4] | (e[5] << 16), e[6] | (e[7] << 16));
            }
        }
        R.b[i] = v;
    }
}

__device__ inline void store_tiles(const Regs& R, uint16_t* a, uint16_t* b) {
    const int t = threadIdx.x;
#pragma unroll
    for (int i = 0; i < 4; ++i) *(uint4*)(a + a_off((t >> 3) + 64 * i, t & 7)) = R.a[i];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int kr = (t >> 5) + 16 * i;
        *(uint4*)(b + b_off(kr, (t & 31) << 3)) = R.b[i];
    }
}

__device__ inline void compute(const uint16_t* a, const uint16_t* b, f32x16 (&acc)[4][2], int wm, int wn) {
    const int l = threadIdx.x & 63;
    const int h = l >> 5;
    // transpose-read supplier roles of this lane
    const int q = l >> 4, rr = (l >> 2) & 3, c = l & 3;
#pragma unroll
    for (int s = 0; s < BK / 16; ++s) {
        bf16x8 af[4], bfr[2];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = 128 * wm + 32 * i + (l & 31);
            af[i] = *(const bf16x8*)(a + a_off(r, 2 * s + h));
        }
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int nn = 64 * wn + 32 * j + 16 * (q & 1) + 4 * c;
            const int kr0 = 16 * s + 8 * (q >> 1) + rr;
            i16x4 lo = lds_read_tr16(b + b_off(kr0, nn));
            i16x4 hi = lds_read_tr16(b + b_off(kr0 + 4, nn));
            typedef short i16x8 __attribute__((ext_vector_type(8)));
            i16x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
            bfr[j] = __builtin_bit_cast(bf16x8, v);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
}

template <typename OutT>
__device__ inline void store_out(OutT* __restrict__ out, const f32x16 (&acc)[4][2], int row0, int rows_valid,
                                 int col0, int n, int wm, int wn) {
    const int l = threadIdx.x & 63;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int col = col0 + 64 * wn + 32 * j + (l & 31);
            if (col >= n) continue;
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int r = 128 * wm + 32 * i + 8 * (e >> 2) + 4 * (l >> 5) + (e & 3);
                if (r < rows_valid) {
                    OutT* dst = out + (size_t)(row0 + r) * (size_t)n + col;
                    if constexpr (sizeof(OutT) == 2) *dst = f32_to_bf16(acc[i][j][e]);
                    else *dst = acc[i][j][e];
                }
            }
        }
}

template <typename OutT>
__device__ inline void zero_tile(OutT* __restrict__ out, int row0, int row_end, int col0, int n) {
    for (int idx = threadIdx.x; idx < BM * BN; idx += NT) {
        const int r = row0 + idx / BN, c = col0 + idx % BN;
        if (r < row_end && c < n) out[(size_t)r * (size_t)n + c] = (OutT)0;
    }
}

template <bool VEC, typename OutT>
__global__ __launch_bounds__(NT, 1) void kernel(MParams p) {
    __shared__ Smem sm;
    const uint16_t* __restrict__ lhs = (const uint16_t*)p.lhs;
    const uint16_t* __restrict__ rhs = (const uint16_t*)p.rhs;
    OutT* __restrict__ out = (OutT*)p.out;
    const int ntn = cdiv(p.n, BN);
    int gemm_tiles, covered;
    if (p.uniform_rows > 0) {
        gemm_tiles = p.g * cdiv(p.uniform_rows, BM) * ntn;
        covered = p.m;
    } else {
        build_tables<NT>(p.group_sizes, p.g, p.m, BM, ntn, sm.tab, &gemm_tiles, &covered);
        if (blockIdx.x == 0 && threadIdx.x == 0 && p.status) *p.status = sm.tab.flags;
    }
    const int zero_mt = cdiv(p.m - covered, BM);
    const int total = gemm_tiles + zero_mt * ntn;
    const int wave = threadIdx.x >> 6, wm = wave >> 2, wn = wave & 3;
    const int nk = cdiv(p.k, BK);

    for (int t = xcd_virtual_id(blockIdx.x, gridDim.x); t < total; t += gridDim.x) {
        if (t >= gemm_tiles) {   // rows past the covered ones: zeros
            const int z = t - gemm_tiles;
            zero_tile(out, covered + (z % zero_mt) * BM, p.m, (z / zero_mt) * BN, p.n);
            continue;
        }
        int grp, row0, size;
        int local;
        if (p.uniform_rows > 0) {
            const int per = cdiv(p.uniform_rows, BM) * ntn;
            grp = t / per;
            local = t - grp * per;
            row0 = grp * p.uniform_rows;
            size = p.uniform_rows;
        } else {
            grp = find_group(sm.tab.tile_off, p.g, t);
            local = t - sm.tab.tile_off[grp];
            row0 = sm.tab.row_off[grp];
            size = sm.tab.row_off[grp + 1] - row0;
        }
        const int mtg = cdiv(size, BM);
        int mt, nt;
        if (size <= p.n) { mt = local % mtg; nt = local / mtg; }   // weights stream once
        else { nt = local % ntn; mt = local / ntn; }               // rows stream once
        row0 += mt * BM;
        const int rows_valid = min(BM, size - mt * BM);
        const int col0 = nt * BN;
        const uint16_t* rhs_g = rhs + (size_t)grp * (size_t)p.k * (size_t)p.n;

        f32x16 acc[4][2];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

        Regs R;
        if (nk > 0) {
            load_tiles<VEC>(R, lhs, rhs_g, row0, rows_valid, col0, 0, p.k, p.n);
            store_tiles(R, sm.a[0], sm.b[0]);
            __syncthreads();
        }
        for (int kt = 0; kt < nk; ++kt) {
            const int cur = kt & 1;
            if (kt + 1 < nk) load_tiles<VEC>(R, lhs, rhs_g, row0, rows_valid, col0, (kt + 1) * BK, p.k, p.n);
            compute(sm.a[cur], sm.b[cur], acc, wm, wn);
            if (kt + 1 < nk) store_tiles(R, sm.a[cur ^ 1], sm.b[cur ^ 1]);
            __syncthreads();
        }
        store_out(out, acc, row0, rows_valid, col0, p.n, wm, wn);
    }
}
}  // namespace mbf16

TileShape tiles_m_bf16() { return {mbf16::BM, mbf16::BN}; }

hipError_t launch_ragged_m_bf16(const MParams& p, int grid, bool vec, hipStream_t s) {
    if (p.out_f32) {
        if (vec) hipLaunchKernelGGL((mbf16::kernel<true, float>), dim3(grid), dim3(mbf16::NT), 0, s, p);
        else hipLaunchKernelGGL((mbf16::kernel<false, float>), dim3(grid), dim3(mbf16::NT), 0, s, p);
    } else {
        if (vec) hipLaunchKernelGGL((mbf16::kernel<true, uint16_t>), dim3(grid), dim3(mbf16::NT), 0, s, p);
        else hipLaunchKernelGGL((mbf16::kernel<false, uint16_t>), dim3(grid), dim3(mbf16::NT), 0, s, p);
    }
    return hipGetLastError();
}

// =======================================================================================
// fp32 inputs: 64 x 64 tile, k step 16, 4 waves (2 x 2) of 2 x 2 v_mfma_f32_16x16x4_f32
// blocks.  Element-wise masked loads; this family serves small and unaligned problems.
// =======================================================================================
namespace mf32 {
constexpr int BM = 64, BN = 64, BK = 16, NT = 256;

struct Smem {
    float a[BM][BK + 1];
    float b[BK][BN + 1];
    Tables tab;
};

__global__ __launch_bounds__(NT) void kernel(MParams p) {
    __shared__ Smem sm;
    const float* __restrict__ lhs = (const float*)p.lhs;
    const float* __restrict__ rhs = (const float*)p.rhs;
    float* __restrict__ out = (float*)p.out;
    const int ntn = cdiv(p.n, BN);
    int gemm_tiles, covered;
    if (p.uniform_rows > 0) {
        gemm_tiles = p.g * cdiv(p.uniform_rows, BM) * ntn;
        covered = p.m;
    } else {
        build_tables<NT>(p.group_sizes, p.g, p.m, BM, ntn, sm.tab, &gemm_tiles, &covered);
        if (blockIdx.x == 0 && threadIdx.x == 0 && p.status) *p.status = sm.tab.flags;
    }
    const int zero_mt = cdiv(p.m - covered, BM);
    const int total = gemm_tiles + zero_mt * ntn;
    const int l = threadIdx.x & 63, wave = threadIdx.x >> 6, wm = wave >> 1, wn = wave & 1;

    for (int t = xcd_virtual_id(blockIdx.x, gridDim.x); t < total; t += gridDim.x) {
        if (t >= gemm_tiles) {
            const int z = t - gemm_tiles;
            const int r0 = covered + (z % zero_mt) * BM, c0 = (z / zero_mt) * BN;
            for (int idx = threadIdx.x; idx < BM * BN; idx += NT) {
                const int r = r0 + idx / BN, c = c0 + idx % BN;
                if (r < p.m && c < p.n) out[(size_t)r * p.n + c] = 0.f;
            }
            continue;
        }
        int grp, row0, size, local;
        if (p.uniform_rows > 0) {
            const int per = cdiv(p.uniform_rows, BM) * ntn;
            grp = t / per; local = t - grp * per; row0 = grp * p.uniform_rows; size = p.uniform_rows;
        } else {
            grp = find_group(sm.tab.tile_off, p.g, t);
            local = t - sm.tab.tile_off[grp];
            row0 = sm.tab.row_off[grp];
            size = sm.tab.row_off[grp + 1] - row0;
        }
        const int mtg = cdiv(size, BM);
        const int mt = local % mtg, nt = local / mtg;
        row0 += mt * BM;
        const int rows_valid = min(BM, size - mt * BM);
        const int col0 = nt * BN;
        const float* rhs_g = rhs + (size_t)grp * (size_t)p.k * (size_t)p.n;
        f32x4 acc[2][2];
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
        for (int kk = 0; kk < p.k; kk += BK) {
            for (int idx = threadIdx.x; idx < BM * BK; idx += NT) {
                const int r = idx / BK, c = idx % BK;
                sm.a[r][c] = (r < rows_valid && kk + c < p.k) ? lhs[(size_t)(row0 + r) * p.k + kk + c] : 0.f;
            }
            for (int idx = threadIdx.x; idx < BK * BN; idx += NT) {
                const int r = idx / BN, c = idx % BN;
                sm.b[r][c] = (kk + r < p.k && col0 + c < p.n) ? rhs_g[(size_t)(kk + r) * p.n + col0 + c] : 0.f;
            }
            __syncthreads();
#pragma unroll
            for (int s = 0; s < BK / 4; ++s)
#pragma unroll
                for (int i = 0; i < 2; ++i)
#pragma unroll
                    for (int j = 0; j < 2; ++j) {
                        const float av = sm.a[32 * wm + 16 * i + (l & 15)][4 * s + (l >> 4)];
                        const float bv = sm.b[4 * s + (l >> 4)][32 * wn + 16 * j + (l & 15)];
                        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(av, bv, acc[i][j], 0, 0, 0);
                    }
            __syncthreads();
        }
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const int col = col0 + 32 * wn + 16 * j + (l & 15);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int r = 32 * wm + 16 * i + 4 * (l >> 4) + e;
                    if (r < rows_valid && col < p.n) out[(size_t)(row0 + r) * p.n + col] = acc[i][j][e];
                }
            }
    }
}
}  // namespace mf32

TileShape tiles_m_f32() { return {mf32::BM, mf32::BN}; }

hipError_t launch_ragged_m_f32(const MParams& p, int grid, hipStream_t s) {
    hipLaunchKernelGGL(mf32::kernel, dim3(grid), dim3(mf32::NT), 0, s, p);
    return hipGetLastError();
}

// =======================================================================================
// MXFP8 inputs (OCP e4m3 + E8M0 per 32 along k): 256 x 256 tile, k step 128, 8 waves of
// 4 x 2 v_mfma_scale_f32_32x32x64_f8f6f4 blocks.  The block scales go to the MFMA's own
// scale operands, so operands stay fp8 ("[Triton/Gluon] Merge MoE MXFP8 GEMM ...", the
// follow-up commits: dequantising to fp32 first is never a win).
// LDS: A [256][128] and B [128][256] bytes, double buffered (128 KiB).
// =======================================================================================
namespace mmx {
constexpr int BM = 256, BN = 256, BK = 128, NT = 512;

struct Smem {
    uint8_t a[2][BM * BK];
    uint8_t b[2][BK * BN];
    Tables tab;
};

// A (r, 16-byte chunk c of 8): chunks XOR-swizzled by (r >> 1) & 7.
__device__ inline int a_off(int r, int chunk) { return r * BK + ((chunk ^ ((r >> 1) & 7)) << 4); }
// B (kr, byte nn of 256): 16-byte chunks XOR-swizzled in 32-byte units by row bits 0..2.
__device__ inline int b_off(int kr, int nn) { return kr * BN + ((((nn >> 4) ^ ((kr & 7) << 1))) << 4) + (nn & 15); }

struct Regs { uint4 a[4]; uint4 b[4]; };

__device__ inline void load_tiles(Regs& R, const uint8_t* __restrict__ lhs, const uint8_t* __restrict__ rhs_g,
                                  int row0, int rows_valid, int col0, int kk, int k, int n, bool vec_n) {
    const int t = threadIdx.x;
    // A: 256 rows x 8 chunks; thread t -> chunk t&7 of rows (t>>3) + 64 i   (k % 32 == 0)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int r = (t >> 3) + 64 * i;
        const int kc = kk + ((t & 7) << 4);
        uint4 v = make_uint4(0, 0, 0, 0);
        if (r < rows_valid && kc < k) {   // k % 32 == 0 holds, so a 16-byte chunk never crosses k
            v = *(const uint4*)(lhs + (size_t)(row0 + r) * (size_t)k + kc);
        }
        R.a[i] = v;
    }
    // B: 128 rows x 16 chunks; thread t -> chunk t&15 of rows (t>>4) + 32 i
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int kr = kk + (t >> 4) + 32 * i;
        const int nc = col0 + ((t & 15) << 4);
        uint4 v = make_uint4(0, 0, 0, 0);
        if (kr < k) {
            const uint8_t* src = rhs_g + (size_t)kr * (size_t)n + nc;
            if (vec_n) {
                if (nc < n) v = *(const uint4*)src;
            } else {
                uint8_t e[16];
#pragma unroll
                for (int q = 0; q < 16; ++q) e[q] = (nc + q < n) ? src[q] : (uint8_t)0;
                v = *(const uint4*)e;
            }
        }
        R.b[i] = v;
    }
}

__device__ inline void store_tiles(const Regs& R, uint8_t* a, uint8_t* b) {
    const int t = threadIdx.x;
#pragma unroll
    for (int i = 0; i < 4; ++i) *(uint4*)(a + a_off((t >> 3) + 64 * i, t & 7)) = R.a[i];
#pragma unroll
    for (int i = 0; i < 4; ++i) *(uint4*)(b + b_off((t >> 4) + 32 * i, (t & 15) << 4)) = R.b[i];
}

__device__ inline void compute(const uint8_t* a, const uint8_t* b, const uint8_t* __restrict__ ls,
                               const uint8_t* __restrict__ rs_g, f32x16 (&acc)[4][2], int wm, int wn,
                               int row0, int rows_valid, int col0, int kk, int k, int n) {
    const int l = threadIdx.x & 63;
    const int h = l >> 5;
    const int q = l >> 4, rr = (l >> 1) & 7, c = l & 1;
    const int kb = k >> 5;
#pragma unroll
    for (int s = 0; s < BK / 64; ++s) {
        const int kblk = (kk >> 5) + 2 * s + h;       // 32-wide k block of this lane's scale
        const bool kin = kk + 64 * s < k;             // whole 64-slice inside k (k % 32 == 0)
        i32x8 af[4], bfr[2];
        int sa[4], sb[2];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = 128 * wm + 32 * i + (l & 31);
            const i32x4 lo = *(const i32x4*)(a + a_off(r, 4 * s + h));
            const i32x4 hi = *(const i32x4*)(a + a_off(r, 4 * s + 2 + h));
            af[i] = i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
            sa[i] = (r < rows_valid && kblk < kb) ? (int)ls[(size_t)(row0 + r) * kb + kblk] : 127;
        }
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int nn = 64 * wn + 32 * j + 16 * (q & 1) + 8 * c;
            const int kbase = 64 * s + 16 * (q >> 1) + rr;
            const i32x2 p0 = lds_read_tr8(b + b_off(kbase, nn));
            const i32x2 p1 = lds_read_tr8(b + b_off(kbase + 8, nn));
            const i32x2 p2 = lds_read_tr8(b + b_off(kbase + 32, nn));
            const i32x2 p3 = lds_read_tr8(b + b_off(kbase + 40, nn));
            bfr[j] = i32x8{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
            const int col = col0 + 64 * wn + 32 * j + (l & 31);
            sb[j] = (col < n && kblk < kb) ? (int)rs_g[(size_t)kblk * n + col] : 127;
        }
        if (kin) {
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(af[i], bfr[j], acc[i][j], 0, 0, 0, sa[i],
                                                                               0, sb[j]);
        }
    }
}

template <typename OutT>
__global__ __launch_bounds__(NT, 1) void kernel(MParams p) {
    __shared__ Smem sm;
    const uint8_t* __restrict__ lhs = (const uint8_t*)p.lhs;
    const uint8_t* __restrict__ rhs = (const uint8_t*)p.rhs;
    OutT* __restrict__ out = (OutT*)p.out;
    const int ntn = cdiv(p.n, BN);
    int gemm_tiles, covered;
    if (p.uniform_rows > 0) {
        gemm_tiles = p.g * cdiv(p.uniform_rows, BM) * ntn;
        covered = p.m;
    } else {
        build_tables<NT>(p.group_sizes, p.g, p.m, BM, ntn, sm.tab, &gemm_tiles, &covered);
        if (blockIdx.x == 0 && threadIdx.x == 0 && p.status) *p.status = sm.tab.flags;
    }
    const int zero_mt = cdiv(p.m - covered, BM);
    const int total = gemm_tiles + zero_mt * ntn;
    const int wave = threadIdx.x >> 6, wm = wave >> 2, wn = wave & 3;
    const int nk = cdiv(p.k, BK);
    const bool vec_n = (p.n & 15) == 0;

    for (int t = xcd_virtual_id(blockIdx.x, gridDim.x); t < total; t += gridDim.x) {
        if (t >= gemm_tiles) {
            const int z = t - gemm_tiles;
            mbf16::zero_tile(out, covered + (z % zero_mt) * BM, p.m, (z / zero_mt) * BN, p.n);
            continue;
        }
        int grp, row0, size, local;
        if (p.uniform_rows > 0) {
            const int per = cdiv(p.uniform_rows, BM) * ntn;
            grp = t / per; local = t - grp * per; row0 = grp * p.uniform_rows; size = p.uniform_rows;
        } else {
            grp = find_group(sm.tab.tile_off, p.g, t);
            local = t - sm.tab.tile_off[grp];
            row0 = sm.tab.row_off[grp];
            size = sm.tab.row_off[grp + 1] - row0;
        }
        const int mtg = cdiv(size, BM);
        int mt, nt;
        if (size <= p.n) { mt = local % mtg; nt = local / mtg; }
        else { nt = local % ntn; mt = local / ntn; }
        row0 += mt * BM;
        const int rows_valid = min(BM, size - mt * BM);
        const int col0 = nt * BN;
        const uint8_t* rhs_g = rhs + (size_t)grp * (size_t)p.k * (size_t)p.n;
        const uint8_t* rs_g = p.rhs_scale + (size_t)grp * (size_t)(p.k >> 5) * (size_t)p.n;

        f32x16 acc[4][2];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;
        Regs R;
        if (nk > 0) {
            load_tiles(R, lhs, rhs_g, row0, rows_valid, col0, 0, p.k, p.n, vec_n);
            store_tiles(R, sm.a[0], sm.b[0]);
            __syncthreads();
        }
        for (int kt = 0; kt < nk; ++kt) {
            const int cur = kt & 1;
            if (kt + 1 < nk) load_tiles(R, lhs, rhs_g, row0, rows_valid, col0, (kt + 1) * BK, p.k, p.n, vec_n);
            compute(sm.a[cur], sm.b[cur], p.lhs_scale, rs_g, acc, wm, wn, row0, rows_valid, col0, kt * BK, p.k, p.n);
            if (kt + 1 < nk) store_tiles(R, sm.a[cur ^ 1], sm.b[cur ^ 1]);
            __syncthreads();
        }
        mbf16::store_out(out, acc, row0, rows_valid, col0, p.n, wm, wn);
    }
}
}  // namespace mmx

TileShape tiles_m_e4m3() { return {mmx::BM, mmx::BN}; }

hipError_t launch_ragged_m_e4m3(const MParams& p, int grid, hipStream_t s) {
    if (p.out_f32) hipLaunchKernelGGL((mmx::kernel<float>), dim3(grid), dim3(mmx::NT), 0, s, p);
    else hipLaunchKernelGGL((mmx::kernel<uint16_t>), dim3(grid), dim3(mmx::NT), 0, s, p);
    return hipGetLastError();
}

}  // namespace gg
