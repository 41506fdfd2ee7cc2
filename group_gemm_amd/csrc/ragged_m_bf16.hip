// ragged_m_bf16.hip -- the bf16 non-contracting ragged dot on gfx950, vectorised path
// (16-byte aligned operands, k and n multiples of 8).  The element-wise fallback for other
// shapes lives in ragged_m.hip.
//
// "Group-GEMM in XLA: Making Mixture-of-Experts Fast and Memory-Efficient" (AMD ROCm blog),
// Part 3 "Non-Contracting (the MoE Case)": per output tile, find the group from the prefix
// table, select that expert's weights, accumulate over k, masked store.  Tiles here are
// group-aligned and walked by a persistent grid (see ragged_m.hip for the schedule notes).
//
// Kernel shape: 256 x 256 output tile, 4 waves in a 2 x 2 grid, each wave a 128 x 128
// sub-tile of 4 x 4 v_mfma_f32_32x32x16_bf16 blocks (fp32 accumulators in AGPRs).
// Operands stream through a 4-slot LDS ring of 32-wide k slices, filled by buffer loads
// that write LDS directly (no staging registers); loads run three slices ahead of the
// MFMAs, which is what hides HBM latency.  The buffer descriptors bound the group's rows
// and the weight matrix, so rows past the group and the k / n tails arrive as zeros.
// The MFMA takes the weight fragment as its first operand, which gives every lane 4
// consecutive output columns; the epilogue stages the bf16 tile in LDS and writes whole
// 16-byte row segments.
#include "common.hpp"
#include "launch.hpp"

namespace gg {
namespace mb3 {

constexpr int BM = 256, BN = 256, BK = 32, STAGES = 4, NT = 256;
constexpr int CP = BN + 8;               // pitch (elements) of the staged output tile
constexpr int SLICE = BM * BK;           // elements of one A (= one B) k slice: 16 KiB
constexpr uint32_t kOOB = 0x80000000u;   // a buffer offset past every num_records
constexpr int kRsrcWord3 = 0x00020000;   // raw buffer, 32-bit data format (gfx9 family)

struct Smem {
    union {
        struct {
            uint16_t a[STAGES][SLICE];
            uint16_t b[STAGES][SLICE];
        } ring;
        uint16_t c[BM * CP];
    };
    Tables tab;
};

typedef __amdgpu_buffer_rsrc_t rsrc_t;

__device__ inline rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, kRsrcWord3);
}
__device__ inline void bstore(rsrc_t r, uint32_t off, i32x4 v) { __builtin_amdgcn_raw_buffer_store_b128(v, r, off, 0, 0); }
// 16 bytes per lane from the buffer straight into LDS at lds + 16 * lane
__device__ inline void load_lds16(rsrc_t r, const uint16_t* lds, uint32_t off) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 16, off, 0, 0, 0);
}
// barrier that waits for this wave's LDS accesses only; ring loads stay in flight
__device__ inline void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }
// wait until at most `later` k slices (8 loads each per thread) are still in flight
__device__ inline void wait_slices(int later) {
    if (later >= 2) asm volatile("s_waitcnt vmcnt(16)" ::: "memory");
    else if (later == 1) asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
    else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

// LDS layouts (element offsets); chunks are 8 bf16 = 16 bytes.
// A slice [256 rows][32 k], 64-byte rows: chunk XOR (row >> 2) & 3, so the 16 rows one
// 16-lane phase of a fragment read touches cover all 64 banks.
__device__ inline int a_off(int r, int chunk) { return r * BK + ((chunk ^ ((r >> 2) & 3)) << 3); }
// B slice [32 k][256 n], 512-byte rows: chunk XOR'ed in 64-byte units by a 3-bit function
// of the row, so the rows one transpose read touches land in distinct 64-byte bank groups.
__device__ inline int b_swz(int kr) { return ((kr & 3) | (((kr >> 3) & 1) << 2)) << 2; }
__device__ inline int b_off(int kr, int nn) { return kr * BN + (((nn >> 3) ^ b_swz(kr)) << 3) + (nn & 7); }

struct Frags { bf16x8 a[4]; bf16x8 b[4]; };

// fragments of 16-wide k step s (0 or 1) of a slice
__device__ inline void read_frags(Frags& f, const uint16_t* a, const uint16_t* b, int s, int wm, int wn) {
    const int l = threadIdx.x & 63, h = l >> 5;
    const int q = l >> 4, rr = (l >> 2) & 3, c = l & 3;
#pragma unroll
    for (int i = 0; i < 4; ++i) f.a[i] = *(const bf16x8*)(a + a_off(128 * wm + 32 * i + (l & 31), 2 * s + h));
    const int kr0 = 16 * s + 8 * (q >> 1) + rr;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int nn = 128 * wn + 32 * j + 16 * (q & 1) + 4 * c;
        const i16x4 lo = lds_read_tr16(b + b_off(kr0, nn));
        const i16x4 hi = lds_read_tr16(b + b_off(kr0 + 4, nn));
        typedef short i16x8 __attribute__((ext_vector_type(8)));
        const i16x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        f.b[j] = __builtin_bit_cast(bf16x8, v);
    }
}

__device__ inline void mma(const Frags& f, f32x16 (&acc)[4][4]) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.b[j], f.a[i], acc[i][j], 0, 0, 0);
}

template <typename OutT>
__global__ __launch_bounds__(NT, 1) void kernel(MParams p) {
    __shared__ Smem sm;
    const int t = threadIdx.x, l = t & 63, wave = t >> 6, wm = wave >> 1, wn = wave & 1, h = l >> 5;
    const int ntn = cdiv(p.n, BN);
    int gemm_tiles, covered;
    if (p.uniform_rows > 0) {
        gemm_tiles = p.g * cdiv(p.uniform_rows, BM) * ntn;
        covered = p.m;
    } else {
        build_tables<NT>(p.group_sizes, p.g, p.m, BM, ntn, sm.tab, &gemm_tiles, &covered);
        if (blockIdx.x == 0 && t == 0 && p.status) *p.status = sm.tab.flags;
    }
    const int zero_mt = cdiv(p.m - covered, BM);
    const int total = gemm_tiles + zero_mt * ntn;
    const int nk = cdiv(p.k, BK);
    const uint32_t k2 = (uint32_t)p.k * 2u, n2 = (uint32_t)p.n * 2u;
    constexpr int osz = sizeof(OutT);

    // Ring-load roles (fixed per thread).  Wave w fills 1 KiB blocks 4w..4w+3 of each
    // slice; lane l of block b writes LDS bytes [16 l, 16 l + 16) of it.
    //   A block b = rows 16b..16b+15; lane l -> row 16b + l/4, physical chunk l%4, which
    //     holds logical chunk (l%4) ^ ((row >> 2) & 3) = (l & 3) ^ ((l >> 4) & 3).
    //   B block b = rows 2b, 2b+1; lane l -> row 2b + l/32, physical chunk l%32, which
    //     holds logical chunk (l & 31) ^ b_swz(row).
    const int a_chunk = (l & 3) ^ ((l >> 4) & 3);
    int b_row[4], b_chunk[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        b_row[u] = 2 * (4 * wave + u) + (l >> 5);
        b_chunk[u] = (l & 31) ^ b_swz(b_row[u]);
    }

    for (int tile = xcd_virtual_id(blockIdx.x, gridDim.x); tile < total; tile += gridDim.x) {
        if (tile >= gemm_tiles) {   // rows past the covered ones: zeros, 16-byte stores
            const int z = tile - gemm_tiles;
            const int r0 = covered + (z % zero_mt) * BM, c0 = (z / zero_mt) * BN;
            const int rows = min(BM, p.m - r0);
            const rsrc_t ro = make_rsrc((const char*)p.out + (size_t)r0 * p.n * osz, (uint32_t)(rows * p.n * osz));
            constexpr int per_row = BN * osz / 16;
            for (int idx = t; idx < BM * per_row; idx += NT) {
                const int r = idx / per_row, cc = idx % per_row;
                const int col = c0 + cc * (16 / osz);
                bstore(ro, col < p.n ? (uint32_t)(r * p.n + col) * osz : kOOB, i32x4{0, 0, 0, 0});
            }
            continue;
        }
        int grp, row0, size, local;
        if (p.uniform_rows > 0) {
            const int per = cdiv(p.uniform_rows, BM) * ntn;
            grp = tile / per; local = tile - grp * per; row0 = grp * p.uniform_rows; size = p.uniform_rows;
        } else {
            grp = find_group(sm.tab.tile_off, p.g, tile);
            local = tile - sm.tab.tile_off[grp];
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

        const rsrc_t ra = make_rsrc((const uint16_t*)p.lhs + (size_t)row0 * p.k, (uint32_t)rows_valid * k2);
        const rsrc_t rb = make_rsrc((const uint16_t*)p.rhs + (size_t)grp * p.k * p.n, (uint32_t)p.k * n2);
        uint32_t a_voff[4], b_voff[4];
        bool b_ok[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int row = 16 * (4 * wave + u) + (l >> 2);
            a_voff[u] = (uint32_t)row * k2 + (uint32_t)a_chunk * 16u;
            const int col = col0 + 8 * b_chunk[u];
            b_ok[u] = col < p.n;
            b_voff[u] = (uint32_t)b_row[u] * n2 + (uint32_t)col * 2u;
        }
        auto issue = [&](int stage) {
            const int kk = stage * BK, slot = stage & (STAGES - 1);
            const bool a_ok = kk + 8 * a_chunk < p.k;
#pragma unroll
            for (int u = 0; u < 4; ++u)
                load_lds16(ra, sm.ring.a[slot] + (4 * wave + u) * 512, a_ok ? a_voff[u] + (uint32_t)kk * 2u : kOOB);
#pragma unroll
            for (int u = 0; u < 4; ++u)
                load_lds16(rb, sm.ring.b[slot] + (4 * wave + u) * 512, b_ok[u] ? b_voff[u] + (uint32_t)kk * n2 : kOOB);
        };

        f32x16 acc[4][4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

        Frags f0, f1;
        if (nk > 0) {
            const int pre = min(STAGES - 1, nk);
            for (int s = 0; s < pre; ++s) issue(s);
            wait_slices(pre - 1);
            lds_barrier();
            read_frags(f0, sm.ring.a[0], sm.ring.b[0], 0, wm, wn);
        }
        for (int kt = 0; kt < nk; ++kt) {
            const int slot = kt & (STAGES - 1);
            if (kt + STAGES - 1 < nk) issue(kt + STAGES - 1);
            read_frags(f1, sm.ring.a[slot], sm.ring.b[slot], 1, wm, wn);
            mma(f0, acc);
            if (kt + 1 < nk) {
                wait_slices(min(nk - 1, kt + STAGES - 1) - (kt + 1));
                lds_barrier();
                const int ns = (kt + 1) & (STAGES - 1);
                read_frags(f0, sm.ring.a[ns], sm.ring.b[ns], 0, wm, wn);
            }
            mma(f1, acc);
        }
        lds_barrier();   // every wave is done with the ring before it is reused

        // epilogue: acc[i][j][4q + e] = C[128wm + 32i + (l & 31)][128wn + 32j + 8q + 4h + e]
        const rsrc_t ro = make_rsrc((const char*)p.out + (size_t)row0 * p.n * osz, (uint32_t)(rows_valid * p.n * osz));
        if constexpr (osz == 2) {
            const int m_l = 128 * wm + (l & 31);
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j)
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
                        bf16x4 v = {(__bf16)acc[i][j][4 * q], (__bf16)acc[i][j][4 * q + 1], (__bf16)acc[i][j][4 * q + 2],
                                    (__bf16)acc[i][j][4 * q + 3]};
                        const int n_l = 128 * wn + 32 * j + 8 * q + 4 * h;
                        *(bf16x4*)(sm.c + (m_l + 32 * i) * CP + n_l) = v;
                    }
            lds_barrier();
            const int cc = t & 31;
            const int col = col0 + cc * 8;
#pragma unroll 4
            for (int it = 0; it < BM / 8; ++it) {
                const int r = it * 8 + (t >> 5);
                const i32x4 v = *(const i32x4*)(sm.c + r * CP + cc * 8);
                bstore(ro, col < p.n ? (uint32_t)(r * p.n + col) * 2u : kOOB, v);
            }
            lds_barrier();
        } else {
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j)
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const int r = 128 * wm + 32 * i + (l & 31);
                        const int col = col0 + 128 * wn + 32 * j + 8 * q + 4 * h;
                        const i32x4 v = {__float_as_int(acc[i][j][4 * q]), __float_as_int(acc[i][j][4 * q + 1]),
                                         __float_as_int(acc[i][j][4 * q + 2]), __float_as_int(acc[i][j][4 * q + 3])};
                        bstore(ro, col < p.n ? (uint32_t)(r * p.n + col) * 4u : kOOB, v);
                    }
        }
    }
}

}  // namespace mb3

bool ragged_m_bf16_fast_ok(const MParams& p) {
    // 32-bit buffer offsets: one expert's weights and one tile's rows must fit in 2 GiB
    const uint64_t w = (uint64_t)p.k * (uint64_t)p.n * 2u;
    const uint64_t a = (uint64_t)mb3::BM * (uint64_t)p.k * 2u;
    const uint64_t o = (uint64_t)mb3::BM * (uint64_t)p.n * 4u;
    return p.k % 8 == 0 && p.n % 8 == 0 && w < (1ull << 31) && a < (1ull << 31) && o < (1ull << 31);
}

hipError_t launch_ragged_m_bf16_fast(const MParams& p, int grid, hipStream_t s) {
    if (p.out_f32) hipLaunchKernelGGL((mb3::kernel<float>), dim3(grid), dim3(mb3::NT), 0, s, p);
    else hipLaunchKernelGGL((mb3::kernel<uint16_t>), dim3(grid), dim3(mb3::NT), 0, s, p);
    return hipGetLastError();
}

}  // namespace gg
