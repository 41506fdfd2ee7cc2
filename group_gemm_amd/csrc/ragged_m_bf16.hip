// ragged_m_bf16.hip -- the bf16 non-contracting ragged dot on gfx950, vectorised path
// (16-byte aligned operands, k and n multiples of 8).  The element-wise fallback for other
// shapes lives in ragged_m.hip.
//
// "Group-GEMM in XLA: Making Mixture-of-Experts Fast and Memory-Efficient" (AMD ROCm blog),
// Part 3 "Non-Contracting (the MoE Case)": per output tile, find the group from the prefix
// table, select that expert's weights, accumulate over k, masked store.  Tiles here are
// group-aligned and walked by a persistent grid (see ragged_m.hip for the schedule notes).
//
// Tile: 256 x 256 outputs per workgroup, 4 waves in a 2 x 2 grid, each a 128 x 128
// sub-tile of 4 x 4 v_mfma_f32_32x32x16_bf16 blocks (fp32 accumulators in AGPRs); k is
// consumed in 32-wide slices.  The kernel is a template over tile rows, wave layout and
// ring depth so other shapes can be timed; one shape is instantiated (see GG_TILE).
//  * Operands stream through an LDS ring filled by buffer loads that write LDS directly
//    (no staging registers), STAGES - 1 slices ahead of the MFMAs.  The buffer
//    descriptors bound the group's rows and the weight matrix, so rows past the group and
//    the k / n tails arrive as zeros without branches.
//  * A rows (k-contiguous) feed the MFMA through ds_read_b128; B rows are n-contiguous
//    (rhs as given, no per-call relayout) and ds_read_b64_tr_b16 turns them into
//    k-consecutive fragments.
//  * Each half slice is one pinned instruction sequence: every MFMA is followed by at
//    most one ring load and one fragment read for the next half slice, in the order the
//    next MFMAs need them, so LDS and memory traffic issue while the MFMAs run.
//  * 32-row MFMA blocks that lie wholly past a group's last row are skipped (their A
//    fragments are not read either): a group's last, partly filled tile, and tiles of
//    short groups, cost only the blocks they need.  The block count is a template
//    parameter of the main loop, so each variant is straight-line code.
//  * The MFMA takes the weight fragment as its first operand, which gives every lane 4
//    consecutive output columns; fp32 results are stored straight from AGPRs, bf16
//    results pass through a wave-private fp32 strip in LDS (see the epilogue).
#include "common.hpp"
#include "launch.hpp"
#include "ring.hpp"

namespace gg {
namespace mb {
using namespace ring;

constexpr int BN = 256, BK = 32;
constexpr int BSLICE = BK * BN;          // elements of one B slice: 16 KiB

// B slice [32 k][256 n], 512-byte rows: 16-byte chunks XOR'ed in 64-byte units by a 3-bit
// function of the row, so the rows one transpose read touches land in distinct bank groups.
__device__ inline int b_swz(int kr) { return ((kr & 3) | (((kr >> 3) & 1) << 2)) << 2; }
__device__ inline int b_off(int kr, int nn) { return kr * BN + (((nn >> 3) ^ b_swz(kr)) << 3) + (nn & 7); }
// A slice [BM rows][32 k], 64-byte rows: 16-byte chunk XOR (row >> 1) & 3.  Measured on
// gfx950 with the fragment reads below (32 consecutive rows, one chunk per lane half), this
// swizzle runs ds_read_b128 at ~115 B/clk per CU against ~76 for an XOR by (row >> 2) & 3.
__device__ inline int a_off(int r, int chunk) { return r * BK + ((chunk ^ ((r >> 1) & 3)) << 3); }

template <int BM, int WAVES_M, int STAGES, int NW>
struct Cfg {
    static constexpr int BM_ROWS = BM;
    static constexpr int NT = 64 * NW;                            // threads of a workgroup
    static constexpr int WAVES_N = NW / WAVES_M;
    static constexpr int WROWS = BM / WAVES_M, WCOLS = BN / WAVES_N;
    static constexpr int MI = WROWS / 32, NJ = WCOLS / 32;       // MFMA blocks per wave
    static constexpr int ASLICE = BM * BK;
    static constexpr int A_LOADS = BM / 16 / NW;                  // 1 KiB A blocks (16 rows) per wave
    static constexpr int B_LOADS = 16 / NW;                       // 1 KiB B blocks per wave
    static constexpr int PER = A_LOADS + B_LOADS;                 // ring loads per thread per slice
    static_assert(BM % (16 * NW) == 0 && 16 % NW == 0 && NW % WAVES_M == 0, "wave roles");
    static_assert(BM % 64 == 0 && WROWS % 32 == 0 && WCOLS % 32 == 0, "tile shape");
    static_assert(PER * (STAGES - 1) <= 63, "vmcnt range");
};

template <int BM, int WAVES_M, int STAGES, int NW>
struct Smem {
    typedef Cfg<BM, WAVES_M, STAGES, NW> C;
    struct {
        uint16_t a[STAGES][C::ASLICE];
        uint16_t b[STAGES][BSLICE];
    } ring;
    Tables tab;
    int next_tile;
};

template <int MI, int NJ>
struct Frags { bf16x8 a[MI]; bf16x8 b[NJ]; };

// acc[i][j] += B-fragment j x A-fragment i for the first NB row blocks
template <int MI, int NJ, int NB>
__device__ inline void mma(const Frags<MI, NJ>& f, f32x16 (&acc)[MI][NJ]) {
#pragma unroll
    for (int i = 0; i < NB; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.b[j], f.a[i], acc[i][j], 0, 0, 0);
}


// fragment read number R of k step s, in the order the MFMAs (column block major) first
// need them: B block 0, A blocks 0 .. NB - 1, then B blocks 1 .. NJ - 1
template <int MI, int NJ, int NB, int R, bool B_NK>
__device__ inline void read_one(Frags<MI, NJ>& f, const uint16_t* a, const uint16_t* b, int s, int r0, int c0) {
    const int l = threadIdx.x & 63, h = l >> 5;
    if constexpr (R >= 1 && R <= NB) {
        f.a[R - 1] = *(const bf16x8*)(a + a_off(r0 + 32 * (R - 1) + (l & 31), 2 * s + h));
    } else if constexpr (B_NK) {
        // k-contiguous weights: the slice is [256 n][32 k] in the A layout
        constexpr int j = R == 0 ? 0 : R - NB;
        f.b[j] = *(const bf16x8*)(b + a_off(c0 + 32 * j + (l & 31), 2 * s + h));
    } else {
        constexpr int j = R == 0 ? 0 : R - NB;
        const int q = l >> 4, rr = (l >> 2) & 3, c = l & 3;
        const int kr0 = 16 * s + 8 * (q >> 1) + rr;
        const int nn = c0 + 32 * j + 16 * (q & 1) + 4 * c;
        const i16x4 lo = lds_read_tr16(b + b_off(kr0, nn));
        const i16x4 hi = lds_read_tr16(b + b_off(kr0 + 4, nn));
        typedef short i16x8 __attribute__((ext_vector_type(8)));
        const i16x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        f.b[j] = __builtin_bit_cast(bf16x8, v);
    }
}


template <int BM, int WAVES_M, int STAGES, int NW, bool B_NK, bool EPI, typename OutT>
__global__ __launch_bounds__(64 * NW, 1) void kernel(MParams p) {
    typedef Cfg<BM, WAVES_M, STAGES, NW> C;
    constexpr int MI = C::MI, NJ = C::NJ, NT = C::NT;
    __shared__ Smem<BM, WAVES_M, STAGES, NW> sm;
    const int t = threadIdx.x, l = t & 63, wave = t >> 6, h = l >> 5;
    const int wm = wave / C::WAVES_N, wn = wave % C::WAVES_N;
    const int r0w = wm * C::WROWS, c0w = wn * C::WCOLS;   // this wave's sub-tile origin
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

    // Ring-load roles (fixed per thread).  A slice: 1 KiB blocks of 16 rows, wave w fills
    // blocks A_LOADS*w + u; lane l writes physical chunk l % 4 of row 16 b + l / 4, which
    // holds logical chunk (l & 3) ^ ((row >> 1) & 3) = (l & 3) ^ ((l >> 3) & 3).
    // B slice: 1 KiB blocks of 2 rows, wave w fills blocks B_LOADS w + u; lane l writes
    // physical chunk l % 32 of row 2b + l / 32, which holds logical chunk (l & 31) ^ b_swz.
    const int a_chunk = (l & 3) ^ ((l >> 3) & 3);
    // this wave's first 1 KiB block in A / B slot 0 (wave-uniform, scalar registers)
    const int wave_u = __builtin_amdgcn_readfirstlane(wave);
    const uint32_t lds_a = lds_u32(&sm.ring.a[0][0]) + (uint32_t)(C::A_LOADS * wave_u) * 1024u;
    const uint32_t lds_b = lds_u32(&sm.ring.b[0][0]) + (uint32_t)(C::B_LOADS * wave_u) * 1024u;
    // per-lane parts of the ring-load offsets (the wave- and tile-uniform parts are added
    // at each load, in scalar registers)
    const uint32_t a_lane = (uint32_t)(l >> 2) * k2 + (uint32_t)a_chunk * 16u;
    uint32_t b_lane[C::B_LOADS];
    int b_ch8[C::B_LOADS];
#pragma unroll
    for (int u = 0; u < C::B_LOADS; ++u) {
        const int b_row = 2 * (C::B_LOADS * wave + u) + (l >> 5);
        b_ch8[u] = 8 * ((l & 31) ^ b_swz(b_row));
        b_lane[u] = (uint32_t)(l >> 5) * n2 + (uint32_t)b_ch8[u] * 2u;
    }

    // tile walk: per-XCD queues when the launcher provides them (see ring.hpp)
    const bool queued = queued_walk(p.tile_queue);
    for (int tile = first_tile(queued);; tile += gridDim.x) {
        if (queued) tile = queue_next(p.tile_queue, &sm.next_tile);
        if (tile >= total) break;
        if (tile >= gemm_tiles) {   // rows past the covered ones: zeros
            const int z = tile - gemm_tiles;
            zero_tile<BM, BN, NT, OutT>(p.out, covered + (z % zero_mt) * BM, p.m, (z / zero_mt) * BN, p.n);
            continue;
        }
        int grp, row0, size, local, mt, nt;
        if (p.uniform_rows > 0) {
            const int per = cdiv(p.uniform_rows, BM) * ntn;
            grp = tile / per; local = tile - grp * per; row0 = grp * p.uniform_rows; size = p.uniform_rows;
        } else {
            grp = find_group(sm.tab.tile_off, p.g, tile);
            local = tile - sm.tab.tile_off[grp];
            row0 = sm.tab.row_off[grp];
            size = sm.tab.row_off[grp + 1] - row0;
        }
        // Within a group the tile that shares the streamed operand runs next (consecutive
        // tiles land on one XCD): weights stream once per column when the group is short,
        // rows stream once per row block when it is tall.  A group's partly filled last
        // m-tile stays beside the full ones of its column, so its weight reads hit L2.
        const int mtg = cdiv(size, BM);
        if (size <= p.n) { mt = local % mtg; nt = local / mtg; }
        else { nt = local % ntn; mt = local / ntn; }
        row0 += mt * BM;
        const int rows_valid = min(BM, size - mt * BM);
        const int col0 = nt * BN;
        // 32-row blocks of this wave that hold any of the tile's rows
        const int nb = max(0, min(MI, cdiv(rows_valid - r0w, 32)));

        const i32x4 ra = make_rsrc_v((const uint16_t*)p.lhs + (size_t)row0 * p.k, (uint32_t)rows_valid * k2);
        const i32x4 rb = make_rsrc_v((const uint16_t*)p.rhs + (size_t)grp * p.k * p.n, (uint32_t)p.k * n2);
        // ring load number d (A blocks first, then B) of k slice `stage` into its slot;
        // slices past k are zero-filled into the slot no one reads, which keeps the number
        // of loads per iteration, and so every wait count, constant
        auto dma_one = [&](auto d_c, int stage) {
            constexpr int d = decltype(d_c)::value;
            const int kk = stage * BK, slot = stage % STAGES;
            const bool live = stage < nk;
            if constexpr (d < C::A_LOADS) {
                // row 16 (A_LOADS wave + d) + l / 4 of the tile, chunk a_chunk
                const bool ok = live && kk + 8 * a_chunk < p.k;
                const uint32_t wpart = (uint32_t)(16 * (C::A_LOADS * wave_u + d)) * k2 + (uint32_t)kk * 2u;
                load_lds16(ra, lds_a + (uint32_t)slot * (C::ASLICE * 2) + d * 1024u, ok ? a_lane + wpart : kOOB);
            } else if constexpr (B_NK) {
                // [n][k] weights: row col0 + 16 (4 wave + u) + l / 4, chunk a_chunk (the A roles);
                // rows past n fall outside the descriptor
                constexpr int u = d - C::A_LOADS;
                const bool ok = live && kk + 8 * a_chunk < p.k;
                const uint32_t wpart = (uint32_t)(col0 + 16 * (C::B_LOADS * wave_u + u)) * k2 + (uint32_t)kk * 2u;
                load_lds16(rb, lds_b + (uint32_t)slot * (BSLICE * 2) + u * 1024u, ok ? a_lane + wpart : kOOB);
            } else {
                // k row kk + 2 (4 wave + u) + l / 32, columns col0 + b_ch8 .. + 7
                constexpr int u = d - C::A_LOADS;
                const bool ok = live && b_ch8[u] < p.n - col0;
                const uint32_t wpart = (uint32_t)(kk + 2 * (C::B_LOADS * wave_u + u)) * n2 + (uint32_t)col0 * 2u;
                load_lds16(rb, lds_b + (uint32_t)slot * (BSLICE * 2) + u * 1024u, ok ? b_lane[u] + wpart : kOOB);
            }
        };

        f32x16 acc[MI][NJ];
#pragma unroll
        for (int i = 0; i < MI; ++i)
#pragma unroll
            for (int j = 0; j < NJ; ++j)
#pragma unroll
                for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

        // One half slice: the MFMAs on `cur` with, after some, one ring load of slice `stage`
        // and, after each, at most one fragment read of `nxt` (k step s of slot a / b).  HALF
        // selects the ring loads: 0 none, 1 the first PER / 2 (the A blocks), 2 the rest; they
        // are spread evenly over the MFMAs, so the four waves' loads reach the memory pipeline
        // one at a time rather than in a burst.  The order is pinned so the loads and reads
        // issue while the MFMAs run.
        auto phase = [&](auto nb_c, auto half_c, Frags<MI, NJ>& cur, Frags<MI, NJ>& nxt, const uint16_t* a,
                         const uint16_t* b, int s, int stage) {
            constexpr int NB = decltype(nb_c)::value;
            constexpr int HALF = decltype(half_c)::value;
            constexpr int NM = NB * NJ, NR = NB > 0 ? NB + NJ : 0, ND = HALF ? C::PER / 2 : 0;
            constexpr int SP = ND > 0 && NM >= ND ? NM / ND : 1;   // MFMAs between two ring loads
            constexpr int LD = ND > 0 ? (ND - 1) * SP + 1 : 0;
            constexpr int NOPS = NM > NR ? (NM > LD ? NM : LD) : (NR > LD ? NR : LD);
            static_for<0, NOPS>([&](auto o_c) {
                constexpr int o = decltype(o_c)::value;
                if constexpr (o < NM) {   // column block major: block (o % NB, o / NB)
                    constexpr int i = o % (NB > 0 ? NB : 1), j = o / (NB > 0 ? NB : 1);
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(cur.b[j], cur.a[i], acc[i][j], 0, 0, 0);
                }
                if constexpr (ND > 0 && o % SP == 0 && o / SP < ND)
                    dma_one(std::integral_constant<int, (HALF - 1) * (C::PER / 2) + o / SP>{}, stage);
                if constexpr (o < NR) read_one<MI, NJ, NB, o, B_NK>(nxt, a, b, s, r0w, c0w);
                __builtin_amdgcn_sched_barrier(0);
            });
        };

        // Slice s is loaded in two halves: the first in the second half slice of iteration
        // s - 4 (its slot, read last in the first half slice of that iteration, is free once
        // the iteration's barrier has passed), the second in the first half slice of
        // iteration s - 3.  Either way PER * (STAGES - 2) loads are issued after slice kt + 1's
        // last one by the time iteration kt waits for it.
        static_assert(STAGES == 4 && C::PER % 2 == 0, "the split ring loads assume a 4-slot ring");
        auto run = [&](auto nb_c) {
            constexpr int NB = decltype(nb_c)::value;
            constexpr std::integral_constant<int, 0> none{};
            constexpr std::integral_constant<int, 1> first{};
            constexpr std::integral_constant<int, 2> second{};
            Frags<MI, NJ> f0, f1;
            static_for<0, STAGES - 1>([&](auto st_c) { static_for<0, C::PER>([&](auto d_c) { dma_one(d_c, decltype(st_c)::value); }); });
            static_for<0, C::PER / 2>([&](auto d_c) { dma_one(d_c, STAGES - 1); });
            // slice 0 in LDS.  Loads complete in issue order among themselves; output stores of
            // the previous tile still in flight only raise the count, so this can only wait longer.
            wait_vm<C::PER * (STAGES - 2) + C::PER / 2>();
            lds_barrier();
            if constexpr (NB > 0)
                static_for<0, NB + NJ>([&](auto r_c) { read_one<MI, NJ, NB, decltype(r_c)::value, B_NK>(f0, sm.ring.a[0], sm.ring.b[0], 0, r0w, c0w); });
            for (int kt = 0; kt + 1 < nk; ++kt) {
                const int slot = kt % STAGES, ns = (kt + 1) % STAGES;
                phase(nb_c, second, f0, f1, sm.ring.a[slot], sm.ring.b[slot], 1, kt + STAGES - 1);
                wait_vm<C::PER * (STAGES - 2)>();   // slice kt + 1 in LDS
                lds_barrier();
                phase(nb_c, first, f1, f0, sm.ring.a[ns], sm.ring.b[ns], 0, kt + STAGES);
            }
            const int last = (nk - 1) % STAGES;
            phase(nb_c, none, f0, f1, sm.ring.a[last], sm.ring.b[last], 1, 0);
            mma<MI, NJ, NB>(f1, acc);
        };
        if (nk > 0) with_nb<MI>(nb, run);
        // Every ring load has landed (the zero-fill loads of slices past the end may still be
        // in flight, and the epilogue strips overlap their slots) and every wave is done
        // reading the ring before it is reused.
        wait_vm<0>();
        lds_barrier();

        const rsrc_t ro = make_rsrc((const char*)p.out + (size_t)row0 * p.n * osz, (uint32_t)(rows_valid * p.n * osz));
        static_assert(NW * 32 * (C::WCOLS + 4) * 4 <= (int)sizeof(sm.ring), "epilogue strips fit the ring");
        const EpiTile ep{p.bias ? p.bias + (size_t)grp * p.bias_stride : nullptr, p.alpha, p.beta};
        store_acc<MI, NJ, C::WCOLS, OutT, EPI>(acc, reinterpret_cast<float*>(&sm.ring) + wave * 32 * (C::WCOLS + 4), ro, p.n,
                                               col0, r0w, c0w, ep);
        if constexpr (osz == 2 || EPI) lds_barrier();   // strips read before the next tile's ring loads land there
    }
    wait_vm<0>();   // no ring load may still be writing LDS when the workgroup ends
}

// tile shape: (rows, waves along rows, ring slots, waves).  256 x 256 with a 4-slot ring and
// four waves is the fastest of the shapes the template allows (64 / 128 / 256 rows, 1 / 2 / 4
// row waves, 3-7 slots, 4 or 8 waves) both on groups of ~1000 rows, where the MFMA bounds
// it, and on Zipf-skewed groups of ~128 rows, where the weight stream does: blocks past a
// group's last row are skipped, so tall tiles cost short groups little, while they halve
// the B fragment reads per flop.  (Eight waves, two per SIMD with the accumulators in
// VGPRs, ran 5 % slower on the first and 25 % on the second.)
#define GG_TILE 256, 2, 4, 4

}  // namespace mb

int ragged_m_bf16_fast_bm(const MParams&) { return mb::Cfg<GG_TILE>::BM_ROWS; }

bool ragged_m_bf16_fast_ok(const MParams& p) {
    // 32-bit buffer offsets: one expert's weights and one tile's rows must fit in 2 GiB
    const uint64_t w = (uint64_t)p.k * (uint64_t)p.n * 2u;
    const uint64_t a = 256ull * (uint64_t)p.k * 2u;
    const uint64_t o = 256ull * (uint64_t)p.n * 4u;
    return p.k % 8 == 0 && p.n % 8 == 0 && w < (1ull << 31) && a < (1ull << 31) && o < (1ull << 31);
}

__global__ void clear_queues(int* q) {
    if (threadIdx.x < 8) q[threadIdx.x] = 0;
}

hipError_t launch_clear_queues(int* q, hipStream_t s) {
    hipLaunchKernelGGL(clear_queues, dim3(1), dim3(64), 0, s, q);
    return hipGetLastError();
}

template <bool B_NK, bool EPI>
static void launch_mb(const MParams& p, int grid, hipStream_t s) {
    if (p.tile_queue) launch_clear_queues(p.tile_queue, s);
    constexpr int nt = mb::Cfg<GG_TILE>::NT;
    if (p.out_f32) hipLaunchKernelGGL((mb::kernel<GG_TILE, B_NK, EPI, float>), dim3(grid), dim3(nt), 0, s, p);
    else hipLaunchKernelGGL((mb::kernel<GG_TILE, B_NK, EPI, uint16_t>), dim3(grid), dim3(nt), 0, s, p);
}

hipError_t launch_ragged_m_bf16_fast(const MParams& p, int grid, hipStream_t s) {
    if (p.rhs_nk) {
        if (p.epi) launch_mb<true, true>(p, grid, s);
        else launch_mb<true, false>(p, grid, s);
    } else {
        if (p.epi) launch_mb<false, true>(p, grid, s);
        else launch_mb<false, false>(p, grid, s);
    }
    return hipGetLastError();
}

}  // namespace gg
