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
//    (no staging registers): B (weights) one k slice per slot, three slices ahead of the
//    MFMAs; A (rows) two k slices per slot, so that every load moves 128 contiguous bytes
//    of a row, landing two iterations before use.  The buffer descriptors bound the
//    group's rows and the weight matrix, so rows past the group and the k / n tails
//    arrive as zeros without branches.  A group with a single m-tile streams its weights
//    with the nontemporal hint (nothing else reads them).
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
// [rows][32 k] slice, 64-byte rows (the [n][k] weights of the data-gradient form): 16-byte
// chunk XOR (row >> 2) & 3.  The LDS serves a 16-byte-per-lane read 16 lanes at a time over
// its 64 banks; the fragment reads below give those 16 lanes 16 consecutive rows and one
// logical chunk, so the row's position in its 256-byte bank period (row & 3) and the XOR
// ((row >> 2) & 3) together place them on all 64 banks once (rocprofv3 SQ_LDS_BANK_CONFLICT:
// zero, against 0.5 conflict cycles per access with an XOR by (row >> 1) & 3).
__device__ inline int a_off(int r, int chunk) { return r * BK + ((chunk ^ ((r >> 2) & 3)) << 3); }
// A pair [BM rows][64 k] (two k slices), 128-byte rows: 16-byte chunk XOR (row >> 1) & 7, so
// the 16 rows a quarter of a fragment read touches fill the 64 banks once.  The A ring holds
// pairs because a load of 128 contiguous bytes per row moves twice the data per row as one of
// 64: measured on gfx950 with loads straight into LDS from L2-resident data, 16 rows x 64 B
// per instruction stream at ~30 B/clk per CU, 8 rows x 128 B at ~60.
__device__ inline int ap_off(int r, int chunk) { return r * (2 * BK) + ((chunk ^ ((r >> 1) & 7)) << 3); }

template <int BM, int WAVES_M, int STAGES, int NW>
struct Cfg {
    static constexpr int BM_ROWS = BM;
    static constexpr int NT = 64 * NW;                            // threads of a workgroup
    static constexpr int WAVES_N = NW / WAVES_M;
    static constexpr int WROWS = BM / WAVES_M, WCOLS = BN / WAVES_N;
    static constexpr int MI = WROWS / 32, NJ = WCOLS / 32;       // MFMA blocks per wave
    static constexpr int APAIR = BM * 2 * BK;                     // elements of one A pair (two k slices)
    static constexpr int A_LOADS = BM / 8 / NW;                   // 1 KiB A blocks (8 rows x 128 B) per wave and pair
    static constexpr int A_HALF = A_LOADS / 2;                    // A loads per iteration
    static constexpr int B_LOADS = 16 / NW;                       // 1 KiB B blocks per wave and slice
    static constexpr int BNK_LOADS = BN / 16 / NW;                // [n][k] weights: 1 KiB blocks of 16 rows
    static_assert(STAGES == 3 && NW == 4 && BM == 256, "the ring schedule assumes 3 slots, 4 waves, 256 rows");
    static_assert(BM % (8 * NW) == 0 && A_LOADS % 2 == 0 && 16 % NW == 0 && NW % WAVES_M == 0, "wave roles");
    static_assert(A_HALF == B_LOADS && BNK_LOADS == B_LOADS, "as many A as B loads per iteration");
    static_assert(BM % 64 == 0 && WROWS % 32 == 0 && WCOLS % 32 == 0, "tile shape");
};

template <int BM, int WAVES_M, int STAGES, int NW>
struct Smem {
    typedef Cfg<BM, WAVES_M, STAGES, NW> C;
    struct {
        uint16_t a[STAGES][C::APAIR];   // A pairs of k slices
        uint16_t b[STAGES][BSLICE];     // B slices
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


// fragment read number R of k step s of a slice, in the order the MFMAs (column block
// major) first need them: B block 0, A blocks 0 .. NB - 1, then B blocks 1 .. NJ - 1.  `a` is
// the slice's A pair and ac = 4 (slice parity) + 2 s its first 16-byte chunk of the step.
template <int MI, int NJ, int NB, int R, bool B_NK>
__device__ inline void read_one(Frags<MI, NJ>& f, const uint16_t* a, const uint16_t* b, int ac, int s, int r0, int c0) {
    const int l = threadIdx.x & 63, h = l >> 5;
    if constexpr (R >= 1 && R <= NB) {
        f.a[R - 1] = *(const bf16x8*)(a + ap_off(r0 + 32 * (R - 1) + (l & 31), ac + h));
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

    // Ring-load roles (fixed per thread).
    // A pair [256 rows][64 k]: 1 KiB blocks of 8 rows x 128 B, wave w fills blocks
    // A_LOADS w + e; lane l writes physical chunk l % 8 of row 8 b + l / 8, which holds
    // logical chunk (l & 7) ^ ((row >> 1) & 7) = (l & 7) ^ ((4 (e & 1) + l / 16) & 7).
    // B slice [32 k][256 n]: 1 KiB blocks of 2 rows, wave w fills blocks B_LOADS w + u; lane
    // l writes physical chunk l % 32 of row 2 b + l / 32, which holds logical chunk
    // (l & 31) ^ b_swz.  [n][k] weights (B_NK): 1 KiB blocks of 16 rows x 64 B; lane l writes
    // physical chunk l % 4 of row 16 b + l / 4, logical chunk (l & 3) ^ ((row >> 2) & 3).
    int ap_ch[2];
    uint32_t ap_lane[2];
#pragma unroll
    for (int e = 0; e < 2; ++e) {
        ap_ch[e] = (l & 7) ^ ((4 * e + (l >> 4)) & 7);
        ap_lane[e] = (uint32_t)(l >> 3) * k2 + (uint32_t)ap_ch[e] * 16u;
    }
    const int nk_chunk = (l & 3) ^ ((l >> 4) & 3);
    const uint32_t nk_lane = (uint32_t)(l >> 2) * k2 + (uint32_t)nk_chunk * 16u;
    // this wave's first 1 KiB block in A / B slot 0 (wave-uniform, scalar registers)
    const int wave_u = __builtin_amdgcn_readfirstlane(wave);
    const uint32_t lds_a = lds_u32(&sm.ring.a[0][0]) + (uint32_t)(C::A_LOADS * wave_u) * 1024u;
    const uint32_t lds_b = lds_u32(&sm.ring.b[0][0]) + (uint32_t)(C::B_LOADS * wave_u) * 1024u;
    // per-lane parts of the B ring-load offsets (the wave- and tile-uniform parts are added
    // at each load, in scalar registers)
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
        if (queued) tile = queue_next(p.tile_queue, &sm.next_tile, total);
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
        // A group with one m-tile reads each weight slice once (no other tile of it shares the
        // slice), so its weight loads carry the nontemporal hint: they stream past L2 instead of
        // evicting the rows that the group's other n-tiles read again (DeepSeek-like workload:
        // 0.27 GB less fetched per call, 1.2-1.6 % faster; the others have no such group).
        const bool b_stream = __builtin_amdgcn_readfirstlane(mtg == 1 ? 1 : 0) != 0;
        // 32-row blocks of this wave that hold any of the tile's rows
        const int nb = max(0, min(MI, cdiv(rows_valid - r0w, 32)));

        const i32x4 ra = make_rsrc_v((const uint16_t*)p.lhs + (size_t)row0 * p.k, (uint32_t)rows_valid * k2);
        const i32x4 rb = make_rsrc_v((const uint16_t*)p.rhs + (size_t)grp * p.k * p.n, (uint32_t)p.k * n2);
        // Ring loads.  Every iteration issues the same number, and loads past the end of k
        // read zeros into a slot no one reads, so every wait count is a compile-time constant.
        // A block e of pair `pr` (k slices 2 pr, 2 pr + 1): rows 8 (A_LOADS wave + e) + l / 8
        // of the tile, logical chunk ap_ch[e & 1]
        // (the caller passes the ring slot, pslot = pr % STAGES, as a constant where it can)
        // FULL: the caller guarantees the load lies in whole k slices, and the k check goes
        auto dma_a = [&](auto e_c, int pr, int pslot, auto full_c) {
            constexpr int e = decltype(e_c)::value;
            constexpr bool FULL = decltype(full_c)::value;
            // (the k offset goes through readfirstlane, opaque to loop strength reduction: left
            // visible, every load's lane offset becomes a vector induction variable, and the
            // registers they take spill, each reload a wait for every ring load in flight; this
            // one change made the Mixtral-like call 6 % faster and the DeepSeek-like 3.6 %)
            const int kk = __builtin_amdgcn_readfirstlane(pr * 2 * BK);
            const bool ok = FULL || kk + 8 * ap_ch[e & 1] < p.k;
            const uint32_t wpart = (uint32_t)(8 * (C::A_LOADS * wave_u + e)) * k2 + (uint32_t)kk * 2u;
            load_lds16(ra, lds_a + (uint32_t)pslot * (C::APAIR * 2) + e * 1024u, ok ? ap_lane[e & 1] + wpart : kOOB);
        };
        // B block u of k slice st into ring slot bslot = st % STAGES (NT: with the nontemporal hint)
        auto dma_b = [&](auto u_c, int st, auto nt_c, int bslot, auto full_c) {
            constexpr int u = decltype(u_c)::value;
            constexpr bool NT_HINT = decltype(nt_c)::value;
            constexpr bool FULL = decltype(full_c)::value;
            auto load = [&](uint32_t dst, uint32_t off) {
                if constexpr (NT_HINT) load_lds16_nt(rb, dst, off);
                else load_lds16(rb, dst, off);
            };
            const int kk = __builtin_amdgcn_readfirstlane(st * BK);   // (see dma_a)
            const uint32_t dst = lds_b + (uint32_t)bslot * (BSLICE * 2) + u * 1024u;
            if constexpr (B_NK) {
                // [n][k] weights: row col0 + 16 (4 wave + u) + l / 4, chunk nk_chunk; rows past n
                // fall outside the descriptor
                const bool ok = FULL || kk + 8 * nk_chunk < p.k;
                const uint32_t wpart = (uint32_t)(col0 + 16 * (C::B_LOADS * wave_u + u)) * k2 + (uint32_t)kk * 2u;
                load(dst, ok ? nk_lane + wpart : kOOB);
            } else {
                // k row kk + 2 (4 wave + u) + l / 32, columns col0 + b_ch8 .. + 7.  Unchecked: rows
                // past k lie past the descriptor's end and read zeros, and columns past n read
                // other weights that reach only output columns that are never stored.
                const uint32_t wpart = (uint32_t)(kk + 2 * (C::B_LOADS * wave_u + u)) * n2 + (uint32_t)col0 * 2u;
                load(dst, b_lane[u] + wpart);
            }
        };

        f32x16 acc[MI][NJ];
#pragma unroll
        for (int i = 0; i < MI; ++i)
#pragma unroll
            for (int j = 0; j < NJ; ++j)
#pragma unroll
                for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

        // One half slice: the MFMAs on `cur` with, after each, at most one fragment read of
        // `nxt` (k step s: chunk ac of A pair a, step s of B slot b) and, spread evenly over
        // the MFMAs, ND ring loads mem(d) for d = 0 .. ND - 1, so the four waves' loads reach
        // the memory pipeline one at a time rather than in a burst.  The order is pinned so
        // the loads and reads issue while the MFMAs run.
        auto phase = [&](auto nb_c, auto nd_c, auto&& mem, Frags<MI, NJ>& cur, Frags<MI, NJ>& nxt, const uint16_t* a,
                         int ac, const uint16_t* b, int s) {
            constexpr int NB = decltype(nb_c)::value;
            constexpr int ND = decltype(nd_c)::value;
            constexpr int NM = NB * NJ, NR = NB > 0 ? NB + NJ : 0;
            constexpr int SP = ND > 0 && NM >= ND ? NM / (ND > 0 ? ND : 1) : 1;   // MFMAs between two ring loads
            constexpr int LD = ND > 0 ? (ND - 1) * SP + 1 : 0;
            constexpr int NOPS = NM > NR ? (NM > LD ? NM : LD) : (NR > LD ? NR : LD);
            static_for<0, NOPS>([&](auto o_c) {
                constexpr int o = decltype(o_c)::value;
                if constexpr (o < NM) {   // column block major: block (o % NB, o / NB)
                    constexpr int i = o % (NB > 0 ? NB : 1), j = o / (NB > 0 ? NB : 1);
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(cur.b[j], cur.a[i], acc[i][j], 0, 0, 0);
                }
                if constexpr (ND > 0 && o % SP == 0 && o / SP < ND) mem(std::integral_constant<int, o / SP>{});
                if constexpr (o < NR) read_one<MI, NJ, NB, o, B_NK>(nxt, a, b, ac, s, r0w, c0w);
                __builtin_amdgcn_sched_barrier(0);
            });
        };

        // Iteration kt runs k step 0 of slice kt, waits for slice kt + 1, then runs step 1
        // while reading step 0 of slice kt + 1.  Ring loads, four per half slice:
        //  * B slice kt + 3 in the second half slice of iteration kt.  Its slot held slice
        //    kt, whose last reads came before this iteration's barrier.
        //  * A pair j (slices 2 j, 2 j + 1) in the first half slices of iterations 2 j - 4
        //    (blocks 0-3) and 2 j - 3 (blocks 4-7).  Its slot held pair j - 3, read last before
        //    the barrier of iteration 2 j - 5.
        // At the barrier of iteration kt slice kt + 1's B blocks, issued in iteration kt - 2,
        // are followed by 12 loads (its A pair by at least 16), so a wait for 12 outstanding
        // loads covers both; loads complete in issue order among themselves, and output
        // stores of the previous tile still in flight only raise the count.
        constexpr int AH = C::A_HALF, BL = C::B_LOADS;
        constexpr int W_STEADY = 2 * AH + BL;   // B of slice kt + 1 is followed by A, B, A
        auto run = [&](auto nb_c, auto nt_c) {
            constexpr int NB = decltype(nb_c)::value;
            constexpr std::integral_constant<int, 0> zero{};
            constexpr std::integral_constant<int, AH> nd_a{};
            constexpr std::integral_constant<int, BL> nd_b{};
            Frags<MI, NJ> f0, f1;
            // what iterations before the first would have issued, in an order that leaves at
            // least W_STEADY loads behind slice 1's B blocks before the first barrier
            constexpr std::false_type chk{};
            static_for<0, BL>([&](auto u_c) { dma_b(u_c, 0, nt_c, 0, chk); });
            static_for<0, 2 * AH>([&](auto e_c) { dma_a(e_c, 0, 0, chk); });
            static_for<0, BL>([&](auto u_c) { dma_b(u_c, 1, nt_c, 1, chk); });
            static_for<0, 2 * AH>([&](auto e_c) { dma_a(e_c, 1, 1, chk); });
            static_for<0, BL>([&](auto u_c) { dma_b(u_c, 2, nt_c, 2, chk); });
            wait_vm<2 * BL + 2 * AH>();   // slice 0's B blocks and pair 0 in LDS
            lds_barrier();
            if constexpr (NB > 0)
                static_for<0, NB + NJ>([&](auto r_c) { read_one<MI, NJ, NB, decltype(r_c)::value, B_NK>(f0, sm.ring.a[0], sm.ring.b[0], 0, 0, r0w, c0w); });
            __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0): exact wait counts at the loop head
            // Iteration kt, for kt = R (mod 6) with R a compile-time constant.  Six is the least
            // common multiple of the slice parity (which picks the A chunk and the A blocks a
            // half slice loads) and the three ring slots, so every slot index, and with it
            // every LDS offset of the fragment reads and ring loads, is a constant.  With the
            // slots taken mod 3 at run time the Mixtral-like loop issued 6.1 instructions per
            // MFMA, and a wave alone on its SIMD spent the MFMAs' issue slots on them; unrolled
            // by six it issues 3.9 (7 % faster, DeepSeek-like 4 %, results bit-identical).
            // (forced inline: with three call sites the inliner would keep it out of line, and
            // the fragment registers it works on would go to memory)
            auto iter = [&](auto r_c, int kt, auto full_c) __attribute__((always_inline)) {
                constexpr int R = decltype(r_c)::value, P = R & 1;
                constexpr int pa = (R >> 1) % STAGES, pn = ((R + 1) >> 1) % STAGES;   // A pairs of slices kt, kt + 1
                constexpr int slot = R % STAGES, ns = (R + 1) % STAGES;                // B slices kt, kt + 1
                constexpr int ps = ((R + 4) >> 1) % STAGES, bs = (R + 3) % STAGES;      // slots loaded
                const int pr = (kt + 4) >> 1;   // A pair kt / 2 + 2, blocks 4 P .. 4 P + 3
                phase(nb_c, nd_a, [&](auto d_c) { dma_a(std::integral_constant<int, P * AH + decltype(d_c)::value>{}, pr, ps, full_c); },
                      f0, f1, sm.ring.a[pa], 4 * P + 2, sm.ring.b[slot], 1);
                wait_vm<W_STEADY>();   // slice kt + 1 in LDS
                lds_barrier();
                phase(nb_c, nd_b, [&](auto d_c) { dma_b(d_c, kt + 3, nt_c, bs, full_c); }, f1, f0, sm.ring.a[pn], 4 * (1 - P), sm.ring.b[ns], 0);
            };
            // Six iterations from kt (even) load B slices up to kt + 8 and A pairs up to slices
            // kt + 8, kt + 9; while those lie before slice nk - 1, the last and possibly partial
            // one, no load needs its k check (the A loads' and the [n][k] weights' per-lane
            // checks go: forward 664 -> 640, data gradient 628 -> 538 instructions per six
            // iterations; Mixtral-like 0.9 % and DeepSeek-like 0.7 % faster, bit-identical).
            int kt = 0;
            for (; kt + 11 <= nk; kt += 6) static_for<0, 6>([&](auto r_c) { iter(r_c, kt + decltype(r_c)::value, std::true_type{}); });
            for (; kt + 6 < nk; kt += 6) static_for<0, 6>([&](auto r_c) { iter(r_c, kt + decltype(r_c)::value, chk); });
            static_for<0, 5>([&](auto r_c) {   // the last nk - 1 - kt < 6 iterations (kt = 0 mod 6)
                if (kt + decltype(r_c)::value + 1 < nk) iter(r_c, kt + decltype(r_c)::value, chk);
            });
            const int last = nk - 1;
            const uint16_t* al = sm.ring.a[(last >> 1) % STAGES];
            const uint16_t* bl = sm.ring.b[last % STAGES];
            phase(nb_c, zero, [&](auto) {}, f0, f1, al, 4 * (last & 1) + 2, bl, 1);
            mma<MI, NJ, NB>(f1, acc);
        };
        // the hint is a compile-time choice: a branch around each load inside the pinned
        // schedule measured 8 % slower
        if (nk > 0) {
            if (b_stream) with_nb<MI>(nb, [&](auto nb_c) { run(nb_c, std::true_type{}); });
            else with_nb<MI>(nb, [&](auto nb_c) { run(nb_c, std::false_type{}); });
        }
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

// tile shape: (rows, waves along rows, ring slots, waves).  256 x 256 with four waves was the
// fastest shape (64 / 128 / 256 rows, 1 / 2 / 4 row waves, 3-7 single-slice slots, 4 or 8
// waves, timed with an earlier ring of one k slice per slot) both on groups of ~1000 rows,
// where the MFMA bounds it, and on Zipf-skewed groups of ~128 rows, where the weight stream
// does: blocks past a group's last row are skipped, so tall tiles cost short groups
// little, while they halve the B fragment reads per flop.  (Eight waves, two per SIMD with
// the accumulators in VGPRs, ran 5 % slower on the first and 25 % on the second.)  The
// three A-pair and three B slots take 144 KiB of the 160 KiB of LDS.
#define GG_TILE 256, 2, 3, 4

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
    if (p.tile_queue && launch_clear_queues(p.tile_queue, s) != hipSuccess) return;   // reported by the caller
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
