// ragged_k_bf16.hip -- bf16 contracting ragged dot (the weight-gradient case) on gfx950,
// vectorised path (16-byte aligned operands and output, k and n multiples of 8):
//   out[h] = lhs[rows of h, :]^T . dout[rows of h, :]    -> out [g, k, n]
// ragged_k.hip holds the general kernel.
//
// "Group-GEMM in XLA: Making Mixture-of-Experts Fast and Memory-Efficient" (AMD ROCm blog),
// Part 3 "Contracting": the group index is an output dimension, so (group, k-tile,
// n-tile) triples are the parallel axis, and each group reduces only over its own slice
// [start, end) of the contracted row axis, read from the prefix table.
//
// The non-contracting ring kernel's machine (ragged_m_bf16.hip): a 256 x 256 output tile
// per workgroup, 4 waves of 128 x 128 (4 x 4 blocks of v_mfma_f32_32x32x16_bf16), a 4-slot
// LDS ring of 32-row slices filled by direct-to-LDS loads, two pinned half-slice phases.
// Both operands have the contracted rows as their slow axis, so both slices are
// [32 rows][256 columns] in the layout of the non-contracting kernel's weight slice, and
// both are read with ds_read_b64_tr_b16 into row-consecutive fragments.  The ring loads'
// buffer descriptors cover only the group's rows (one 32-row slice at a time when lhs or dout
// spans 2 GiB or more, so a group of any size stays within 32-bit offsets), and the last
// slice's rows past the group read as zeros.  An empty group still owns its tiles: they store exact zeros.
// Order: groups longest first (even rounds for the persistent walk), and within a group
// 4 x 8 (k-tile, n-tile) super-tiles, so the 32 tiles running on one XCD share operand
// slices in L2.
#include "common.hpp"
#include "launch.hpp"
#include "ring.hpp"

namespace gg {
namespace kr {
using namespace ring;

constexpr int BM = 256, BN = 256, BR = 32, NT = 256, STAGES = 4;   // BM along k (output rows), BN along n
constexpr int MI = 4, NJ = 4, WCOLS = 128;
constexpr int SLICE = BR * 256;          // elements of one operand slice: 16 KiB
constexpr int PER = 8;                   // ring loads per thread per slice: 4 lhs + 4 dout
constexpr int LPT_MAX_G = 256;           // longest-first order up to this many groups (O(g^2) ranking)
constexpr int SJ = 8;                    // n-tiles per super-tile column
static_assert(PER * (STAGES - 1) <= 63, "vmcnt range");

struct Smem {
    struct {
        uint16_t a[STAGES][SLICE];
        uint16_t b[STAGES][SLICE];
    } ring;
    Tables tab;
    int order[LPT_MAX_G];
};

// slice [32 rows][256 columns], 512-byte rows: 16-byte chunks XOR'ed in 64-byte units by a
// 3-bit function of the row, so the rows one transpose read touches land in distinct banks
__device__ inline int swz(int kr) { return ((kr & 3) | (((kr >> 3) & 1) << 2)) << 2; }
__device__ inline int off(int kr, int nn) { return kr * 256 + (((nn >> 3) ^ swz(kr)) << 3) + (nn & 7); }

struct Frags { bf16x8 a[MI]; bf16x8 b[NJ]; };

// fragment of 16-row step s for columns c0 + 32 j + (lane & 31) of a slice (rows 8 (lane / 32)
// .. + 7 of the step), from two 8-byte transpose reads
__device__ inline bf16x8 frag(const uint16_t* sl, int s, int c0, int j) {
    const int l = threadIdx.x & 63, q = l >> 4, rr = (l >> 2) & 3, c = l & 3;
    const int kr0 = 16 * s + 8 * (q >> 1) + rr;
    const int nn = c0 + 32 * j + 16 * (q & 1) + 4 * c;
    const i16x4 lo = lds_read_tr16(sl + off(kr0, nn));
    const i16x4 hi = lds_read_tr16(sl + off(kr0 + 4, nn));
    typedef short i16x8 __attribute__((ext_vector_type(8)));
    const i16x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    return __builtin_bit_cast(bf16x8, v);
}
// read number R of a step, in the order the MFMAs (column block major) first need them:
// dout block 0, lhs blocks 0 .. NB - 1, then dout blocks 1 .. NJ - 1
template <int NB, int R>
__device__ inline void read_one(Frags& f, const uint16_t* a, const uint16_t* b, int s, int r0w, int c0w) {
    if constexpr (R >= 1 && R <= NB) f.a[R - 1] = frag(a, s, r0w, R - 1);
    else f.b[R == 0 ? 0 : R - NB] = frag(b, s, c0w, R == 0 ? 0 : R - NB);
}

template <bool EPI, typename OutT, bool REBASE>
__global__ __launch_bounds__(NT, 1) void kernel(KParams p) {
    __shared__ Smem sm;
    const int t = threadIdx.x, l = t & 63, wave = t >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int r0w = 128 * wm, c0w = 128 * wn;   // wave's sub-tile: output rows (k) r0w.., columns (n) c0w..
    const int nti = cdiv(p.k, BM), ntj = cdiv(p.n, BN);
    const int per = nti * ntj;
    const int total = p.g * per;
    const bool lpt = p.uniform_rows == 0 && p.g <= LPT_MAX_G;
    if (p.uniform_rows == 0) {
        int gemm_tiles, covered;
        build_tables<NT>(p.group_sizes, p.g, p.m, 1, 0, sm.tab, &gemm_tiles, &covered);
        if (blockIdx.x == 0 && t == 0 && p.status) *p.status = sm.tab.flags;
        if (lpt) {   // rank of every group by (size desc, index asc)
            for (int h = t; h < p.g; h += NT) {
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
    const uint32_t k2 = (uint32_t)p.k * 2u, n2 = (uint32_t)p.n * 2u;
    constexpr int osz = sizeof(OutT);

    // ring-load roles: slice [32 rows][256 cols] in 1 KiB blocks of 2 rows; wave w fills
    // blocks 4 w + u; lane l writes physical chunk l % 32 of row 2 (4 w + u) + l / 32, which
    // holds logical chunk (l & 31) ^ swz(row)
    const int wave_u = __builtin_amdgcn_readfirstlane(wave);
    int ch8[4];
    uint32_t a_lane[4], b_lane[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const int row = 2 * (4 * wave + u) + (l >> 5);
        ch8[u] = 8 * ((l & 31) ^ swz(row));
        a_lane[u] = (uint32_t)(l >> 5) * k2 + (uint32_t)ch8[u] * 2u;
        b_lane[u] = (uint32_t)(l >> 5) * n2 + (uint32_t)ch8[u] * 2u;
    }
    const uint32_t lds_a = lds_u32(&sm.ring.a[0][0]) + (uint32_t)(4 * wave_u) * 1024u;
    const uint32_t lds_b = lds_u32(&sm.ring.b[0][0]) + (uint32_t)(4 * wave_u) * 1024u;

    for (int tile = xcd_virtual_id(blockIdx.x, gridDim.x); tile < total; tile += gridDim.x) {
        const int pg = tile / per;
        int local = tile - pg * per;
        const int grp = lpt ? sm.order[pg] : pg;
        int row_base, size;
        if (p.uniform_rows > 0) { row_base = grp * p.uniform_rows; size = p.uniform_rows; }
        else { row_base = sm.tab.row_off[grp]; size = sm.tab.row_off[grp + 1] - row_base; }
        // (k-tile, n-tile) in super-tiles of SJ n-tiles: consecutive tiles share lhs columns
        // within a super-tile row and dout columns down it
        const int full_sc = ntj / SJ;
        int it, jt;
        if (local < full_sc * SJ * nti) {
            const int sc = local / (SJ * nti), lo = local - sc * SJ * nti;
            it = lo / SJ; jt = sc * SJ + lo % SJ;
        } else {
            const int wl = ntj - full_sc * SJ, lo = local - full_sc * SJ * nti;
            it = lo / wl; jt = full_sc * SJ + lo % wl;
        }
        const int i0 = it * BM, j0 = jt * BN;
        const int rows_valid = min(BM, p.k - i0);   // output rows of the tile
        const int nb = max(0, min(MI, cdiv(rows_valid - r0w, 32)));
        const int nk = cdiv(size, BR);

        // ring load d (lhs blocks 0-3, dout blocks 4-7) of row slice `stage`.  Each load's buffer
        // descriptor starts at the slice's first row and covers only its rows of the group, so
        // the 32-bit offsets span one slice whatever the group's size, and rows past the group
        // (and slices past its end) read as zeros into the slot no one reads.
        // Buffer descriptors of the ring loads: with REBASE each covers one 32-row slice (its
        // rows of the group), so a group of any size stays within 32-bit offsets; otherwise one
        // pair covers the group's rows (every row of lhs / dout spans less than 2 GiB).  Either
        // way rows past the group, and slices past its end, read as zeros into a slot no one reads.
        struct SliceRsrc { i32x4 a, b; };
        const SliceRsrc group_rs = REBASE ? SliceRsrc{} : SliceRsrc{
            make_rsrc_v((const uint16_t*)p.lhs + (size_t)row_base * p.k, (uint32_t)size * k2),
            make_rsrc_v((const uint16_t*)p.dout + (size_t)row_base * p.n, (uint32_t)size * n2)};
        auto slice_rsrc = [&](int stage) {
            if constexpr (!REBASE) return group_rs;
            const bool live = stage < nk;
            const int srows = live ? min(BR, size - stage * BR) : 0;
            const size_t row0 = (size_t)row_base + (size_t)(live ? stage * BR : 0);
            return SliceRsrc{make_rsrc_v((const uint16_t*)p.lhs + row0 * p.k, (uint32_t)srows * k2),
                             make_rsrc_v((const uint16_t*)p.dout + row0 * p.n, (uint32_t)srows * n2)};
        };
        // ring load d (lhs blocks 0-3, dout blocks 4-7) of row slice `stage`
        // FULL: the slice lies inside the group (stage < nk), and the loads skip the column checks
        // too: columns past k or n then read the next row's values (or zeros past the
        // descriptor), which only reach output rows or columns that are never stored
        auto dma_one = [&](auto d_c, int stage, const SliceRsrc& r, auto full_c) {
            constexpr int d = decltype(d_c)::value;
            constexpr bool FULL = decltype(full_c)::value;
            constexpr int u = d & 3;
            const int slot = stage % STAGES;
            const bool live = stage < nk;
            // row within the descriptor
            // (the slice offset goes through readfirstlane, opaque to loop strength reduction, so
            // the lane offsets stay one scalar add per load instead of vector induction
            // variables; with those the unrolled loop below spilled registers and ran 9 % slower)
            const uint32_t rrow = (uint32_t)((REBASE ? 0 : __builtin_amdgcn_readfirstlane(stage * BR)) + 2 * (4 * wave_u + u));
            if constexpr (d < 4) {
                const bool ok = live && ch8[u] < p.k - i0;
                load_lds16(r.a, lds_a + (uint32_t)slot * (SLICE * 2) + u * 1024u, FULL || ok ? a_lane[u] + rrow * k2 + (uint32_t)i0 * 2u : kOOB);
            } else {
                const bool ok = live && ch8[u] < p.n - j0;
                load_lds16(r.b, lds_b + (uint32_t)slot * (SLICE * 2) + u * 1024u, FULL || ok ? b_lane[u] + rrow * n2 + (uint32_t)j0 * 2u : kOOB);
            }
        };

        f32x16 acc[MI][NJ];
#pragma unroll
        for (int i = 0; i < MI; ++i)
#pragma unroll
            for (int j = 0; j < NJ; ++j)
#pragma unroll
                for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

        // one half slice: MFMAs on `cur`, each followed by at most one ring load and one
        // fragment read of `nxt` (step s of slot a / b), in a pinned order
        auto phase = [&](auto nb_c, auto half_c, Frags& cur, Frags& nxt, const uint16_t* a, const uint16_t* b, int s,
                         int stage, auto full_c) {
            constexpr int NB = decltype(nb_c)::value;
            constexpr int HALF = decltype(half_c)::value;   // ring loads: 0 none, 1 the first PER / 2, 2 the rest
            constexpr int NM = NB * NJ, NR = NB > 0 ? NB + NJ : 0, ND = HALF ? PER / 2 : 0;
            constexpr int SP = ND > 0 && NM >= ND ? NM / (ND > 0 ? ND : 1) : 1;   // MFMAs between two ring loads
            constexpr int LD = ND > 0 ? (ND - 1) * SP + 1 : 0;
            constexpr int NOPS = NM > NR ? (NM > LD ? NM : LD) : (NR > LD ? NR : LD);
            const SliceRsrc rs = slice_rsrc(stage);
            static_for<0, NOPS>([&](auto o_c) {
                constexpr int o = decltype(o_c)::value;
                if constexpr (o < NM) {
                    constexpr int i = o % (NB > 0 ? NB : 1), j = o / (NB > 0 ? NB : 1);
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(cur.b[j], cur.a[i], acc[i][j], 0, 0, 0);
                }
                if constexpr (ND > 0 && o % SP == 0 && o / SP < ND)
                    dma_one(std::integral_constant<int, (HALF - 1) * (PER / 2) + o / SP>{}, stage, rs, full_c);
                if constexpr (o < NR) read_one<NB, o>(nxt, a, b, s, r0w, c0w);
                __builtin_amdgcn_sched_barrier(0);
            });
        };
        static_assert(STAGES == 4 && PER % 2 == 0, "the split ring loads assume a 4-slot ring");
        auto run = [&](auto nb_c) {
            constexpr int NB = decltype(nb_c)::value;
            Frags f0, f1;
            // slice s is loaded in two halves, spread over the MFMAs: the first in the second
            // half slice of iteration s - 4 (its slot is free once that iteration's barrier has
            // passed), the rest in the first half slice of iteration s - 3; either way
            // PER * (STAGES - 2) loads follow slice kt + 1's last one when iteration kt waits
            static_for<0, STAGES - 1>([&](auto st_c) {
                const SliceRsrc rs = slice_rsrc(decltype(st_c)::value);
                static_for<0, PER>([&](auto d_c) { dma_one(d_c, decltype(st_c)::value, rs, std::false_type{}); });
            });
            const SliceRsrc rs3 = slice_rsrc(STAGES - 1);
            static_for<0, PER / 2>([&](auto d_c) { dma_one(d_c, STAGES - 1, rs3, std::false_type{}); });
            wait_vm<PER * (STAGES - 2) + PER / 2>();   // slice 0 in LDS
            lds_barrier();
            if constexpr (NB > 0) static_for<0, NB + NJ>([&](auto r_c) { read_one<NB, decltype(r_c)::value>(f0, sm.ring.a[0], sm.ring.b[0], 0, r0w, c0w); });
            __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0): exact wait counts at the loop head
            auto iter = [&](int kt, auto full_c) {
                const int slot = kt % STAGES, ns = (kt + 1) % STAGES;
                phase(nb_c, std::integral_constant<int, 2>{}, f0, f1, sm.ring.a[slot], sm.ring.b[slot], 1, kt + STAGES - 1, full_c);
                wait_vm<PER * (STAGES - 2)>();   // slice kt + 1 in LDS
                lds_barrier();
                phase(nb_c, std::integral_constant<int, 1>{}, f1, f0, sm.ring.a[ns], sm.ring.b[ns], 0, kt + STAGES, full_c);
            };
            // Iterations whose ring loads all fall inside the group skip the range checks (one
            // select and its condition per load: 165 instead of 184 instructions per iteration,
            // 2 % faster), and run unrolled by four, the ring's slot count, so every slot index and
            // LDS offset is a constant (3.6 instead of 5.2 instructions per MFMA, 3 % faster; both
            // bit-identical).  The last iterations, up to six, take the slots at run time and keep
            // the checks.
            auto iter_c = [&](auto r_c, int kt) {
                constexpr int R = decltype(r_c)::value, slot = R % STAGES, ns = (R + 1) % STAGES;
                phase(nb_c, std::integral_constant<int, 2>{}, f0, f1, sm.ring.a[slot], sm.ring.b[slot], 1, kt + STAGES - 1, std::true_type{});
                wait_vm<PER * (STAGES - 2)>();
                lds_barrier();
                phase(nb_c, std::integral_constant<int, 1>{}, f1, f0, sm.ring.a[ns], sm.ring.b[ns], 0, kt + STAGES, std::true_type{});
            };
            int kt = 0;
            for (; kt + 3 + STAGES < nk; kt += 4) static_for<0, 4>([&](auto r_c) { iter_c(r_c, kt + decltype(r_c)::value); });
            for (; kt + 1 < nk; ++kt) iter(kt, std::false_type{});
            const int last = (nk - 1) % STAGES;
            phase(nb_c, std::integral_constant<int, 0>{}, f0, f1, sm.ring.a[last], sm.ring.b[last], 1, 0, std::false_type{});
            static_for<0, NB * NJ>([&](auto o_c) {   // the last half slice's MFMAs
                constexpr int o = decltype(o_c)::value, i = o % (NB > 0 ? NB : 1), j = o / (NB > 0 ? NB : 1);
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f1.b[j], f1.a[i], acc[i][j], 0, 0, 0);
            });
        };
        if (nk > 0) with_nb<MI>(nb, run);
        // Every ring load has landed (the zero-fill loads of slices past the end may still be
        // in flight, and the epilogue strips overlap their slots) and every wave is done
        // reading the ring before it is reused.
        wait_vm<0>();
        lds_barrier();

        const rsrc_t ro = make_rsrc((const char*)p.out + ((size_t)grp * p.k + i0) * p.n * osz, (uint32_t)(rows_valid * p.n * osz));
        static_assert(4 * 32 * (WCOLS + 4) * 4 <= (int)sizeof(sm.ring), "epilogue strips fit the ring");
        const EpiTile ep{nullptr, p.alpha, p.beta};
        store_acc<MI, NJ, WCOLS, OutT, EPI, true>(acc, reinterpret_cast<float*>(&sm.ring) + wave * 32 * (WCOLS + 4), ro, p.n, j0,
                                                  r0w, c0w, ep);
        lds_barrier();   // strips read before the next tile's ring loads land there
    }
    wait_vm<0>();   // no ring load may still be writing LDS when the workgroup ends
}

}  // namespace kr

bool ragged_k_bf16_fast_ok(const KParams& p) {
    // 32-bit buffer offsets over one 32-row slice of lhs / dout and one 256-row output tile
    const uint64_t a = 33ull * (uint64_t)p.k * 2u;
    const uint64_t b = 33ull * (uint64_t)p.n * 2u;
    const uint64_t o = 256ull * (uint64_t)p.n * 4u;
    return p.k % 8 == 0 && p.n % 8 == 0 && a < (1ull << 31) && b < (1ull << 31) && o < (1ull << 31);
}

template <bool REBASE>
static void launch_kr(const KParams& p, int grid, hipStream_t s) {
    if (p.epi) {
        if (p.out_f32) hipLaunchKernelGGL((kr::kernel<true, float, REBASE>), dim3(grid), dim3(kr::NT), 0, s, p);
        else hipLaunchKernelGGL((kr::kernel<true, uint16_t, REBASE>), dim3(grid), dim3(kr::NT), 0, s, p);
    } else {
        if (p.out_f32) hipLaunchKernelGGL((kr::kernel<false, float, REBASE>), dim3(grid), dim3(kr::NT), 0, s, p);
        else hipLaunchKernelGGL((kr::kernel<false, uint16_t, REBASE>), dim3(grid), dim3(kr::NT), 0, s, p);
    }
}

hipError_t launch_ragged_k_bf16_fast(const KParams& p, int grid, hipStream_t s) {
    // one descriptor per group while all of lhs and dout (a group may own every row) spans
    // less than 2 GiB; per-slice descriptors beyond that
    const uint64_t a = (uint64_t)p.m * (uint64_t)p.k * 2u + 64ull * p.k * 2u;
    const uint64_t b = (uint64_t)p.m * (uint64_t)p.n * 2u + 64ull * p.n * 2u;
    if (a < (1ull << 31) && b < (1ull << 31)) launch_kr<false>(p, grid, s);
    else launch_kr<true>(p, grid, s);
    return hipGetLastError();
}

}  // namespace gg
