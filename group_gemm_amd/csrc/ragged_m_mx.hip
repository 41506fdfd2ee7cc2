// ragged_m_mx.hip -- the MXFP8 non-contracting ragged dot on gfx950, vectorised path:
// OCP e4m3 operands with one E8M0 scale per 32 elements along k (lhs_scale [m, k/32],
// rhs_scale [g, k/32, n]), fp32 accumulation, bf16 or fp32 output.  Requires k % 128 == 0,
// n % 16 == 0 and 16-byte aligned operands; ragged_m.hip holds the general kernel.
//
// "Group-GEMM in XLA: Making Mixture-of-Experts Fast and Memory-Efficient" (AMD ROCm blog),
// Part 3 "Non-Contracting (the MoE Case)", with the block-scaled product of the MX formats
// (each 32-element k block of a row and of a column carries its own power-of-two scale).
//
// Same machine as the bf16 ring kernel (ragged_m_bf16.hip): a 256 x 256 tile per
// workgroup, 4 waves in a 2 x 2 grid, each a 128 x 128 sub-tile of 4 x 4 blocks of
// v_mfma_scale_f32_32x32x64_f8f6f4 (fp32 accumulators in AGPRs); k is consumed in 64-byte
// slices streamed through a 4-slot LDS ring by direct-to-LDS buffer loads.  A slot holds
// A [256 rows][64 k] (16 KiB), B [64 k][256 n] (16 KiB), the rows' E8M0 scales (the
// aligned 4-byte group holding the slice's two k blocks, per row) and the slice's two
// k-block rows of column scales (twice: one copy per wave pair), all loaded by the ring,
// so every wait count is a constant.  One slice is two pinned phases:
//   phase 1: MFMAs of column blocks 0, 1; ring loads of slice kt + 3; reads of this slot's
//            B blocks 2, 3 and their scales;
//   slice kt + 1 complete (own loads, then barrier);
//   phase 2: MFMAs of column blocks 2, 3; reads of slot kt + 1's A blocks (each right after
//            the block's last MFMA, into the same registers), B blocks 0, 1 and scales.
// The MFMA takes the column operand first (and its scale), so every lane holds 4
// consecutive output columns; the epilogue is the bf16 kernel's.
#include "common.hpp"
#include "launch.hpp"
#include "ring.hpp"

namespace gg {
namespace mx {
using namespace ring;

constexpr int BM = 256, BN = 256, BK = 64, NT = 256, STAGES = 4;
constexpr int MI = 4, NJ = 4, WCOLS = 128;
constexpr int A_BYTES = BM * BK, B_BYTES = BK * BN;
constexpr int AS_BYTES = BM * 4;        // per row: the 4 scale bytes of k blocks 4c .. 4c + 3
constexpr int BS_BYTES = 2 * 2 * BN;    // 2 copies x the slice's 2 k-block rows of column scales
constexpr int PER = 4 + 4 + 1 + 1;      // ring loads per thread per slice: A, B, A scales, B scales
static_assert(PER * (STAGES - 1) <= 63, "vmcnt range");

struct alignas(16) Slot {
    uint8_t a[A_BYTES];
    uint8_t b[B_BYTES];
    uint8_t as[AS_BYTES];
    uint8_t bs[BS_BYTES];
};
// Row scales in blocks of 8 k slices (AS8, when k % 512 == 0 and the scales are 16-byte
// aligned): the 16 bytes of a row's 16 k blocks come in one 16-byte load per row, issued
// with the block's first slice into one of two buffers, instead of 4 bytes per row with
// every slice.  A load straight into LDS costs about the same per cache line touched
// whatever it moves of the line (measured on gfx950: ~0.5 lines per clock per CU), and the
// per-slice form touches one line per row for 4 bytes, as many lines as the A data itself.
// The other slices issue an out-of-range load into a dummy area, so every slice still
// issues the same number of loads and every wait count stays constant.
constexpr int AS8_BYTES = BM * 16;      // one block: 16 bytes per row
struct Smem {
    Slot ring[STAGES];
    uint8_t asb[2][AS8_BYTES];           // AS8: row scales of blocks j (buffer j % 2)
    uint8_t asdummy[AS8_BYTES];          // AS8: target of the placeholder loads
    Tables tab;
};

// A slot [256 rows][64 k bytes]: 16-byte chunk XOR (row >> 2) & 3 (the bf16 kernel's [n][k]
// weight layout, byte for byte: 16 consecutive rows of one chunk cover the 64 LDS banks once).
__device__ inline int a_off(int r, int chunk) { return r * BK + ((chunk ^ ((r >> 2) & 3)) << 4); }
// B slot [64 k][256 n bytes]: 16-byte chunks XOR'ed by 2 (k & 7), so the 8 k rows one
// 8-byte transpose read gathers fall in different bank groups.
__device__ inline int b_off(int kr, int nn) { return kr * BN + ((((nn >> 4) ^ ((kr & 7) << 1))) << 4) + (nn & 15); }

struct Frags {
    i32x8 a[MI];
    i32x8 b[NJ];
    int sa[MI];
    int sb[NJ];
};

// A block i of a slot: lane l holds row r0w + 32 i + (l & 31), k bytes 16 h .. 16 h + 15 and
// 32 + 16 h .. + 15 (h = l / 32), as the 32x32x64 f8f6f4 operand layout wants
template <bool AS8>
__device__ inline void read_a(Frags& f, int i, const Slot& s, const Smem& sm, int r0w, int ks) {
    const int l = threadIdx.x & 63, h = l >> 5;
    const int r = r0w + 32 * i + (l & 31);
    const i32x4 lo = *(const i32x4*)(s.a + a_off(r, h));
    const i32x4 hi = *(const i32x4*)(s.a + a_off(r, 2 + h));
    f.a[i] = i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    // E8M0 of (row, k block 2 ks + h)
    if constexpr (AS8) f.sa[i] = sm.asb[(ks >> 3) & 1][16 * r + 2 * (ks & 7) + h];
    else f.sa[i] = s.as[4 * r + 2 * (ks & 1) + h];
}
// B block j: lane l holds column c0w + 32 j + (l & 31) for the same k bytes, gathered by
// four 8-byte transpose reads (lane j of a 16-lane group takes byte j % 8 of rows 2r + j / 8)
__device__ inline void read_b(Frags& f, int j, const Slot& s, int c0w, int cp) {
    const int l = threadIdx.x & 63, h = l >> 5, q = l >> 4;
    const int nn = c0w + 32 * j + 16 * (q & 1) + 8 * (l & 1);
    const int kb = 16 * (q >> 1) + ((l >> 1) & 7);
    const i32x2 p0 = lds_read_tr8(s.b + b_off(kb, nn));
    const i32x2 p1 = lds_read_tr8(s.b + b_off(kb + 8, nn));
    const i32x2 p2 = lds_read_tr8(s.b + b_off(kb + 32, nn));
    const i32x2 p3 = lds_read_tr8(s.b + b_off(kb + 40, nn));
    f.b[j] = i32x8{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
    f.sb[j] = s.bs[cp * 2 * BN + h * BN + c0w + 32 * j + (l & 31)];   // E8M0 of (column, k block 2 ks + h)
}

template <bool AS8, bool EPI, typename OutT>
__global__ __launch_bounds__(NT, 1) void kernel(MParams p) {
    __shared__ Smem sm;
    const int t = threadIdx.x, l = t & 63, wave = t >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int r0w = 128 * wm, c0w = 128 * wn;
    const int cp = wave >> 1;   // which copy of the column scales this wave reads
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
    const int kb = p.k >> 5;   // k blocks per row
    constexpr int osz = sizeof(OutT);

    // per-lane parts of the ring-load offsets
    const int wave_u = __builtin_amdgcn_readfirstlane(wave);
    const int a_chunk = (l & 3) ^ ((l >> 4) & 3);   // A: row 16 b + l / 4 holds chunk (l & 3) ^ ((row >> 2) & 3)
    const uint32_t a_lane = (uint32_t)(l >> 2) * (uint32_t)p.k + (uint32_t)a_chunk * 16u;
    uint32_t b_lane[4];
    int b_col[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {   // B: row 4 (4 wave + u) + l / 16 holds chunk (l & 15) ^ 2 (row & 7)
        const int kr = 4 * u + (l >> 4);   // row & 7 does not depend on the wave
        b_col[u] = 16 * ((l & 15) ^ ((kr & 7) << 1));
        b_lane[u] = (uint32_t)(l >> 4) * (uint32_t)p.n + (uint32_t)b_col[u];
    }
    const uint32_t lds0 = lds_u32(&sm.ring[0]);
    const uint32_t lds_asb = lds_u32(&sm.asb[0][0]), lds_asd = lds_u32(&sm.asdummy[0]);
    constexpr uint32_t SLOT = sizeof(Slot);
    constexpr uint32_t OFF_B = offsetof(Slot, b), OFF_AS = offsetof(Slot, as), OFF_BS = offsetof(Slot, bs);

    for (int tile = xcd_virtual_id(blockIdx.x, gridDim.x); tile < total; tile += gridDim.x) {
        if (tile >= gemm_tiles) {
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
        const int mtg = cdiv(size, BM);
        if (size <= p.n) { mt = local % mtg; nt = local / mtg; }
        else { nt = local % ntn; mt = local / ntn; }
        row0 += mt * BM;
        const int rows_valid = min(BM, size - mt * BM);
        const int col0 = nt * BN;
        const int nb = max(0, min(MI, cdiv(rows_valid - r0w, 32)));

        const i32x4 ra = make_rsrc_v((const uint8_t*)p.lhs + (size_t)row0 * p.k, (uint32_t)rows_valid * (uint32_t)p.k);
        const i32x4 rb = make_rsrc_v((const uint8_t*)p.rhs + (size_t)grp * p.k * p.n, (uint32_t)p.k * (uint32_t)p.n);
        const i32x4 rsa = make_rsrc_v(p.lhs_scale + (size_t)row0 * kb, (uint32_t)rows_valid * (uint32_t)kb);
        const i32x4 rsb = make_rsrc_v(p.rhs_scale + (size_t)grp * kb * p.n, (uint32_t)kb * (uint32_t)p.n);

        // ring load number d of k slice `stage` (A 0-3, B 4-7, row scales 8, column
        // scales 9); slices past k are zero-filled into the slot no one reads
        auto dma_one = [&](auto d_c, int stage_v, int slot_i, auto full_c) {
            constexpr int d = decltype(d_c)::value;
            // (the slice index goes through readfirstlane, opaque to loop strength reduction, so
            // the lane offsets stay one scalar add per load instead of vector induction variables,
            // which spilled registers once the loop below was unrolled)
            const int stage = __builtin_amdgcn_readfirstlane(stage_v);
            // FULL: the slice lies inside k, so the checks below always pass for A and the row
            // scales; B and column-scale loads past n (the last n-tile of a ragged n) then read
            // the next row's bytes, or zeros past the buffer, which only reach output columns that
            // are never stored
            constexpr bool FULL = decltype(full_c)::value;
            const int kk = stage * BK;
            const uint32_t slot = lds0 + (uint32_t)slot_i * SLOT;
            const bool live = stage < nk;
            if constexpr (d < 4) {
                const bool ok = live && kk + 16 * a_chunk < p.k;
                const uint32_t wpart = (uint32_t)(16 * (4 * wave_u + d)) * (uint32_t)p.k + (uint32_t)kk;
                load_lds16(ra, slot + (uint32_t)(4 * wave_u + d) * 1024u, FULL ? a_lane + wpart : (ok ? a_lane + wpart : kOOB));
            } else if constexpr (d < 8) {
                constexpr int u = d - 4;
                const bool ok = live && b_col[u] < p.n - col0;
                const uint32_t wpart = (uint32_t)(kk + 4 * (4 * wave_u + u)) * (uint32_t)p.n + (uint32_t)col0;
                load_lds16(rb, slot + OFF_B + (uint32_t)(4 * wave_u + u) * 1024u, FULL ? b_lane[u] + wpart : (ok ? b_lane[u] + wpart : kOOB));
            } else if constexpr (d == 8 && AS8) {
                // rows 64 wave + l: the 16 scale bytes of k blocks 16 (stage / 8) .. + 15 with
                // the block's first slice, a placeholder load with the others
                const bool real = live && (stage & 7) == 0;
                const uint32_t off = (uint32_t)(64 * wave_u + l) * (uint32_t)kb + (uint32_t)(16 * (stage >> 3));
                const uint32_t dst = (real ? lds_asb + (uint32_t)((stage >> 3) & 1) * AS8_BYTES : lds_asd) + (uint32_t)wave_u * 1024u;
                load_lds16(rsa, dst, real ? off : kOOB);
            } else if constexpr (d == 8) {
                // rows 64 wave + l: the 4 scale bytes of k blocks 4 (stage / 2) .. + 3
                const uint32_t off = (uint32_t)(64 * wave_u + l) * (uint32_t)kb + (uint32_t)(4 * (stage >> 1));
                load_lds4(rsa, slot + OFF_AS + (uint32_t)wave_u * 256u, FULL || live ? off : kOOB);
            } else {
                // k-block row 2 stage + (wave & 1), columns col0 + 4 l .. + 3, into copy wave / 2
                const bool ok = live && 4 * l < p.n - col0;
                const uint32_t off = (uint32_t)(2 * stage + (wave_u & 1)) * (uint32_t)p.n + (uint32_t)(col0 + 4 * l);
                load_lds4(rsb, slot + OFF_BS + (uint32_t)((wave_u >> 1) * 2 * BN + (wave_u & 1) * BN), FULL ? off : (ok ? off : kOOB));
            }
        };

        f32x16 acc[MI][NJ];
#pragma unroll
        for (int i = 0; i < MI; ++i)
#pragma unroll
            for (int j = 0; j < NJ; ++j)
#pragma unroll
                for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

        auto mfma = [&](Frags& f, int i, int j) {
            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(f.b[j], f.a[i], acc[i][j], 0, 0, 0, f.sb[j], 0,
                                                                        f.sa[i]);
        };

        auto run = [&](auto nb_c) {
            constexpr int NB = decltype(nb_c)::value;
            Frags f;
            // Slice s is loaded in two halves: ring loads 0 .. PER/2 - 1 in phase 2 of iteration
            // s - 4 (its slot, read last in phase 1 of that iteration, is free once the
            // iteration's barrier has passed), the rest in phase 1 of iteration s - 3, so the
            // loads are spread over all the slice's MFMAs.  Either way PER * (STAGES - 2)
            // loads are issued after slice kt + 1's last one by the time iteration kt waits.
            constexpr std::false_type chk{};
            static_for<0, STAGES - 1>([&](auto st_c) { static_for<0, PER>([&](auto d_c) { dma_one(d_c, decltype(st_c)::value, decltype(st_c)::value, chk); }); });
            static_for<0, PER / 2>([&](auto d_c) { dma_one(d_c, STAGES - 1, STAGES - 1, chk); });
            wait_vm<PER * (STAGES - 2) + PER / 2>();   // slice 0 in LDS
            lds_barrier();
            if constexpr (NB > 0) {
                static_for<0, NB>([&](auto i_c) { read_a<AS8>(f, decltype(i_c)::value, sm.ring[0], sm, r0w, 0); });
                read_b(f, 0, sm.ring[0], c0w, cp);
                read_b(f, 1, sm.ring[0], c0w, cp);
            }
            // Nothing of the prologue's reads stays pending into the loop: the compiler's wait
            // counts at the loop head merge both ways in, and the prologue's order (reads
            // just issued) would otherwise make every iteration wait for all reads in flight.
            __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0)
            // phase 1 of slice kt: MFMAs (i, 0..1), the second half of the ring loads of slice
            // `stage` (when DMA), reads of B blocks 2, 3 of slot kt
            auto phase1 = [&](auto dma_c, const Slot& s, int stage, int sslot, auto full_c) {
                constexpr bool DMA = decltype(dma_c)::value;
                constexpr int NM = 2 * NB, ND = DMA ? PER - PER / 2 : 0, NR = NB > 0 ? 2 : 0;
                constexpr int NOPS = ND + NR;
                constexpr int PERM = NM > 0 ? (NOPS + NM - 1) / (NM > 0 ? NM : 1) : NOPS;   // ops after each MFMA
                constexpr int NSLOT = NM > 0 ? NM : 1;
                static_for<0, NSLOT>([&](auto m_c) {
                    constexpr int m = decltype(m_c)::value;
                    if constexpr (NM > 0) mfma(f, m >> 1, m & 1);
                    static_for<m * PERM, (m + 1) * PERM < NOPS ? (m + 1) * PERM : NOPS>([&](auto o_c) {
                        constexpr int o = decltype(o_c)::value;
                        // the two B reads go early (ops RB2, RB3), so phase 2 never waits on them;
                        // the rest are ring loads in order
                        constexpr int RB2 = ND > 0 ? 1 : 0, RB3 = ND > 0 ? 3 : 1;
                        if constexpr (NR > 0 && o == RB2) read_b(f, 2, s, c0w, cp);
                        else if constexpr (NR > 0 && o == RB3) read_b(f, 3, s, c0w, cp);
                        else {
                            constexpr int d = o - (NR > 0 ? (o > RB3 ? 2 : (o > RB2 ? 1 : 0)) : 0);
                            static_assert(d >= 0 && d < ND, "op index");
                            dma_one(std::integral_constant<int, PER / 2 + d>{}, stage, sslot, full_c);
                        }
                    });
                    __builtin_amdgcn_sched_barrier(0);
                });
            };
            // phase 2 of slice kt: MFMAs (i, 2..3), reads of slot kt + 1 (A block i after its
            // last MFMA, B blocks 0, 1 spread over the first MFMAs) when NEXT, and the first half
            // of the ring loads of slice `stage`, spread over the MFMAs
            auto phase2 = [&](auto next_c, const Slot& s, int ks1, int stage, int sslot, auto full_c) {
                constexpr bool NEXT = decltype(next_c)::value;
                constexpr int NM = 2 * NB, ND = NEXT ? PER / 2 : 0;
                static_for<0, NM>([&](auto m_c) {
                    constexpr int m = decltype(m_c)::value;
                    mfma(f, m >> 1, 2 + (m & 1));
                    if constexpr (NEXT) {
                        if constexpr (m == 0) read_b(f, 0, s, c0w, cp);
                        if constexpr (m == 2 || (NB == 1 && m == 1)) read_b(f, 1, s, c0w, cp);
                        if constexpr (m & 1) read_a<AS8>(f, m >> 1, s, sm, r0w, ks1);
                        // ring load q after MFMA q * NM / ND (several after the last when NM < ND)
                        static_for<0, ND>([&](auto q_c) {
                            constexpr int q = decltype(q_c)::value;
                            constexpr int at = q * NM / ND;
                            if constexpr (at == m) dma_one(q_c, stage, sslot, full_c);
                        });
                    }
                    __builtin_amdgcn_sched_barrier(0);
                });
                if constexpr (NM == 0 && NEXT) static_for<0, ND>([&](auto q_c) { dma_one(q_c, stage, sslot, full_c); });
            };
            auto iter = [&](int kt, auto full_c) {
                phase1(std::true_type{}, sm.ring[kt % STAGES], kt + STAGES - 1, (kt + STAGES - 1) % STAGES, full_c);
                wait_vm<PER * (STAGES - 2)>();   // slice kt + 1 in LDS
                lds_barrier();
                phase2(std::true_type{}, sm.ring[(kt + 1) % STAGES], kt + 1, kt + STAGES, kt % STAGES, full_c);
            };
            auto iter_c = [&](auto r_c, int kt) {
                constexpr int R = decltype(r_c)::value;
                phase1(std::true_type{}, sm.ring[R % STAGES], kt + STAGES - 1, (R + STAGES - 1) % STAGES, std::true_type{});
                wait_vm<PER * (STAGES - 2)>();
                lds_barrier();
                phase2(std::true_type{}, sm.ring[(R + 1) % STAGES], kt + 1, kt + STAGES, R % STAGES, std::true_type{});
            };
            int kt = 0;
            // Iterations whose ring loads all fall inside k skip the range checks (one select and
            // its condition per load: 175 instead of 190 instructions per slice; 2-3 % faster),
            // and run unrolled by four, the ring's slot count, so every slot index and LDS offset
            // is a constant (128 instead of 175 instructions per slice, 1.4 % faster; both
            // bit-identical).  The last iterations take the slots at run time, and the last three
            // keep the checks.
            for (; kt + 3 + STAGES < nk; kt += 4) static_for<0, 4>([&](auto r_c) { iter_c(r_c, kt + decltype(r_c)::value); });
            for (; kt + STAGES < nk; ++kt) iter(kt, std::true_type{});
            for (; kt + 1 < nk; ++kt) iter(kt, chk);
            phase1(std::false_type{}, sm.ring[(nk - 1) % STAGES], 0, 0, chk);
            phase2(std::false_type{}, sm.ring[0], 0, 0, 0, chk);
        };
        if (nk > 0) with_nb<MI>(nb, run);
        // Every ring load has landed (the zero-fill loads of slices past the end may still be
        // in flight, and the epilogue strips overlap their slots) and every wave is done
        // reading the ring before it is reused.
        wait_vm<0>();
        lds_barrier();

        const rsrc_t ro = make_rsrc((const char*)p.out + (size_t)row0 * p.n * osz, (uint32_t)(rows_valid * p.n * osz));
        static_assert(4 * 32 * (WCOLS + 4) * 4 <= (int)sizeof(sm.ring), "epilogue strips fit the ring");
        const EpiTile ep{p.bias ? p.bias + (size_t)grp * p.bias_stride : nullptr, p.alpha, p.beta};
        store_acc<MI, NJ, WCOLS, OutT, EPI>(acc, reinterpret_cast<float*>(&sm.ring[0]) + wave * 32 * (WCOLS + 4), ro, p.n, col0,
                                            r0w, c0w, ep);
        if constexpr (osz == 2 || EPI) lds_barrier();   // strips read before the next tile's ring loads land there
    }
    wait_vm<0>();   // no ring load may still be writing LDS when the workgroup ends
}

}  // namespace mx

// row scales in blocks of 8 k slices: 16-byte loads of 16-byte aligned rows
static bool as8_ok(const MParams& p) { return p.k % 512 == 0 && ((uintptr_t)p.lhs_scale & 15) == 0; }

bool ragged_m_mx_fast_ok(const MParams& p) {
    // 16-byte ring loads of A and B, 4-byte loads of both scale arrays; 32-bit offsets
    const uint64_t w = (uint64_t)p.k * (uint64_t)p.n;
    const uint64_t a = 256ull * (uint64_t)p.k;
    const uint64_t o = 256ull * (uint64_t)p.n * 4u;
    return p.k % 128 == 0 && p.n % 16 == 0 && w + 64ull * p.n < (1ull << 31) && a < (1ull << 31) && o < (1ull << 31);
}

template <bool AS8>
static void launch_mx(const MParams& p, int grid, hipStream_t s) {
    if (p.epi) {
        if (p.out_f32) hipLaunchKernelGGL((mx::kernel<AS8, true, float>), dim3(grid), dim3(mx::NT), 0, s, p);
        else hipLaunchKernelGGL((mx::kernel<AS8, true, uint16_t>), dim3(grid), dim3(mx::NT), 0, s, p);
    } else {
        if (p.out_f32) hipLaunchKernelGGL((mx::kernel<AS8, false, float>), dim3(grid), dim3(mx::NT), 0, s, p);
        else hipLaunchKernelGGL((mx::kernel<AS8, false, uint16_t>), dim3(grid), dim3(mx::NT), 0, s, p);
    }
}

hipError_t launch_ragged_m_mx_fast(const MParams& p, int grid, hipStream_t s) {
    if (as8_ok(p)) launch_mx<true>(p, grid, s);
    else launch_mx<false>(p, grid, s);
    return hipGetLastError();
}

}  // namespace gg
