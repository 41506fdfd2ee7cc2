// ragged_m_gated.hip -- the fused gate/up projection of an MoE expert block on gfx950:
//   out[r, :] = act(lhs[r, :] . w0[h] + b0[h]) * (lhs[r, :] . w1[h] + b1[h])
// for every row r of group h (rows past sum(group_sizes) are 0); bf16 operands, fp32
// accumulation, bf16 or fp32 output, act = SiLU or tanh-GELU.
//
// "Group-GEMM in XLA: Making Mixture-of-Experts Fast and Memory-Efficient" (AMD ROCm blog):
// Part 1's dense formulation computes the gate and up projections of the same inputs with
// two weight tensors and multiplies activation(gate) by up; Part 4's MaxText layer body
// calls the grouped up-projection with both weights and their biases, then applies the FFN
// activation, writing one intermediate.  Fusing both products and the activation into one
// kernel reads each lhs row once for both projections and writes only the [m, n]
// intermediate instead of two [m, n] products.
//
// The bf16 ring kernel's machine (ragged_m_bf16.hip) with a 256 x 128 output tile: each
// ring slot holds A [256 rows][32 k] and the two weight slices w0, w1 [32 k][128 n]
// (16 KiB together, so the ring, its loads and the 16 MFMAs per wave and half slice are
// those of the plain kernel).  4 waves in a 2 x 2 grid; a wave owns 128 rows x 64 output
// columns and keeps both accumulators (gate blocks j = 0, 1 and up blocks j = 2, 3:
// 16 blocks of 32 x 32, 256 AGPRs).  The epilogue writes both to the wave's LDS strip
// straight from AGPRs, reads 8 gate and 8 up columns back per lane, applies the
// activation and stores 16 bytes of output per lane.
#include "common.hpp"
#include "launch.hpp"
#include "ring.hpp"

namespace gg {
namespace mg {
using namespace ring;

constexpr int BM = 256, ON = 128, BK = 32, NT = 256, STAGES = 4;
constexpr int MI = 4, NJ = 4, WCOLS = 128;   // strip width: 64 gate + 64 up columns
constexpr int ASLICE = BM * BK;               // elements: 16 KiB
constexpr int WSLICE = BK * ON;               // elements of one weight sub-slice: 8 KiB
constexpr int PER = 4 + 4;                    // ring loads per thread per slice: A, w0 + w1
static_assert(PER * (STAGES - 1) <= 63, "vmcnt range");

struct Smem {
    struct {
        uint16_t a[STAGES][ASLICE];
        uint16_t w[STAGES][2][WSLICE];
    } ring;
    Tables tab;
};

// A slice [256 rows][32 k], 64-byte rows: 16-byte chunk XOR (row >> 2) & 3 (the plain kernel's
// [n][k] weight layout: 16 consecutive rows of one chunk cover the 64 LDS banks once)
__device__ inline int a_off(int r, int chunk) { return r * BK + ((chunk ^ ((r >> 2) & 3)) << 3); }
// weight sub-slice [32 k][128 n], 256-byte rows: 16-byte chunk XOR 4 (k & 3), so the 4 rows
// of one transpose read land in different 64-byte quarters of the banks
__device__ inline int w_off(int kr, int nn) { return kr * ON + (((nn >> 3) ^ ((kr & 3) << 2)) << 3) + (nn & 7); }

struct Frags { bf16x8 a[MI]; bf16x8 b[NJ]; };

// fragment read R of k step s: B block 0 (gate columns c0 ..), A blocks 0 .. NB - 1, then
// B blocks 1 .. 3 (j = 1 gate, j = 2, 3 up)
template <int NB, int R>
__device__ inline void read_one(Frags& f, const uint16_t* a, const uint16_t* w, int s, int r0, int c0) {
    const int l = threadIdx.x & 63, h = l >> 5;
    if constexpr (R >= 1 && R <= NB) {
        f.a[R - 1] = *(const bf16x8*)(a + a_off(r0 + 32 * (R - 1) + (l & 31), 2 * s + h));
    } else {
        constexpr int j = R == 0 ? 0 : R - NB;
        const uint16_t* sub = w + (j >> 1) * WSLICE;   // j 0, 1: w0; j 2, 3: w1
        const int q = l >> 4, rr = (l >> 2) & 3, c = l & 3;
        const int kr0 = 16 * s + 8 * (q >> 1) + rr;
        const int nn = c0 + 32 * (j & 1) + 16 * (q & 1) + 4 * c;
        const i16x4 lo = lds_read_tr16(sub + w_off(kr0, nn));
        const i16x4 hi = lds_read_tr16(sub + w_off(kr0 + 4, nn));
        typedef short i16x8 __attribute__((ext_vector_type(8)));
        const i16x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        f.b[j] = __builtin_bit_cast(bf16x8, v);
    }
}

template <int ACT>
__device__ inline float act_fn(float x) {
    if constexpr (ACT == GG_ACT_SILU) return x / (1.f + __expf(-x));   // x * sigmoid(x)
    else return 0.5f * x * (1.f + tanhf(0.7978845608028654f * (x + 0.044715f * x * x * x)));   // tanh-GELU
}

template <int ACT, typename OutT>
__global__ __launch_bounds__(NT, 1) void kernel(GParams p) {
    __shared__ Smem sm;
    const int t = threadIdx.x, l = t & 63, wave = t >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int r0w = 128 * wm, c0w = 64 * wn;   // wave's rows, and its output columns within the tile
    const int ntn = cdiv(p.n, ON);
    int gemm_tiles, covered;
    build_tables<NT>(p.group_sizes, p.g, p.m, BM, ntn, sm.tab, &gemm_tiles, &covered);
    if (blockIdx.x == 0 && t == 0 && p.status) *p.status = sm.tab.flags;
    const int zero_mt = cdiv(p.m - covered, BM);
    const int total = gemm_tiles + zero_mt * ntn;
    const int nk = cdiv(p.k, BK);
    const uint32_t k2 = (uint32_t)p.k * 2u, n2 = (uint32_t)p.n * 2u;
    constexpr int osz = sizeof(OutT);

    // ring-load roles.  A: as the plain kernel (wave w fills 1 KiB blocks 4w + u, lane l
    // writes chunk l % 4 of row 16 b + l / 4).  Weights: 1 KiB blocks of 4 rows of one
    // sub-slice; wave w fills rows 4 (2 w + u') .. + 3 of w0 (u = u' = 0, 1) and of w1
    // (u = 2, 3, u' = u - 2); lane l writes physical chunk l % 16 of row 4 b + l / 16,
    // which holds logical chunk (l & 15) ^ 4 ((l >> 4) & 3).
    const int wave_u = __builtin_amdgcn_readfirstlane(wave);
    const int a_chunk = (l & 3) ^ ((l >> 4) & 3);
    const uint32_t a_lane = (uint32_t)(l >> 2) * k2 + (uint32_t)a_chunk * 16u;
    const int w_ch8 = 8 * ((l & 15) ^ (((l >> 4) & 3) << 2));
    const uint32_t w_lane = (uint32_t)(l >> 4) * n2 + (uint32_t)w_ch8 * 2u;
    const uint32_t lds_a = lds_u32(&sm.ring.a[0][0]) + (uint32_t)(4 * wave_u) * 1024u;
    const uint32_t lds_w = lds_u32(&sm.ring.w[0][0][0]);

    for (int tile = xcd_virtual_id(blockIdx.x, gridDim.x); tile < total; tile += gridDim.x) {
        if (tile >= gemm_tiles) {
            const int z = tile - gemm_tiles;
            zero_tile<BM, ON, NT, OutT>(p.out, covered + (z % zero_mt) * BM, p.m, (z / zero_mt) * ON, p.n);
            continue;
        }
        const int grp = find_group(sm.tab.tile_off, p.g, tile);
        const int local = tile - sm.tab.tile_off[grp];
        int row0 = sm.tab.row_off[grp];
        const int size = sm.tab.row_off[grp + 1] - row0;
        const int mtg = cdiv(size, BM);
        int mt, nt;
        if (size <= p.n) { mt = local % mtg; nt = local / mtg; }
        else { nt = local % ntn; mt = local / ntn; }
        row0 += mt * BM;
        const int rows_valid = min(BM, size - mt * BM);
        const int col0 = nt * ON;
        const int nb = max(0, min(MI, cdiv(rows_valid - r0w, 32)));

        const i32x4 ra = make_rsrc_v((const uint16_t*)p.lhs + (size_t)row0 * p.k, (uint32_t)rows_valid * k2);
        const i32x4 rw0 = make_rsrc_v((const uint16_t*)p.w0 + (size_t)grp * p.k * p.n, (uint32_t)p.k * n2);
        const i32x4 rw1 = make_rsrc_v((const uint16_t*)p.w1 + (size_t)grp * p.k * p.n, (uint32_t)p.k * n2);
        // ring load d of k slice `stage` into ring slot `slot` = stage % STAGES (a constant where
        // the caller knows it)
        auto dma_one = [&](auto d_c, int stage, int slot) {
            constexpr int d = decltype(d_c)::value;
            // (the k offset goes through readfirstlane, opaque to loop strength reduction: left
            // visible, the lane offsets become vector induction variables, one of them spilled,
            // and its reload before the main loop made the loop wait for every ring load in
            // flight once per four iterations)
            const int kk = __builtin_amdgcn_readfirstlane(stage * BK);
            if constexpr (d < 4) {
                const bool ok = kk + 8 * a_chunk < p.k;
                const uint32_t wpart = (uint32_t)(16 * (4 * wave_u + d)) * k2 + (uint32_t)kk * 2u;
                load_lds16(ra, lds_a + (uint32_t)slot * (ASLICE * 2) + d * 1024u, ok ? a_lane + wpart : kOOB);
            } else {
                constexpr int u = d - 4, mat = u >> 1, up = u & 1;
                const int row = 4 * (2 * wave_u + up);   // first of this block's 4 k rows
                // unchecked: k rows past the end lie past the descriptor's end and read zeros, and
                // columns past n read other weights, which reach only output columns never stored
                const uint32_t wpart = (uint32_t)(kk + row) * n2 + (uint32_t)col0 * 2u;
                const uint32_t dst = lds_w + (uint32_t)(slot * 2 + mat) * (WSLICE * 2) + (uint32_t)(row >> 2) * 1024u;
                load_lds16(mat ? rw1 : rw0, dst, w_lane + wpart);
            }
        };

        f32x16 acc[MI][NJ];
#pragma unroll
        for (int i = 0; i < MI; ++i)
#pragma unroll
            for (int j = 0; j < NJ; ++j)
#pragma unroll
                for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

        auto phase = [&](auto nb_c, auto dma_c, Frags& cur, Frags& nxt, const uint16_t* a, const uint16_t* w, int s,
                         int stage, int sslot) {
            constexpr int NB = decltype(nb_c)::value;
            constexpr bool DMA = decltype(dma_c)::value;
            constexpr int NM = NB * NJ, NR = NB > 0 ? NB + NJ : 0, ND = DMA ? PER : 0;
            constexpr int NOPS = NM > NR ? (NM > ND ? NM : ND) : (NR > ND ? NR : ND);
            static_for<0, NOPS>([&](auto o_c) {
                constexpr int o = decltype(o_c)::value;
                if constexpr (o < NM) {
                    constexpr int i = o % (NB > 0 ? NB : 1), j = o / (NB > 0 ? NB : 1);
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(cur.b[j], cur.a[i], acc[i][j], 0, 0, 0);
                }
                if constexpr (o < ND) dma_one(o_c, stage, sslot);
                if constexpr (o < NR) read_one<NB, o>(nxt, a, w, s, r0w, c0w);
                __builtin_amdgcn_sched_barrier(0);
            });
        };
        auto run = [&](auto nb_c) {
            constexpr int NB = decltype(nb_c)::value;
            Frags f0, f1;
            static_for<0, STAGES - 1>([&](auto st_c) {
                static_for<0, PER>([&](auto d_c) { dma_one(d_c, decltype(st_c)::value, decltype(st_c)::value); });
            });
            wait_vm<PER * (STAGES - 2)>();   // slice 0 in LDS
            lds_barrier();
            if constexpr (NB > 0)
                static_for<0, NB + NJ>([&](auto r_c) { read_one<NB, decltype(r_c)::value>(f0, sm.ring.a[0], sm.ring.w[0][0], 0, r0w, c0w); });
            __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0): exact wait counts at the loop head
            // Iteration kt for kt = R (mod 4), R a compile-time constant, so the ring slots and
            // the LDS offsets of every read and load are constants: 3.8 instead of 5.2 instructions
            // per MFMA (the wave is alone on its SIMD, and what it issues besides MFMAs competes
            // with them for issue cycles); 2 % faster, results bit-identical.
            auto iter = [&](auto r_c, int kt) {
                constexpr int R = decltype(r_c)::value, slot = R % STAGES, ns = (R + 1) % STAGES;
                constexpr int ls = (R + STAGES - 1) % STAGES;   // slot of slice kt + 3
                phase(nb_c, std::true_type{}, f0, f1, sm.ring.a[slot], sm.ring.w[slot][0], 1, kt + STAGES - 1, ls);
                wait_vm<PER * (STAGES - 2)>();   // slice kt + 1 in LDS
                lds_barrier();
                phase(nb_c, std::false_type{}, f1, f0, sm.ring.a[ns], sm.ring.w[ns][0], 0, 0, 0);
            };
            int kt = 0;
            for (; kt + 4 < nk; kt += 4) static_for<0, 4>([&](auto r_c) { iter(r_c, kt + decltype(r_c)::value); });
            static_for<0, 3>([&](auto r_c) {   // the last nk - 1 - kt < 4 iterations (kt = 0 mod 4)
                if (kt + decltype(r_c)::value + 1 < nk) iter(r_c, kt + decltype(r_c)::value);
            });
            const int last = (nk - 1) % STAGES;
            phase(nb_c, std::false_type{}, f0, f1, sm.ring.a[last], sm.ring.w[last][0], 1, 0, 0);
            static_for<0, NB * NJ>([&](auto o_c) {   // the last half slice's MFMAs
                constexpr int o = decltype(o_c)::value, i = o % (NB > 0 ? NB : 1), j = o / (NB > 0 ? NB : 1);
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f1.b[j], f1.a[i], acc[i][j], 0, 0, 0);
            });
        };
        if (nk > 0) with_nb<MI>(nb, run);
        // every ring load has landed (zero-fill loads past k may still be in flight, and the
        // strips overlap their slots) and every wave is done reading the ring
        wait_vm<0>();
        lds_barrier();

        // epilogue: strip columns 0..63 gate, 64..127 up (strip column of block j is 32 j + ..)
        constexpr int SP = WCOLS + 4, LPR = 8, RPS = 64 / LPR;
        float* strip = reinterpret_cast<float*>(&sm.ring) + wave * 32 * SP;
        static_assert(4 * 32 * SP * 4 <= (int)sizeof(sm.ring), "strips fit the ring");
        const rsrc_t ro = make_rsrc((const char*)p.out + (size_t)row0 * p.n * osz, (uint32_t)(rows_valid * p.n * osz));
        const int h = l >> 5, rr = l / LPR, g8 = l % LPR;
        const int col = col0 + c0w + 8 * g8;
        const bool col_ok = col < p.n;
        const float* b0 = p.bias0 ? p.bias0 + (size_t)grp * p.bias_stride : nullptr;
        const float* b1 = p.bias1 ? p.bias1 + (size_t)grp * p.bias_stride : nullptr;
#pragma unroll
        for (int i = 0; i < MI; ++i) {
#pragma unroll
            for (int j = 0; j < NJ; ++j)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const f32x4 v = {acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]};
                    *(f32x4*)(strip + (l & 31) * SP + 32 * j + 8 * q + 4 * h) = v;
                }
#pragma unroll
            for (int t2 = 0; t2 < 32 / RPS; ++t2) {
                const int rs = t2 * RPS + rr;
                const f32x4 g_lo = *(const f32x4*)(strip + rs * SP + 8 * g8);
                const f32x4 g_hi = *(const f32x4*)(strip + rs * SP + 8 * g8 + 4);
                const f32x4 u_lo = *(const f32x4*)(strip + rs * SP + 64 + 8 * g8);
                const f32x4 u_hi = *(const f32x4*)(strip + rs * SP + 64 + 8 * g8 + 4);
                const float gv[8] = {g_lo[0], g_lo[1], g_lo[2], g_lo[3], g_hi[0], g_hi[1], g_hi[2], g_hi[3]};
                const float uv[8] = {u_lo[0], u_lo[1], u_lo[2], u_lo[3], u_hi[0], u_hi[1], u_hi[2], u_hi[3]};
                float y[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const bool in = col + e < p.n;
                    const float gb = gv[e] + (b0 && in ? b0[col + e] : 0.f);
                    const float ub = uv[e] + (b1 && in ? b1[col + e] : 0.f);
                    y[e] = act_fn<ACT>(gb) * ub;
                }
                const int r = r0w + 32 * i + rs;
                const uint32_t off = col_ok ? (uint32_t)(r * p.n + col) * (uint32_t)osz : kOOB;
                if constexpr (osz == 2) {
                    bstore(ro, off, i32x4{(int)pack_bf16(y[0], y[1]), (int)pack_bf16(y[2], y[3]), (int)pack_bf16(y[4], y[5]),
                                          (int)pack_bf16(y[6], y[7])});
                } else {
                    bstore(ro, off, i32x4{__float_as_int(y[0]), __float_as_int(y[1]), __float_as_int(y[2]), __float_as_int(y[3])});
                    bstore(ro, col_ok ? off + 16u : kOOB,
                           i32x4{__float_as_int(y[4]), __float_as_int(y[5]), __float_as_int(y[6]), __float_as_int(y[7])});
                }
            }
        }
        lds_barrier();   // strips read before the next tile's ring loads land there
    }
    wait_vm<0>();   // no ring load may still be writing LDS when the workgroup ends
}

}  // namespace mg

bool ragged_m_gated_ok(const GParams& p) {
    const uint64_t w = (uint64_t)p.k * (uint64_t)p.n * 2u;
    const uint64_t a = 256ull * (uint64_t)p.k * 2u;
    const uint64_t o = 256ull * (uint64_t)p.n * 4u;
    return p.k % 8 == 0 && p.n % 8 == 0 && w < (1ull << 31) && a < (1ull << 31) && o < (1ull << 31);
}

hipError_t launch_ragged_m_gated(const GParams& p, int grid, hipStream_t s) {
    if (p.act == GG_ACT_SILU) {
        if (p.out_f32) hipLaunchKernelGGL((mg::kernel<GG_ACT_SILU, float>), dim3(grid), dim3(mg::NT), 0, s, p);
        else hipLaunchKernelGGL((mg::kernel<GG_ACT_SILU, uint16_t>), dim3(grid), dim3(mg::NT), 0, s, p);
    } else {
        if (p.out_f32) hipLaunchKernelGGL((mg::kernel<GG_ACT_GELU_TANH, float>), dim3(grid), dim3(mg::NT), 0, s, p);
        else hipLaunchKernelGGL((mg::kernel<GG_ACT_GELU_TANH, uint16_t>), dim3(grid), dim3(mg::NT), 0, s, p);
    }
    return hipGetLastError();
}

}  // namespace gg
