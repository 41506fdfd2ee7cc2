// permute.hip -- the pre- and post-processing around the Group-GEMM of an MoE layer, on the
// device and without host synchronisation.
//
// "Group-GEMM in XLA: Making Mixture-of-Experts Fast and Memory-Efficient" (AMD ROCm blog),
// Part 4 "The Three MoE Compute Paths in MaxText", Path 1 (sparse / ragged-dot):
//   permute    -- each token is repeated top_k times (copy i = token * top_k + j), the
//                 copies are ordered by a stable argsort of the flattened expert ids, their
//                 rows gathered in that order, and a bincount of the ids gives group_sizes;
//   un-permute -- the inverse order brings the expert outputs back to copy order and each
//                 token's top_k rows are summed, weighted by the router weights.
// The blog's closing section names this pre/post-processing as what caps the end-to-end
// gain of the Group-GEMM.
//
// Permute is a stable counting sort and a row copy in three launches.  The M copies are cut
// into nblk chunks of `chunk` copies (a multiple of 1024, nblk <= kMaxChunks):
//   1. histogram: per-chunk expert counts -> counts[c][e] (LDS atomics); ids outside [0, g)
//      are not routed and only mark the chunk in bad[c];
//   2. rank (one 1024-thread workgroup per chunk): the chunk's first position for expert e is
//      (copies of experts < e) + (copies of e in earlier chunks), from the counts; the chunk
//      is then walked 1024 copies at a time, each copy ranked among equal ids of its wave by
//      ballots over the id bits and among earlier waves by per-wave counts in LDS, which
//      keeps the order of equal ids (a stable sort).  Writes copy_to_sorted, sorted_to_copy;
//      chunk 0 also writes group_sizes, the routed total and the status word;
//   3. scatter: token t's row is read once and stored to the sorted rows of its top_k copies
//      (copy_to_sorted), 16-byte vectors; rows past the routed total are zero (and their
//      index -1), so every output element is written.
// Un-permute gives each token WPR waves, fp32 accumulation of its top_k rows in copy order.
#include "common.hpp"
#include "launch.hpp"
#include "ring.hpp"

namespace gg {
namespace perm {

constexpr int NT = 1024;    // threads of the histogram and rank workgroups
constexpr int NW = NT / 64;
// Cache policy of the row copies: each sorted row is written once and each expert-output row
// read once, so these accesses carry gfx950's nontemporal (`nt`) hint, which streams them
// past the caches (measured +13 % on the permute, +12 % on the un-permute).  The GEMM
// kernels' output stores do not use it: there it measured neutral to twice as slow.
constexpr int kNontemporal = 2;
// row kernels (scatter, combine): 256-thread workgroups, WPR waves share one token's row
constexpr int WPR = 2;
constexpr int TPB = 4 / WPR;   // tokens per workgroup

__global__ __launch_bounds__(NT) void histogram(const int32_t* __restrict__ experts, int M, int g, int chunk,
                                                 int* __restrict__ counts, int* __restrict__ bad) {
    __shared__ int hist[GG_MAX_GROUPS];
    const int t = threadIdx.x, c = blockIdx.x;
    for (int e = t; e < g; e += NT) hist[e] = 0;
    __syncthreads();
    const int end = min(M, (c + 1) * chunk);
    int nbad = 0;
    for (int i = c * chunk + t; i < end; i += NT) {
        const int e = experts[i];
        if (e >= 0 && e < g) atomicAdd(&hist[e], 1);
        else ++nbad;
    }
    const int any_bad = __syncthreads_or(nbad);
    for (int e = t; e < g; e += NT) counts[(size_t)c * g + e] = hist[e];
    if (t == 0) bad[c] = any_bad;
}

__global__ __launch_bounds__(NT) void rank(const int32_t* __restrict__ experts, int M, int g, int chunk, int nblk,
                                           const int* __restrict__ counts, const int* __restrict__ bad,
                                           int32_t* __restrict__ copy_to_sorted, int32_t* __restrict__ sorted_to_copy,
                                           int32_t* __restrict__ group_sizes, int* __restrict__ total_routed,
                                           uint32_t* __restrict__ status) {
    __shared__ int run[GG_MAX_GROUPS];       // next sorted position of each expert
    __shared__ int cnt[NW][GG_MAX_GROUPS];   // copies of each expert per wave, current step
    __shared__ int part[NW];
    const int t = threadIdx.x, lane = t & 63, w = t >> 6, c = blockIdx.x;

    // 1. start of this chunk's copies of expert e
    int total = 0, before = 0;
    if (t < g) {
        // eight chunks' counts in flight at a time (they come from other CUs' caches)
        int b = 0;
        for (; b + 8 <= nblk; b += 8) {
            int x[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) x[u] = counts[(size_t)(b + u) * g + t];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                total += x[u];
                before += b + u < c ? x[u] : 0;
            }
        }
        for (; b < nblk; ++b) {
            const int x = counts[(size_t)b * g + t];
            total += x;
            before += b < c ? x : 0;
        }
    }
    for (int idx = t; idx < NW * GG_MAX_GROUPS; idx += NT) (&cnt[0][0])[idx] = 0;
    int inc = total;   // inclusive scan of the totals over experts (thread = expert)
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const int u = __shfl_up(inc, d, 64);
        if (lane >= d) inc += u;
    }
    if (lane == 63) part[w] = inc;
    const int any_bad = __syncthreads_or(t < nblk && bad[t] != 0);
    int prev = 0, all = 0;
#pragma unroll
    for (int v = 0; v < NW; ++v) {
        prev += v < w ? part[v] : 0;
        all += part[v];
    }
    if (t < g) run[t] = prev + inc - total + before;
    if (c == 0) {
        if (t < g) group_sizes[t] = total;
        if (t == 0) {
            *total_routed = all;
            if (status) *status = any_bad ? GG_DEV_BAD_EXPERT : 0u;
        }
    }
    __syncthreads();

    // 2. rank the chunk's copies, NT at a time, in index order
    const int nbits = g > 1 ? 32 - __clz(g - 1) : 0;
    const uint64_t lt = (1ull << lane) - 1ull;
    const int end = min(M, (c + 1) * chunk);
    for (int s0 = c * chunk; s0 < end; s0 += NT) {
        const int i = s0 + t;
        int e = -1;
        if (i < end) {
            const int x = experts[i];
            e = (x >= 0 && x < g) ? x : -1;
        }
        // lanes of this wave holding the same expert id
        uint64_t peers = __ballot(e >= 0);
        for (int bit = 0; bit < nbits; ++bit) {
            const bool set = (e >> bit) & 1;
            const uint64_t m1 = __ballot(set);
            peers &= set ? m1 : ~m1;
        }
        const int r = __popcll(peers & lt);
        if (e >= 0 && r == 0) cnt[w][e] = __popcll(peers);
        __syncthreads();
        if (e >= 0) {
            int pos = run[e] + r;
            for (int v = 0; v < w; ++v) pos += cnt[v][e];
            copy_to_sorted[i] = pos;
            sorted_to_copy[pos] = i;
        } else if (i < end) {
            copy_to_sorted[i] = -1;
        }
        __syncthreads();
        if (t < g) {
            int sum = 0;
#pragma unroll
            for (int v = 0; v < NW; ++v) {
                sum += cnt[v][t];
                cnt[v][t] = 0;
            }
            run[t] += sum;
        }
        __syncthreads();
    }
}

// Rows to their sorted places, in copy order: the WPR waves of token t read its row once and
// store it to the sorted row of each of its top_k copies, and its scale row likewise.  The last `zero_blocks` workgroups write zeros (and index -1)
// to the sorted rows past the routed total, a grid-stride loop over [total, M).
// the same address, marked wave-uniform (it is: one token or row per wave), so buffer
// descriptors built from it live in scalar registers
template <typename T>
__device__ inline T* uniform_ptr(T* p) {
    const uint64_t a = (uint64_t)(uintptr_t)p;
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
    return (T*)(uintptr_t)(((uint64_t)hi << 32) | lo);
}

template <bool VEC>
__device__ inline void copy_row(const uint8_t* __restrict__ src, int64_t rb, const int32_t* __restrict__ pos, int top_k,
                                int M, uint8_t* __restrict__ dst0, int h, int l) {
    if constexpr (VEC) {
        // 8 KiB pieces of the row, piece q to wave q % WPR of the token: eight 16-byte loads
        // per lane, one wait, then the stores to every destination.  Buffer accesses past
        // the row's end read zeros and write nothing, so there is no branch around them.
        for (int64_t o0 = (int64_t)h * 8192; o0 < rb; o0 += WPR * 8192) {
            const int64_t rem = rb - o0;
            const uint32_t len = rem < 8192 ? (uint32_t)rem : 8192u;
            const ring::rsrc_t rs = ring::make_rsrc(uniform_ptr(src + o0), len);
            i32x4 v[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) v[u] = __builtin_amdgcn_raw_buffer_load_b128(rs, u * 1024 + 16 * l, 0, 0);
            for (int j = 0; j < top_k; ++j) {
                const int p = pos[j];
                if (p < 0 || p >= M) continue;
                const ring::rsrc_t rd = ring::make_rsrc(uniform_ptr(dst0 + (size_t)p * rb + o0), len);
#pragma unroll
                for (int u = 0; u < 8; ++u) __builtin_amdgcn_raw_buffer_store_b128(v[u], rd, u * 1024 + 16 * l, 0, kNontemporal);
            }
        }
    } else {
        for (int64_t o = h * 64 + l; o < rb; o += WPR * 64) {
            const uint8_t v = src[o];
            for (int j = 0; j < top_k; ++j) {
                const int p = pos[j];
                if (p >= 0 && p < M) dst0[(size_t)p * rb + o] = v;
            }
        }
    }
}

template <bool VEC>
__device__ inline void zero_row(uint8_t* __restrict__ dst, int64_t rb, int l) {
    if constexpr (VEC) {
        for (int64_t o = 16 * l; o < rb; o += 1024) *(uint4*)(dst + o) = make_uint4(0, 0, 0, 0);
    } else {
        for (int64_t o = l; o < rb; o += 64) dst[o] = 0;
    }
}

template <bool VEC>
__global__ __launch_bounds__(256) void scatter(const uint8_t* __restrict__ x, const uint8_t* __restrict__ xs, int T,
                                               int top_k, int64_t rb, int64_t srb, const int32_t* __restrict__ c2s,
                                               const int* __restrict__ total_routed, int zero_blocks,
                                               int32_t* __restrict__ s2c, uint8_t* __restrict__ sorted_x,
                                               uint8_t* __restrict__ sorted_s) {
    const int M = T * top_k, l = threadIdx.x & 63;
    const int tok_blocks = (int)gridDim.x - zero_blocks;
    if ((int)blockIdx.x < tok_blocks) {
        // wave-uniform token, so the copy positions come in through scalar loads
        const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
        const int t = blockIdx.x * TPB + wv / WPR, h = wv % WPR;
        if (t >= T) return;
        const int32_t* pos = c2s + (size_t)t * top_k;
        copy_row<VEC>(x + (size_t)t * rb, rb, pos, top_k, M, sorted_x, h, l);
        if (xs) copy_row<VEC>(xs + (size_t)t * srb, srb, pos, top_k, M, sorted_s, h, l);
        return;
    }
    const int zw = (blockIdx.x - tok_blocks) * 4 + (threadIdx.x >> 6), nzw = zero_blocks * 4;
    for (int p = *total_routed + zw; p < M; p += nzw) {
        if (l == 0) s2c[p] = -1;
        zero_row<VEC>(sorted_x + (size_t)p * rb, rb, l);
        if (sorted_s) zero_row<VEC>(sorted_s + (size_t)p * srb, srb, l);
    }
}

// out[t, :] = sum_j w[t, j] * y[copy_to_sorted[t * top_k + j], :], fp32 sum in j order;
// entries outside [0, rows) contribute nothing.  WPR waves per token; VEC: 8 consecutive
// columns per lane with 16-byte (bf16) or 2 x 16-byte (fp32) accesses.
// (streaming accesses: each expert-output row is read once and each token row written once,
// so they bypass the caches' retention with nontemporal hints)
template <typename InT>
__device__ inline void load8(const InT* p, float (&v)[8]) {
    if constexpr (sizeof(InT) == 2) {
        const i32x4 q = __builtin_nontemporal_load((const i32x4*)p);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            v[2 * e] = __uint_as_float((uint32_t)q[e] << 16);
            v[2 * e + 1] = __uint_as_float((uint32_t)q[e] & 0xffff0000u);
        }
    } else {
        const f32x4 a = __builtin_nontemporal_load((const f32x4*)p), b = __builtin_nontemporal_load((const f32x4*)(p + 4));
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            v[e] = a[e];
            v[4 + e] = b[e];
        }
    }
}
template <typename OutT>
__device__ inline void store8(OutT* p, const float (&v)[8]) {
    if constexpr (sizeof(OutT) == 2) {
        i32x4 q;
#pragma unroll
        for (int e = 0; e < 4; ++e) q[e] = (int)(f32_to_bf16(v[2 * e]) | ((uint32_t)f32_to_bf16(v[2 * e + 1]) << 16));
        __builtin_nontemporal_store(q, (i32x4*)p);
    } else {
        __builtin_nontemporal_store(f32x4{v[0], v[1], v[2], v[3]}, (f32x4*)p);
        __builtin_nontemporal_store(f32x4{v[4], v[5], v[6], v[7]}, (f32x4*)(p + 4));
    }
}
__device__ inline float ld1(const uint16_t* p) { return __uint_as_float((uint32_t)*p << 16); }
__device__ inline float ld1(const float* p) { return *p; }
__device__ inline void st1(uint16_t* p, float v) { *p = f32_to_bf16(v); }
__device__ inline void st1(float* p, float v) { *p = v; }

template <typename InT, typename OutT, bool VEC>
__global__ __launch_bounds__(256) void combine(const InT* __restrict__ y, int rows, const int32_t* __restrict__ c2s,
                                               const float* __restrict__ w, int T, int top_k, int n,
                                               OutT* __restrict__ out) {
    // wave-uniform token: positions and weights come in through scalar loads
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), l = threadIdx.x & 63;
    const int t = blockIdx.x * TPB + wv / WPR, h = wv % WPR;
    if (t >= T) return;
    const int32_t* pos = c2s + (size_t)t * top_k;
    const float* wt = w + (size_t)t * top_k;
    OutT* orow = out + (size_t)t * n;
    if constexpr (VEC) {
        // eight copies at a time.  Copies without a sorted row (and slots past top_k) read
        // row 0 and are replaced by zeros with a select, so the eight loads issue back to
        // back with no branch between them.
        struct Eight { int p[8]; bool ok[8]; float w[8]; };
        auto fetch = [&](int j0, Eight& q) {
#pragma unroll
            for (int jj = 0; jj < 8; ++jj) {
                const int j = j0 + jj;
                const int p = j < top_k ? pos[j] : -1;
                q.ok[jj] = p >= 0 && p < rows;
                q.p[jj] = q.ok[jj] ? p : 0;
                q.w[jj] = q.ok[jj] ? wt[j] : 0.f;
            }
        };
        auto accumulate = [&](const Eight& q, int c0, float (&acc)[8]) {
            float v[8][8];
#pragma unroll
            for (int jj = 0; jj < 8; ++jj) load8(y + (size_t)q.p[jj] * n + c0, v[jj]);
#pragma unroll
            for (int jj = 0; jj < 8; ++jj)
#pragma unroll
                for (int e = 0; e < 8; ++e) acc[e] = __builtin_fmaf(q.w[jj], q.ok[jj] ? v[jj][e] : 0.f, acc[e]);
        };
        Eight first;
        fetch(0, first);
        for (int c0 = 512 * h + 8 * l; c0 < n; c0 += WPR * 512) {
            float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
            accumulate(first, c0, acc);
            for (int j0 = 8; j0 < top_k; j0 += 8) {
                Eight more;
                fetch(j0, more);
                accumulate(more, c0, acc);
            }
            store8(orow + c0, acc);
        }
    } else {
        for (int c = 64 * h + l; c < n; c += WPR * 64) {
            float acc = 0.f;
            for (int j = 0; j < top_k; ++j) {
                const int p = pos[j];
                if (p < 0 || p >= rows) continue;
                acc = __builtin_fmaf(wt[j], ld1(y + (size_t)p * n + c), acc);
            }
            st1(orow + c, acc);
        }
    }
}

template <typename InT, typename OutT>
hipError_t launch_combine_t(const void* y, int rows, const int32_t* c2s, const float* w, int T, int top_k, int n,
                            void* out, bool vec, hipStream_t s) {
    const dim3 grid((T + TPB - 1) / TPB), block(256);
    if (vec)
        hipLaunchKernelGGL((combine<InT, OutT, true>), grid, block, 0, s, (const InT*)y, rows, c2s, w, T, top_k, n, (OutT*)out);
    else
        hipLaunchKernelGGL((combine<InT, OutT, false>), grid, block, 0, s, (const InT*)y, rows, c2s, w, T, top_k, n, (OutT*)out);
    return hipGetLastError();
}

}  // namespace perm

PermuteGeometry permute_geometry(int64_t M) {
    PermuteGeometry pg;
    const int64_t per = (M + kMaxChunks - 1) / kMaxChunks;
    pg.chunk = (int)((per + perm::NT - 1) / perm::NT * perm::NT);
    if (pg.chunk < perm::NT) pg.chunk = perm::NT;
    pg.nblk = (int)((M + pg.chunk - 1) / pg.chunk);
    return pg;
}

hipError_t launch_permute(const PermuteArgs& a, hipStream_t s) {
    const int M = a.tokens * a.top_k;
    const PermuteGeometry pg = permute_geometry(M);
    if (pg.nblk > 0)
        hipLaunchKernelGGL(perm::histogram, dim3(pg.nblk), dim3(perm::NT), 0, s, a.experts, M, a.g, pg.chunk, a.counts,
                           a.bad);
    // at least one workgroup, so group_sizes, the routed total and the status are written
    hipLaunchKernelGGL(perm::rank, dim3(pg.nblk > 0 ? pg.nblk : 1), dim3(perm::NT), 0, s, a.experts, M, a.g, pg.chunk,
                       pg.nblk, a.counts, a.bad, a.copy_to_sorted, a.sorted_to_copy, a.group_sizes, a.total_routed,
                       a.status);
    if (M == 0) return hipGetLastError();
    const bool vec = (uintptr_t)a.x % 16 == 0 && (uintptr_t)a.sorted_x % 16 == 0 && a.row_bytes % 16 == 0 &&
                     (!a.x_scale || ((uintptr_t)a.x_scale % 16 == 0 && (uintptr_t)a.sorted_scale % 16 == 0 &&
                                     a.scale_row_bytes % 16 == 0));
    const int tok_blocks = (a.tokens + perm::TPB - 1) / perm::TPB;
    const int zero_blocks = min((M + 3) / 4, 256);
    const dim3 grid(tok_blocks + zero_blocks), block(256);
    const uint8_t* xs = a.x_scale && a.scale_row_bytes > 0 ? (const uint8_t*)a.x_scale : nullptr;
    uint8_t* ss = xs ? (uint8_t*)a.sorted_scale : nullptr;
    if (vec)
        hipLaunchKernelGGL(perm::scatter<true>, grid, block, 0, s, (const uint8_t*)a.x, xs, a.tokens, a.top_k,
                           a.row_bytes, a.scale_row_bytes, a.copy_to_sorted, a.total_routed, zero_blocks,
                           a.sorted_to_copy, (uint8_t*)a.sorted_x, ss);
    else
        hipLaunchKernelGGL(perm::scatter<false>, grid, block, 0, s, (const uint8_t*)a.x, xs, a.tokens, a.top_k,
                           a.row_bytes, a.scale_row_bytes, a.copy_to_sorted, a.total_routed, zero_blocks,
                           a.sorted_to_copy, (uint8_t*)a.sorted_x, ss);
    return hipGetLastError();
}

hipError_t launch_combine(const void* y, bool y_bf16, int rows, const int32_t* c2s, const float* w, int T, int top_k,
                          int n, void* out, bool out_bf16, hipStream_t s) {
    if (T == 0 || n == 0) return hipSuccess;
    const size_t ey = y_bf16 ? 2 : 4, eo = out_bf16 ? 2 : 4;
    const bool vec = n % 8 == 0 && (uintptr_t)y % 16 == 0 && (uintptr_t)out % 16 == 0 && (n * ey) % 16 == 0 &&
                     (n * eo) % 16 == 0;
    if (y_bf16)
        return out_bf16 ? perm::launch_combine_t<uint16_t, uint16_t>(y, rows, c2s, w, T, top_k, n, out, vec, s)
                        : perm::launch_combine_t<uint16_t, float>(y, rows, c2s, w, T, top_k, n, out, vec, s);
    return out_bf16 ? perm::launch_combine_t<float, uint16_t>(y, rows, c2s, w, T, top_k, n, out, vec, s)
                    : perm::launch_combine_t<float, float>(y, rows, c2s, w, T, top_k, n, out, vec, s);
}

}  // namespace gg
