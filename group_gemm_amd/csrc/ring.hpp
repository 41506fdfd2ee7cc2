// ring.hpp -- building blocks shared by the direct-to-LDS ring kernels (bf16 and MXFP8
// non-contracting ragged dot): buffer descriptors, ring loads issued outside the
// compiler's wait tracking, the waits and barrier that order them, compile-time loops,
// and the tile epilogue.
#pragma once

#include <type_traits>

#include "common.hpp"

namespace gg {
namespace ring {

constexpr uint32_t kOOB = 0x80000000u;   // a buffer offset past every num_records
constexpr int kRsrcWord3 = 0x00020000;   // raw buffer, 32-bit data format (gfx9 family)

typedef __amdgpu_buffer_rsrc_t rsrc_t;

__device__ inline rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, kRsrcWord3);
}
// the same descriptor as four scalar registers, for the inline-asm ring loads
__device__ inline i32x4 make_rsrc_v(const void* base, uint32_t bytes) {
    const uint64_t a = (uint64_t)(uintptr_t)base;
    i32x4 r;
    r[0] = __builtin_amdgcn_readfirstlane((int)(uint32_t)a);
    r[1] = __builtin_amdgcn_readfirstlane((int)((uint32_t)(a >> 32) & 0xffffu));
    r[2] = __builtin_amdgcn_readfirstlane((int)bytes);
    r[3] = kRsrcWord3;
    return r;
}
// output stores carry the nontemporal hint (cache-policy bit 1, `nt`): each output line is written
// once and never read back by the kernel, so it need not displace operand panels in L2
__device__ inline void bstore(rsrc_t r, uint32_t off, i32x4 v) { __builtin_amdgcn_raw_buffer_store_b128(v, r, off, 0, 2); }
// two floats -> two bf16 (round to nearest even), low element in the low half
__device__ inline uint32_t pack_bf16(float a, float b) {
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    const bf16x2 v = {(__bf16)a, (__bf16)b};
    return __builtin_bit_cast(uint32_t, v);
}

// Ring loads: 16 (or 4) bytes per lane from the buffer straight into LDS at
// lds_addr + 16 * lane (+ 4 * lane).  Issued from inline asm so the compiler does not track
// them as LDS writes: its alias rule would make every LDS read wait for all outstanding
// loads.  The kernels order these loads themselves (explicit vmcnt waits, then a barrier)
// and issue no other vector-memory loads while a ring runs, so the counts they wait on are
// exact.  lds_addr is a wave-uniform LDS byte address; out-of-range offsets read zeros.
__device__ inline void load_lds16(i32x4 r, uint32_t lds_addr, uint32_t off) {
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                 :: "s"(lds_addr), "v"(off), "s"(r) : "memory", "m0");
}
// the same with the nontemporal hint: for data read once, streamed past the caches so it
// does not evict operands that other tiles will read again
__device__ inline void load_lds16_nt(i32x4 r, uint32_t lds_addr, uint32_t off) {
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen nt lds"
                 :: "s"(lds_addr), "v"(off), "s"(r) : "memory", "m0");
}
__device__ inline void load_lds4(i32x4 r, uint32_t lds_addr, uint32_t off) {
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dword %1, %2, 0 offen lds"
                 :: "s"(lds_addr), "v"(off), "s"(r) : "memory", "m0");
}
// LDS byte address of a pointer into a __shared__ object
__device__ inline uint32_t lds_u32(const void* p) {
    return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const void*)p;
}
// Barrier that waits for this wave's LDS accesses only; ring loads stay in flight.  The
// builtin wait tells the compiler's own wait tracking that LDS reads issued before the
// barrier are complete (it cannot see into the asm, and would otherwise make later
// MFMAs wait on reads they do not use); the asm keeps the wait and the barrier together.
__device__ inline void lds_barrier() {
    __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0); vmcnt and expcnt at their maximum: no wait
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}
// wait until at most N vector-memory operations of this thread are outstanding
template <int N>
__device__ inline void wait_vm() {
    static_assert(N >= 0 && N <= 63, "vmcnt range");
    asm volatile("s_waitcnt vmcnt(%0)" :: "n"(N) : "memory");
}

// calls f(std::integral_constant<int, I>) for I = B .. E - 1, in order
template <int B, int E, typename F>
__device__ inline void static_for(F&& f) {
    if constexpr (B < E) {
        f(std::integral_constant<int, B>{});
        static_for<B + 1, E>(f);
    }
}
// calls fn(std::integral_constant<int, NB>) for the runtime value nb in [0, MAX] (forced inline:
// kept out of line, the per-NB bodies would pass their fragment registers through memory)
template <int MAX, typename F>
__device__ __attribute__((always_inline)) inline void with_nb(int nb, F&& fn) {
    if constexpr (MAX > 0) {
        if (nb >= MAX) { fn(std::integral_constant<int, MAX>{}); return; }
        with_nb<MAX - 1>(nb, fn);
    } else {
        fn(std::integral_constant<int, 0>{});
    }
}

// Tile walk of the persistent ring kernels.  With queues (8 device ints, one per XCD,
// zeroed by launch_clear_queues before the launch): the tiles are dealt to the 8 XCDs in
// chunks of kQueueChunk consecutive tiles (chunk c to XCD c % 8; workgroup w runs on XCD
// w % 8) and every workgroup takes its XCD's next tile from an atomic counter (another XCD's
// once its own are gone).  A chunk's tiles share a row or weight panel and run side by side
// on one XCD, and workgroups that drew cheap tiles (a short group, a group's partly filled
// last m-tile) take more, where the static walk hands every workgroup the same number of
// tiles whatever they cost.
// Without queues, or with a grid that is not a multiple of 8: a static round-robin over
// virtual ids that keeps consecutive tiles on one XCD.  All threads call these together.
constexpr int kQueueChunk = 8;
__device__ inline bool queued_walk(const int* queues) { return queues != nullptr && (gridDim.x & 7) == 0; }
__device__ inline int first_tile(bool queued) { return queued ? 0 : xcd_virtual_id(blockIdx.x, gridDim.x); }
// The next tile of a queued walk (>= total once every queue is empty); `slot` is an int in
// LDS.  A workgroup whose own XCD's queue is empty takes the next tile of another XCD's queue,
// so an XCD that runs at a lower clock does not hold up the end of the call: counter value c
// of queue x is tile ((c / kQueueChunk) * 8 + x) * kQueueChunk + c % kQueueChunk, increasing
// in c, so every tile is handed out exactly once and a queue, once past the last tile, stays
// past it (the extra increments only move its counter further).
__device__ inline int queue_next(int* queues, int* slot, int total) {
    __syncthreads();   // every thread has read the previous index
    if (threadIdx.x == 0) {
        const int xcd = blockIdx.x & 7;
        int tile = total;
        for (int o = 0; o < 8 && tile >= total; ++o) {   // own queue first, then the others
            const int x = (xcd + o) & 7;
            const int c = atomicAdd(queues + x, 1);
            tile = ((c / kQueueChunk) * 8 + x) * kQueueChunk + c % kQueueChunk;
        }
        *slot = tile;
    }
    __syncthreads();
    return *slot;
}

// Optional epilogue of the tile: out = alpha * acc + bias_row[col] + beta * out (in place).
struct EpiTile {
    const float* bias_row;   // this group's bias row, or nullptr
    float alpha, beta;
};

// Epilogue of one wave's MI x NJ blocks of 32 x 32 fp32 results laid out as
// acc[i][j][4q + e] = C[r0w + 32i + (lane & 31)][c0w + 32j + 8q + 4h + e], h = lane / 32
// (the MFMA took the column operand first).  `ro` covers the tile's valid rows of the
// output; col0 is the tile's first column.  With STRIP (always for bf16 results and for an
// epilogue) results go through `strip`, a wave-private 32 x (WCOLS + 4) fp32 area of LDS:
// the accumulators are written there straight from AGPRs, come back 8 columns per lane
// (8 consecutive ones for bf16, two runs of 4 for fp32), are converted or scaled (EPI), and
// leave as 16-byte stores, a whole row segment per WCOLS / 8 lanes.  Converting or scaling in registers would copy every accumulator
// through VGPRs.  Without STRIP, fp32 results are stored straight from AGPRs, a quarter
// cache line per row and instruction: fewer registers, but slower writes (the fp32
// weight-gradient kernel, whose output dominates its traffic, takes the strip: 12 % faster).
// The row pitch WCOLS + 4 floats spreads the 32 rows one write touches over all banks.  The
// caller synchronises the waves before the strip's memory is reused.
template <int MI, int NJ, int WCOLS, typename OutT, bool EPI, bool STRIP = (sizeof(OutT) == 2 || EPI)>
__device__ inline void store_acc(const f32x16 (&acc)[MI][NJ], float* strip, rsrc_t ro, int n, int col0, int r0w, int c0w,
                                 const EpiTile& ep) {
    const int l = threadIdx.x & 63, h = l >> 5;
    constexpr bool osz2 = sizeof(OutT) == 2;
    static_assert(STRIP || !(osz2 || EPI), "bf16 results and epilogues go through the strip");
    if constexpr (!STRIP) {
#pragma unroll
        for (int i = 0; i < MI; ++i)
#pragma unroll
            for (int j = 0; j < NJ; ++j)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int r = r0w + 32 * i + (l & 31);
                    const int col = col0 + c0w + 32 * j + 8 * q + 4 * h;
                    const i32x4 v = {__float_as_int(acc[i][j][4 * q]), __float_as_int(acc[i][j][4 * q + 1]),
                                     __float_as_int(acc[i][j][4 * q + 2]), __float_as_int(acc[i][j][4 * q + 3])};
                    bstore(ro, col < n ? (uint32_t)(r * n + col) * 4u : kOOB, v);
                }
        return;
    }
    constexpr int SP = WCOLS + 4, LPR = WCOLS / 8, RPS = 64 / LPR;
    const int rr = l / LPR, g = l % LPR;
    // Columns of x[0..3] and x[4..7]: eight consecutive ones for bf16 (one 16-byte store), two
    // runs of four for fp32, 4 g and WCOLS / 2 + 4 g, so that each 16-byte store instruction
    // writes whole 128-byte lines (16 lanes cover 64 consecutive columns of a row) instead of
    // every other 16 bytes of twice as many lines.  n % 8 == 0, so a run is in or out whole.
    constexpr int HALF = WCOLS / 2;
    const int sA = osz2 ? 8 * g : 4 * g, sB = osz2 ? 8 * g + 4 : HALF + 4 * g;   // strip columns
    const int colA = col0 + c0w + sA, colB = col0 + c0w + sB;
    const bool okA = colA < n, okB = colB < n;
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
            const int rs = t2 * RPS + rr;   // row within the strip
            const f32x4 lo = *(const f32x4*)(strip + rs * SP + sA);
            const f32x4 hi = *(const f32x4*)(strip + rs * SP + sB);
            float x[8] = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
            const int r = r0w + 32 * i + rs;
            const uint32_t offA = okA ? (uint32_t)(r * n + colA) * (uint32_t)sizeof(OutT) : kOOB;
            const uint32_t offB = okB ? (uint32_t)(r * n + colB) * (uint32_t)sizeof(OutT) : kOOB;
            if constexpr (EPI) {
                float old[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) old[e] = 0.f;
                if (ep.beta != 0.f) {   // rows past the tile and columns past n read as 0
                    if constexpr (osz2) {
                        const i32x4 c = __builtin_amdgcn_raw_buffer_load_b128(ro, offA, 0, 0);
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            old[2 * e] = __uint_as_float((uint32_t)c[e] << 16);
                            old[2 * e + 1] = __uint_as_float((uint32_t)c[e] & 0xffff0000u);
                        }
                    } else {
                        const i32x4 c0 = __builtin_amdgcn_raw_buffer_load_b128(ro, offA, 0, 0);
                        const i32x4 c1 = __builtin_amdgcn_raw_buffer_load_b128(ro, offB, 0, 0);
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            old[e] = __int_as_float(c0[e]);
                            old[4 + e] = __int_as_float(c1[e]);
                        }
                    }
                }
                // the bias row is re-read per output row (cached) to keep few registers live
                float bias[8];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    bias[e] = ep.bias_row && okA ? ep.bias_row[colA + e] : 0.f;
                    bias[4 + e] = ep.bias_row && okB ? ep.bias_row[colB + e] : 0.f;
                }
#pragma unroll
                for (int e = 0; e < 8; ++e) x[e] = ep.alpha * x[e] + bias[e] + ep.beta * old[e];
            }
            if constexpr (osz2) {
                const i32x4 v = {(int)pack_bf16(x[0], x[1]), (int)pack_bf16(x[2], x[3]), (int)pack_bf16(x[4], x[5]),
                                 (int)pack_bf16(x[6], x[7])};
                bstore(ro, offA, v);
            } else {
                bstore(ro, offA, i32x4{__float_as_int(x[0]), __float_as_int(x[1]), __float_as_int(x[2]), __float_as_int(x[3])});
                bstore(ro, offB, i32x4{__float_as_int(x[4]), __float_as_int(x[5]), __float_as_int(x[6]), __float_as_int(x[7])});
            }
        }
    }
}

// Output rows past the groups' total are zeros: one BM x BN tile of them, 16-byte stores.
template <int BM, int BN, int NT, typename OutT>
__device__ inline void zero_tile(void* out, int r0, int m, int c0, int n) {
    constexpr int osz = sizeof(OutT);
    const int rows = min(BM, m - r0);
    const rsrc_t ro = make_rsrc((const char*)out + (size_t)r0 * n * osz, (uint32_t)(rows * n * osz));
    constexpr int per_row = BN * osz / 16;
    for (int idx = threadIdx.x; idx < BM * per_row; idx += NT) {
        const int r = idx / per_row, cc = idx % per_row;
        const int col = c0 + cc * (16 / osz);
        bstore(ro, col < n ? (uint32_t)(r * n + col) * osz : kOOB, i32x4{0, 0, 0, 0});
    }
}

}  // namespace ring
}  // namespace gg
