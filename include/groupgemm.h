/*
 * groupgemm.h -- C ABI of the MI355X (gfx950) ragged-dot Group-GEMM library.
 *
 * The operation is ragged-dot lowered to one Group-GEMM: a set of independent GEMMs whose
 * row counts are known only at run time, computed in one launch with no padding.
 * Sources (page titles and sections):
 *   "Group-GEMM in XLA: Making Mixture-of-Experts Fast and Memory-Efficient" (AMD ROCm blog):
 *     Part 1 "The Ragged-Dot Operation" (lhs [m,k], rhs [g,k,n], group_sizes [g], 2-D out),
 *     "Why Group-GEMM Is the Suitable Solution", "The Naive Support, and Why It Hurts:
 *     Padded-Dot"; Part 3 "Non-Contracting (the MoE Case)", "Contracting", "Batch";
 *     Part 4 Table 7 (fwd / dgrad / wgrad classes).
 *   "[Triton/Gluon] Merge MoE MXFP8 GEMM into existing _moe_gemm_a8w8 kernel" (ROCm/aiter
 *     pull request 5658): OCP e4m3 with one E8M0 scale per 32 elements along k, a
 *     zero-filled output, and a routing conversion with no host synchronisation.
 *
 * Conventions shared by every call
 *   - All tensors are caller-owned device memory, dense row-major (last index fastest).
 *     `out` must not overlap any input.  The library allocates and frees nothing.
 *   - Work is enqueued on `stream` (a hipStream_t; NULL = the null stream) and the call
 *     returns once it is enqueued.  No call synchronises with the host, reads group_sizes
 *     on the host, or allocates, so every call may be captured in a HIP graph.
 *   - group_sizes is int32[g] in device memory.  Group h owns the contiguous rows
 *     [sum_{j<h} gs_j, sum_{j<=h} gs_j).  Bad sizes are a device-side condition: a negative
 *     size counts as 0 and the groups are cut off at row m (no access out of bounds); the
 *     device status word of the workspace records it (GG_DEV_*).
 *   - Host-detectable errors return a code and enqueue nothing.
 *   - The workspace carries per-call state (the status word; the forward kernels' tile
 *     queue counters, which each call resets on its stream): calls that share a workspace
 *     must not run concurrently -- issue them on one stream or give each its own.
 *   - Accumulation is fp32.  bf16 outputs are rounded to nearest-even.
 *   - Tensors must be aligned to their element size (e4m3 operands: 16 bytes) and the
 *     workspace to 16 bytes.  16-byte aligned bf16 operands whose rows are whole multiples
 *     of 16 bytes take the vectorised path (the one performance figures assume); any other
 *     k and n take an element-wise path.
 */
#ifndef GROUPGEMM_H
#define GROUPGEMM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define GG_ABI_VERSION 5

/* Each enumeration below also names the ends of the int32 range, so that every int32 value a
 * caller passes (from C, through an FFI, ...) is a valid value of the type; the calls refuse the
 * ones they do not know with an error code. */

typedef enum {
    GG_OK = 0,
    GG_ERR_NULL_PTR = 1,           /* a required pointer is NULL                          */
    GG_ERR_BAD_SHAPE = 2,          /* negative m/k/n, g < 1, g above GG_MAX_GROUPS, ...    */
    GG_ERR_BAD_DTYPE = 3,          /* unsupported in/out element type combination          */
    GG_ERR_MISALIGNED = 4,         /* a pointer is not aligned to its element (16 B for e4m3) */
    GG_ERR_WORKSPACE_TOO_SMALL = 5,
    GG_ERR_UNSUPPORTED = 6,        /* e.g. MXFP8 with k not a multiple of 32               */
    GG_ERR_HIP = 7,                /* a HIP runtime call failed (launch, device query)      */
    GG_STATUS_RANGE_MIN = INT32_MIN, GG_STATUS_RANGE_MAX = INT32_MAX
} gg_status;

typedef enum {
    GG_DT_F32 = 0,                 /* IEEE binary32                                         */
    GG_DT_BF16 = 1,                /* bfloat16                                              */
    GG_DT_E4M3 = 2,                /* OCP float8 e4m3 ("e4m3fn"), with E8M0 block scales    */
    GG_DT_RANGE_MIN = INT32_MIN, GG_DT_RANGE_MAX = INT32_MAX
} gg_dtype;

typedef enum {
    GG_OP_RAGGED_M = 0,            /* ragged_dot_m                                          */
    GG_OP_RAGGED_K = 1,            /* ragged_dot_k                                          */
    GG_OP_PADDED_M = 2,            /* padded_dot, non-contracting form                      */
    GG_OP_PADDED_K = 3,            /* padded_dot, contracting form                          */
    GG_OP_PERMUTE = 4,             /* moe_permute (m = tokens * top_k copies)               */
    GG_OP_RANGE_MIN = INT32_MIN, GG_OP_RANGE_MAX = INT32_MAX
} gg_op;

typedef enum {
    GG_ACT_SILU = 0,               /* x * sigmoid(x)  (SwiGLU when applied to the gate)     */
    GG_ACT_GELU_TANH = 1,          /* 0.5 x (1 + tanh(sqrt(2/pi) (x + 0.044715 x^3)))       */
    GG_ACT_RANGE_MIN = INT32_MIN, GG_ACT_RANGE_MAX = INT32_MAX
} gg_activation;

/* Device status bits (read back with gg_read_device_status). */
#define GG_DEV_NEGATIVE_SIZE 0x1u  /* some group_sizes[h] < 0 (treated as 0)               */
#define GG_DEV_SUM_EXCEEDS_M 0x2u  /* sum(group_sizes) > m (groups cut off at row m)       */
#define GG_DEV_OVER_CAPACITY 0x4u  /* padded_dot: a group had more rows than `capacity`    */
#define GG_DEV_BAD_EXPERT    0x8u  /* moe_permute: an expert id outside [0, g) (not routed)  */

/* Largest group count any call accepts. */
#define GG_MAX_GROUPS 1024

/* Workspace bytes a call needs.  Tiny (a few hundred bytes) for the ragged calls; for
 * padded_dot it holds the padded operands and result ([g, capacity, .] buffers).
 * in_dtype selects the element size of the padded buffers.  Returns 0 on bad arguments. */
size_t gg_workspace_bytes(gg_op op, int64_t m, int64_t k, int64_t n, int32_t g, int64_t capacity,
                          gg_dtype in_dtype);

/* ragged_dot_m -- non-contracting (m-ragged) ragged dot, the MoE forward case.
 * ("Group-GEMM in XLA", Part 1 "The Ragged-Dot Operation"; Part 3 "Non-Contracting".)
 *   out[r, :] = lhs[r, :] . rhs[h]   for every row r of group h;   rows r >= sum(sizes) = 0.
 *   lhs  [m, k]      in_dtype        (fp32, bf16 or e4m3)
 *   rhs  [g, k, n]   in_dtype        one weight matrix per group, n fastest
 *   out  [m, n]      out_dtype       fp32 for fp32 inputs; bf16 or fp32 otherwise
 *   lhs_scale [m, k/32], rhs_scale [g, k/32, n]: E8M0 bytes, required for e4m3 inputs
 *     (value = e4m3 * 2^(scale - 127)), NULL otherwise; e4m3 needs k % 32 == 0.
 * The table-7 class fwd_wo is the same call with k and n renamed.  Every element of out is
 * written on every call. */
gg_status ragged_dot_m(const void* lhs, const void* rhs, const int32_t* group_sizes, void* out,
                       int64_t m, int64_t k, int64_t n, int32_t g, gg_dtype in_dtype,
                       gg_dtype out_dtype, const uint8_t* lhs_scale, const uint8_t* rhs_scale,
                       void* workspace, size_t workspace_bytes, void* stream);

/* ragged_dot_m_noalloc -- ragged_dot_m for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc): no
 * workspace argument.  The per-call state that ragged_dot_m keeps in its workspace (256
 * bytes: the status word and the forward kernels' tile-queue counters) lives in a static
 * 256-byte device array of the library instead, one per GPU, held until the process ends;
 * the call allocates nothing, and a size whose state would not fit returns
 * GG_ERR_WORKSPACE_TOO_SMALL (no shape does at present).
 *   status: optional device uint32 that receives the GG_DEV_* bits of this call (NULL: they
 *     stay in the library's array, where no call reads them).
 * Other arguments, results and errors as ragged_dot_m (same kernels, bit-identical output).
 * Every no-allocation call on one GPU shares that array: calls that overlap in time on one
 * GPU (different streams, or host threads) race and must not be issued.  The first call on
 * a device looks up the array's address there (not a stream operation). */
gg_status ragged_dot_m_noalloc(const void* lhs, const void* rhs, const int32_t* group_sizes, void* out,
                               int64_t m, int64_t k, int64_t n, int32_t g, gg_dtype in_dtype,
                               gg_dtype out_dtype, const uint8_t* lhs_scale, const uint8_t* rhs_scale,
                               uint32_t* status, void* stream);

/* ragged_dot_m_nk -- ragged_dot_m with each group's matrix stored [n, k] (k contiguous):
 * the data-gradient classes, which contract the weight's output-feature axis.
 * ("Group-GEMM in XLA", Part 4 Table 7, classes dgrad_wi and dgrad_wo: rhs contracting
 * dimension 2, so the weights are used as stored, with no transposed copy.)
 *   out[r, :] = lhs[r, :] . rhs_nk[h]^T   for every row r of group h;   rows r >= sum(sizes) = 0.
 *   lhs    [m, k]      bf16            e.g. dgrad_wi: the output gradient [M, N_fwd]
 *   rhs_nk [g, n, k]   bf16            e.g. dgrad_wi: the forward weights [E, K_fwd, N_fwd]
 *   out    [m, n]      bf16 or fp32    e.g. dgrad_wi: the input gradient [M, K_fwd]
 * Requires 16-byte aligned lhs, rhs_nk and out and k % 8 == 0, n % 8 == 0; other element
 * types or shapes return GG_ERR_UNSUPPORTED.  Workspace, status and errors as
 * ragged_dot_m. */
gg_status ragged_dot_m_nk(const void* lhs, const void* rhs_nk, const int32_t* group_sizes, void* out,
                          int64_t m, int64_t k, int64_t n, int32_t g, gg_dtype in_dtype,
                          gg_dtype out_dtype, void* workspace, size_t workspace_bytes, void* stream);

/* ragged_dot_m_epilogue -- ragged_dot_m with a fused epilogue, in place on out:
 *   out[r, :] = alpha * (lhs[r, :] . rhs[h]) + bias[h, :] + beta * out[r, :]
 * for every row r of group h; rows r >= sum(sizes) are 0 as in ragged_dot_m.
 * ("Group-GEMM in XLA", Part 2: the grouped-GEMM configuration carries alpha and beta;
 * "[Triton/Gluon] Merge MoE MXFP8 GEMM into existing _moe_gemm_a8w8 kernel", review: a
 * per-expert bias [E, N] indexed with its real row stride.)
 *   bias [g, bias_stride] fp32 (bias_stride >= n, 4-byte aligned), or NULL for none.
 *   beta != 0 reads out (bf16 or fp32, as written by a previous call) before writing it.
 * Other arguments as ragged_dot_m.  A non-trivial epilogue (bias, alpha != 1 or beta != 0)
 * runs on the vectorised bf16 / MXFP8 paths (16-byte aligned operands and output; k, n % 8
 * for bf16; k % 128, n % 16 for e4m3) and returns GG_ERR_UNSUPPORTED elsewhere. */
gg_status ragged_dot_m_epilogue(const void* lhs, const void* rhs, const int32_t* group_sizes, void* out,
                                int64_t m, int64_t k, int64_t n, int32_t g, gg_dtype in_dtype,
                                gg_dtype out_dtype, const uint8_t* lhs_scale, const uint8_t* rhs_scale,
                                const float* bias, int64_t bias_stride, float alpha, float beta,
                                void* workspace, size_t workspace_bytes, void* stream);

/* ragged_dot_k_epilogue -- ragged_dot_k with out[h] = alpha * (lhs_h^T . dout_h) + beta * out[h],
 * in place: beta = 1 accumulates weight gradients over gradient-accumulation micro-steps
 * ("Group-GEMM in XLA", Part 4 Tables 4/5: the models train with grad-accum up to 16).
 * An empty group gives beta * out[h].  Other arguments as ragged_dot_k; a non-trivial
 * epilogue runs on the vectorised bf16 path (16-byte aligned, k, n % 8) and returns
 * GG_ERR_UNSUPPORTED elsewhere. */
gg_status ragged_dot_k_epilogue(const void* lhs, const void* dout, const int32_t* group_sizes, void* out,
                                int64_t m, int64_t k, int64_t n, int32_t g, gg_dtype in_dtype,
                                gg_dtype out_dtype, float alpha, float beta, void* workspace,
                                size_t workspace_bytes, void* stream);

/* ragged_dot_m_gated -- the fused gate/up projection of an MoE expert block:
 *   out[r, :] = act(lhs[r, :] . w0[h] + bias0[h, :]) * (lhs[r, :] . w1[h] + bias1[h, :])
 * for every row r of group h; rows r >= sum(sizes) are 0.
 * ("Group-GEMM in XLA", Part 1: the dense formulation's gate/up einsums and
 * activation(layer_w0) * layer_w1; Part 4: the MaxText layer's gmm_up(x, w0, w1, w0_bias,
 * w1_bias) followed by apply_ffn_activation, fused here into one pass.)
 *   lhs [m, k], w0 / w1 [g, k, n]: bf16; out [m, n]: bf16 or fp32.
 *   bias0 / bias1: fp32 [g, bias_stride] (bias_stride >= n, 4-byte aligned) or NULL.
 *   act: GG_ACT_SILU or GG_ACT_GELU_TANH.
 * Requires 16-byte aligned lhs, w0, w1, out and k % 8 == 0, n % 8 == 0; other shapes
 * return GG_ERR_UNSUPPORTED.  Workspace, status and errors as ragged_dot_m. */
gg_status ragged_dot_m_gated(const void* lhs, const void* w0, const void* w1, const int32_t* group_sizes,
                             void* out, int64_t m, int64_t k, int64_t n, int32_t g, gg_dtype in_dtype,
                             gg_dtype out_dtype, gg_activation act, const float* bias0,
                             const float* bias1, int64_t bias_stride, void* workspace,
                             size_t workspace_bytes, void* stream);

/* ragged_dot_k -- contracting ragged dot, the weight-gradient case: the contracted
 * dimension m is ragged and the group index appears in the output.
 * ("Group-GEMM in XLA", Part 3 "Contracting"; Part 4 Table 7, class wgrad_wi.)
 *   out[h] = lhs[rows of h, :]^T . dout[rows of h, :]   for every group h; empty group -> 0
 *   lhs  [m, k]      in_dtype (fp32 or bf16)
 *   dout [m, n]      in_dtype
 *   out  [g, k, n]   out_dtype (fp32, or bf16 for bf16 inputs); every element written.
 * wgrad_wo is the same call with the operands' roles swapped. */
gg_status ragged_dot_k(const void* lhs, const void* dout, const int32_t* group_sizes, void* out,
                       int64_t m, int64_t k, int64_t n, int32_t g, gg_dtype in_dtype,
                       gg_dtype out_dtype, void* workspace, size_t workspace_bytes, void* stream);

/* padded_dot -- the capacity-padded baseline the Group-GEMM replaces.
 * ("Group-GEMM in XLA", Part 1 "The Naive Support, and Why It Hurts: Padded-Dot" and Part 4:
 * expand the ragged operand into g padded matrices, one batched GEMM, compact again.)
 *   mode GG_OP_PADDED_M: a = lhs [m,k], b = rhs [g,k,n], out [m,n]; same result as
 *     ragged_dot_m when capacity >= max(group_sizes).
 *   mode GG_OP_PADDED_K: a = lhs [m,k], b = dout [m,n], out [g,k,n]; same result as
 *     ragged_dot_k when capacity >= max(group_sizes).
 *   Rows of a group past `capacity` are dropped (they contribute nothing and their output
 *   rows are 0) and GG_DEV_OVER_CAPACITY is set.  Steps: scatter into the zeroed
 *   [g, capacity, .] buffers of the workspace, one uniform batched GEMM, gather.
 *   a_scale / b_scale: as lhs_scale / rhs_scale of ragged_dot_m (mode M with e4m3 only). */
gg_status padded_dot(gg_op mode, const void* a, const void* b, const int32_t* group_sizes,
                     void* out, int64_t m, int64_t k, int64_t n, int32_t g, int64_t capacity,
                     gg_dtype in_dtype, gg_dtype out_dtype, const uint8_t* a_scale,
                     const uint8_t* b_scale, void* workspace, size_t workspace_bytes,
                     void* stream);

/* moe_permute -- the MoE pre-processing that feeds ragged_dot_m: sort the tokens' top-k
 * copies by expert, gather their rows, and count the rows of every expert.
 * ("Group-GEMM in XLA", Part 4 "The Three MoE Compute Paths in MaxText", Path 1: repeat
 * each token top_k times, argsort the flattened expert ids, sort the activations with that
 * order, bincount the ids into group_sizes.)  M = tokens * top_k copies; copy i is token
 * i / top_k routed to experts[i].
 *   x              [tokens, k]      dtype (fp32, bf16 or e4m3)
 *   x_scale        [tokens, k/32]   E8M0 bytes, e4m3 only (k % 32 == 0), else NULL
 *   experts        [tokens, top_k]  int32 expert ids; an id outside [0, g) is not routed
 *                                   (that copy gets no row) and sets GG_DEV_BAD_EXPERT
 *   sorted_x       [M, k]           dtype: the routed copies' rows grouped by expert, equal
 *                                   ids in copy order (a stable sort); rows past the routed
 *                                   total are zero
 *   sorted_scale   [M, k/32]        e4m3 only, else NULL: the scale rows in the same order
 *   group_sizes    [g]   int32      rows per expert (the bincount); sums to the routed total
 *   sorted_to_copy [M]   int32      copy index of each sorted row (the pages' argsort
 *                                   result), -1 past the routed total
 *   copy_to_sorted [M]   int32      sorted row of each copy (the inverse order), -1 if the
 *                                   copy was not routed
 * Every output element is written on every call; with tokens == 0 only group_sizes (zeros)
 * is written and the other pointers may be NULL.  All computed on the device (histogram,
 * scan, rank, gather); nothing is read back.  tokens * top_k <= 2^30.  Workspace:
 * gg_workspace_bytes(GG_OP_PERMUTE, tokens * top_k, k, 0, g, 0, dtype) bytes, 16-byte
 * aligned; its status word is rewritten by every call. */
gg_status moe_permute(const void* x, const uint8_t* x_scale, const int32_t* experts, void* sorted_x,
                      uint8_t* sorted_scale, int32_t* group_sizes, int32_t* sorted_to_copy,
                      int32_t* copy_to_sorted, int64_t tokens, int32_t top_k, int64_t k, int32_t g,
                      gg_dtype dtype, void* workspace, size_t workspace_bytes, void* stream);

/* moe_unpermute -- the MoE post-processing: bring the expert outputs back to token order and
 * sum each token's top-k rows weighted by the router weights.
 * ("Group-GEMM in XLA", Part 4 "The Three MoE Compute Paths in MaxText", Path 1: un-sort
 * with the inverse order, reshape to [tokens, top_k, n], weighted sum over top_k.)
 *   y              [tokens * top_k, n]  in_dtype (fp32 or bf16): rows in sorted order
 *   copy_to_sorted [tokens * top_k]     int32, as written by moe_permute; an entry outside
 *                                       [0, tokens * top_k) (-1: not routed) adds nothing
 *   weights        [tokens, top_k]      fp32 router weights
 *   out            [tokens, n]          out_dtype (fp32 or bf16):
 *     out[t, :] = sum_j weights[t, j] * y[copy_to_sorted[t * top_k + j], :]
 * fp32 accumulation in j order, one rounding.  No workspace. */
gg_status moe_unpermute(const void* y, const int32_t* copy_to_sorted, const float* weights, void* out,
                        int64_t tokens, int32_t top_k, int64_t n, gg_dtype in_dtype,
                        gg_dtype out_dtype, void* stream);

/* gg_schedule -- runs only the group_sizes -> offsets scan that opens every launch, and
 * writes its tables, so the scan can be tested on its own.
 * ("Group-GEMM in XLA", Part 2 "The Compile-Time vs. Runtime Problem": a block scan over
 * the group sizes gives every group its start; Part 3 "Non-Contracting": exclusive
 * prefix = start rows, inclusive = end rows.)
 *   row_off  int32[g+1]  device: clamped exclusive prefix of the sizes; row_off[g] = rows used
 *   tile_off int32[g+1]  device: exclusive prefix of per-group tile counts
 *                        ceil(size_h / block_m) * ceil(n / block_n)
 *   status   uint32[1]   device: GG_DEV_* bits
 *   block_m, block_n in [1, 4096]. */
gg_status gg_schedule(const int32_t* group_sizes, int64_t m, int64_t n, int32_t g, int32_t block_m,
                      int32_t block_n, int32_t* row_off, int32_t* tile_off, uint32_t* status,
                      void* stream);

/* Synchronises `stream`, then copies the device status word of `workspace` (written by the
 * last call that used it) into *flags.  For tests and debugging. */
gg_status gg_read_device_status(const void* workspace, uint32_t* flags, void* stream);

/* Static text for a status code. */
const char* gg_status_string(gg_status s);

/* GG_ABI_VERSION of the built library. */
int gg_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* GROUPGEMM_H */
