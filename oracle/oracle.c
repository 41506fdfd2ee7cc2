/*
 * oracle.c -- plain, slow CPU reference for ragged-dot.  TEST INFRASTRUCTURE ONLY.
 *
 * Only the test-suite, the smoke check and the benchmark's CPU-baseline leg load this
 * library.  It shares no code, header, table or constant with the GPU library: every
 * definition below is restated here from the pages' text and from the public OCP
 * FP8 / Microscaling (MX) format specifications.
 *
 * Sources (page titles and sections):
 *  [XLA]   "Group-GEMM in XLA: Making Mixture-of-Experts Fast and Memory-Efficient"
 *          (AMD ROCm blog), Part 1 "The Ragged-Dot Operation", "Why Group-GEMM Is the
 *          Suitable Solution"; Part 3 "Non-Contracting (the MoE Case)", "Contracting";
 *          Part 4 Table 7 (the six ragged-dot classes).
 *  [AITER] "[Triton/Gluon] Merge MoE MXFP8 GEMM into existing _moe_gemm_a8w8 kernel"
 *          (ROCm/aiter pull request 5658): OCP float8 e4m3 on gfx950, E8M0 scales, one
 *          scale per 32 contiguous elements along k.
 *
 * What is computed (fp64 accumulation, summation order t = 0, 1, ..., in the order the
 * definition writes the sum):
 *  ragged_dot_m: out[r, j] = sum_t lhs[r, t] * rhs[g(r), t, j], where g(r) is the group
 *                whose contiguous row block [start_g, start_g + m_g) holds r; rows not
 *                covered by any group are 0.
 *  ragged_dot_k: out[g, i, j] = sum over rows r of group g of lhs[r, i] * dout[r, j];
 *                an empty group gives exactly 0.
 *
 * Readings where the pages are silent (each also listed in the design notes):
 *  - rows at or past sum(group_sizes) are written as 0 (the aiter PR zero-fills the
 *    output; the XLA blog says they are "left unwritten");
 *  - a negative group size counts as 0, and a group is cut off at row m when the running
 *    sum passes m (the pages only say invalid sizes corrupt memory accesses);
 *  - MXFP8 value = e4m3(code) * 2^(scale - 127); lhs_scale is [m, k/32] and rhs_scale is
 *    [g, k/32, n], both row-major bytes.
 *
 * Parallelism: OpenMP splits independent output rows across threads; each output
 * element is still one sequential fp64 sum over t.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* element codes understood by the oracle (its own numbering) */
#define ORC_F32 0
#define ORC_BF16 1
#define ORC_E4M3 2

/* ---- element decoding (exact in double) ------------------------------------------ */

/* bfloat16: the upper 16 bits of an IEEE-754 binary32. */
double orc_decode_bf16(uint16_t bits) {
    uint32_t w = ((uint32_t)bits) << 16;
    float f;
    memcpy(&f, &w, sizeof f);
    return (double)f;
}

/* OCP 8-bit float E4M3 ("e4m3fn"): 1 sign, 4 exponent (bias 7), 3 mantissa bits.
 * exponent field 0 is subnormal (m/8 * 2^-6); S.1111.111 is NaN; there are no
 * infinities, so exponent field 15 with mantissa 0..6 is a normal number (max 448). */
double orc_decode_e4m3(uint8_t code) {
    int sign = (code >> 7) & 1;
    int e = (code >> 3) & 0xF;
    int mant = code & 0x7;
    double v;
    if (e == 0xF && mant == 0x7) return NAN;
    if (e == 0)
        v = ldexp((double)mant / 8.0, -6);
    else
        v = ldexp(1.0 + (double)mant / 8.0, e - 7);
    return sign ? -v : v;
}

/* OCP MX E8M0 scale: an unsigned biased exponent, value 2^(s - 127); 0xFF is NaN. */
double orc_decode_e8m0(uint8_t s) {
    if (s == 0xFF) return NAN;
    return ldexp(1.0, (int)s - 127);
}

static double load_elem(int dtype, const void* base, size_t idx) {
    switch (dtype) {
        case ORC_F32: return (double)((const float*)base)[idx];
        case ORC_BF16: return orc_decode_bf16(((const uint16_t*)base)[idx]);
        case ORC_E4M3: return orc_decode_e4m3(((const uint8_t*)base)[idx]);
        default: return NAN;
    }
}

/* ---- group partition --------------------------------------------------------------- */

/* Effective row block of every group: start[h] and size[h] after the clamping reading
 * (negative -> 0, truncated at row m).  Returns the covered row count S. */
static int64_t group_blocks(const int32_t* group_sizes, int32_t g, int64_t m, int64_t* start,
                            int64_t* size) {
    int64_t run = 0;
    for (int32_t h = 0; h < g; ++h) {
        int64_t s = group_sizes[h] < 0 ? 0 : (int64_t)group_sizes[h];
        if (run + s > m) s = m - run;
        start[h] = run;
        size[h] = s;
        run += s;
    }
    return run;
}

/* ---- ragged_dot, non-contracting (m-ragged) ---------------------------------------- */

/* out[nrows, n] (row-major double) receives rows `rows[0..nrows)` of the [m, n] result;
 * rows == NULL means every row 0..m-1.  lhs is [m, k], rhs is [g, k, n], row-major.
 * For dtype ORC_E4M3, lhs_scale [m, k/32] and rhs_scale [g, k/32, n] are E8M0 bytes and
 * k must be a multiple of 32.  Returns 0, or -1 on a bad argument. */
int oracle_ragged_dot_m(int dtype, const void* lhs, const void* rhs, const uint8_t* lhs_scale,
                        const uint8_t* rhs_scale, const int32_t* group_sizes, int64_t m,
                        int64_t k, int64_t n, int32_t g, const int64_t* rows, int64_t nrows,
                        double* out) {
    if (g < 1 || m < 0 || k < 0 || n < 0) return -1;
    if (dtype == ORC_E4M3 && (k % 32 != 0 || !lhs_scale || !rhs_scale)) return -1;
    if (!rows) nrows = m;
    int64_t* start = (int64_t*)malloc(sizeof(int64_t) * (size_t)g);
    int64_t* size = (int64_t*)malloc(sizeof(int64_t) * (size_t)g);
    if (!start || !size) { free(start); free(size); return -1; }
    group_blocks(group_sizes, g, m, start, size);
    int bad = 0;

#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t q = 0; q < nrows; ++q) {
        int64_t r = rows ? rows[q] : q;
        double* orow = out + (size_t)q * (size_t)n;
        for (int64_t j = 0; j < n; ++j) orow[j] = 0.0;
        if (r < 0 || r >= m) { bad = 1; continue; }
        /* the group whose contiguous block holds row r */
        int32_t grp = -1;
        for (int32_t h = 0; h < g; ++h)
            if (size[h] > 0 && r >= start[h] && r < start[h] + size[h]) { grp = h; break; }
        if (grp < 0) continue; /* uncovered row: stays 0 */
        const size_t rhs_base = (size_t)grp * (size_t)k * (size_t)n;
        for (int64_t t = 0; t < k; ++t) {
            double a = load_elem(dtype, lhs, (size_t)r * (size_t)k + (size_t)t);
            if (dtype == ORC_E4M3) a *= orc_decode_e8m0(lhs_scale[(size_t)r * (size_t)(k / 32) + (size_t)(t / 32)]);
            for (int64_t j = 0; j < n; ++j) {
                double b = load_elem(dtype, rhs, rhs_base + (size_t)t * (size_t)n + (size_t)j);
                if (dtype == ORC_E4M3)
                    b *= orc_decode_e8m0(rhs_scale[((size_t)grp * (size_t)(k / 32) + (size_t)(t / 32)) * (size_t)n + (size_t)j]);
                orow[j] += a * b;
            }
        }
    }
    free(start);
    free(size);
    return bad ? -1 : 0;
}

/* ---- ragged_dot, contracting (ragged contraction dim, group index in the output) ---- */

/* out[npairs, n] receives out[g_q, i_q, :] for the (group, k-index) pairs given in
 * pairs[2q], pairs[2q+1]; pairs == NULL means every (g, i) in g-major order, i.e. the
 * whole [g, k, n] result.  lhs is [m, k], dout is [m, n], row-major. */
int oracle_ragged_dot_k(int dtype, const void* lhs, const void* dout, const int32_t* group_sizes,
                        int64_t m, int64_t k, int64_t n, int32_t g, const int64_t* pairs,
                        int64_t npairs, double* out) {
    if (g < 1 || m < 0 || k < 0 || n < 0) return -1;
    if (dtype != ORC_F32 && dtype != ORC_BF16) return -1;
    if (!pairs) npairs = (int64_t)g * k;
    int64_t* start = (int64_t*)malloc(sizeof(int64_t) * (size_t)g);
    int64_t* size = (int64_t*)malloc(sizeof(int64_t) * (size_t)g);
    if (!start || !size) { free(start); free(size); return -1; }
    group_blocks(group_sizes, g, m, start, size);
    int bad = 0;

#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t q = 0; q < npairs; ++q) {
        int64_t grp = pairs ? pairs[2 * q] : q / (k > 0 ? k : 1);
        int64_t i = pairs ? pairs[2 * q + 1] : q % (k > 0 ? k : 1);
        double* orow = out + (size_t)q * (size_t)n;
        for (int64_t j = 0; j < n; ++j) orow[j] = 0.0;
        if (grp < 0 || grp >= g || i < 0 || i >= k) { bad = 1; continue; }
        for (int64_t r = start[grp]; r < start[grp] + size[grp]; ++r) {
            double a = load_elem(dtype, lhs, (size_t)r * (size_t)k + (size_t)i);
            for (int64_t j = 0; j < n; ++j)
                orow[j] += a * load_elem(dtype, dout, (size_t)r * (size_t)n + (size_t)j);
        }
    }
    free(start);
    free(size);
    return bad ? -1 : 0;
}

/* number of OpenMP threads a parallel region would use (reported with timings) */
int oracle_num_threads(void) {
#ifdef _OPENMP
    extern int omp_get_max_threads(void);
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* sets the OpenMP thread count of later calls (the benchmark times a one-thread run) */
void oracle_set_num_threads(int n) {
#ifdef _OPENMP
    extern void omp_set_num_threads(int);
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}
