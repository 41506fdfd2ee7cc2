/*
 * oracle_driver.c -- exercises every entry point of the CPU oracle (oracle/oracle.c) under
 * AddressSanitizer and UndefinedBehaviorSanitizer on the host: valid calls of every element
 * type and argument combination, and the invalid ones the oracle must refuse or clamp
 * (negative group sizes, sizes past m, rows or (group, k-index) pairs out of range, empty
 * dimensions).  Any out-of-bounds access or undefined operation aborts the run; a wrong
 * value on the small worked cases exits with status 2.  Test infrastructure only.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int oracle_ragged_dot_m(int dtype, const void* lhs, const void* rhs, const uint8_t* lhs_scale,
                        const uint8_t* rhs_scale, const int32_t* group_sizes, int64_t m, int64_t k, int64_t n,
                        int32_t g, const int64_t* rows, int64_t nrows, double* out);
int oracle_ragged_dot_k(int dtype, const void* lhs, const void* dout, const int32_t* group_sizes, int64_t m,
                        int64_t k, int64_t n, int32_t g, const int64_t* pairs, int64_t npairs, double* out);
double orc_decode_bf16(uint16_t bits);
double orc_decode_e4m3(uint8_t code);
double orc_decode_e8m0(uint8_t s);
int oracle_num_threads(void);
void oracle_set_num_threads(int n);

static int failures = 0;
#define CHECK(c) do { if (!(c)) { fprintf(stderr, "check failed line %d: %s\n", __LINE__, #c); ++failures; } } while (0)

/* exact-sized heap buffers, so any overrun is caught by the sanitizer */
static void* xmalloc(size_t n) { void* p = malloc(n ? n : 1); if (!p) abort(); return p; }

static uint32_t lcg = 12345u;
static float frand(void) { lcg = lcg * 1664525u + 1013904223u; return (float)((lcg >> 8) & 0xffff) / 32768.0f - 1.0f; }

int main(void) {
    /* decoders over every code */
    for (int c = 0; c < 256; ++c) { (void)orc_decode_e4m3((uint8_t)c); (void)orc_decode_e8m0((uint8_t)c); }
    for (int c = 0; c < 65536; ++c) (void)orc_decode_bf16((uint16_t)c);
    CHECK(orc_decode_e4m3(0x38) == 1.0 && orc_decode_e4m3(0x7E) == 448.0 && isnan(orc_decode_e4m3(0x7F)));
    CHECK(orc_decode_e8m0(127) == 1.0 && isnan(orc_decode_e8m0(255)));

    /* the worked example: lhs 5x4, rhs 2x4x3, sizes [3, 2] */
    const float L[20] = {1, .5f, 0, 1, 0, 1, .2f, 0, 1, 1, 0, 1, .1f, .2f, .3f, .4f, .5f, 0, 0, 0};
    float R[24];
    for (int i = 0; i < 24; ++i) R[i] = (float)(i % 5) * 0.25f;
    int32_t gs2[2] = {3, 2};
    double out[5 * 3];
    CHECK(oracle_ragged_dot_m(0, L, R, NULL, NULL, gs2, 5, 4, 3, 2, NULL, 0, out) == 0);
    for (int r = 0; r < 5; ++r)
        for (int j = 0; j < 3; ++j) {
            const int h = r < 3 ? 0 : 1;
            double want = 0.0;
            for (int t = 0; t < 4; ++t) want += (double)L[r * 4 + t] * (double)R[h * 12 + t * 3 + j];
            CHECK(fabs(out[r * 3 + j] - want) < 1e-12);
        }

    /* every element type, several shapes, clamped sizes, row selections and pairs */
    const int64_t shapes[][3] = {{37, 64, 9}, {1, 32, 1}, {64, 96, 17}, {5, 0, 3}, {0, 32, 4}, {8, 32, 0}};
    const int32_t sizes[][4] = {{10, 0, 20, 7}, {-3, 5, 40, 2}, {0, 0, 0, 0}, {100, 0, 0, 0}};
    for (size_t si = 0; si < sizeof shapes / sizeof shapes[0]; ++si) {
        const int64_t m = shapes[si][0], k = shapes[si][1], n = shapes[si][2];
        const int32_t g = 4;
        for (int dt = 0; dt < 3; ++dt) {
            const size_t es = dt == 0 ? 4 : dt == 1 ? 2 : 1;
            uint8_t* lhs = xmalloc((size_t)(m * k) * es);
            uint8_t* rhs = xmalloc((size_t)(g * k * n) * es);
            uint8_t* dout = xmalloc((size_t)(m * n) * es);
            for (size_t i = 0; i < (size_t)(m * k) * es; ++i) lhs[i] = (uint8_t)(lcg = lcg * 1664525u + 1013904223u) >> 3;
            for (size_t i = 0; i < (size_t)(g * k * n) * es; ++i) rhs[i] = (uint8_t)((lcg = lcg * 1664525u + 1013904223u) >> 5);
            for (size_t i = 0; i < (size_t)(m * n) * es; ++i) dout[i] = (uint8_t)((lcg = lcg * 1664525u + 1013904223u) >> 7);
            if (dt == 0) {
                for (int64_t i = 0; i < m * k; ++i) ((float*)lhs)[i] = frand();
                for (int64_t i = 0; i < g * k * n; ++i) ((float*)rhs)[i] = frand();
                for (int64_t i = 0; i < m * n; ++i) ((float*)dout)[i] = frand();
            }
            uint8_t* ls = xmalloc((size_t)(m * (k / 32)));
            uint8_t* rs = xmalloc((size_t)(g * (k / 32) * n));
            for (int64_t i = 0; i < m * (k / 32); ++i) ls[i] = (uint8_t)(120 + i % 14);
            for (int64_t i = 0; i < g * (k / 32) * n; ++i) rs[i] = (uint8_t)(118 + i % 17);
            for (size_t zi = 0; zi < sizeof sizes / sizeof sizes[0]; ++zi) {
                double* o = xmalloc(sizeof(double) * (size_t)(m * n));
                int rc = oracle_ragged_dot_m(dt, lhs, rhs, ls, rs, sizes[zi], m, k, n, g, NULL, 0, o);
                CHECK(rc == 0);
                free(o);
                int64_t rows[3] = {0, m - 1, m > 2 ? m / 2 : 0};
                double* o2 = xmalloc(sizeof(double) * 3 * (size_t)n);
                rc = oracle_ragged_dot_m(dt, lhs, rhs, ls, rs, sizes[zi], m, k, n, g, rows, m > 0 ? 3 : 0, o2);
                CHECK(rc == 0);
                int64_t bad_rows[2] = {-1, m};   /* refused, nothing read out of range */
                rc = oracle_ragged_dot_m(dt, lhs, rhs, ls, rs, sizes[zi], m, k, n, g, bad_rows, 2, o2);
                CHECK(rc == -1);
                free(o2);
                if (dt < 2) {
                    double* ok = xmalloc(sizeof(double) * (size_t)(g * k * n));
                    CHECK(oracle_ragged_dot_k(dt, lhs, dout, sizes[zi], m, k, n, g, NULL, 0, ok) == 0);
                    free(ok);
                    int64_t pairs[6] = {0, 0, 3, k > 0 ? k - 1 : 0, 1, k / 2};
                    double* op = xmalloc(sizeof(double) * 3 * (size_t)n);
                    CHECK(oracle_ragged_dot_k(dt, lhs, dout, sizes[zi], m, k, n, g, pairs, k > 0 ? 3 : 0, op) == 0);
                    int64_t bad_pairs[4] = {4, 0, 0, k};
                    CHECK(oracle_ragged_dot_k(dt, lhs, dout, sizes[zi], m, k, n, g, bad_pairs, 2, op) == -1);
                    free(op);
                }
            }
            free(lhs); free(rhs); free(dout); free(ls); free(rs);
        }
    }
    /* refused arguments */
    double tiny[4];
    float one[4] = {1, 1, 1, 1};
    int32_t gs1[1] = {2};
    CHECK(oracle_ragged_dot_m(0, one, one, NULL, NULL, gs1, 2, 1, 2, 0, NULL, 0, tiny) == -1);   /* g < 1 */
    CHECK(oracle_ragged_dot_m(2, one, one, NULL, NULL, gs1, 2, 16, 1, 1, NULL, 0, tiny) == -1);  /* e4m3: k % 32, no scales */
    CHECK(oracle_ragged_dot_k(2, one, one, gs1, 2, 1, 2, 1, NULL, 0, tiny) == -1);              /* e4m3 not taken */
    oracle_set_num_threads(1);
    CHECK(oracle_num_threads() == 1);
    printf("oracle driver: %d failures\n", failures);
    return failures ? 2 : 0;
}
