/* The fp64 oracle (oracle/fa_ref.c) on exact-size heap buffers, built with AddressSanitizer
 * and UndefinedBehaviorSanitizer by tests/test_host_asan.py and run on the CPU.
 *
 * Shapes cover one row and one key, ragged sizes, causal and not, grouped K/V heads, key
 * ranges and explicit row lists.  Besides what the sanitizers report, each call is checked
 * against facts that hold for any inputs: with every value row equal to a constant vector the
 * output is that vector; causal row 0 sees key 0 alone, so its output is v[0] and its LSE
 * is scale * q0.k0; and bad arguments are refused without writing.  Exit status 0 when all
 * hold, 1 otherwise.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

int fa_ref_rows_kv(const double* q, const double* k, const double* v, double* o, double* lse, int B, int Hq,
                   int Hkv, int Nq, int Nk, int d, int causal, double scale, int k_lo, int k_hi,
                   const int64_t* rows, int64_t nrows);
int fa_ref_rows(const double* q, const double* k, const double* v, double* o, double* lse, int B, int Hq, int Hkv,
                int N, int d, int causal, double scale, const int64_t* rows, int64_t nrows);
int fa_ref_fwd(const double* q, const double* k, const double* v, double* o, double* lse, int B, int Hq, int Hkv,
               int N, int d, int causal, double scale);

static int failures = 0;
static uint64_t state = 0x9E3779B97F4A7C15ull;

static double uniform(void)
{
    state ^= state << 13;
    state ^= state >> 7;
    state ^= state << 17;
    return (double)(state >> 11) / 9007199254740992.0 * 2.0 - 1.0;
}

static double* filled(size_t n)
{
    double* p = (double*)malloc(n ? n * sizeof(double) : 1);
    for (size_t i = 0; i < n; ++i) p[i] = uniform();
    return p;
}

static void check(int ok, const char* what, int line)
{
    if (!ok) {
        printf("line %d: %s\n", line, what);
        ++failures;
    }
}
#define CHECK(x) check((x), #x, __LINE__)

static void shape(int B, int Hq, int Hkv, int Nq, int Nk, int d, int causal)
{
    const size_t nq = (size_t)B * Hq * Nq, nk = (size_t)B * Hkv * Nk;
    double* q = filled(nq * d);
    double* k = filled(nk * d);
    double* v = filled(nk * d);
    double* o = filled(nq * d);
    double* lse = filled(nq);
    const double scale = 1.0 / sqrt((double)d);
    /* every value row the same vector: every output row is that vector */
    for (size_t j = 0; j < nk; ++j)
        for (int c = 0; c < d; ++c) v[j * d + c] = 0.25 * c - 1.0;
    CHECK(fa_ref_rows_kv(q, k, v, o, lse, B, Hq, Hkv, Nq, Nk, d, causal, scale, 0, Nk, NULL, (int64_t)nq) == 0);
    for (size_t r = 0; r < nq; ++r) {
        CHECK(isfinite(lse[r]));
        for (int c = 0; c < d; ++c) CHECK(fabs(o[r * d + c] - (0.25 * c - 1.0)) < 1e-12);
    }
    if (Nq == Nk && causal && Nq > 0) {
        /* row 0 of head 0 sees key 0 alone */
        for (size_t j = 0; j < nk * d; ++j) v[j] = uniform();
        int64_t row0 = 0;
        double o0[256], l0;
        CHECK(fa_ref_rows(q, k, v, o0, &l0, B, Hq, Hkv, Nq, d, 1, scale, &row0, 1) == 0);
        double s = 0.0;
        for (int c = 0; c < d; ++c) s += q[c] * k[c];
        CHECK(fabs(l0 - scale * s) < 1e-12);
        for (int c = 0; c < d; ++c) CHECK(o0[c] == v[c]);
        CHECK(fa_ref_fwd(q, k, v, o, lse, B, Hq, Hkv, Nq, d, causal, scale) == 0);
    }
    if (Nk >= 2 && nq > 0) {
        /* a key range and a reversed list of rows */
        int64_t* rows = (int64_t*)malloc(nq * sizeof(int64_t));
        for (size_t r = 0; r < nq; ++r) rows[r] = (int64_t)(nq - 1 - r);
        CHECK(fa_ref_rows_kv(q, k, v, o, lse, B, Hq, Hkv, Nq, Nk, d, 0, scale, 1, Nk, rows, (int64_t)nq) == 0);
        free(rows);
    }
    free(q);
    free(k);
    free(v);
    free(o);
    free(lse);
}

int main(void)
{
    shape(1, 1, 1, 1, 1, 64, 0);
    shape(1, 1, 1, 1, 1, 64, 1);
    shape(1, 2, 1, 37, 37, 64, 1);
    shape(2, 4, 2, 33, 33, 128, 1);
    shape(1, 8, 2, 5, 70, 64, 0);
    shape(1, 8, 8, 3, 130, 128, 1);
    shape(3, 2, 2, 0, 9, 64, 0);

    /* refused arguments leave the outputs untouched */
    double q[64], k[64], v[64], o[64], lse = 7.0;
    for (int i = 0; i < 64; ++i) q[i] = k[i] = v[i] = o[i] = 1.0;
    int64_t bad_row = 1;
    CHECK(fa_ref_rows(NULL, k, v, o, &lse, 1, 1, 1, 1, 64, 0, 1.0, NULL, 1) == 1);
    CHECK(fa_ref_rows(q, k, v, o, &lse, 1, 3, 2, 1, 64, 0, 1.0, NULL, 1) == 1);
    CHECK(fa_ref_rows(q, k, v, o, &lse, 1, 1, 1, 1, 64, 2, 1.0, NULL, 1) == 1);
    CHECK(fa_ref_rows(q, k, v, o, &lse, 1, 1, 1, 1, 64, 0, NAN, NULL, 1) == 1);
    CHECK(fa_ref_rows(q, k, v, o, &lse, 1, 1, 1, 1, 64, 0, 1.0, &bad_row, 1) == 1);
    CHECK(fa_ref_rows(q, k, v, o, &lse, 1, 1, 1, 1, 64, 0, 1.0, NULL, 2) == 1);
    CHECK(fa_ref_rows_kv(q, k, v, o, &lse, 1, 1, 1, 1, 1, 64, 0, 1.0, 1, 0, NULL, 1) == 1);
    CHECK(lse == 7.0 && o[0] == 1.0);

    if (failures) printf("%d oracle checks failed\n", failures);
    else printf("oracle checks passed\n");
    return failures ? 1 : 0;
}
