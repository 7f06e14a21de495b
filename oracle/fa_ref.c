/*
 * fa_ref.c -- the oracle: exact scaled-dot-product attention in fp64, the slow
 * and obvious way.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or call
 * this file: only the tests, the package's smoke check and the benchmark's CPU
 * baseline do.  It shares no code, header, table or constant with the HIP
 * library; the two meet only through the seeded inputs the tests hand to both.
 *
 * What it computes, for every query row (b, h, i) of q[B][Hq][N][d]:
 *
 *   kv head      hk = h / (Hq / Hkv)        consecutive query heads share one
 *                                           K/V head (grouped-query reading)
 *   visible keys J  = {0..N-1}, or {0..i} when causal (key j visible iff j <= i)
 *   scores       s_j = scale * sum_t q[b][h][i][t] * k[b][hk][j][t],  j in J
 *   pass 1       m   = max_j s_j
 *   pass 2       l   = sum_j exp(s_j - m)
 *   pass 3       w_j = exp(s_j - m) / l,   O[b][h][i][:] = sum_j w_j * v[b][hk][j][:]
 *   LSE[b][h][i] = m + ln(l)
 *
 * The general entry (fa_ref_rows_kv) takes Nq query rows against Nk keys and
 * cuts J to a key range [k_lo, k_hi):
 *   causal       key j visible to query i iff j <= i + (Nk - Nq): the queries
 *                are the last Nq positions of the key sequence (Nq == Nk gives
 *                j <= i above)
 *   J            = {j in [k_lo, k_hi) : j visible}
 *   empty J      no weight at all: the empty state of the merge (m = -inf,
 *                l = 0), written as O = 0 and LSE = -inf
 * A row's result over a key range is the partial state (m, l, acc) of the
 * pages in normalised form: O = acc / l, LSE = m + ln l.
 *
 * Sources, cited by page and section:
 *  - subtracting the row maximum leaves softmax unchanged because the common
 *    factor exp(-m) cancels: kbwen.com FlashAttention feed, "All four scores at
 *    once"; spicyshark.co online-softmax lesson, "The fix: subtract the maximum".
 *  - the three passes (max, sum, output): spicyshark.co lesson, "The cost: three
 *    passes".
 *  - the attention form s_j = q.k_j / sqrt(d) and output = sum exp(s_j - m) v_j /
 *    sum exp(s_j - m): spicyshark.co lesson, "From softmax to attention".
 *  - the reference is computed in float64: spicyshark.co lesson, the
 *    attention_reference function of its code listing.
 *  - causal masking gives masked keys no weight (a score of -inf): spicyshark.co
 *    lesson, "The implementation".  Here masked keys are simply left out of J,
 *    which is the same thing written without infinities.
 *  - grouped-query attention, fewer K/V heads than query heads:
 *    paweldubiel.com FlashAttention note, "Averaging block results is not
 *    enough" (last paragraph).  The pages give no head mapping; the reading
 *    used is hk = h / (Hq/Hkv).
 *  - LSE (natural log, in units of the scaled score) is not on the pages; they
 *    carry m and l, and m + ln l is the log of the normaliser they define.
 *  - a state built from part of the keys, and its value when the keys end
 *    there: kbwen.com FlashAttention feed, "Two blocks" (the first block alone
 *    gives the output for a query with only those keys); states of disjoint
 *    key sets combine by the merge: spicyshark.co lesson, "From softmax to
 *    attention" (two workers) and the answer in "Check yourself".
 *  - the causal offset for Nq < Nk and the empty-set convention are readings:
 *    the pages have only square, top-left causal masks and never an empty row.
 *
 * Plain C99 + OpenMP over rows; libm exp/log; no blocking, no fusion, no
 * reordering beyond the definition.  The score row of the query being computed
 * is held in a per-thread buffer: this is the textbook method the pages
 * contrast with FlashAttention, which is exactly what an oracle should be.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define FA_REF_OK 0
#define FA_REF_BAD_ARG 1
#define FA_REF_NO_MEMORY 2

/* Threads the OpenMP runtime will use for the next parallel region. */
int fa_ref_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* One query row against the keys j_lo .. j_hi-1 (the visible set J).  s is a
 * scratch buffer indexed by key, at least j_hi doubles long. */
static void attend_one_row(const double* qi, const double* kh, const double* vh,
                           int d, int j_lo, int j_hi, double scale,
                           double* s, double* out, double* lse_out)
{
    int j, t;
    double m, l;

    if (j_hi <= j_lo) {
        /* no visible key: the empty state, which carries no weight */
        for (t = 0; t < d; ++t) out[t] = 0.0;
        *lse_out = -INFINITY;
        return;
    }

    /* scores against every visible key */
    for (j = j_lo; j < j_hi; ++j) {
        const double* kj = kh + (int64_t)j * d;
        double dot = 0.0;
        for (t = 0; t < d; ++t) dot += qi[t] * kj[t];
        s[j] = scale * dot;
    }

    /* pass 1: the row maximum */
    m = -INFINITY;
    for (j = j_lo; j < j_hi; ++j)
        if (s[j] > m) m = s[j];

    /* pass 2: the normaliser, measured against the maximum */
    l = 0.0;
    for (j = j_lo; j < j_hi; ++j) l += exp(s[j] - m);

    /* pass 3: the softmax weights, then the weighted sum of the values */
    for (t = 0; t < d; ++t) out[t] = 0.0;
    for (j = j_lo; j < j_hi; ++j) {
        const double w = exp(s[j] - m) / l;
        const double* vj = vh + (int64_t)j * d;
        for (t = 0; t < d; ++t) out[t] += w * vj[t];
    }
    *lse_out = m + log(l);
}

/*
 * fa_ref_rows_kv: attention for a list of query rows, Nq queries against Nk keys,
 * keys restricted to [k_lo, k_hi).
 *
 *   q  [B][Hq][Nq][d], k and v [B][Hkv][Nk][d]: fp64, contiguous, read only.
 *   rows: flat row ids r = (b*Hq + h)*Nq + i, or NULL for every row in order.
 *   o   [nrows][d] and lse [nrows]: written in the order of `rows` (with rows ==
 *       NULL, nrows must be B*Hq*Nq and o/lse are laid out as [B][Hq][Nq](d)).
 *
 * Returns 0, or 1 for a bad argument (nothing written), or 2 when a scratch
 * row could not be allocated.
 */
int fa_ref_rows_kv(const double* q, const double* k, const double* v,
                   double* o, double* lse,
                   int B, int Hq, int Hkv, int Nq, int Nk, int d, int causal, double scale,
                   int k_lo, int k_hi, const int64_t* rows, int64_t nrows)
{
    int64_t total, r;
    int group, failed = 0;

    if (!q || !k || !v || !o || !lse) return FA_REF_BAD_ARG;
    if (B < 0 || Nq < 0 || Nk < 0 || Hq < 1 || Hkv < 1 || d < 1 || Hq % Hkv != 0)
        return FA_REF_BAD_ARG;
    if (causal != 0 && causal != 1) return FA_REF_BAD_ARG;
    if (!isfinite(scale)) return FA_REF_BAD_ARG;
    if (k_lo < 0 || k_hi < k_lo || k_hi > Nk) return FA_REF_BAD_ARG;
    total = (int64_t)B * Hq * Nq;
    if (rows == NULL && nrows != total) return FA_REF_BAD_ARG;
    if (nrows < 0) return FA_REF_BAD_ARG;
    if (rows)
        for (r = 0; r < nrows; ++r)
            if (rows[r] < 0 || rows[r] >= total) return FA_REF_BAD_ARG;
    if (nrows == 0) return FA_REF_OK;
    group = Hq / Hkv;

#pragma omp parallel reduction(| : failed)
    {
        double* s = (double*)malloc(sizeof(double) * (size_t)(Nk > 0 ? Nk : 1));
        if (!s) {
            failed = 1;
        } else {
            int64_t idx;
#pragma omp for schedule(dynamic, 8)
            for (idx = 0; idx < nrows; ++idx) {
                const int64_t row = rows ? rows[idx] : idx;
                const int i = (int)(row % Nq);
                const int64_t bh = row / Nq;
                const int h = (int)(bh % Hq);
                const int b = (int)(bh / Hq);
                const int hk = h / group;
                const double* qi = q + row * d;
                const double* kh = k + ((int64_t)b * Hkv + hk) * Nk * d;
                const double* vh = v + ((int64_t)b * Hkv + hk) * Nk * d;
                const int last = causal ? i + (Nk - Nq) : Nk - 1;   /* last visible key */
                const int j_lo = k_lo;
                const int j_hi = last + 1 < k_hi ? last + 1 : k_hi;
                attend_one_row(qi, kh, vh, d, j_lo, j_hi, scale, s, o + idx * d, lse + idx);
            }
            free(s);
        }
    }
    return failed ? FA_REF_NO_MEMORY : FA_REF_OK;
}

/* Square attention (Nq == Nk == N) over every key: the forward the library computes. */
int fa_ref_rows(const double* q, const double* k, const double* v,
                double* o, double* lse,
                int B, int Hq, int Hkv, int N, int d, int causal, double scale,
                const int64_t* rows, int64_t nrows)
{
    return fa_ref_rows_kv(q, k, v, o, lse, B, Hq, Hkv, N, N, d, causal, scale,
                          0, N > 0 ? N : 0, rows, nrows);
}

/* Every row: o [B][Hq][N][d], lse [B][Hq][N]. */
int fa_ref_fwd(const double* q, const double* k, const double* v,
               double* o, double* lse,
               int B, int Hq, int Hkv, int N, int d, int causal, double scale)
{
    return fa_ref_rows(q, k, v, o, lse, B, Hq, Hkv, N, d, causal, scale,
                       NULL, (int64_t)B * (Hq > 0 ? Hq : 0) * (N > 0 ? N : 0));
}
