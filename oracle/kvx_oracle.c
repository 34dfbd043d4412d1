/*
 * CPU ORACLE for the query-free KV-cache eviction step -- TEST INFRASTRUCTURE.
 *
 * Only the test-suite, the smoke entry and the benchmark's oracle leg may
 * load this file's library.  The product path (the HIP library and its Python
 * binding) never calls it and shares no code with it.
 *
 * What it computes, per (layer, batch, KV head) group, for one incoming block of
 * S key/value rows:
 *
 *  1. score each incoming key once (Q-Filters page, "How it works", step 3;
 *     L2Norm page, "How it works", step 1):
 *       L2 mode:          s = ||k||_2
 *       projection mode:  s = sign * (k . f)      (f = frozen per-head filter)
 *     The sum runs in fp64 over the exactly widened key elements, d = 0..D-1 in
 *     order, and is rounded once to float32, the precision the pages give for
 *     stored scores.  A -0 result is stored as +0 (the pages are silent; IEEE
 *     compares the two equal, so they must tie).
 *  2. append the incoming rows after the kept rows, with absolute positions
 *     tokens_seen + i (Q-Filters page, "How it works", step 1; "RoPE positions
 *     had to be fixed first").
 *  3. if the concatenation holds more rows than the budget (strictly more),
 *     keep every protected row -- the first n_sink rows and the last `recent`
 *     rows -- plus the (budget - #protected) best other rows, best meaning the
 *     highest score (keep-high) or the lowest score (keep-low), ties going to
 *     the lower row, i.e. the earlier position (Q-Filters page, "How it works",
 *     step 4 and "Metal kernels", the tie paragraph; L2Norm page, "How it
 *     works", step 3).  The ranking is a plain sort of the unprotected rows on
 *     (score, row); this is the "one top-k" of the pages.
 *  4. emit the kept rows in row order (= temporal order), carrying each row's
 *     K and V bytes, stored score and position unchanged (Q-Filters page,
 *     "Adaptation notes": no renumbering, keys copied bit-identically).
 *
 * Nothing here is blocked, fused or reordered beyond those steps.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_OK 0
#define ORC_EINVAL -1
#define ORC_ENOMEM -2
#define ORC_ENONFINITE -3

/*
 * dtype: 0 = float32 rows, 1 = bfloat16 rows, 2 = IEEE binary16 rows (raw
 * uint16 bits for both 16-bit types).  Widening is exact.
 */
static double half_bits_to_double(uint16_t h)
{
    int sign = h >> 15, e = (h >> 10) & 0x1F, m = h & 0x3FF;
    double v;
    if (e == 0)
        v = ldexp((double)m, -24);                /* zero or subnormal: m * 2^-24 */
    else if (e == 31)
        v = m ? NAN : INFINITY;
    else
        v = ldexp((double)(m | 0x400), e - 25);   /* (1.m) * 2^(e-15) */
    return sign ? -v : v;
}

static double widen(const void *rows, int dtype, int64_t i)
{
    if (dtype == 1) {
        uint32_t u = (uint32_t)((const uint16_t *)rows)[i] << 16;
        float f;
        memcpy(&f, &u, sizeof f);
        return (double)f;
    }
    if (dtype == 2)
        return half_bits_to_double(((const uint16_t *)rows)[i]);
    return (double)((const float *)rows)[i];
}

static int64_t esize(int dtype) { return dtype == 0 ? 4 : 2; }

/* Score n rows of D elements.  mode 0 = L2 norm, 1 = projection onto f with sign. */
int orc_score(const void *k, int dtype, int64_t n, int64_t D, int mode,
              const float *f, int sign, float *out)
{
    if ((dtype < 0 || dtype > 2) || (mode != 0 && mode != 1) || D <= 0 || n < 0)
        return ORC_EINVAL;
    if (mode == 1 && (f == NULL || (sign != 1 && sign != -1)))
        return ORC_EINVAL;
    for (int64_t r = 0; r < n; ++r) {
        double acc = 0.0;
        for (int64_t d = 0; d < D; ++d) {
            double x = widen(k, dtype, r * D + d);
            if (!isfinite(x))
                return ORC_ENONFINITE;
            acc += (mode == 0) ? x * x : x * (double)f[d];
        }
        float s = (mode == 0) ? (float)sqrt(acc) : (float)((double)sign * acc);
        if (s == 0.0f)
            s = 0.0f; /* -0 -> +0 */
        if (!isfinite(s))
            return ORC_ENONFINITE;
        out[r] = s;
    }
    return ORC_OK;
}

typedef struct {
    float s;
    int64_t row;
} orc_item;

static int by_high(const void *a, const void *b)
{
    const orc_item *x = a, *y = b;
    if (x->s > y->s) return -1;
    if (x->s < y->s) return 1;
    return (x->row > y->row) - (x->row < y->row);
}

static int by_low(const void *a, const void *b)
{
    const orc_item *x = a, *y = b;
    if (x->s < y->s) return -1;
    if (x->s > y->s) return 1;
    return (x->row > y->row) - (x->row < y->row);
}

/* Validation shared by every entry below (same rules the pages raise on). */
static int check_params(int64_t budget, int64_t n_sink, int64_t recent, int keep_low)
{
    if (budget < 1 || n_sink < 0 || recent < 0 || n_sink + recent >= budget)
        return ORC_EINVAL;
    if (keep_low != 0 && keep_low != 1)
        return ORC_EINVAL;
    return ORC_OK;
}

/*
 * Selection on the concatenated scores s[0..n_total).  Writes the kept row
 * indices, ascending, to keep_idx and their count to *n_out.
 */
int orc_select(const float *s, int64_t n_total, int64_t budget, int64_t n_sink,
               int64_t recent, int keep_low, int64_t *keep_idx, int64_t *n_out)
{
    int rc = check_params(budget, n_sink, recent, keep_low);
    if (rc != ORC_OK || n_total < 0)
        return ORC_EINVAL;
    for (int64_t r = 0; r < n_total; ++r)
        if (!isfinite(s[r]))
            return ORC_ENONFINITE;
    if (n_total <= budget) {
        for (int64_t r = 0; r < n_total; ++r)
            keep_idx[r] = r;
        *n_out = n_total;
        return ORC_OK;
    }
    unsigned char *keep = calloc((size_t)n_total, 1);
    orc_item *items = malloc(sizeof(orc_item) * (size_t)n_total);
    if (!keep || !items) {
        free(keep);
        free(items);
        return ORC_ENOMEM;
    }
    int64_t n_prot = 0, n_cand = 0;
    for (int64_t r = 0; r < n_total; ++r) {
        int prot = (r < n_sink) || (r >= n_total - recent);
        if (prot) {
            keep[r] = 1;
            ++n_prot;
        } else {
            items[n_cand].s = s[r];
            items[n_cand].row = r;
            ++n_cand;
        }
    }
    qsort(items, (size_t)n_cand, sizeof(orc_item), keep_low ? by_low : by_high);
    int64_t take = budget - n_prot;
    for (int64_t i = 0; i < take; ++i)
        keep[items[i].row] = 1;
    int64_t j = 0;
    for (int64_t r = 0; r < n_total; ++r)
        if (keep[r])
            keep_idx[j++] = r;
    *n_out = j;
    free(keep);
    free(items);
    return ORC_OK;
}

/*
 * One group's cache state.  Buffers hold `cap` rows (cap >= budget); rows
 * [0, n) are valid and in temporal order.
 */
typedef struct {
    int64_t n;           /* kept rows */
    int64_t tokens_seen; /* absolute tokens absorbed so far (the true offset) */
    void *k;             /* [cap, D] */
    void *v;             /* [cap, D] */
    float *s;            /* [cap]    stored scores */
    int32_t *pos;        /* [cap]    absolute positions */
} orc_group;

/*
 * Absorb one block of S rows into a group.  scores_in, when not NULL, supplies
 * the new rows' scores instead of computing them (used to replay the selection
 * and compaction rules on another implementation's scores).
 */
int orc_group_update(orc_group *st, int64_t D, int dtype, int mode, const float *f, int sign,
                     int64_t budget, int64_t n_sink, int64_t recent, int keep_low,
                     const void *k_new, const void *v_new, int64_t S, const float *scores_in)
{
    int rc = check_params(budget, n_sink, recent, keep_low);
    if (rc != ORC_OK || S < 0 || st->n < 0 || st->n > budget)
        return ORC_EINVAL;
    int64_t es = esize(dtype), row = D * es;
    int64_t nk = st->n, nt = nk + S;
    float *s_all = malloc(sizeof(float) * (size_t)(nt ? nt : 1));
    int32_t *p_all = malloc(sizeof(int32_t) * (size_t)(nt ? nt : 1));
    unsigned char *k_all = malloc((size_t)(nt ? nt : 1) * (size_t)row);
    unsigned char *v_all = malloc((size_t)(nt ? nt : 1) * (size_t)row);
    int64_t *keep = malloc(sizeof(int64_t) * (size_t)(nt ? nt : 1));
    if (!s_all || !p_all || !k_all || !v_all || !keep) {
        rc = ORC_ENOMEM;
        goto done;
    }
    /* step 1: score the incoming rows only; stored scores are reused. */
    if (scores_in) {
        memcpy(s_all + nk, scores_in, sizeof(float) * (size_t)S);
    } else {
        rc = orc_score(k_new, dtype, S, D, mode, f, sign, s_all + nk);
        if (rc != ORC_OK)
            goto done;
    }
    /* step 2: concatenate kept rows, then incoming rows with fresh positions. */
    memcpy(s_all, st->s, sizeof(float) * (size_t)nk);
    memcpy(p_all, st->pos, sizeof(int32_t) * (size_t)nk);
    memcpy(k_all, st->k, (size_t)(nk * row));
    memcpy(v_all, st->v, (size_t)(nk * row));
    memcpy(k_all + nk * row, k_new, (size_t)(S * row));
    memcpy(v_all + nk * row, v_new, (size_t)(S * row));
    for (int64_t i = 0; i < S; ++i)
        p_all[nk + i] = (int32_t)(st->tokens_seen + i);
    /* step 3: protected top-k. */
    int64_t n_out = 0;
    rc = orc_select(s_all, nt, budget, n_sink, recent, keep_low, keep, &n_out);
    if (rc != ORC_OK)
        goto done;
    /* step 4: compact in row order. */
    for (int64_t j = 0; j < n_out; ++j) {
        int64_t r = keep[j];
        ((float *)st->s)[j] = s_all[r];
        st->pos[j] = p_all[r];
        memcpy((unsigned char *)st->k + j * row, k_all + r * row, (size_t)row);
        memcpy((unsigned char *)st->v + j * row, v_all + r * row, (size_t)row);
    }
    st->n = n_out;
    st->tokens_seen += S;
done:
    free(s_all);
    free(p_all);
    free(k_all);
    free(v_all);
    free(keep);
    return rc;
}

/*
 * Many independent groups at once, laid out with fixed strides:
 *   k_state/v_state [G, cap, D], s_state/pos_state [G, cap], n_kept/tokens [G],
 *   k_new/v_new [G, S, D], filters [G, D] (projection mode; NULL for L2),
 *   scores_in [G, S] or NULL.
 * Groups are processed in parallel with OpenMP when the library is built with it;
 * each group's computation is exactly orc_group_update.
 */
int orc_groups_update(int64_t G, int64_t cap, int64_t D, int dtype, int mode,
                      const float *filters, int sign, int64_t budget, int64_t n_sink,
                      int64_t recent, int keep_low, void *k_state, void *v_state,
                      float *s_state, int32_t *pos_state, int64_t *n_kept, int64_t *tokens,
                      const void *k_new, const void *v_new, int64_t S, const float *scores_in)
{
    if (cap < budget)
        return ORC_EINVAL;
    int64_t row = D * esize(dtype);
    int rc_all = ORC_OK;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t g = 0; g < G; ++g) {
        orc_group st;
        st.n = n_kept[g];
        st.tokens_seen = tokens[g];
        st.k = (unsigned char *)k_state + g * cap * row;
        st.v = (unsigned char *)v_state + g * cap * row;
        st.s = s_state + g * cap;
        st.pos = pos_state + g * cap;
        int rc = orc_group_update(&st, D, dtype, mode, filters ? filters + g * D : NULL, sign,
                                  budget, n_sink, recent, keep_low,
                                  (const unsigned char *)k_new + g * S * row,
                                  (const unsigned char *)v_new + g * S * row, S,
                                  scores_in ? scores_in + g * S : NULL);
        if (rc != ORC_OK) {
#pragma omp critical
            rc_all = rc;
        }
        n_kept[g] = st.n;
        tokens[g] = st.tokens_seen;
    }
    return rc_all;
}

int orc_num_threads(void)
{
#ifdef _OPENMP
    extern int omp_get_max_threads(void);
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Threads the next parallel loops use (timing baselines only). */
int orc_set_num_threads(int n)
{
#ifdef _OPENMP
    extern void omp_set_num_threads(int);
    if (n < 1) return -1;
    omp_set_num_threads(n);
    return 0;
#else
    return n == 1 ? 0 : -1;
#endif
}
