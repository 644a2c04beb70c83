/*
 * orc.c -- plain fp64 CPU oracle for the banded block-sparse attention forward.
 *
 * TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only the tests, the smoke check and the
 * CPU-baseline leg of the benchmark may load this library.  It shares no code,
 * header, table or helper with the HIP library, and it never touches a GPU.
 *
 * What it computes follows the NucleoByte project page ("NucleoByte:
 * GPU-Accelerated Block-Sparse Genomic Language Model"):
 *   - section 3, "Localized Block-Sparse Attention Matrix": with block size B,
 *     query block i scores only key blocks j with |i - j| <= R;
 *   - section 3, "Softmax Normalization & Online Numerical Stability": scores
 *     S = Q K^T / sqrt(d_k) followed by a softmax over the scored keys, kept
 *     stable by a running maximum, a running denominator and a running output;
 *   - section 2, item 2 ("Dynamic Ceiling Hardware Alignment"): each batch is
 *     padded up to a multiple of the block size, so keys past a sequence's
 *     length are padding and are never attended to.
 *
 * The online recurrence on that page is an exact rewriting of an ordinary
 * softmax, so the main routine here is the plain definition, done in two passes
 * per query row over the set of keys the row may attend to:
 *
 *   A(b,t) = { s : 0 <= s < len_b,  |floor(t/B) - floor(s/B)| <= R,
 *              and s <= t when the causal flag is set }
 *   S_ts   = scale * sum_c Q[b,h,t,c] K[b,h,s,c]
 *   O[b,h,t,:] = sum_{s in A} exp(S_ts - M_t) V[b,h,s,:] / sum_{s in A} exp(S_ts - M_t)
 *   M_t    = max_{s in A} S_ts,   lse_t = M_t + ln sum_{s in A} exp(S_ts - M_t)
 *   rows t >= len_b are padding: O = 0, lse = -inf.
 *
 * A second routine, orc_forward_recurrence_f64, walks the page's running
 * (m, d, O) update block by block, in the page's order, and divides by the
 * denominator once after the last block (the page never writes that division;
 * it is the only reading under which the probabilities sum to one).  The tests
 * compare the two routines; they are independent formulations of one result.
 *
 * The backward routines (orc_backward_f64, orc_backward_blocks_f64) follow the
 * same page's section 3, "Custom Backpropagation": a per-row correction
 * D_t = sum_c dO_tc O_tc and dS_ts = P_ts (dO_t . V_s - D_t), with P the
 * softmax above.  The page leaves the remaining gradients to the chain rule
 * through S = scale Q K^T and O = P V, written out plainly:
 *   dV_s = sum_t P_ts dO_t,  dQ_t = scale sum_s dS_ts K_s,  dK_s = scale sum_t dS_ts Q_t
 * with t over valid rows and s over A(b,t); padded rows and keys get zero.
 * O and P are recomputed here from Q, K, V in double (the exact forward).
 *
 * orc_kmer_tokenize follows the same page's section 2, item 1 ("Fused 2-Bit
 * Tokenization") and section 1 ("Token Blur": a hard-coded, bit-packed sliding
 * window instead of a learned vocabulary), with the k-mer size and vocabulary of
 * section 5 (6-mers, 4096 k-mer IDs plus padding/mask entries; the usage example
 * of section 6 builds the model with 4100 entries).  Each base is two bits
 * (A = 0, C = 1, G = 2, T = 3, first base most significant); the page's printed
 * IDs (TGGGAC = 3745, TGAAGT = 3595, GGCCCC = 2645) fix that code.  Window t of
 * a sequence covers bases t .. t+k-1 (stride one: a sliding window); its ID is
 *     id_t = sum_{p=0}^{k-1} code(base[t+p]) * 4^(k-1-p),
 * or UNK when one of its bases is not A, C, G or T (either case).  Rows are
 * padded to n_out tokens with PAD.  Special IDs: PAD = 4^k, MASK = 4^k + 1,
 * UNK = 4^k + 2, 4^k + 3 reserved (4^k + 4 entries: 4100 for k = 6).
 *
 * The _w entry points take a token window W as well (section 2, item 3 of the
 * page bounds the receptive field by a local neighbourhood W and says no more
 * of it; read plainly, key s is in reach of query t when |t - s| <= W): A(b,t) is then
 *   { s : 0 <= s < len_b, |t - s| <= W, (causal => s <= t) },
 * searched within the block band of radius ceil(W / B), the widest band such a
 * window reaches.  W = -1 leaves the block band alone.
 *
 * Inputs are float (the exact bf16- or fp32-rounded values a GPU consumes);
 * every product and sum is taken in double.  Q, K, V, O are [batch][heads][n][d]
 * contiguous.  All routines return 0 on success and a negative code on bad
 * arguments, before writing anything.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_E_INVALID (-1)
#define ORC_E_NOMEM (-2)

int orc_version(void) { return 1; }

/* ---------------------------------------------------------------- validation */

static int check_shape(int batch, int n, int bsize, int radius, const int32_t *seqlens)
{
    if (batch < 0 || n < 0 || bsize < 1 || radius < 0)
        return ORC_E_INVALID;
    if (n % bsize != 0)
        return ORC_E_INVALID;
    if (seqlens) {
        for (int b = 0; b < batch; ++b)
            if (seqlens[b] < 0 || seqlens[b] > n)
                return ORC_E_INVALID;
    }
    return 0;
}

/* A token window must fit inside the block band that is searched for it. */
static int check_window(int window, int radius, int bsize)
{
    if (window < -1)
        return ORC_E_INVALID;
    if (window >= 0 && radius < (window + bsize - 1) / bsize)
        return ORC_E_INVALID;
    return 0;
}

static int seq_len(const int32_t *seqlens, int b, int n) { return seqlens ? seqlens[b] : n; }

/* Number of blocks that hold at least one real token: the padded length of a
 * sequence rounded up to the block size, divided by it (section 2, item 2). */
static int blocks_of(int len, int bsize) { return (len + bsize - 1) / bsize; }

/* Is key block j in the band of query block i, inside the sequence, and (causal)
 * not after i?  Section 3's band rule |i - j| <= R. */
static int block_in_band(int i, int j, int radius, int nb, int causal)
{
    if (i >= nb || j < 0 || j >= nb)
        return 0;
    if (abs(i - j) > radius)
        return 0;
    if (causal && j > i)
        return 0;
    return 1;
}

/* Is token pair (query t, key s) kept: the token-level set A(b,t) above.  With
 * a token window (window >= 0) the pair must also lie within window tokens of
 * each other, |t - s| <= window; callers then pass radius = ceil(window / B),
 * the widest block band such a window reaches. */
static int pair_kept(int t, int s, int len, int bsize, int radius, int causal, int window)
{
    if (t < 0 || t >= len || s < 0 || s >= len)
        return 0;
    if (abs(t / bsize - s / bsize) > radius)
        return 0;
    if (window >= 0 && abs(t - s) > window)
        return 0;
    if (causal && s > t)
        return 0;
    return 1;
}

/* ------------------------------------------------------------- block lists */

/* active[b][i][0 .. 2R]: the key blocks query block i of sequence b visits, in
 * ascending order, padded with -1.  Empty (all -1) for blocks that hold no real
 * token. */
int orc_active_blocks(int batch, int n, int bsize, int radius, int causal,
                      const int32_t *seqlens, int32_t *active)
{
    int rc = check_shape(batch, n, bsize, radius, seqlens);
    if (rc)
        return rc;
    if (batch > 0 && n > 0 && !active)
        return ORC_E_INVALID;
    const int nblk = n / bsize, width = 2 * radius + 1;
    for (int b = 0; b < batch; ++b) {
        const int nb = blocks_of(seq_len(seqlens, b, n), bsize);
        for (int i = 0; i < nblk; ++i) {
            int32_t *row = active + ((int64_t)b * nblk + i) * width;
            int used = 0;
            for (int j = i - radius; j <= i + radius; ++j)
                if (block_in_band(i, j, radius, nb, causal))
                    row[used++] = j;
            for (; used < width; ++used)
                row[used] = -1;
        }
    }
    return 0;
}

/* masks[b][i][slot][r], bit c: for the slot-th active key block j of query block
 * i, key j*B + c is kept for query i*B + r.  Zero for unused slots and for query
 * rows past the sequence.  Needs B <= 32 (one 32-bit word per query row). */
int orc_masks_w(int batch, int n, int bsize, int radius, int causal, int window,
                const int32_t *seqlens, const int32_t *active, uint32_t *masks)
{
    int rc = check_shape(batch, n, bsize, radius, seqlens);
    if (rc)
        return rc;
    rc = check_window(window, radius, bsize);
    if (rc)
        return rc;
    if (bsize > 32)
        return ORC_E_INVALID;
    if (batch > 0 && n > 0 && (!active || !masks))
        return ORC_E_INVALID;
    const int nblk = n / bsize, width = 2 * radius + 1;
    for (int b = 0; b < batch; ++b) {
        const int len = seq_len(seqlens, b, n);
        for (int i = 0; i < nblk; ++i) {
            for (int slot = 0; slot < width; ++slot) {
                const int64_t at = ((int64_t)b * nblk + i) * width + slot;
                const int j = active[at];
                uint32_t *words = masks + at * bsize;
                for (int r = 0; r < bsize; ++r) {
                    uint32_t w = 0;
                    if (j >= 0)
                        for (int c = 0; c < bsize; ++c)
                            if (pair_kept(i * bsize + r, j * bsize + c, len, bsize, radius, causal,
                                          window))
                                w |= (uint32_t)1 << c;
                    words[r] = w;
                }
            }
        }
    }
    return 0;
}

/* --------------------------------------------------- two-pass definition */

typedef struct {
    int batch, heads, n, d, bsize, radius, causal;
    double scale;
    const int32_t *seqlens;
    const float *q, *k, *v;
    int window; /* < 0: the block band alone */
} problem;

/* One query row t of (b, h): the plain definition above.  o_row gets d values;
 * *lse and *psum (sum of the normalised probabilities) may be NULL. */
static void row_definition(const problem *p, int b, int h, int t, double *sbuf,
                           int32_t *sidx, double *o_row, double *lse, double *psum)
{
    const int len = seq_len(p->seqlens, b, p->n);
    const int64_t base = ((int64_t)b * p->heads + h) * p->n;
    const int d = p->d;
    if (t >= len) {
        for (int c = 0; c < d; ++c)
            o_row[c] = 0.0;
        if (lse)
            *lse = -INFINITY;
        if (psum)
            *psum = 0.0;
        return;
    }
    /* keys that can be in A(b,t): the blocks within R of t's block */
    const int ib = t / p->bsize;
    int s_lo = (ib - p->radius) * p->bsize;
    int s_hi = (ib + p->radius + 1) * p->bsize; /* exclusive */
    if (s_lo < 0)
        s_lo = 0;
    if (s_hi > len)
        s_hi = len;
    const float *qt = p->q + (base + t) * d;

    /* pass 1: scores of every kept key, and their maximum */
    int cnt = 0;
    double m = -INFINITY;
    for (int s = s_lo; s < s_hi; ++s) {
        if (!pair_kept(t, s, len, p->bsize, p->radius, p->causal, p->window))
            continue;
        const float *ks = p->k + (base + s) * d;
        double dot = 0.0;
        for (int c = 0; c < d; ++c)
            dot += (double)qt[c] * (double)ks[c];
        const double sc = p->scale * dot;
        sbuf[cnt] = sc;
        sidx[cnt] = s;
        ++cnt;
        if (sc > m)
            m = sc;
    }
    /* pass 2: exponentials, denominator, weighted sum of values */
    double l = 0.0;
    for (int c = 0; c < d; ++c)
        o_row[c] = 0.0;
    for (int e = 0; e < cnt; ++e) {
        const double w = exp(sbuf[e] - m);
        sbuf[e] = w;
        l += w;
        const float *vs = p->v + (base + sidx[e]) * d;
        for (int c = 0; c < d; ++c)
            o_row[c] += w * (double)vs[c];
    }
    for (int c = 0; c < d; ++c)
        o_row[c] /= l;
    if (lse)
        *lse = m + log(l);
    if (psum) {
        double ps = 0.0;
        for (int e = 0; e < cnt; ++e)
            ps += sbuf[e] / l;
        *psum = ps;
    }
}

/* Work list for the thread pool: query blocks given as (b, h, i) triples.  Each
 * output row block is [bsize][d] (o), [bsize] (lse, psum). */
typedef struct {
    const problem *p;
    int64_t nsel;
    const int32_t *sel; /* [nsel][3] or NULL = every block in order */
    double *o, *lse, *psum;
    int64_t next;
    pthread_mutex_t lock;
    int failed;
} job;

static int64_t take(job *jb, int64_t chunk, int64_t *end)
{
    pthread_mutex_lock(&jb->lock);
    int64_t at = jb->next;
    jb->next += chunk;
    pthread_mutex_unlock(&jb->lock);
    *end = at + chunk < jb->nsel ? at + chunk : jb->nsel;
    return at;
}

static void *worker(void *arg)
{
    job *jb = (job *)arg;
    const problem *p = jb->p;
    const int nblk = p->n / p->bsize;
    const int maxkeys = (2 * p->radius + 1) * p->bsize;
    double *sbuf = (double *)malloc(sizeof(double) * (size_t)maxkeys);
    int32_t *sidx = (int32_t *)malloc(sizeof(int32_t) * (size_t)maxkeys);
    if (!sbuf || !sidx) {
        free(sbuf);
        free(sidx);
        pthread_mutex_lock(&jb->lock);
        jb->failed = 1;
        pthread_mutex_unlock(&jb->lock);
        return NULL;
    }
    for (;;) {
        int64_t end, at = take(jb, 4, &end);
        if (at >= jb->nsel)
            break;
        for (int64_t w = at; w < end; ++w) {
            int b, h, i;
            if (jb->sel) {
                b = jb->sel[3 * w];
                h = jb->sel[3 * w + 1];
                i = jb->sel[3 * w + 2];
            } else {
                i = (int)(w % nblk);
                h = (int)((w / nblk) % p->heads);
                b = (int)(w / ((int64_t)nblk * p->heads));
            }
            for (int r = 0; r < p->bsize; ++r) {
                const int64_t row = w * p->bsize + r;
                row_definition(p, b, h, i * p->bsize + r, sbuf, sidx, jb->o + row * p->d,
                               jb->lse ? jb->lse + row : NULL, jb->psum ? jb->psum + row : NULL);
            }
        }
    }
    free(sbuf);
    free(sidx);
    return NULL;
}

static int run_pool(job *jb, int nthreads)
{
    if (nthreads < 1)
        nthreads = 1;
    if (nthreads > 1024)
        nthreads = 1024;
    pthread_mutex_init(&jb->lock, NULL);
    jb->next = 0;
    jb->failed = 0;
    pthread_t *tid = (pthread_t *)malloc(sizeof(pthread_t) * (size_t)nthreads);
    if (!tid)
        return ORC_E_NOMEM;
    int started = 0;
    for (int t = 0; t < nthreads; ++t) {
        if (pthread_create(&tid[t], NULL, worker, jb) != 0)
            break;
        ++started;
    }
    if (started == 0)
        worker(jb);
    for (int t = 0; t < started; ++t)
        pthread_join(tid[t], NULL);
    free(tid);
    pthread_mutex_destroy(&jb->lock);
    return jb->failed ? ORC_E_NOMEM : 0;
}

static int check_problem(const problem *p)
{
    int rc = check_shape(p->batch, p->n, p->bsize, p->radius, p->seqlens);
    if (rc)
        return rc;
    rc = check_window(p->window, p->radius, p->bsize);
    if (rc)
        return rc;
    if (p->heads < 0 || p->d < 1)
        return ORC_E_INVALID;
    if (!(p->scale > 0.0) || !isfinite(p->scale))
        return ORC_E_INVALID;
    return 0;
}

/* scale <= 0 selects 1/sqrt(d), the scaling of section 3's score formula. */
static double pick_scale(double scale, int d) { return scale > 0.0 ? scale : 1.0 / sqrt((double)d); }

/* Full forward: o [batch][heads][n][d], lse and psum [batch][heads][n] (either
 * may be NULL). */
int orc_forward_w_f64(int batch, int heads, int n, int d, int bsize, int radius, int causal,
                      int window, double scale, const int32_t *seqlens, const float *q,
                      const float *k, const float *v, double *o, double *lse, double *psum,
                      int nthreads)
{
    problem p = {batch, heads, n, d, bsize, radius, causal, pick_scale(scale, d), seqlens, q, k, v,
                 window};
    int rc = check_problem(&p);
    if (rc)
        return rc;
    const int64_t nwork = (int64_t)batch * heads * (n / bsize);
    if (nwork == 0)
        return 0;
    if (!q || !k || !v || !o)
        return ORC_E_INVALID;
    job jb;
    memset(&jb, 0, sizeof jb);
    jb.p = &p;
    jb.nsel = nwork;
    jb.sel = NULL;
    jb.o = o;
    jb.lse = lse;
    jb.psum = psum;
    return run_pool(&jb, nthreads);
}

/* Selected query blocks only: sel[w] = (b, h, i).  o [nsel][bsize][d], lse and
 * psum [nsel][bsize].  The inputs are the full-size tensors. */
int orc_forward_blocks_w_f64(int batch, int heads, int n, int d, int bsize, int radius,
                             int causal, int window, double scale, const int32_t *seqlens,
                             const float *q, const float *k, const float *v, int64_t nsel,
                             const int32_t *sel, double *o, double *lse, double *psum,
                             int nthreads)
{
    problem p = {batch, heads, n, d, bsize, radius, causal, pick_scale(scale, d), seqlens, q, k, v,
                 window};
    int rc = check_problem(&p);
    if (rc)
        return rc;
    if (nsel < 0)
        return ORC_E_INVALID;
    if (nsel == 0)
        return 0;
    if (!q || !k || !v || !o || !sel)
        return ORC_E_INVALID;
    for (int64_t w = 0; w < nsel; ++w) {
        const int32_t *s = sel + 3 * w;
        if (s[0] < 0 || s[0] >= batch || s[1] < 0 || s[1] >= heads || s[2] < 0 ||
            s[2] >= n / bsize)
            return ORC_E_INVALID;
    }
    job jb;
    memset(&jb, 0, sizeof jb);
    jb.p = &p;
    jb.nsel = nsel;
    jb.sel = sel;
    jb.o = o;
    jb.lse = lse;
    jb.psum = psum;
    return run_pool(&jb, nthreads);
}

/* ------------------------------------------- the page's running recurrence */

/* Section 3's update taken block by block, in order of ascending key block:
 *   m_new = max(m_old, max_c S_ic)
 *   d_new = d_old * exp(m_old - m_new) + sum_c exp(S_ic - m_new)
 *   O_new = O_old * exp(m_old - m_new) + sum_c exp(S_ic - m_new) V_c
 * per query row, starting from m = -inf, d = 0, O = 0, with masked scores set to
 * -inf; after the last block O / d is the output.  Single threaded. */
int orc_forward_recurrence_w_f64(int batch, int heads, int n, int d, int bsize, int radius,
                                 int causal, int window, double scale, const int32_t *seqlens,
                                 const float *q, const float *k, const float *v, double *o)
{
    problem p = {batch, heads, n, d, bsize, radius, causal, pick_scale(scale, d), seqlens, q, k, v,
                 window};
    int rc = check_problem(&p);
    if (rc)
        return rc;
    const int nblk = n / bsize;
    if ((int64_t)batch * heads * nblk == 0)
        return 0;
    if (!q || !k || !v || !o)
        return ORC_E_INVALID;
    double *sblk = (double *)malloc(sizeof(double) * (size_t)bsize);
    double *acc = (double *)malloc(sizeof(double) * (size_t)d);
    if (!sblk || !acc) {
        free(sblk);
        free(acc);
        return ORC_E_NOMEM;
    }
    for (int b = 0; b < batch; ++b) {
        const int len = seq_len(seqlens, b, n);
        const int nb = blocks_of(len, bsize);
        for (int h = 0; h < heads; ++h) {
            const int64_t base = ((int64_t)b * heads + h) * n;
            for (int t = 0; t < n; ++t) {
                double *out = o + (base + t) * d;
                if (t >= len) {
                    for (int c = 0; c < d; ++c)
                        out[c] = 0.0;
                    continue;
                }
                const int i = t / bsize;
                double m_old = -INFINITY, den = 0.0;
                for (int c = 0; c < d; ++c)
                    acc[c] = 0.0;
                for (int j = i - radius; j <= i + radius; ++j) {
                    if (!block_in_band(i, j, radius, nb, causal))
                        continue;
                    double bmax = -INFINITY;
                    for (int c = 0; c < bsize; ++c) {
                        const int s = j * bsize + c;
                        double sc = -INFINITY;
                        if (pair_kept(t, s, len, bsize, radius, causal, window)) {
                            double dot = 0.0;
                            for (int e = 0; e < d; ++e)
                                dot += (double)q[(base + t) * d + e] * (double)k[(base + s) * d + e];
                            sc = p.scale * dot;
                        }
                        sblk[c] = sc;
                        if (sc > bmax)
                            bmax = sc;
                    }
                    const double m_new = bmax > m_old ? bmax : m_old;
                    if (m_new == -INFINITY)
                        continue; /* every key of this block masked: nothing to add */
                    const double corr = exp(m_old - m_new); /* 0 on the first block */
                    double add = 0.0;
                    for (int e = 0; e < d; ++e)
                        acc[e] *= corr;
                    for (int c = 0; c < bsize; ++c) {
                        const double w = exp(sblk[c] - m_new);
                        if (w == 0.0)
                            continue;
                        add += w;
                        const float *vs = v + (base + (int64_t)j * bsize + c) * d;
                        for (int e = 0; e < d; ++e)
                            acc[e] += w * (double)vs[e];
                    }
                    den = den * corr + add;
                    m_old = m_new;
                }
                for (int c = 0; c < d; ++c)
                    out[c] = acc[c] / den;
            }
        }
    }
    free(sblk);
    free(acc);
    return 0;
}

/* The entry points without a token window: the block band alone. */
int orc_masks(int batch, int n, int bsize, int radius, int causal, const int32_t *seqlens,
              const int32_t *active, uint32_t *masks)
{
    return orc_masks_w(batch, n, bsize, radius, causal, -1, seqlens, active, masks);
}

int orc_forward_f64(int batch, int heads, int n, int d, int bsize, int radius, int causal,
                    double scale, const int32_t *seqlens, const float *q, const float *k,
                    const float *v, double *o, double *lse, double *psum, int nthreads)
{
    return orc_forward_w_f64(batch, heads, n, d, bsize, radius, causal, -1, scale, seqlens, q, k, v,
                             o, lse, psum, nthreads);
}

int orc_forward_blocks_f64(int batch, int heads, int n, int d, int bsize, int radius, int causal,
                           double scale, const int32_t *seqlens, const float *q, const float *k,
                           const float *v, int64_t nsel, const int32_t *sel, double *o,
                           double *lse, double *psum, int nthreads)
{
    return orc_forward_blocks_w_f64(batch, heads, n, d, bsize, radius, causal, -1, scale, seqlens,
                                    q, k, v, nsel, sel, o, lse, psum, nthreads);
}

int orc_forward_recurrence_f64(int batch, int heads, int n, int d, int bsize, int radius,
                               int causal, double scale, const int32_t *seqlens, const float *q,
                               const float *k, const float *v, double *o)
{
    return orc_forward_recurrence_w_f64(batch, heads, n, d, bsize, radius, causal, -1, scale,
                                        seqlens, q, k, v, o);
}

/* ------------------------------------------------------------ backward pass */

typedef struct {
    problem fw;
    const float *dout;
} bproblem;

/* Gradient contributions of query row t of (b, h), from the definition:
 * recompute the row's kept keys, P and O, then D_t, dS_ts, and add
 *   dq_row += scale * dS_ts K_s                      (always)
 *   dk[s], dv[s] += scale * dS_ts Q_t, P_ts dO_t     (for keys s in [klo, khi))
 * dk and dv point at key row klo.  Rows t >= len contribute nothing. */
static void row_backward(const bproblem *bp, int b, int h, int t, double *sbuf, int32_t *sidx,
                         double *orow, double *dq_row, int klo, int khi, double *dk, double *dv)
{
    const problem *p = &bp->fw;
    const int len = seq_len(p->seqlens, b, p->n);
    if (t >= len)
        return;
    const int64_t base = ((int64_t)b * p->heads + h) * p->n;
    const int d = p->d;
    /* P (in sbuf, over the kept keys sidx) and O of this row */
    double lse;
    row_definition(p, b, h, t, sbuf, sidx, orow, &lse, NULL);
    int cnt = 0;
    {
        /* row_definition leaves exp(S - M) in sbuf for the kept keys in
         * ascending order; recount them and normalise */
        const int ib = t / p->bsize;
        int s_lo = (ib - p->radius) * p->bsize, s_hi = (ib + p->radius + 1) * p->bsize;
        if (s_lo < 0)
            s_lo = 0;
        if (s_hi > len)
            s_hi = len;
        for (int s = s_lo; s < s_hi; ++s)
            if (pair_kept(t, s, len, p->bsize, p->radius, p->causal, p->window))
                ++cnt;
        double l = 0.0;
        for (int e = 0; e < cnt; ++e)
            l += sbuf[e];
        for (int e = 0; e < cnt; ++e)
            sbuf[e] /= l;
    }
    const float *q_row = p->q + (base + t) * d;
    const float *dot_ = bp->dout + (base + t) * d;
    double Dt = 0.0;
    for (int c = 0; c < d; ++c)
        Dt += (double)dot_[c] * orow[c];
    for (int e = 0; e < cnt; ++e) {
        const int s = sidx[e];
        const double P = sbuf[e];
        const float *vs = p->v + (base + s) * d;
        double dP = 0.0;
        for (int c = 0; c < d; ++c)
            dP += (double)dot_[c] * (double)vs[c];
        const double dS = P * (dP - Dt);
        const float *ks = p->k + (base + s) * d;
        if (dq_row)
            for (int c = 0; c < d; ++c)
                dq_row[c] += p->scale * dS * (double)ks[c];
        if (s >= klo && s < khi) {
            double *dks = dk + (int64_t)(s - klo) * d, *dvs = dv + (int64_t)(s - klo) * d;
            for (int c = 0; c < d; ++c) {
                dks[c] += p->scale * dS * (double)q_row[c];
                dvs[c] += P * (double)dot_[c];
            }
        }
    }
}

typedef struct {
    const bproblem *bp;
    int64_t nwork;
    const int32_t *sel; /* NULL: every (b, h) slice; else (b, h, i) triples */
    double *dq, *dk, *dv;
    int64_t next;
    pthread_mutex_t lock;
    int failed;
} bjob;

static void *bworker(void *arg)
{
    bjob *jb = (bjob *)arg;
    const problem *p = &jb->bp->fw;
    const int maxkeys = (2 * p->radius + 1) * p->bsize;
    const int d = p->d, B = p->bsize, nblk = p->n / B;
    double *sbuf = (double *)malloc(sizeof(double) * (size_t)maxkeys);
    int32_t *sidx = (int32_t *)malloc(sizeof(int32_t) * (size_t)maxkeys);
    double *orow = (double *)malloc(sizeof(double) * (size_t)d);
    if (!sbuf || !sidx || !orow) {
        free(sbuf);
        free(sidx);
        free(orow);
        pthread_mutex_lock(&jb->lock);
        jb->failed = 1;
        pthread_mutex_unlock(&jb->lock);
        return NULL;
    }
    for (;;) {
        pthread_mutex_lock(&jb->lock);
        const int64_t w = jb->next++;
        pthread_mutex_unlock(&jb->lock);
        if (w >= jb->nwork)
            break;
        if (!jb->sel) {
            /* whole slice (b, h): every row adds into its slice of dq, dk, dv */
            const int b = (int)(w / p->heads), h = (int)(w % p->heads);
            const int64_t off = ((int64_t)b * p->heads + h) * p->n * d;
            for (int t = 0; t < p->n; ++t)
                row_backward(jb->bp, b, h, t, sbuf, sidx, orow, jb->dq + off + (int64_t)t * d, 0,
                             p->n, jb->dk + off, jb->dv + off);
        } else {
            /* one block index i: dQ of query block i, dK and dV of key block i;
             * the latter gather every row whose band holds key block i */
            const int b = jb->sel[3 * w], h = jb->sel[3 * w + 1], i = jb->sel[3 * w + 2];
            double *dq = jb->dq + w * (int64_t)B * d;
            double *dk = jb->dk + w * (int64_t)B * d, *dv = jb->dv + w * (int64_t)B * d;
            for (int r = 0; r < B; ++r)
                row_backward(jb->bp, b, h, i * B + r, sbuf, sidx, orow, dq + (int64_t)r * d, 0, 0,
                             NULL, NULL);
            for (int qi = i - p->radius; qi <= i + p->radius; ++qi) {
                if (qi < 0 || qi >= nblk)
                    continue;
                for (int r = 0; r < B; ++r)
                    row_backward(jb->bp, b, h, qi * B + r, sbuf, sidx, orow, NULL, i * B,
                                 (i + 1) * B, dk, dv);
            }
        }
    }
    free(sbuf);
    free(sidx);
    free(orow);
    return NULL;
}

static int run_bpool(bjob *jb, int nthreads)
{
    if (nthreads < 1)
        nthreads = 1;
    if (nthreads > 1024)
        nthreads = 1024;
    pthread_mutex_init(&jb->lock, NULL);
    jb->next = 0;
    jb->failed = 0;
    pthread_t *tid = (pthread_t *)malloc(sizeof(pthread_t) * (size_t)nthreads);
    if (!tid)
        return ORC_E_NOMEM;
    int started = 0;
    for (int t = 0; t < nthreads; ++t) {
        if (pthread_create(&tid[t], NULL, bworker, jb) != 0)
            break;
        ++started;
    }
    if (started == 0)
        bworker(jb);
    for (int t = 0; t < started; ++t)
        pthread_join(tid[t], NULL);
    free(tid);
    pthread_mutex_destroy(&jb->lock);
    return jb->failed ? ORC_E_NOMEM : 0;
}

/* Full backward: dq, dk, dv [batch][heads][n][d] (overwritten), from the
 * forward's inputs and the output gradient dout [batch][heads][n][d].  With
 * window >= 0 the forward is the token-window one (radius = ceil(W / B)). */
int orc_backward_w_f64(int batch, int heads, int n, int d, int bsize, int radius, int causal,
                       int window, double scale, const int32_t *seqlens, const float *q,
                       const float *k, const float *v, const float *dout, double *dq, double *dk,
                       double *dv, int nthreads)
{
    bproblem bp = {{batch, heads, n, d, bsize, radius, causal, pick_scale(scale, d), seqlens, q, k, v,
                    window},
                   dout};
    int rc = check_problem(&bp.fw);
    if (rc)
        return rc;
    rc = check_window(window, radius, bsize);
    if (rc)
        return rc;
    const int64_t total = (int64_t)batch * heads * n * d;
    if (total == 0)
        return 0;
    if (!q || !k || !v || !dout || !dq || !dk || !dv)
        return ORC_E_INVALID;
    memset(dq, 0, sizeof(double) * (size_t)total);
    memset(dk, 0, sizeof(double) * (size_t)total);
    memset(dv, 0, sizeof(double) * (size_t)total);
    bjob jb;
    memset(&jb, 0, sizeof jb);
    jb.bp = &bp;
    jb.nwork = (int64_t)batch * heads;
    jb.dq = dq;
    jb.dk = dk;
    jb.dv = dv;
    return run_bpool(&jb, nthreads);
}

/* Selected block indices sel[w] = (b, h, i): dq [nsel][bsize][d] gets the rows
 * of query block i, dk and dv [nsel][bsize][d] the rows of key block i. */
int orc_backward_blocks_w_f64(int batch, int heads, int n, int d, int bsize, int radius,
                              int causal, int window, double scale, const int32_t *seqlens,
                              const float *q, const float *k, const float *v, const float *dout,
                              int64_t nsel, const int32_t *sel, double *dq, double *dk, double *dv,
                              int nthreads)
{
    bproblem bp = {{batch, heads, n, d, bsize, radius, causal, pick_scale(scale, d), seqlens, q, k, v,
                    window},
                   dout};
    int rc = check_problem(&bp.fw);
    if (rc)
        return rc;
    rc = check_window(window, radius, bsize);
    if (rc)
        return rc;
    if (nsel < 0)
        return ORC_E_INVALID;
    if (nsel == 0)
        return 0;
    if (!q || !k || !v || !dout || !dq || !dk || !dv || !sel)
        return ORC_E_INVALID;
    for (int64_t w = 0; w < nsel; ++w) {
        const int32_t *s = sel + 3 * w;
        if (s[0] < 0 || s[0] >= batch || s[1] < 0 || s[1] >= heads || s[2] < 0 ||
            s[2] >= n / bsize)
            return ORC_E_INVALID;
    }
    const size_t per = sizeof(double) * (size_t)nsel * (size_t)bsize * (size_t)d;
    memset(dq, 0, per);
    memset(dk, 0, per);
    memset(dv, 0, per);
    bjob jb;
    memset(&jb, 0, sizeof jb);
    jb.bp = &bp;
    jb.nwork = nsel;
    jb.sel = sel;
    jb.dq = dq;
    jb.dk = dk;
    jb.dv = dv;
    return run_bpool(&jb, nthreads);
}

/* The backward entry points without a token window: the block band alone. */
int orc_backward_f64(int batch, int heads, int n, int d, int bsize, int radius, int causal,
                     double scale, const int32_t *seqlens, const float *q, const float *k,
                     const float *v, const float *dout, double *dq, double *dk, double *dv,
                     int nthreads)
{
    return orc_backward_w_f64(batch, heads, n, d, bsize, radius, causal, -1, scale, seqlens, q, k,
                              v, dout, dq, dk, dv, nthreads);
}

int orc_backward_blocks_f64(int batch, int heads, int n, int d, int bsize, int radius, int causal,
                            double scale, const int32_t *seqlens, const float *q, const float *k,
                            const float *v, const float *dout, int64_t nsel, const int32_t *sel,
                            double *dq, double *dk, double *dv, int nthreads)
{
    return orc_backward_blocks_w_f64(batch, heads, n, d, bsize, radius, causal, -1, scale, seqlens,
                                     q, k, v, dout, nsel, sel, dq, dk, dv, nthreads);
}

/* ------------------------------------------------------------------ k-mers */

/* The two-bit code of one base, or -1 for anything that is not a base. */
static int base_code(uint8_t c)
{
    switch (c) {
    case 'A': case 'a': return 0;
    case 'C': case 'c': return 1;
    case 'G': case 'g': return 2;
    case 'T': case 't': return 3;
    default: return -1;
    }
}

/* bases: the sequences' ASCII bytes back to back; starts[batch + 1]: sequence b
 * is bytes [starts[b], starts[b+1]).  ids [batch][n_out] receives window IDs
 * (PAD past the sequence's last window), ntok[batch] the number of windows
 * written: min(max(len - k + 1, 0), n_out). */
int orc_kmer_tokenize(int batch, const uint8_t *bases, const int64_t *starts, int k, int n_out,
                      int32_t *ids, int32_t *ntok)
{
    if (batch < 0 || k < 1 || k > 12 || n_out < 0 || !starts || (batch > 0 && (!ids || !ntok)))
        return ORC_E_INVALID;
    if (starts[0] < 0)
        return ORC_E_INVALID;
    for (int b = 0; b < batch; ++b)
        if (starts[b + 1] < starts[b])
            return ORC_E_INVALID;
    if (batch > 0 && starts[batch] > starts[0] && !bases)
        return ORC_E_INVALID;
    const int32_t four_k = 1 << (2 * k);
    const int32_t pad = four_k, unk = four_k + 2;
    for (int b = 0; b < batch; ++b) {
        const int64_t len = starts[b + 1] - starts[b];
        int64_t nt = len - k + 1;
        if (nt < 0)
            nt = 0;
        if (nt > n_out)
            nt = n_out;
        ntok[b] = (int32_t)nt;
        const uint8_t *seq = bases + starts[b];
        for (int64_t t = 0; t < n_out; ++t) {
            int32_t id = pad;
            if (t < nt) {
                int64_t value = 0, place = 1;
                int bad = 0;
                for (int p = k - 1; p >= 0; --p) {   /* last base is the least significant */
                    const int c = base_code(seq[t + p]);
                    if (c < 0)
                        bad = 1;
                    else
                        value += c * place;
                    place *= 4;
                }
                id = bad ? unk : (int32_t)value;
            }
            ids[(int64_t)b * n_out + t] = id;
        }
    }
    return 0;
}
