/*
 * spec_oracle.c -- CPU oracle for the verify/accept step of block speculative
 * decoding (greedy accept and lossless speculative-sampling accept).
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the slow, plain, single-threaded,
 * double-precision statement of what the GPU path must compute.  Only the
 * test suite, the smoke check and the benchmark's CPU-baseline leg load it.
 * It shares no source, header, table or helper with the HIP library.
 *
 * Sources for what is computed:
 *  - "dspark-mlx 0.1.0" wheel diff, dspark_mlx/adapter.py, module docstring
 *    ("Logit conventions (one decode cycle)"): row 0 of the target block is
 *    p_1 from the anchor step, rows 1..K are p_2..p_{K+1} from one verify
 *    forward, row K being the bonus position; the accept policy consumes the
 *    [K+1, V] block.  BaseModelAdapter.kv_rollback(n_keep) consumes the
 *    accepted count.
 *  - same page, dspark_mlx/__init__.py: the policy exports greedy_accept,
 *    speculative_sample_accept and AcceptResult (bodies not on the page).
 *  - "mlx-dspark 0.0.1" sdist diff, README "How it works": greedy output is
 *    identical to plain greedy decoding (target argmax chain) up to near-tie
 *    floating-point tie-breaking; benchmark.py takes the plain greedy token
 *    as the argmax of the raw last-position logits.
 *  - "DeepSeek-V4-Flash DSpark drafter" model card: decoding is lossless, the
 *    target's verify forward being the sole token source.
 *  - The sampling rule itself is the published speculative-sampling rule
 *    (Leviathan, Kalman & Matias, ICML 2023; Chen et al., 2023): accept draft
 *    token x with probability min(1, p(x)/q(x)); on rejection resample from
 *    normalise(max(0, p - q)); if all K drafts are accepted draw one more
 *    token from the last target distribution.
 *  - Uniforms: Philox4x32-10 (Salmon, Moraes, Dror & Shaw, "Parallel Random
 *    Numbers: As Easy as 1, 2, 3", SC'11), keyed by the 64-bit seed, counter
 *    (position, batch row, tag, 0).
 *
 * Readings where the pages are silent (each is also listed in the design
 * notes): lowest index wins an exact argmax tie; greedy compares raw logits;
 * temperature divides the logits of both sides; the accept test is strict
 * u < min(1, r); p(x) = 0 rejects, q(x) = 0 < p(x) accepts; the resample and
 * the bonus use their own uniform (tag 1) at the slot they fill; the CDF
 * search walks ascending vocabulary index and returns the first v whose
 * running sum exceeds t = u' * R; a row holding NaN or +inf, or only -inf,
 * makes its sequence invalid (n = -1, all tokens -1).
 *
 * Numerics: every logit is widened exactly to double (bf16 bits << 16, or
 * fp32), all arithmetic is in double, every sum runs sequentially in
 * ascending vocabulary index.
 */
/*
 * Planted-mistake builds, used only by the tests' negative controls to show
 * that a pin has the power to catch a plausible error (never the default):
 *   ORACLE_MUTANT=1  resample a rejected slot from p_n, not the residual
 *   ORACLE_MUTANT=2  residual with its sign flipped, max(0, q - p)
 *   ORACLE_MUTANT=3  bonus drawn from p_K instead of p_{K+1}
 *   ORACLE_MUTANT=4  greedy ties go to the last maximal index
 *   ORACLE_MUTANT=5  temperature applied to the target side only
 *   ORACLE_MUTANT=6  zero residual mass draws from the block's last row
 *                    p_{Ks+1} instead of p_n
 *   ORACLE_MUTANT=7  zero residual mass has no fallback (the draw finds no
 *                    token)
 *   ORACLE_MUTANT=8  the rounding fallback takes the FIRST entry of positive
 *                    weight instead of the last
 */
#ifndef ORACLE_MUTANT
#define ORACLE_MUTANT 0
#endif

#include <math.h>
#include <stdint.h>
#include <string.h>
#include <stdlib.h>

#define OR_F32 0
#define OR_BF16 1

/* ------------------------------------------------------------------------ */
/* Input widening.                                                           */

static double logit_at(const void *base, int dtype, int64_t idx)
{
    if (dtype == OR_F32) {
        return (double)((const float *)base)[idx];
    }
    uint32_t bits = (uint32_t)((const uint16_t *)base)[idx] << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
}

/* ------------------------------------------------------------------------ */
/* Philox4x32-10, from the SC'11 paper's definition: each round multiplies   */
/* counter words 0 and 2 by the two round multipliers, keeps the 64-bit      */
/* products split into high and low halves, xors the high halves with the    */
/* other two counter words and the round key, and permutes; the key is       */
/* bumped by the two Weyl constants between rounds.                          */

void oracle_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2],
                          uint32_t out[4])
{
    const uint32_t M0 = 0xD2511F53u, M1 = 0xCD9E8D57u;
    const uint32_t W0 = 0x9E3779B9u, W1 = 0xBB67AE85u;
    uint32_t c0 = ctr[0], c1 = ctr[1], c2 = ctr[2], c3 = ctr[3];
    uint32_t k0 = key[0], k1 = key[1];
    for (int round = 0; round < 10; ++round) {
        if (round > 0) {
            k0 += W0;
            k1 += W1;
        }
        uint64_t prod0 = (uint64_t)M0 * (uint64_t)c0;
        uint64_t prod1 = (uint64_t)M1 * (uint64_t)c2;
        uint32_t hi0 = (uint32_t)(prod0 >> 32), lo0 = (uint32_t)prod0;
        uint32_t hi1 = (uint32_t)(prod1 >> 32), lo1 = (uint32_t)prod1;
        uint32_t n0 = hi1 ^ c1 ^ k0;
        uint32_t n1 = lo1;
        uint32_t n2 = hi0 ^ c3 ^ k1;
        uint32_t n3 = lo0;
        c0 = n0; c1 = n1; c2 = n2; c3 = n3;
    }
    out[0] = c0; out[1] = c1; out[2] = c2; out[3] = c3;
}

/* U(seed, row, pos, tag): word 0 of Philox4x32-10 at counter
 * (pos, row, tag, 0) under key (low 32 bits of seed, high 32 bits of seed),
 * keeping its top 24 bits: U = (w >> 8) * 2^-24, a value in [0, 1 - 2^-24]
 * that is exact in both float and double. */
double oracle_uniform(uint64_t seed, uint32_t row, uint32_t pos, uint32_t tag)
{
    uint32_t ctr[4] = {pos, row, tag, 0u};
    uint32_t key[2] = {(uint32_t)(seed & 0xFFFFFFFFu), (uint32_t)(seed >> 32)};
    uint32_t out[4];
    oracle_philox4x32_10(ctr, key, out);
    return (double)(out[0] >> 8) * (1.0 / 16777216.0);
}

/* The same uniforms on a grid of counters: out[r * npos + p] =
 * U(seed, row0 + r, pos0 + p, tag), row and position wrapping mod 2^32. */
void oracle_uniform_grid(uint64_t seed, uint32_t row0, int nrow, uint32_t pos0, int npos,
                         uint32_t tag, double *out)
{
    for (int r = 0; r < nrow; ++r) {
        for (int p = 0; p < npos; ++p) {
            out[(int64_t)r * npos + p] = oracle_uniform(seed, row0 + (uint32_t)r,
                                                        pos0 + (uint32_t)p, tag);
        }
    }
}

/* ------------------------------------------------------------------------ */
/* Row validity: a row is usable when it holds no NaN, no +inf and at least  */
/* one finite value (-inf entries are masked vocabulary and are allowed).    */

static int row_is_valid(const void *base, int dtype, int64_t off, int V)
{
    int any_finite = 0;
    for (int v = 0; v < V; ++v) {
        double z = logit_at(base, dtype, off + v);
        if (isnan(z) || z == INFINITY) {
            return 0;
        }
        if (z != -INFINITY) {
            any_finite = 1;
        }
    }
    return any_finite;
}

/* First index of the largest raw logit (numpy / torch argmax convention). */
static int32_t row_argmax(const void *base, int dtype, int64_t off, int V)
{
    int32_t best = 0;
    double best_z = logit_at(base, dtype, off);
    for (int v = 1; v < V; ++v) {
        double z = logit_at(base, dtype, off + v);
#if ORACLE_MUTANT == 4
        if (z >= best_z) {
#else
        if (z > best_z) {
#endif
            best_z = z;
            best = v;
        }
    }
    return best;
}

/* Log-normaliser of softmax(z / T), kept as the pair (M, L) with
 * M = max_v z_v (the raw logits) and L = ln sum_v exp((z_v - M) / T), so that
 * ln p(v) = (z_v - M) / T - L.  This is the log-sum-exp of z / T with the
 * row maximum subtracted before the division: z_v - M is exact in double for
 * float inputs, where z_v / T - (m + ln S) would lose |z / T| 2^-53 to the
 * magnitude (1e-4 relative in p at |z / T| = 1e12). */
typedef struct {
    double M, L;
} RowNorm;

static RowNorm row_log_normaliser(const void *base, int dtype, int64_t off,
                                  int V, double T)
{
    RowNorm n;
    n.M = -INFINITY;
    for (int v = 0; v < V; ++v) {
        double z = logit_at(base, dtype, off + v);
        if (z > n.M) {
            n.M = z;
        }
    }
    double S = 0.0;
    for (int v = 0; v < V; ++v) {
        S += exp((logit_at(base, dtype, off + v) - n.M) / T);
    }
    n.L = log(S);
    return n;
}

/* ln p(v) of logit z under the row's log-normaliser. */
static double log_prob(double z, RowNorm n, double T)
{
    return (z - n.M) / T - n.L;
}

/* ------------------------------------------------------------------------ */
/* Greedy accept.                                                            */
/* For each sequence: A_i = argmax of target row i (i = 0..K); n = length of  */
/* the longest prefix with x_i == A_i; committed tokens x_0..x_{n-1}, A_n,    */
/* then -1 up to K+1 entries.                                                */
/* A sequence may carry only Ks <= K draft tokens (a shorter block): then     */
/* rows 0..Ks and tokens 0..Ks-1 are its block, row Ks its bonus position,    */
/* and the rest of its [K+1] / [K] storage is not read.  K is the stride.     */

static void greedy_sequence(const void *target, int dtype,
                            int64_t t_batch_stride, int64_t t_row_stride,
                            const int32_t *draft_tokens, int s, int K, int Ks, int V,
                            int32_t *n_accepted, int32_t *tokens,
                            int32_t *target_argmax)
{
    int valid = 1;
    int32_t *A = (int32_t *)calloc((size_t)(K + 1), sizeof(int32_t));
    for (int i = 0; i <= K; ++i) {
        A[i] = -1;
    }
    for (int i = 0; i <= Ks; ++i) {
        int64_t off = (int64_t)s * t_batch_stride + (int64_t)i * t_row_stride;
        if (!row_is_valid(target, dtype, off, V)) {
            valid = 0;
            A[i] = -1;
        } else {
            A[i] = row_argmax(target, dtype, off, V);
        }
    }
    for (int i = 0; i < Ks; ++i) {
        int32_t x = draft_tokens[(int64_t)s * K + i];
        if (x < 0 || x >= V) {
            valid = 0;
        }
    }
    int32_t *tok = tokens + (int64_t)s * (K + 1);
    for (int j = 0; j <= K; ++j) {
        tok[j] = -1;
    }
    if (target_argmax) {
        for (int i = 0; i <= K; ++i) {
            target_argmax[(int64_t)s * (K + 1) + i] = valid ? A[i] : -1;
        }
    }
    if (!valid) {
        n_accepted[s] = -1;
        free(A);
        return;
    }
    int n = 0;
    while (n < Ks && draft_tokens[(int64_t)s * K + n] == A[n]) {
        ++n;
    }
    for (int j = 0; j < n; ++j) {
        tok[j] = draft_tokens[(int64_t)s * K + j];
    }
    tok[n] = A[n];
    n_accepted[s] = n;
    free(A);
}

int oracle_greedy_accept(const void *target, int dtype,
                         int64_t t_batch_stride, int64_t t_row_stride,
                         const int32_t *draft_tokens, int b, int K, int V,
                         int32_t *n_accepted, int32_t *tokens,
                         int32_t *target_argmax)
{
    if (b < 1 || K < 1 || V < 1 || (dtype != OR_F32 && dtype != OR_BF16)) {
        return 1;
    }
    for (int s = 0; s < b; ++s) {
        greedy_sequence(target, dtype, t_batch_stride, t_row_stride, draft_tokens, s, K, K, V,
                        n_accepted, tokens, target_argmax);
    }
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Speculative-sampling accept.                                              */

/* Weight w_v of vocabulary entry v for the token drawn at a slot, given the
 * log-normalisers of that slot's rows: the residual max(0, p(v) - q(v)) when
 * `residual` is set, else the target probability p(v) (the bonus from
 * p_{K+1}, or a rejected slot whose residual mass is zero). */
static double draw_weight(const void *target, const void *draft, int dtype,
                          int64_t t_off, int64_t d_off, int v, double T,
                          RowNorm Ct, RowNorm Cd, int residual)
{
    double p = exp(log_prob(logit_at(target, dtype, t_off + v), Ct, T));
    if (!residual) {
        return p;
    }
    double q = exp(log_prob(logit_at(draft, dtype, d_off + v), Cd, T));
#if ORACLE_MUTANT == 1
    double w = p + 0.0 * q;
#elif ORACLE_MUTANT == 2
    double w = q - p;
#else
    double w = p - q;
#endif
    return w > 0.0 ? w : 0.0;
}

/* Per-sequence diagnostics written by oracle_sample_accept when `diag` is
 * not NULL: diag[s * (2K + 4) + ...] =
 *   [0 .. K)      r_i = exp(d_i), the accept ratio of slot i (all slots)
 *   [K .. 2K)     u_i = U(seed_s, s, i, 0)
 *   2K            t   = u' * R for the drawn token
 *   2K + 1        R   = total draw mass
 *   2K + 2        u'  = U(seed_s, s, n, 1)
 *   2K + 3        1 when the draw used the residual, 0 for p (bonus or R=0)
 */
static void sample_sequence(const void *target, const void *draft, int dtype,
                            int64_t t_batch_stride, int64_t t_row_stride,
                            int64_t d_batch_stride, int64_t d_row_stride,
                            const int32_t *draft_tokens, int s, int K, int Ks, int V,
                            double T, const uint64_t *seeds,
                            int32_t *n_accepted, int32_t *tokens,
                            double *p_draft, double *q_draft, double *diag)
{
    const int dstride = 2 * K + 4;
    const int32_t *x = draft_tokens + (int64_t)s * K;
    int32_t *tok = tokens + (int64_t)s * (K + 1);
    for (int j = 0; j <= K; ++j) {
        tok[j] = -1;
    }
    for (int i = 0; i < K; ++i) {          /* slots past the block report NaN */
        p_draft[(int64_t)s * K + i] = NAN;
        q_draft[(int64_t)s * K + i] = NAN;
    }
    if (diag) {
        for (int j = 0; j < dstride; ++j) {
            diag[(int64_t)s * dstride + j] = NAN;
        }
    }
    int valid = 1;
    for (int i = 0; i <= Ks && valid; ++i) {
        int64_t off = (int64_t)s * t_batch_stride + (int64_t)i * t_row_stride;
        valid = row_is_valid(target, dtype, off, V);
    }
    for (int i = 0; i < Ks && valid; ++i) {
        int64_t off = (int64_t)s * d_batch_stride + (int64_t)i * d_row_stride;
        valid = row_is_valid(draft, dtype, off, V);
    }
    for (int i = 0; i < Ks; ++i) {
        if (x[i] < 0 || x[i] >= V) {
            valid = 0;
        }
    }
    if (!valid) {
        n_accepted[s] = -1;
        for (int i = 0; i < K; ++i) {
            p_draft[(int64_t)s * K + i] = NAN;
            q_draft[(int64_t)s * K + i] = NAN;
        }
        if (diag) {
            for (int j = 0; j < dstride; ++j) {
                diag[(int64_t)s * dstride + j] = NAN;
            }
        }
        return;
    }

    /* Step 1: log-normalisers of every target and draft row. */
    RowNorm *Ct = (RowNorm *)malloc(sizeof(RowNorm) * (size_t)(K + 1));
    RowNorm *Cd = (RowNorm *)malloc(sizeof(RowNorm) * (size_t)(K + 1));
    for (int i = 0; i <= Ks; ++i) {
        Ct[i] = row_log_normaliser(target, dtype,
                                   (int64_t)s * t_batch_stride + (int64_t)i * t_row_stride,
                                   V, T);
    }
#if ORACLE_MUTANT == 5
    const double Tq = 1.0;
#else
    const double Tq = T;
#endif
    for (int i = 0; i < Ks; ++i) {
        Cd[i] = row_log_normaliser(draft, dtype,
                                   (int64_t)s * d_batch_stride + (int64_t)i * d_row_stride,
                                   V, Tq);
    }

    /* Step 2: accept test of every slot, stopping the prefix at the first
     * rejection; ratios and probabilities are reported for all Ks slots. */
    int n = Ks;
    for (int i = 0; i < Ks; ++i) {
        int64_t toff = (int64_t)s * t_batch_stride + (int64_t)i * t_row_stride;
        int64_t doff = (int64_t)s * d_batch_stride + (int64_t)i * d_row_stride;
        double lp = log_prob(logit_at(target, dtype, toff + x[i]), Ct[i], T);
        double lq = log_prob(logit_at(draft, dtype, doff + x[i]), Cd[i], Tq);
        double p = exp(lp), q = exp(lq);
        double r;
        if (lp == -INFINITY) {
            r = 0.0;               /* p(x) = 0: never accepted */
        } else if (lq == -INFINITY) {
            r = INFINITY;          /* q(x) = 0 < p(x): always accepted */
        } else {
            r = exp(lp - lq);
        }
        double u = oracle_uniform(seeds[s], (uint32_t)s, (uint32_t)i, 0u);
        p_draft[(int64_t)s * K + i] = p;
        q_draft[(int64_t)s * K + i] = q;
        if (diag) {
            diag[(int64_t)s * dstride + i] = r;
            diag[(int64_t)s * dstride + K + i] = u;
        }
        double accept_prob = r < 1.0 ? r : 1.0;
        if (n == Ks && !(u < accept_prob)) {
            n = i;
        }
    }

    /* Step 3: draw the token at slot n: residual when n < Ks, bonus from
     * the block's last row when n == Ks; inverse CDF in ascending vocabulary
     * order. */
#if ORACLE_MUTANT == 3
    const int draw_row = n < Ks ? n : (Ks > 0 ? Ks - 1 : 0);
#else
    const int draw_row = n;
#endif
    int64_t toff = (int64_t)s * t_batch_stride + (int64_t)draw_row * t_row_stride;
    int64_t doff = (int64_t)s * d_batch_stride + (int64_t)(n < Ks ? n : 0) * d_row_stride;
    int residual = n < Ks;
    RowNorm Cdn = {0.0, 0.0};
    if (residual) {
        Cdn = Cd[n];
    }
    double R = 0.0;
    for (int v = 0; v < V; ++v) {
        R += draw_weight(target, draft, dtype, toff, doff, v, T, Ct[draw_row], Cdn, residual);
    }
    int weight_row = draw_row;     /* the row whose log-normaliser the weights use */
#if ORACLE_MUTANT == 7
    if (0) {
#else
    if (residual && R == 0.0) {
#endif
        residual = 0;              /* no residual mass: draw from p_n */
#if ORACLE_MUTANT == 6
        weight_row = Ks;
        toff = (int64_t)s * t_batch_stride + (int64_t)Ks * t_row_stride;
#endif
        R = 0.0;
        for (int v = 0; v < V; ++v) {
            R += draw_weight(target, draft, dtype, toff, doff, v, T, Ct[weight_row], Cdn, 0);
        }
    }
    double u2 = oracle_uniform(seeds[s], (uint32_t)s, (uint32_t)n, 1u);
    double t = u2 * R;
    int32_t y = -1, last_positive = -1;
    double F = 0.0;
    for (int v = 0; v < V; ++v) {
        double w = draw_weight(target, draft, dtype, toff, doff, v, T, Ct[weight_row], Cdn, residual);
        F += w;
#if ORACLE_MUTANT == 8
        if (w > 0.0 && last_positive < 0) {
#else
        if (w > 0.0) {
#endif
            last_positive = v;
        }
        if (F > t) {
            y = v;
            break;
        }
    }
    if (y < 0) {
        y = last_positive;         /* t at the top end by rounding */
    }

    for (int j = 0; j < n; ++j) {
        tok[j] = x[j];
    }
    tok[n] = y;
    n_accepted[s] = n;
    if (diag) {
        diag[(int64_t)s * dstride + 2 * K] = t;
        diag[(int64_t)s * dstride + 2 * K + 1] = R;
        diag[(int64_t)s * dstride + 2 * K + 2] = u2;
        diag[(int64_t)s * dstride + 2 * K + 3] = residual ? 1.0 : 0.0;
    }
    free(Ct);
    free(Cd);
}

int oracle_sample_accept(const void *target, const void *draft, int dtype,
                         int64_t t_batch_stride, int64_t t_row_stride,
                         int64_t d_batch_stride, int64_t d_row_stride,
                         const int32_t *draft_tokens, int b, int K, int V,
                         double T, const uint64_t *seeds,
                         int32_t *n_accepted, int32_t *tokens,
                         double *p_draft, double *q_draft, double *diag)
{
    if (b < 1 || K < 1 || V < 1 || !(T > 0.0) || isinf(T) ||
        (dtype != OR_F32 && dtype != OR_BF16)) {
        return 1;
    }
    for (int s = 0; s < b; ++s) {
        sample_sequence(target, draft, dtype, t_batch_stride, t_row_stride,
                        d_batch_stride, d_row_stride, draft_tokens, s, K, K, V, T, seeds,
                        n_accepted, tokens, p_draft, q_draft, diag);
    }
    return 0;
}

/* Mixed batch: sequence s follows the greedy rule when temps[s] == 0 and the
 * sampling rule at temperature temps[s] when temps[s] > 0 is finite (the
 * drafter's temperature 0.0 stands for greedy decoding, "dspark-mlx 0.1.0",
 * dspark_mlx/arch/gemma4.py, Gemma4DSparkArgs); any other value makes the
 * sequence invalid.  Each sequence gets exactly what the single-rule
 * functions compute for it, with its index s in this batch as the Philox
 * row.  Greedy sequences report NaN probabilities; sampling sequences report
 * -1 argmax entries.
 * draft_lengths (or NULL: all K): sequence s uses only Ks = draft_lengths[s]
 * draft tokens, 0 <= Ks <= K -- the adaptive block length of a confidence
 * head, or a --max-draft cap ("mlx-dspark 0.0.1" sdist diff, README "Tuning";
 * __main__.py flags --max-draft and --confidence-threshold).  Its block is
 * then target rows 0..Ks (row Ks the bonus position) and draft rows
 * 0..Ks-1; Ks = 0 is a plain decode step.  Ks outside [0, K] makes the
 * sequence invalid. */
int oracle_mixed_accept(const void *target, const void *draft, int dtype,
                        int64_t t_batch_stride, int64_t t_row_stride,
                        int64_t d_batch_stride, int64_t d_row_stride,
                        const int32_t *draft_tokens, int b, int K, int V,
                        const double *temps, const int32_t *draft_lengths,
                        const uint64_t *seeds,
                        int32_t *n_accepted, int32_t *tokens,
                        double *p_draft, double *q_draft, int32_t *target_argmax,
                        double *diag)
{
    if (b < 1 || K < 1 || V < 1 || (dtype != OR_F32 && dtype != OR_BF16)) {
        return 1;
    }
    const int dstride = 2 * K + 4;
    for (int s = 0; s < b; ++s) {
        const double T = temps[s];
        const int Ks = draft_lengths ? draft_lengths[s] : K;
        const int len_ok = Ks >= 0 && Ks <= K;
        const int greedy = len_ok && T == 0.0;
        const int sampling = len_ok && T > 0.0 && !isinf(T);
        if (greedy) {
            greedy_sequence(target, dtype, t_batch_stride, t_row_stride, draft_tokens, s, K, Ks, V,
                            n_accepted, tokens, target_argmax);
        } else if (sampling) {
            sample_sequence(target, draft, dtype, t_batch_stride, t_row_stride,
                            d_batch_stride, d_row_stride, draft_tokens, s, K, Ks, V, T, seeds,
                            n_accepted, tokens, p_draft, q_draft, diag);
        } else {
            n_accepted[s] = -1;
            for (int j = 0; j <= K; ++j) {
                tokens[(int64_t)s * (K + 1) + j] = -1;
            }
        }
        if (!sampling) {
            for (int i = 0; i < K; ++i) {
                p_draft[(int64_t)s * K + i] = NAN;
                q_draft[(int64_t)s * K + i] = NAN;
            }
            if (diag) {
                for (int j = 0; j < dstride; ++j) {
                    diag[(int64_t)s * dstride + j] = NAN;
                }
            }
        }
        if (!greedy && target_argmax) {
            for (int i = 0; i <= K; ++i) {
                target_argmax[(int64_t)s * (K + 1) + i] = -1;
            }
        }
    }
    return 0;
}

/* Running sums F_v (v = 0..V-1) of the weights the oracle draws the token of
 * slot `slot` from, for sequence s: residual weights when slot < K and
 * `residual` is set, p_slot otherwise.  Used by the tests to tell whether a
 * disagreeing GPU draw sits next to a CDF step of the oracle. */
int oracle_draw_cdf(const void *target, const void *draft, int dtype,
                    int64_t t_batch_stride, int64_t t_row_stride,
                    int64_t d_batch_stride, int64_t d_row_stride,
                    int K, int V, double T, int s, int slot, int residual,
                    double *F_out)
{
    if (slot < 0 || slot > K || V < 1 || !(T > 0.0)) {
        return 1;
    }
    int64_t toff = (int64_t)s * t_batch_stride + (int64_t)slot * t_row_stride;
    RowNorm Ct = row_log_normaliser(target, dtype, toff, V, T);
    RowNorm Cd = {0.0, 0.0};
    int64_t doff = 0;
    if (residual) {
        if (slot >= K) {
            return 1;
        }
        doff = (int64_t)s * d_batch_stride + (int64_t)slot * d_row_stride;
        Cd = row_log_normaliser(draft, dtype, doff, V, T);
    }
    double F = 0.0;
    for (int v = 0; v < V; ++v) {
        F += draw_weight(target, draft, dtype, toff, doff, v, T, Ct, Cd, residual);
        F_out[v] = F;
    }
    return 0;
}

/* Log-normaliser of one row, exposed for the tests that pin it against an
 * independent library routine. */
double oracle_row_log_normaliser(const void *base, int dtype, int V, double T)
{
    RowNorm n = row_log_normaliser(base, dtype, 0, V, T);
    return n.M / T + n.L;
}
