/*
 * Plain fp64 CPU oracle for the Domino head drafting loop.
 *
 * TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only the test suite, the smoke
 * check and the CPU-baseline leg of the benchmark may load this library.
 * It shares no code, header, table or helper with the HIP library; the two
 * meet only in the seeded inputs.
 *
 * What it computes (per batch row; "the pages" are the four web pages on
 * Domino: the paper.oopus.info review, the news.sig.ai article, the
 * researchpapers.dev summary and the Hugging Face papers mirror):
 *
 *   - paper.oopus.info review, section 二 (第二步 Domino Head): a GRU causal
 *     encoder with hidden size h reads the embeddings of the draft tokens of
 *     the preceding positions and yields the causal state S_{i-1}; a
 *     rank-r correction head with SiLU forms
 *         L_final_i = L_base_i + W2 * SiLU(W1 * [H_i ; S_{i-1}])
 *     directly in logit space (no LM-head recomputation).
 *   - news.sig.ai article, section "Domino怎么做": greedy decoding, so the
 *     draft token of position i is the argmax of L_final_i.
 *   - paper.oopus.info review, section 二 (训练策略, Teacher Forcing): given
 *     tokens replace the model's own choices as GRU inputs.
 *   - paper.oopus.info review, section 一, and the researchpapers.dev
 *     summary, "关键结果": the verifier accepts the longest draft prefix that
 *     matches its own tokens.
 *
 * Readings taken where the pages are silent (each is a convention, not a
 * fact the pages fix):
 *   - sigma in the formula is SiLU(x) = x / (1 + exp(-x)) (the review says
 *     the correction head uses SiLU);
 *   - W1 is [r, d+h] row-major; column j < d multiplies H_i[j], column d+j
 *     multiplies S_{i-1}[j]; W1 and W2 carry no bias;
 *   - GRU = PyTorch GRUCell: rows of W_ih/W_hh/b_ih/b_hh in blocks (reset,
 *     update, new); r = sig(Wir x + bir + Whr s + bhr), z likewise,
 *     n = tanh(Win x + bin + r * (Whn s + bhn)), s' = (1 - z) n + z s;
 *     a NULL bias is zero;
 *   - GRU input = row of the token embedding table E for the token;
 *   - anchor step: S_{-1} = S_init (zero when NULL), S_0 = GRU(E[last_tok],
 *     S_{-1}); then for i = 1..K: u_i = SiLU(W1 [H_i; S_{i-1}]),
 *     L_final_i = L_base_i + W2 u_i, t_i = argmax, and for i < K
 *     S_i = GRU(E[x_i], S_{i-1}) with x_i = t_i (free running) or the
 *     teacher token y_i (teacher forced);
 *   - argmax: lowest index among equal maxima; a NaN counts as larger than
 *     every number and the first NaN wins.  The decision is taken on the
 *     logits rounded to float32, the precision the GPU path decides in;
 *   - a last_tok or a used teacher token outside [0, V) makes the row
 *     invalid: all its tokens are -1 and the function returns 1;
 *   - Markov head (markov != 0).  The news.sig.ai article (section
 *     从Domino看DSpark) says DSpark ships a Markov head as its default beside
 *     an RNN head, and that Domino's causal encoder corresponds to the RNN
 *     head; it gives no formula.  Reading taken: a Markov head
 *     conditions each position on the preceding token alone, so the causal
 *     state is the same GRU cell applied to that token's embedding from a
 *     zero state, S_i = GRU(E[x_i], 0) (S_0 = GRU(E[last_tok], 0)); nothing
 *     is carried from earlier positions and S_init is not used.
 *
 * Arithmetic: every weight and input is widened from its stored bits
 * (float32 or bfloat16) to double; every dot product sums in ascending index
 * order in double.  OpenMP splits only independent outputs (vocabulary rows,
 * hidden units), so results do not depend on the thread count.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

typedef struct {
    int32_t d, h, r, V, K;
    int32_t wdtype; /* 0: float32 storage, 1: bfloat16 bit patterns (uint16) */
    const void *W1, *W2, *W_ih, *W_hh, *b_ih, *b_hh, *E;
    int32_t markov; /* 1: Markov head, every GRU step starts from the zero state */
} oracle_head;

static double widen(const void *base, int32_t wdtype, size_t idx)
{
    if (wdtype == 0)
        return (double)((const float *)base)[idx];
    uint32_t bits = ((uint32_t)((const uint16_t *)base)[idx]) << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
}

static double sigmoid(double x) { return 1.0 / (1.0 + exp(-x)); }

/* PyTorch GRUCell on x = E[tok] (widened) and state s; writes s_next[h]. */
static void gru_cell(const oracle_head *hd, int32_t tok, const double *s, double *s_next, int nthreads)
{
    const int32_t d = hd->d, h = hd->h;
    double *x = (double *)malloc(sizeof(double) * (size_t)d);
    for (int32_t k = 0; k < d; ++k)
        x[k] = widen(hd->E, hd->wdtype, (size_t)tok * d + k);
#pragma omp parallel for schedule(static) num_threads(nthreads)
    for (int32_t j = 0; j < h; ++j) {
        double g[3], q[3];
        for (int gate = 0; gate < 3; ++gate) {
            size_t row = (size_t)gate * h + j;
            double acc = hd->b_ih ? widen(hd->b_ih, hd->wdtype, row) : 0.0;
            for (int32_t k = 0; k < d; ++k)
                acc += widen(hd->W_ih, hd->wdtype, row * d + k) * x[k];
            g[gate] = acc;
            double acc2 = hd->b_hh ? widen(hd->b_hh, hd->wdtype, row) : 0.0;
            for (int32_t k = 0; k < h; ++k)
                acc2 += widen(hd->W_hh, hd->wdtype, row * h + k) * s[k];
            q[gate] = acc2;
        }
        double rg = sigmoid(g[0] + q[0]);
        double zg = sigmoid(g[1] + q[1]);
        double ng = tanh(g[2] + rg * q[2]);
        s_next[j] = (1.0 - zg) * ng + zg * s[j];
    }
    free(x);
}

/* float32 order with NaN above everything; returns 1 if a beats b. */
static int beats(float a, float b)
{
    if (isnan(b))
        return 0;
    if (isnan(a))
        return 1;
    return a > b;
}

/*
 * One batch row.
 *   H        [K, d]   wdtype storage
 *   L_base   [K, V]   float32
 *   teacher  [K] or NULL; entries 0..K-2 (tokens y_1..y_{K-1}) are used
 *   S_init   [h] float32 or NULL (not used by a Markov head)
 * Outputs (any pointer but tokens may be NULL):
 *   tokens [K] int32; L_final [K, V] double; gap [K] double (top1 - top2 of
 *   L_final in double, top2 over the other entries); S_out [K, h] double
 *   (S_0..S_{K-1}); u_out [K, r] double (u_1..u_K).
 * Returns 0, or 1 when the row is invalid (tokens set to -1).
 */
int oracle_draft_row(const oracle_head *hd, const void *H, const float *L_base, int32_t last_tok,
                     const int32_t *teacher, const float *S_init, int32_t *tokens, double *L_final,
                     double *gap, double *S_out, double *u_out, int nthreads)
{
    const int32_t d = hd->d, h = hd->h, r = hd->r, V = hd->V, K = hd->K;
    if (nthreads < 1)
        nthreads = 1;
    int bad = (last_tok < 0 || last_tok >= V);
    if (teacher)
        for (int32_t i = 0; i + 1 < K; ++i)
            if (teacher[i] < 0 || teacher[i] >= V)
                bad = 1;
    if (bad) {
        for (int32_t i = 0; i < K; ++i)
            tokens[i] = -1;
        return 1;
    }

    double *s = (double *)malloc(sizeof(double) * (size_t)h);
    double *s_next = (double *)malloc(sizeof(double) * (size_t)h);
    double *zero = (double *)calloc((size_t)h, sizeof(double));
    double *cat = (double *)malloc(sizeof(double) * (size_t)(d + h));
    double *u = (double *)malloc(sizeof(double) * (size_t)r);
    double *lf = (double *)malloc(sizeof(double) * (size_t)V);

    for (int32_t j = 0; j < h; ++j)
        s[j] = (S_init && !hd->markov) ? (double)S_init[j] : 0.0;
    /* anchor step: S_0 = GRU(E[last_tok], S_init) */
    gru_cell(hd, last_tok, s, s_next, nthreads);
    memcpy(s, s_next, sizeof(double) * (size_t)h);

    for (int32_t i = 0; i < K; ++i) {
        if (S_out)
            memcpy(S_out + (size_t)i * h, s, sizeof(double) * (size_t)h);
        /* [H_i ; S_{i-1}] */
        for (int32_t j = 0; j < d; ++j)
            cat[j] = widen(H, hd->wdtype, (size_t)i * d + j);
        for (int32_t j = 0; j < h; ++j)
            cat[d + j] = s[j];
        for (int32_t k = 0; k < r; ++k) {
            double a = 0.0;
            for (int32_t j = 0; j < d + h; ++j)
                a += widen(hd->W1, hd->wdtype, (size_t)k * (d + h) + j) * cat[j];
            u[k] = a * sigmoid(a); /* SiLU */
        }
        if (u_out)
            memcpy(u_out + (size_t)i * r, u, sizeof(double) * (size_t)r);
        const float *lb = L_base + (size_t)i * V;
#pragma omp parallel for schedule(static) num_threads(nthreads)
        for (int32_t v = 0; v < V; ++v) {
            double c = 0.0;
            for (int32_t k = 0; k < r; ++k)
                c += widen(hd->W2, hd->wdtype, (size_t)v * r + k) * u[k];
            lf[v] = (double)lb[v] + c;
        }
        /* greedy choice on float32-rounded logits, lowest index wins ties */
        int32_t best = 0;
        float bestf = (float)lf[0];
        for (int32_t v = 1; v < V; ++v) {
            float f = (float)lf[v];
            if (beats(f, bestf)) {
                best = v;
                bestf = f;
            }
        }
        tokens[i] = best;
        if (gap) {
            double second = -INFINITY;
            int any = 0;
            for (int32_t v = 0; v < V; ++v) {
                if (v == best)
                    continue;
                if (!any || lf[v] > second || isnan(lf[v])) {
                    second = lf[v];
                    any = 1;
                }
            }
            gap[i] = any ? lf[best] - second : INFINITY;
        }
        if (L_final)
            memcpy(L_final + (size_t)i * V, lf, sizeof(double) * (size_t)V);
        if (i + 1 < K) {
            int32_t x_tok = teacher ? teacher[i] : best;
            /* recurrent head: from S_{i-1}; Markov head: from the zero state */
            gru_cell(hd, x_tok, hd->markov ? zero : s, s_next, nthreads);
            memcpy(s, s_next, sizeof(double) * (size_t)h);
        }
    }
    free(s);
    free(s_next);
    free(zero);
    free(cat);
    free(u);
    free(lf);
    return 0;
}

/* Accepted prefix length: first j with draft[b][j] != target[b][j], else K. */
void oracle_accept_len(int32_t B, int32_t K, const int32_t *draft, const int32_t *target, int32_t *out)
{
    for (int32_t b = 0; b < B; ++b) {
        int32_t j = 0;
        while (j < K && draft[(size_t)b * K + j] == target[(size_t)b * K + j])
            ++j;
        out[b] = j;
    }
}

/*
 * Greedy verify step for one drafted block (paper.oopus.info review, section
 * 一: the target model checks the whole draft in one parallel pass and keeps
 * what it would have produced; researchpapers.dev summary, 关键结果 and
 * 常见问题: every accepted token is exactly the target's own token).
 *   logits [B, K+1, V] float32: row j scores the token that follows the
 *          context plus draft[b][0..j-1] (row K follows the whole draft)
 *   draft  [B, K] int32
 * Outputs:
 *   target [B, K+1] int32 (may be NULL): the target's greedy token of each
 *          row, with the draft's argmax rules (beats(); lowest index on ties)
 *   accept [B] int32: first j < K with draft[b][j] != target[b][j], else K
 *   next   [B] int32: target[b][accept[b]], the token the target itself puts
 *          after the accepted prefix (the anchor of the next block)
 * Reading taken: the committed tokens of a step are the accepted prefix plus
 * that one target token; the pages do not spell out the extra token, but it
 * is the target's own greedy choice, so committing it keeps the output
 * identical to plain greedy decoding by the target.
 */
void oracle_verify(int32_t B, int32_t K, int32_t V, const float *logits, const int32_t *draft, int32_t *target,
                   int32_t *accept, int32_t *next)
{
    int32_t *t = (int32_t *)malloc(sizeof(int32_t) * (size_t)(K + 1));
    for (int32_t b = 0; b < B; ++b) {
        for (int32_t j = 0; j <= K; ++j) {
            const float *row = logits + ((size_t)b * (K + 1) + j) * (size_t)V;
            int32_t best = 0;
            for (int32_t v = 1; v < V; ++v)
                if (beats(row[v], row[best]))
                    best = v;
            t[j] = best;
            if (target)
                target[(size_t)b * (K + 1) + j] = best;
        }
        int32_t a = 0;
        while (a < K && draft[(size_t)b * K + a] == t[a])
            ++a;
        accept[b] = a;
        next[b] = t[a];
    }
    free(t);
}

/* Head parameters: W1 [r, d+h], W2 [V, r], W_ih [3h, d], W_hh [3h, h] (+ 2 x 3h GRU biases). */
int64_t oracle_param_count(int64_t d, int64_t h, int64_t r, int64_t V, int32_t with_bias)
{
    int64_t n = r * (d + h) + V * r + 3 * h * d + 3 * h * h;
    if (with_bias)
        n += 6 * h;
    return n;
}

int oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
