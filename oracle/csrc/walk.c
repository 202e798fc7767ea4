/*
 * CPU oracle: Philox4x64-10 uniforms and the root-down rejection-sampling walk
 * over a candidate tree, in plain float64 C.  TEST INFRASTRUCTURE ONLY: only
 * the test suite, the smoke check and the benchmark's CPU-baseline leg load
 * this file's library; the GPU library shares no code with it.
 *
 * What it computes, and where the pages state it:
 *  - radar-34b blog, section 2 (rejection-sampling acceptance condition and its
 *    proof sketch): a draft x drawn from q is accepted when a uniform r falls
 *    below min(1, p(x)/q(x)); on rejection the token is redrawn from the
 *    normalised positive part of p - q and the later drafts are discarded.
 *  - LLM Primer VI ch. 9, section 9.1: one target pass yields a distribution at
 *    every candidate position plus one more, so a fully accepted path still
 *    emits one extra token.
 *  - jisaku.com glossary, SpecInfer paragraph: nodes are accepted or rejected
 *    from the root downwards, depth first.
 *
 * Readings where the pages are silent (each is listed in the design notes):
 *  - children of a node are tried in ascending node index, each against the
 *    running residual; under the i.i.d. sibling rule every child is tested
 *    with the same draft distribution q_u (siblings drawn independently from
 *    q_u), under the without-replacement rule a rejected child's token then
 *    leaves q: its entry is set to zero and the rest is divided by its sum
 *    (siblings drawn from q_u without replacement); if no draft mass is
 *    left, q stays zero and a later child is accepted iff its residual is
 *    positive;
 *  - the test is written without division: accept iff r*q(x) < p_res(x);
 *  - the residual normaliser is summed directly; if it is zero the
 *    distribution is left unchanged;
 *  - the final token is the smallest k with C(k) > r * sum(p), C the running
 *    sum in token order;
 *  - temperature T divides both target and draft logits;
 *  - uniforms come from Philox4x64-10 with counter (offset, b, i, 0) and key
 *    (seed, 0); output word 0 gives the acceptance uniform of node i, word 1
 *    the resampling uniform used if the walk stops at node i; a word w maps to
 *    (w >> 40) * 2^-24.
 *
 * Philox4x64-10 follows J. K. Salmon, M. A. Moraes, R. O. Dror, D. E. Shaw,
 * "Parallel random numbers: as easy as 1, 2, 3", SC'11 (the 4x64 round, its
 * two multipliers and the two Weyl key increments published there).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define PHILOX_M0 0xD2E7470EE14C6C93ULL
#define PHILOX_M1 0xCA5A826395121157ULL
#define PHILOX_W0 0x9E3779B97F4A7C15ULL
#define PHILOX_W1 0xBB67AE8584CAA73BULL

enum {
    ORACLE_RULE_IID = 0,                 /* siblings drawn independently from q */
    ORACLE_RULE_WITHOUT_REPLACEMENT = 1, /* siblings drawn from q without replacement */
};

enum {
    ORACLE_OK = 0,
    ORACLE_BAD_PARENT = 1,
    ORACLE_BAD_TOKEN = 2,
    ORACLE_NONFINITE = 3,
    ORACLE_BAD_ARG = 4,
    ORACLE_NOMEM = 5,
};

static void mulhilo64(uint64_t a, uint64_t b, uint64_t *hi, uint64_t *lo)
{
    unsigned __int128 prod = (unsigned __int128)a * (unsigned __int128)b;
    *hi = (uint64_t)(prod >> 64);
    *lo = (uint64_t)prod;
}

/* Ten Philox rounds on a 4-word counter with a 2-word key. */
void oracle_philox4x64_10(const uint64_t ctr[4], const uint64_t key[2], uint64_t out[4])
{
    uint64_t c0 = ctr[0], c1 = ctr[1], c2 = ctr[2], c3 = ctr[3];
    uint64_t k0 = key[0], k1 = key[1];
    for (int round = 0; round < 10; ++round) {
        if (round > 0) {
            k0 += PHILOX_W0;
            k1 += PHILOX_W1;
        }
        uint64_t hi0, lo0, hi1, lo1;
        mulhilo64(PHILOX_M0, c0, &hi0, &lo0);
        mulhilo64(PHILOX_M1, c2, &hi1, &lo1);
        uint64_t n0 = hi1 ^ c1 ^ k0;
        uint64_t n1 = lo1;
        uint64_t n2 = hi0 ^ c3 ^ k1;
        uint64_t n3 = lo0;
        c0 = n0; c1 = n1; c2 = n2; c3 = n3;
    }
    out[0] = c0; out[1] = c1; out[2] = c2; out[3] = c3;
}

static double word_to_uniform(uint64_t w)
{
    return (double)(w >> 40) * (1.0 / 16777216.0);
}

/* u[0]: acceptance uniform of node i; u[1]: resampling uniform at node i. */
void oracle_node_uniforms(uint64_t seed, uint64_t offset, int64_t b, int64_t i, double u[2])
{
    uint64_t ctr[4] = {offset, (uint64_t)b, (uint64_t)i, 0};
    uint64_t key[2] = {seed, 0};
    uint64_t w[4];
    oracle_philox4x64_10(ctr, key, w);
    u[0] = word_to_uniform(w[0]);
    u[1] = word_to_uniform(w[1]);
}

/* p = softmax(logits / T) in float64. Fails on NaN or an all -inf row. */
static int softmax_row(const float *logits, int32_t V, double T, double *p)
{
    double m = -INFINITY;
    for (int32_t x = 0; x < V; ++x) {
        double v = (double)logits[x] / T;
        if (isnan(v))
            return ORACLE_NONFINITE;
        if (v > m)
            m = v;
    }
    if (!(m > -INFINITY) || isinf(m))
        return ORACLE_NONFINITE;
    double z = 0.0;
    for (int32_t x = 0; x < V; ++x) {
        p[x] = exp((double)logits[x] / T - m);
        z += p[x];
    }
    for (int32_t x = 0; x < V; ++x)
        p[x] /= z;
    return ORACLE_OK;
}

typedef struct {
    int32_t draws;        /* uniforms consumed by decisions */
    int32_t near;         /* of those, how many fell within eps of their boundary */
    int32_t first_near;   /* accepted count when the first near draw happened, or -1 */
    double min_margin;    /* smallest |r - boundary| seen */
} draw_log;

static void log_draw(draw_log *lg, double margin, double eps, int32_t n_acc)
{
    lg->draws += 1;
    if (margin < lg->min_margin)
        lg->min_margin = margin;
    if (margin < eps) {
        if (lg->near == 0)
            lg->first_near = n_acc;
        lg->near += 1;
    }
}

/*
 * Walk one tree.  target/draft: [N][V] rows of this sequence.  Writes path[N]
 * (accepted nodes from the root, -1 padded), out_tokens[N] (emitted tokens,
 * -1 padded) and returns the accepted count through *n_acc_out.
 */
/* Node i's two uniforms: from the caller's table utab[i][0..1] when it gives
 * one, else from Philox. */
static void node_uniforms_or_table(const double *utab, uint64_t seed, uint64_t offset, int64_t b,
                                   int32_t i, double ur[2])
{
    if (utab) {
        ur[0] = utab[2 * (size_t)i];
        ur[1] = utab[2 * (size_t)i + 1];
    } else {
        oracle_node_uniforms(seed, offset, b, i, ur);
    }
}

static int walk_one(const float *target, const float *draft, const int32_t *parent,
                    const int32_t *token, int32_t N, int32_t V, double T, int32_t rule,
                    uint64_t seed, uint64_t offset, int64_t b, double eps, const double *utab,
                    int32_t *path, int32_t *out_tokens, int32_t *n_acc_out,
                    draw_log *lg, double *p, double *q, double *pr)
{
    if (N < 1 || parent[0] != -1)
        return ORACLE_BAD_PARENT;
    for (int32_t i = 1; i < N; ++i) {
        if (parent[i] < 0 || parent[i] >= i)
            return ORACLE_BAD_PARENT;
        if (token[i] < 0 || token[i] >= V)
            return ORACLE_BAD_TOKEN;
    }
    for (int32_t i = 0; i < N; ++i) {
        path[i] = -1;
        out_tokens[i] = -1;
    }

    int32_t u = 0, n_acc = 0;
    path[0] = 0;
    for (;;) {
        int rc = softmax_row(target + (size_t)u * V, V, T, p);
        if (rc)
            return rc;
        const double *final_dist = p;

        int has_child = 0;
        for (int32_t c = u + 1; c < N; ++c)
            if (parent[c] == u) { has_child = 1; break; }

        int accepted = 0;
        if (has_child) {
            rc = softmax_row(draft + (size_t)u * V, V, T, q);
            if (rc)
                return rc;
            memcpy(pr, p, sizeof(double) * (size_t)V);
            for (int32_t c = u + 1; c < N && !accepted; ++c) {
                if (parent[c] != u)
                    continue;
                int32_t x = token[c];
                double ur[2];
                node_uniforms_or_table(utab, seed, offset, b, c, ur);
                double r = ur[0];
                double margin = q[x] > 0.0 ? fabs(r - pr[x] / q[x]) : INFINITY;
                log_draw(lg, margin, eps, n_acc);
                if (r * q[x] < pr[x]) {
                    n_acc += 1;
                    path[n_acc] = c;
                    out_tokens[n_acc - 1] = x;
                    u = c;
                    accepted = 1;
                } else {
                    double z = 0.0;
                    for (int32_t y = 0; y < V; ++y) {
                        double d = pr[y] - q[y];
                        z += d > 0.0 ? d : 0.0;
                    }
                    if (z > 0.0) {
                        for (int32_t y = 0; y < V; ++y) {
                            double d = pr[y] - q[y];
                            pr[y] = (d > 0.0 ? d : 0.0) / z;
                        }
                    }
                    if (rule == ORACLE_RULE_WITHOUT_REPLACEMENT) {
                        q[x] = 0.0;
                        double s = 0.0;
                        for (int32_t y = 0; y < V; ++y)
                            s += q[y];
                        if (s > 0.0)
                            for (int32_t y = 0; y < V; ++y)
                                q[y] /= s;
                    }
                }
            }
            if (accepted)
                continue;
            final_dist = pr;
        }

        /* Inverse-CDF draw from the final distribution at u. */
        double ur[2];
        node_uniforms_or_table(utab, seed, offset, b, u, ur);
        double total = 0.0;
        for (int32_t y = 0; y < V; ++y)
            total += final_dist[y];
        double target_mass = ur[1] * total;
        double run = 0.0;
        int32_t tok = -1;
        double margin = INFINITY;
        for (int32_t y = 0; y < V; ++y) {
            double prev = run;
            run += final_dist[y];
            if (run > target_mass) {
                tok = y;
                double lo = target_mass - prev, hi = run - target_mass;
                margin = (lo < hi ? lo : hi) / total;
                break;
            }
        }
        if (tok < 0) {           /* rounding left the mass short: take the last live token */
            for (int32_t y = V - 1; y >= 0; --y)
                if (final_dist[y] > 0.0) { tok = y; break; }
            margin = 0.0;
        }
        log_draw(lg, margin, eps, n_acc);
        out_tokens[n_acc] = tok;
        *n_acc_out = n_acc;
        return ORACLE_OK;
    }
}

/*
 * Batch entry.  target/draft: float32 [B][N][V]; parent/token: int32 [B][N];
 * rule: ORACLE_RULE_IID or ORACLE_RULE_WITHOUT_REPLACEMENT; uniforms: NULL
 * (Philox from seed and offset) or the uniforms to use, double [B][N][2]
 * (acceptance, resampling), so a test can integrate over them exactly.
 * Outputs: path, out_tokens int32 [B][N]; n_accepted int32 [B]; per sequence
 * draws/near/first_near int32 [B] and min_margin double [B].  Returns 0 or the
 * first error code met (then *bad_seq names the sequence).
 */
int oracle_verify_walk_u(const float *target, const float *draft, const int32_t *parent,
                         const int32_t *token, int64_t B, int32_t N, int32_t V, double T,
                         uint64_t seed, uint64_t offset, double eps, int32_t rule,
                         const double *uniforms, int32_t *path, int32_t *n_accepted,
                         int32_t *out_tokens, int32_t *draws, int32_t *near,
                         int32_t *first_near, double *min_margin, int64_t *bad_seq)
{
    if (B < 0 || N < 1 || V < 1 || !(T > 0.0) ||
        (rule != ORACLE_RULE_IID && rule != ORACLE_RULE_WITHOUT_REPLACEMENT))
        return ORACLE_BAD_ARG;
    double *buf = (double *)malloc(sizeof(double) * (size_t)V * 3);
    if (!buf)
        return ORACLE_NOMEM;
    int rc = ORACLE_OK;
    for (int64_t b = 0; b < B; ++b) {
        draw_log lg = {0, 0, -1, INFINITY};
        size_t row0 = (size_t)b * (size_t)N;
        rc = walk_one(target + row0 * V, draft + row0 * V, parent + row0, token + row0,
                      N, V, T, rule, seed, offset, b, eps, uniforms ? uniforms + row0 * 2 : NULL,
                      path + row0, out_tokens + row0, n_accepted + b, &lg, buf, buf + V,
                      buf + 2 * (size_t)V);
        if (rc) {
            *bad_seq = b;
            break;
        }
        draws[b] = lg.draws;
        near[b] = lg.near;
        first_near[b] = lg.first_near;
        min_margin[b] = lg.min_margin;
    }
    free(buf);
    return rc;
}

int oracle_verify_walk(const float *target, const float *draft, const int32_t *parent,
                       const int32_t *token, int64_t B, int32_t N, int32_t V, double T,
                       uint64_t seed, uint64_t offset, double eps, int32_t rule,
                       int32_t *path, int32_t *n_accepted, int32_t *out_tokens,
                       int32_t *draws, int32_t *near, int32_t *first_near,
                       double *min_margin, int64_t *bad_seq)
{
    return oracle_verify_walk_u(target, draft, parent, token, B, N, V, T, seed, offset, eps,
                                rule, NULL, path, n_accepted, out_tokens, draws, near,
                                first_near, min_margin, bad_seq);
}

/* u[b][i][0..1] for a whole batch (used by tests to cross-check the device). */
void oracle_uniform_table(uint64_t seed, uint64_t offset, int64_t B, int32_t N, double *u)
{
    for (int64_t b = 0; b < B; ++b)
        for (int32_t i = 0; i < N; ++i)
            oracle_node_uniforms(seed, offset, b, i, u + ((size_t)b * N + i) * 2);
}

/* Raw Philox words for a list of counters (4 words each) under one key. */
void oracle_philox_words(const uint64_t *ctrs, int64_t n, uint64_t k0, uint64_t k1,
                         uint64_t *out)
{
    uint64_t key[2] = {k0, k1};
    for (int64_t i = 0; i < n; ++i)
        oracle_philox4x64_10(ctrs + 4 * i, key, out + 4 * i);
}
