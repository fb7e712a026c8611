/*
 * specverify oracle -- a plain, slow, obviously-correct fp64 CPU model of the
 * verify step of speculative sampling.
 *
 * TEST INFRASTRUCTURE ONLY.  The product (the HIP library and its Python
 * binding) never includes, links, loads or calls this file.  Only the test
 * suite, the smoke check and the benchmark's CPU-baseline leg use it.  It
 * shares no code, header, table or helper with the GPU path.
 *
 * What it follows (cited by page title and section):
 *  - "CS3602_FINAL_SpeDec", section 2 (perplexity test) and its proof: with
 *    p the target distribution and q the draft distribution, a guess x ~ q is
 *    accepted with probability min(1, p(x)/q(x)); on rejection the token is
 *    drawn from p'(x) = norm(max(0, p(x) - q(x))), whose normaliser is
 *    1 - beta with beta = sum_x min(p(x), q(x)).
 *  - "Text Generation via Speculative Sampling, KV Caching, and OpenVINO",
 *    section "Prepare autoregressive sampling" (max_fn = norm(max(0, .)),
 *    softmax over the vocabulary, argmax for the greedy decode) and section
 *    "Prepare speculative sampling", steps 3 and 4 (one uniform draw per
 *    draft position compared with the ratio, stop at the first rejection,
 *    one extra token from the last target position when every draft token
 *    was accepted).
 *  - Philox4x32-10: J. K. Salmon, M. A. Moraes, R. O. Dror, D. E. Shaw,
 *    "Parallel Random Numbers: As Easy as 1, 2, 3", SC'11 (the Philox
 *    S-box: two 32x32->64 multiplications per round, Weyl key schedule).
 *
 * Readings taken where the pages are silent:
 *  p = target, q = draft; both are softmaxes at the same temperature T;
 *  top-k keeps every id whose raw logit is >= the k-th largest (ties kept),
 *  applied to each row on its own; accept iff u < min(1, p/q) with u in
 *  [0, 1); q = 0 accepts iff p > 0; the inverse CDF walks ids in ascending
 *  order and picks the first id whose running mass exceeds u * total;
 *  uniforms come from Philox4x32-10 with key (seed lo, seed hi) and counter
 *  (sequence, position, purpose, offset), word 0, 24 high bits.
 *
 * Everything is fp64, libm exp, ascending-id loops, no blocking or fusion.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_DTYPE_F32 0
#define ORC_DTYPE_BF16 1
#define ORC_DTYPE_F16 2

#define ORC_FLAG_ZERO_RESIDUAL 1   /* residual mass <= 0: fell back to p_n   */
#define ORC_FLAG_NO_CROSSING 2     /* rounding: took the last positive id    */
#define ORC_FLAG_BAD_INPUT 4       /* id out of range or degenerate row      */

/* ------------------------------------------------------------------------ */
/* Element decoding: bf16 is the top half of an IEEE binary32, so widening   */
/* is exact.  IEEE binary16 (1 sign, 5 exponent bits with bias 15, 10        */
/* fraction bits) is decoded from its definition: subnormals are             */
/* fraction * 2^-24, normals (1024 + fraction) * 2^(exponent - 25), and the  */
/* all-ones exponent is infinity (fraction 0) or NaN.                        */
/* ------------------------------------------------------------------------ */
static double orc_half_to_double(uint16_t h)
{
    const int sign = h >> 15;
    const int ex = (h >> 10) & 31;
    const int fr = h & 1023;
    double mag;
    if (ex == 0) {
        mag = ldexp((double)fr, -24);
    } else if (ex == 31) {
        mag = fr == 0 ? INFINITY : NAN;
    } else {
        mag = ldexp((double)(1024 + fr), ex - 25);
    }
    return sign ? -mag : mag;
}

double orc_decode(const void* base, int32_t dtype, int64_t i)
{
    if (dtype == ORC_DTYPE_F32) {
        return (double)((const float*)base)[i];
    }
    if (dtype == ORC_DTYPE_F16) {
        return orc_half_to_double(((const uint16_t*)base)[i]);
    }
    uint32_t bits = (uint32_t)((const uint16_t*)base)[i] << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
}

/* ------------------------------------------------------------------------ */
/* Philox4x32-10 (Salmon et al., SC'11).                                     */
/* One round: (hi0, lo0) = M0 * c0, (hi1, lo1) = M1 * c2 (full 64-bit        */
/* products); new counter = (hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0).        */
/* Between rounds the key advances by the Weyl constants.                    */
/* ------------------------------------------------------------------------ */
void orc_philox4x32_10(const uint32_t ctr_in[4], const uint32_t key_in[2], uint32_t out[4])
{
    const uint64_t M0 = 0xD2511F53u, M1 = 0xCD9E8D57u;
    const uint32_t W0 = 0x9E3779B9u, W1 = 0xBB67AE85u;
    uint32_t c[4] = {ctr_in[0], ctr_in[1], ctr_in[2], ctr_in[3]};
    uint32_t k[2] = {key_in[0], key_in[1]};
    for (int round = 0; round < 10; ++round) {
        if (round > 0) {
            k[0] += W0;
            k[1] += W1;
        }
        uint64_t prod0 = M0 * (uint64_t)c[0];
        uint64_t prod1 = M1 * (uint64_t)c[2];
        uint32_t hi0 = (uint32_t)(prod0 >> 32), lo0 = (uint32_t)prod0;
        uint32_t hi1 = (uint32_t)(prod1 >> 32), lo1 = (uint32_t)prod1;
        uint32_t n0 = hi1 ^ c[1] ^ k[0];
        uint32_t n1 = lo1;
        uint32_t n2 = hi0 ^ c[3] ^ k[1];
        uint32_t n3 = lo0;
        c[0] = n0; c[1] = n1; c[2] = n2; c[3] = n3;
    }
    out[0] = c[0]; out[1] = c[1]; out[2] = c[2]; out[3] = c[3];
}

/* u = (first output word >> 8) * 2^-24, a multiple of 2^-24 in [0, 1). */
double orc_uniform(uint64_t seed, uint32_t seq, uint32_t pos, uint32_t purpose, uint32_t offset)
{
    uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
    uint32_t ctr[4] = {seq, pos, purpose, offset};
    uint32_t out[4];
    orc_philox4x32_10(ctr, key, out);
    return (double)(out[0] >> 8) * (1.0 / 16777216.0);
}

/* ------------------------------------------------------------------------ */
/* Row statistics and probabilities.                                         */
/* ------------------------------------------------------------------------ */
static int orc_cmp_desc(const void* a, const void* b)
{
    double x = *(const double*)a, y = *(const double*)b;
    return (x < y) - (x > y);
}

/*
 * prob[v] = softmax(l / T) over the kept set, 0 elsewhere.  The kept set is
 * every id when top_k <= 0 or top_k >= V; otherwise every id whose logit is
 * >= tau, the top_k-th largest logit counted with multiplicity (so ties at
 * tau are all kept).  Then, when top_p < 1, the nucleus (top-p) filter on
 * that distribution, the other sampling filter the SpeDec report's helpers
 * name next to top-K: the kept set shrinks to every id whose logit is >=
 * tau_p, the largest logit value t for which the probability of
 * {v : l_v >= t} reaches top_p (so the smallest such set of highest-logit
 * ids, with ties at tau_p kept), and is renormalised.
 * stats = {m, S, tau, kept_count, tau_p, margin}, where m is the largest
 * kept logit and S = sum over kept v of exp((l_v - m) / T), summed in
 * ascending v (both over the final kept set); margin is the distance of
 * top_p from the cumulative probabilities on either side of tau_p (infinity
 * without top-p).  Returns 0, or -1 when the kept set has no finite logit.
 */
typedef struct {
    double val;
    int64_t idx;
} OrcValIdx;

static int orc_cmp_vi_desc(const void* a, const void* b)
{
    const double x = ((const OrcValIdx*)a)->val, y = ((const OrcValIdx*)b)->val;
    return (x < y) - (x > y);
}

/* The nucleus threshold of prob (kept ids have prob > 0): tau_p and the margin. */
static int orc_nucleus(const double* vals, const double* prob, int64_t V, double top_p, double* tau_p,
                       double* margin)
{
    int64_t n = 0;
    for (int64_t v = 0; v < V; ++v) n += prob[v] > 0.0;
    OrcValIdx* a = (OrcValIdx*)malloc(sizeof(OrcValIdx) * (size_t)(n > 0 ? n : 1));
    if (!a) return -2;
    n = 0;
    for (int64_t v = 0; v < V; ++v)
        if (prob[v] > 0.0) a[n++] = (OrcValIdx){vals[v], v};
    qsort(a, (size_t)n, sizeof(OrcValIdx), orc_cmp_vi_desc);
    /* walk groups of equal logits from the top; cum = P(l >= group value) */
    double cum = 0.0, prev = 0.0;
    *tau_p = n > 0 ? a[n - 1].val : -INFINITY;
    *margin = INFINITY;
    for (int64_t i = 0; i < n;) {
        int64_t j = i;
        double g = 0.0;
        while (j < n && a[j].val == a[i].val) g += prob[a[j++].idx];
        prev = cum;
        cum += g;
        if (cum >= top_p) {
            /* the first group is always kept: below it there is no other choice */
            *tau_p = a[i].val;
            *margin = fmin(cum - top_p, i > 0 ? top_p - prev : INFINITY);
            break;
        }
        i = j;
    }
    free(a);
    return 0;
}

int orc_row_probs_p(const void* row, int32_t dtype, int64_t V, double T, int32_t top_k, double top_p,
                    double* prob, double* stats)
{
    double* vals = (double*)malloc((size_t)V * sizeof(double));
    if (!vals) return -2;
    for (int64_t v = 0; v < V; ++v) vals[v] = orc_decode(row, dtype, v);

    double tau = -INFINITY;
    if (top_k > 0 && top_k < V) {
        double* sorted = (double*)malloc((size_t)V * sizeof(double));
        if (!sorted) { free(vals); return -2; }
        memcpy(sorted, vals, (size_t)V * sizeof(double));
        qsort(sorted, (size_t)V, sizeof(double), orc_cmp_desc);
        tau = sorted[top_k - 1];
        free(sorted);
    }

    double m = -INFINITY;
    int64_t kept = 0;
    for (int64_t v = 0; v < V; ++v) {
        if (vals[v] >= tau) {
            ++kept;
            if (vals[v] > m) m = vals[v];
        }
    }
    if (!(m > -INFINITY) || isinf(m)) {
        for (int64_t v = 0; v < V; ++v) prob[v] = 0.0;
        stats[0] = m; stats[1] = 0.0; stats[2] = tau; stats[3] = (double)kept;
        stats[4] = tau; stats[5] = INFINITY;
        free(vals);
        return -1;
    }

    double S = 0.0;
    for (int64_t v = 0; v < V; ++v) {
        double w = (vals[v] >= tau) ? exp((vals[v] - m) / T) : 0.0;
        prob[v] = w;
        S += w;
    }
    for (int64_t v = 0; v < V; ++v) prob[v] /= S;
    stats[4] = tau;
    stats[5] = INFINITY;
    if (top_p < 1.0) {
        double tau_p, margin;
        if (orc_nucleus(vals, prob, V, top_p, &tau_p, &margin) != 0) { free(vals); return -2; }
        /* the same softmax over the nucleus (m, the largest logit, is in it) */
        S = 0.0;
        kept = 0;
        for (int64_t v = 0; v < V; ++v) {
            double w = (vals[v] >= tau && vals[v] >= tau_p) ? exp((vals[v] - m) / T) : 0.0;
            kept += (vals[v] >= tau && vals[v] >= tau_p);
            prob[v] = w;
            S += w;
        }
        for (int64_t v = 0; v < V; ++v) prob[v] /= S;
        stats[4] = tau_p;
        stats[5] = margin;
    }
    stats[0] = m; stats[1] = S; stats[2] = tau; stats[3] = (double)kept;
    free(vals);
    return 0;
}

int orc_row_probs(const void* row, int32_t dtype, int64_t V, double T, int32_t top_k, double* prob, double* stats)
{
    return orc_row_probs_p(row, dtype, V, T, top_k, 1.0, prob, stats);
}

/* The lowest index among the maxima of the raw logits. */
int64_t orc_row_argmax(const void* row, int32_t dtype, int64_t V)
{
    int64_t best = 0;
    double bv = orc_decode(row, dtype, 0);
    for (int64_t v = 1; v < V; ++v) {
        double x = orc_decode(row, dtype, v);
        if (x > bv) { bv = x; best = v; }
    }
    return best;
}

/* ------------------------------------------------------------------------ */
/* Inverse CDF over non-negative weights w[0..V), ascending id order.        */
/* Returns the first v whose running sum exceeds u * total.  Also reports    */
/* the distance from u to the edges of the chosen id's normalised interval   */
/* and the range of ids whose interval meets [u - eps, u + eps].             */
/* ------------------------------------------------------------------------ */
static int64_t orc_inverse_cdf(const double* w, int64_t V, double u, double eps,
                               double* total_out, double* dist_out,
                               int32_t* lo_out, int32_t* hi_out, int32_t* flags)
{
    double total = 0.0;
    int64_t last_pos = -1;
    for (int64_t v = 0; v < V; ++v) {
        total += w[v];
        if (w[v] > 0.0) last_pos = v;
    }
    *total_out = total;
    if (!(total > 0.0)) {
        *dist_out = 0.0;
        *lo_out = -1;
        *hi_out = -1;
        return -1;
    }
    double target = u * total;
    double cum = 0.0, prev = 0.0;
    int64_t tok = -1;
    for (int64_t v = 0; v < V; ++v) {
        prev = cum;
        cum += w[v];
        if (cum > target) { tok = v; break; }
    }
    if (tok < 0) {
        tok = last_pos;
        *flags |= ORC_FLAG_NO_CROSSING;
        prev = total - w[tok];
        cum = total;
    }
    double d0 = u - prev / total, d1 = cum / total - u;
    *dist_out = d0 < d1 ? d0 : d1;

    /* ids whose interval [c_prev/total, c/total) meets the eps-window */
    double lo_u = u - eps, hi_u = u + eps;
    int32_t lo = -1, hi = -1;
    cum = 0.0;
    for (int64_t v = 0; v < V; ++v) {
        double c0 = cum / total;
        cum += w[v];
        double c1 = cum / total;
        if (w[v] > 0.0 && c1 > lo_u && c0 <= hi_u) {
            if (lo < 0) lo = (int32_t)v;
            hi = (int32_t)v;
        }
    }
    *lo_out = lo;
    *hi_out = hi;
    return tok;
}

/* ------------------------------------------------------------------------ */
/* The verify algorithm for one sequence, uniforms given explicitly.         */
/*                                                                           */
/* P: K+1 target probability rows, Q: K draft probability rows, each of      */
/* length V; x: the K draft ids; u_acc[k]: the accept uniform of position k; */
/* u_res[k]: the residual uniform used if the first rejection is at k;       */
/* u_bonus: the uniform for the extra token when all K are accepted.         */
/* Outputs: tokens[0..K] (x_0..x_{n-1}, the new token, then -1), n, p_k and  */
/* q_k of every draft position, the residual mass Z (0 when all accepted),   */
/* the boundary distances and the eps-window id range of the final draw.     */
/* Returns 0, or -1 on invalid input (id outside [0, V)).                    */
/* ------------------------------------------------------------------------ */
int orc_verify_seq_u(const double* P, const double* Q, const int32_t* x, int32_t K, int64_t V,
                     const double* u_acc, const double* u_res, double u_bonus, double eps,
                     int32_t* tokens, int32_t* n_out, double* p_out, double* q_out,
                     double* z_out, double* d_acc, double* d_fin,
                     int32_t* tok_lo, int32_t* tok_hi, int32_t* flags)
{
    *flags = 0;
    for (int32_t j = 0; j <= K; ++j) tokens[j] = -1;
    for (int32_t k = 0; k < K; ++k) {
        if (x[k] < 0 || (int64_t)x[k] >= V) {
            *flags |= ORC_FLAG_BAD_INPUT;
            *n_out = -1;
            return -1;
        }
    }

    /* Step 3: p, q and the ratio at every draft position. */
    for (int32_t k = 0; k < K; ++k) {
        p_out[k] = P[(int64_t)k * V + x[k]];
        q_out[k] = Q[(int64_t)k * V + x[k]];
        d_acc[k] = INFINITY;
    }

    /* Accept draft k iff u_k < min(1, p/q); stop at the first rejection. */
    int32_t n = K;
    for (int32_t k = 0; k < K; ++k) {
        double p = p_out[k], q = q_out[k];
        double r;
        if (q > 0.0) {
            r = p / q;
            if (r > 1.0) r = 1.0;
        } else {
            r = (p > 0.0) ? 1.0 : 0.0;
        }
        d_acc[k] = fabs(u_acc[k] - r);
        if (!(u_acc[k] < r)) { n = k; break; }
        tokens[k] = x[k];
    }
    *n_out = n;

    double* w = (double*)malloc((size_t)V * sizeof(double));
    if (!w) return -2;
    int64_t tok;
    double total;
    if (n < K) {
        /* Residual p' = norm(max(0, p_n - q_n)). */
        const double* pn = P + (int64_t)n * V;
        const double* qn = Q + (int64_t)n * V;
        for (int64_t v = 0; v < V; ++v) {
            double r = pn[v] - qn[v];
            w[v] = r > 0.0 ? r : 0.0;
        }
        tok = orc_inverse_cdf(w, V, u_res[n], eps, &total, d_fin, tok_lo, tok_hi, flags);
        *z_out = total;
        if (tok < 0) {
            /* No positive residual mass (only reachable through rounding):
               draw from p_n with the same uniform. */
            *flags |= ORC_FLAG_ZERO_RESIDUAL;
            tok = orc_inverse_cdf(pn, V, u_res[n], eps, &total, d_fin, tok_lo, tok_hi, flags);
        }
    } else {
        /* Step 4: every guess accepted, one extra token from p_K. */
        *z_out = 0.0;
        tok = orc_inverse_cdf(P + (int64_t)K * V, V, u_bonus, eps, &total, d_fin,
                              tok_lo, tok_hi, flags);
    }
    free(w);
    if (tok < 0) {
        *flags |= ORC_FLAG_BAD_INPUT;
        return -1;
    }
    tokens[n] = (int32_t)tok;
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Variant with argmax draws ("Text Generation via Speculative Sampling, KV  */
/* Caching, and OpenVINO", "Prepare speculative sampling": step 3 accepts   */
/* with the same probabilistic test but takes the argmax of                  */
/* max_fn(q - p) (in its names; max(0, p - q) here) on a rejection, step 4  */
/* the argmax of the last target position).                                 */
/* ------------------------------------------------------------------------ */

/* First index of the largest w[v] (w >= 0), or -1 when every w is 0.  gap:   */
/* (best - runner-up) / best over the other ids (1 when there is none);     */
/* second: the runner-up's id (-1 when none).                               */
static int64_t orc_argmax_w(const double* w, int64_t V, double* gap, int32_t* second)
{
    int64_t best = -1, sec = -1;
    for (int64_t v = 0; v < V; ++v) {
        if (!(w[v] > 0.0)) continue;
        if (best < 0 || w[v] > w[best]) {
            sec = best;
            best = v;
        } else if (sec < 0 || w[v] > w[sec]) {
            sec = v;
        }
    }
    *second = (int32_t)sec;
    *gap = best < 0 ? 0.0 : (sec < 0 ? 1.0 : (w[best] - w[sec]) / w[best]);
    return best;
}

int orc_verify_argmax_seq(const double* P, const double* Q, const int32_t* x, int32_t K, int64_t V,
                          const double* u_acc, int32_t* tokens, int32_t* n_out, double* p_out, double* q_out,
                          double* z_out, double* d_acc, double* gap, int32_t* second, int32_t* flags)
{
    *flags = 0;
    for (int32_t j = 0; j <= K; ++j) tokens[j] = -1;
    for (int32_t k = 0; k < K; ++k) {
        if (x[k] < 0 || (int64_t)x[k] >= V) {
            *flags |= ORC_FLAG_BAD_INPUT;
            *n_out = -1;
            return -1;
        }
    }
    /* the acceptance test of the sampling variant */
    int32_t n = K;
    for (int32_t k = 0; k < K; ++k) {
        p_out[k] = P[(int64_t)k * V + x[k]];
        q_out[k] = Q[(int64_t)k * V + x[k]];
        d_acc[k] = INFINITY;
    }
    for (int32_t k = 0; k < K; ++k) {
        double p = p_out[k], q = q_out[k];
        double r = q > 0.0 ? (p / q > 1.0 ? 1.0 : p / q) : (p > 0.0 ? 1.0 : 0.0);
        d_acc[k] = fabs(u_acc[k] - r);
        if (!(u_acc[k] < r)) { n = k; break; }
        tokens[k] = x[k];
    }
    *n_out = n;
    int64_t tok;
    if (n < K) {
        double* w = (double*)malloc((size_t)V * sizeof(double));
        if (!w) return -2;
        const double* pn = P + (int64_t)n * V;
        const double* qn = Q + (int64_t)n * V;
        double total = 0.0;
        for (int64_t v = 0; v < V; ++v) {
            double r = pn[v] - qn[v];
            w[v] = r > 0.0 ? r : 0.0;
            total += w[v];
        }
        *z_out = total;
        tok = orc_argmax_w(w, V, gap, second);
        if (tok < 0) {
            /* no positive residual (rounding only): the argmax of p_n */
            *flags |= ORC_FLAG_ZERO_RESIDUAL;
            tok = orc_argmax_w(pn, V, gap, second);
        }
        free(w);
    } else {
        *z_out = 0.0;
        tok = orc_argmax_w(P + (int64_t)K * V, V, gap, second);
    }
    if (tok < 0) {
        *flags |= ORC_FLAG_BAD_INPUT;
        return -1;
    }
    tokens[n] = (int32_t)tok;
    return 0;
}

/* Batch driver of the argmax-draw variant (layout and accept uniforms as      */
/* orc_verify_sample; gap / second per sequence describe the final argmax). */
int orc_verify_argmax(int32_t B, const int32_t* cu, int64_t V, int32_t dtype, const void* target, int64_t t_stride,
                      const void* draft, int64_t d_stride, const int32_t* ids, double T, int32_t top_k,
                      double top_p, uint64_t seed, uint32_t offset, int32_t b_begin, int32_t b_end, int32_t* tokens,
                      int32_t* n_acc, double* probs, double* zmass, double* d_acc, double* gap, int32_t* second,
                      int32_t* flags, double* p_margin)
{
    const size_t esz = dtype == ORC_DTYPE_F32 ? 4 : 2;
    int rc_all = 0;
    double stats[6];
    for (int32_t b = b_begin; b < b_end && b < B; ++b) {
        int32_t K = cu[b + 1] - cu[b];
        int64_t trow0 = (int64_t)cu[b] + b;
        int64_t drow0 = cu[b];
        const size_t k1 = (size_t)(K > 0 ? K : 1);
        double* P = (double*)malloc(sizeof(double) * (size_t)(K + 1) * (size_t)V);
        double* Q = (double*)malloc(sizeof(double) * k1 * (size_t)V);
        double* ua = (double*)malloc(sizeof(double) * k1);
        double* pq = (double*)malloc(sizeof(double) * 2 * k1);
        if (!P || !Q || !ua || !pq) {
            free(P); free(Q); free(ua); free(pq);
            return -2;
        }
        int bad = 0;
        double pm = INFINITY;  /* the sequence's smallest top-p margin */
        for (int32_t k = 0; k <= K; ++k) {
            const char* row = (const char*)target + (size_t)(trow0 + k) * (size_t)t_stride * esz;
            if (orc_row_probs_p(row, dtype, V, T, top_k, top_p, P + (int64_t)k * V, stats) != 0) bad = 1;
            pm = fmin(pm, stats[5]);
        }
        for (int32_t k = 0; k < K; ++k) {
            const char* row = (const char*)draft + (size_t)(drow0 + k) * (size_t)d_stride * esz;
            if (orc_row_probs_p(row, dtype, V, T, top_k, top_p, Q + (int64_t)k * V, stats) != 0) bad = 1;
            pm = fmin(pm, stats[5]);
            ua[k] = orc_uniform(seed, (uint32_t)b, (uint32_t)k, 0u, offset);
        }
        if (p_margin) p_margin[b] = pm;
        int32_t fl = 0;
        int rc = orc_verify_argmax_seq(P, Q, ids + drow0, K, V, ua, tokens + trow0, n_acc + b, pq, pq + k1,
                                       zmass + b, d_acc + drow0, gap + b, second + b, &fl);
        for (int32_t k = 0; k < K; ++k) {
            probs[2 * (drow0 + k)] = pq[k];
            probs[2 * (drow0 + k) + 1] = pq[k1 + k];
        }
        if (bad) fl |= ORC_FLAG_BAD_INPUT;
        flags[b] = fl;
        if (rc != 0 || bad) rc_all = -1;
        free(P); free(Q); free(ua); free(pq);
    }
    return rc_all;
}

/* The same core over many uniform sets (for exhaustive enumeration tests):  */
/* trial t uses u_acc[t*K..], u_res[t*K..] and u_bonus[t].                    */
int orc_verify_seq_u_batch(const double* P, const double* Q, const int32_t* x, int32_t K,
                           int64_t V, int64_t trials, const double* u_acc, const double* u_res,
                           const double* u_bonus, int32_t* tokens, int32_t* n_out)
{
    double* pk = (double*)malloc(sizeof(double) * (size_t)(K + 1));
    double* qk = (double*)malloc(sizeof(double) * (size_t)(K + 1));
    double* dk = (double*)malloc(sizeof(double) * (size_t)(K + 1));
    if (!pk || !qk || !dk) { free(pk); free(qk); free(dk); return -2; }
    int rc = 0;
    for (int64_t t = 0; t < trials; ++t) {
        double z, dfin;
        int32_t lo, hi, fl;
        int r = orc_verify_seq_u(P, Q, x, K, V, u_acc + t * K, u_res + t * K, u_bonus[t], 0.0,
                                 tokens + t * (K + 1), n_out + t, pk, qk, &z, dk, &dfin,
                                 &lo, &hi, &fl);
        if (r != 0) rc = r;
    }
    free(pk); free(qk); free(dk);
    return rc;
}

/* ------------------------------------------------------------------------ */
/* Batched, seeded entry points over a packed ragged batch.                  */
/* Sequence b owns draft rows cu[b]..cu[b+1]-1 and target rows               */
/* cu[b]+b .. cu[b+1]+b; output token slots follow the target rows.          */
/* Uniforms: accept u = U(b, k, 0), residual U(b, n, 1), bonus U(b, K_b, 2). */
/* Only sequences in [b_begin, b_end) are processed (so callers may split    */
/* the batch over threads).                                                  */
/* ------------------------------------------------------------------------ */
int orc_verify_sample(int32_t B, const int32_t* cu, int64_t V, int32_t dtype,
                      const void* target, int64_t t_stride,
                      const void* draft, int64_t d_stride, const int32_t* ids,
                      double T, int32_t top_k, double top_p, uint64_t seed, uint32_t offset, double eps,
                      int32_t b_begin, int32_t b_end,
                      int32_t* tokens, int32_t* n_acc, double* probs, double* zmass,
                      double* d_acc, double* d_fin, int32_t* tok_lo, int32_t* tok_hi,
                      int32_t* flags, double* p_margin)
{
    const size_t esz = dtype == ORC_DTYPE_F32 ? 4 : 2;
    int rc_all = 0;
    double stats[6];
    for (int32_t b = b_begin; b < b_end && b < B; ++b) {
        int32_t K = cu[b + 1] - cu[b];
        int64_t trow0 = (int64_t)cu[b] + b;
        int64_t drow0 = cu[b];
        double* P = (double*)malloc(sizeof(double) * (size_t)(K + 1) * (size_t)V);
        double* Q = (double*)malloc(sizeof(double) * (size_t)(K > 0 ? K : 1) * (size_t)V);
        double* ua = (double*)malloc(sizeof(double) * (size_t)(K > 0 ? K : 1));
        double* ur = (double*)malloc(sizeof(double) * (size_t)(K > 0 ? K : 1));
        double* pq = (double*)malloc(sizeof(double) * 2 * (size_t)(K > 0 ? K : 1));
        if (!P || !Q || !ua || !ur || !pq) {
            free(P); free(Q); free(ua); free(ur); free(pq);
            return -2;
        }
        int bad = 0;
        double pm = INFINITY;  /* the sequence's smallest top-p margin */
        for (int32_t k = 0; k <= K; ++k) {
            const char* row = (const char*)target + (size_t)(trow0 + k) * (size_t)t_stride * esz;
            if (orc_row_probs_p(row, dtype, V, T, top_k, top_p, P + (int64_t)k * V, stats) != 0) bad = 1;
            pm = fmin(pm, stats[5]);
        }
        for (int32_t k = 0; k < K; ++k) {
            const char* row = (const char*)draft + (size_t)(drow0 + k) * (size_t)d_stride * esz;
            if (orc_row_probs_p(row, dtype, V, T, top_k, top_p, Q + (int64_t)k * V, stats) != 0) bad = 1;
            pm = fmin(pm, stats[5]);
            ua[k] = orc_uniform(seed, (uint32_t)b, (uint32_t)k, 0u, offset);
        }
        for (int32_t k = 0; k < K; ++k)
            ur[k] = orc_uniform(seed, (uint32_t)b, (uint32_t)k, 1u, offset);
        double u_bonus = orc_uniform(seed, (uint32_t)b, (uint32_t)K, 2u, offset);

        if (p_margin) p_margin[b] = pm;
        int32_t fl = 0;
        double* dk = d_acc + drow0;
        int rc = orc_verify_seq_u(P, Q, ids + drow0, K, V, ua, ur, u_bonus, eps,
                                  tokens + trow0, n_acc + b, pq, pq + (K > 0 ? K : 1),
                                  zmass + b, dk, d_fin + b, tok_lo + b, tok_hi + b, &fl);
        for (int32_t k = 0; k < K; ++k) {
            probs[2 * (drow0 + k)] = pq[k];
            probs[2 * (drow0 + k) + 1] = pq[(K > 0 ? K : 1) + k];
        }
        if (bad) fl |= ORC_FLAG_BAD_INPUT;
        flags[b] = fl;
        if (rc != 0 || bad) rc_all = -1;
        free(P); free(Q); free(ua); free(ur); free(pq);
    }
    return rc_all;
}

/*
 * Draft-side sampling, the step before verify: the draft model proposes the
 * K guesses one position at a time ("Text Generation via Speculative
 * Sampling, KV Caching, and OpenVINO", "Prepare speculative sampling", step
 * 1, where it takes the argmax), and the acceptance proof of
 * "CS3602_FINAL_SpeDec", section 2, assumes each guess is drawn from q.  So
 * x(b, k) is the inverse-CDF draw (ascending ids) of q_k = softmax(draft row
 * k / T) over its top-k kept set, with U(b, k, 3).  Per draft row: the id,
 * the distance from u to the chosen id's interval edges, the ids whose
 * interval meets [u - eps, u + eps], and flags.
 */
int orc_draft_sample(int32_t B, const int32_t* cu, int64_t V, int32_t dtype, const void* draft, int64_t d_stride,
                     double T, int32_t top_k, double top_p, uint64_t seed, uint32_t offset, double eps,
                     int32_t b_begin, int32_t b_end, int32_t* ids, double* dist, int32_t* tok_lo, int32_t* tok_hi,
                     int32_t* flags, double* p_margin)
{
    const size_t esz = dtype == ORC_DTYPE_F32 ? 4 : 2;
    double* q = (double*)malloc(sizeof(double) * (size_t)V);
    if (!q) return -2;
    double stats[6];
    int rc_all = 0;
    for (int32_t b = b_begin; b < b_end && b < B; ++b) {
        const int32_t K = cu[b + 1] - cu[b];
        for (int32_t k = 0; k < K; ++k) {
            const int64_t r = (int64_t)cu[b] + k;
            const char* row = (const char*)draft + (size_t)r * (size_t)d_stride * esz;
            int32_t fl = 0;
            if (orc_row_probs_p(row, dtype, V, T, top_k, top_p, q, stats) != 0) fl |= ORC_FLAG_BAD_INPUT;
            if (p_margin) p_margin[r] = stats[5];
            const double u = orc_uniform(seed, (uint32_t)b, (uint32_t)k, 3u, offset);
            double total;
            ids[r] = (int32_t)orc_inverse_cdf(q, V, u, eps, &total, dist + r, tok_lo + r, tok_hi + r, &fl);
            flags[r] = fl;
            if (fl & ORC_FLAG_BAD_INPUT) rc_all = -1;
        }
    }
    free(q);
    return rc_all;
}

/*
 * Per-token speculative likelihood: the probability that one speculative
 * step emits a given token y, split as in the proof of
 * "CS3602_FINAL_SpeDec", section 2, and used for that report's perplexity
 * check (its problem analysis, item 1):
 *   beta             = sum_v min(p(v), q(v))                (acceptance mass)
 *   accept part      = q(y) * min(1, p(y) / q(y))           (guess y accepted)
 *   reject part      = (1 - beta) * p'(y),  p' = norm(max(0, p - q))
 *                                                           (guess rejected, y drawn)
 *   P(y)             = accept part + reject part
 * with p = softmax(target row / T) and q = softmax(draft row / T), each over
 * its top-k kept set.  The sum over the vocabulary is taken as written (no
 * shortcut through the identity reject part = p(y) - min(p(y), q(y))); a
 * residual with no positive mass gives a zero reject part.  Position (b, k),
 * k < K_b, is row cu[b] + k of both tensors; nll[b] = -sum_k log P(y_k).
 * Outputs per position: terms[3 r + 0..2] = accept part, reject part, p(y);
 * beta[r].  A sequence with a bad row (no finite kept logit) or a token
 * outside [0, V) gets the bad-input flag and nll = NaN; such a position's
 * terms are NaN, and so is a bad row's beta.
 */
int orc_token_likelihood(int32_t B, const int32_t* cu, int64_t V, int32_t dtype, const void* target,
                         int64_t t_stride, const void* draft, int64_t d_stride, double T, int32_t top_k,
                         double top_p, const int32_t* tokens, int32_t b_begin, int32_t b_end, double* terms,
                         double* beta, double* nll, int32_t* flags, double* p_margin)
{
    const size_t esz = dtype == ORC_DTYPE_F32 ? 4 : 2;
    double* P = (double*)malloc(sizeof(double) * (size_t)V);
    double* Q = (double*)malloc(sizeof(double) * (size_t)V);
    if (!P || !Q) {
        free(P);
        free(Q);
        return -2;
    }
    double stats[6];
    int rc_all = 0;
    for (int32_t b = b_begin; b < b_end && b < B; ++b) {
        const int32_t K = cu[b + 1] - cu[b];
        int32_t fl = 0;
        double s_nll = 0.0;
        for (int32_t k = 0; k < K; ++k) {
            const int64_t r = (int64_t)cu[b] + k;
            const char* trow = (const char*)target + (size_t)r * (size_t)t_stride * esz;
            const char* drow = (const char*)draft + (size_t)r * (size_t)d_stride * esz;
            const int bad_t = orc_row_probs_p(trow, dtype, V, T, top_k, top_p, P, stats) != 0;
            const double pm_t = stats[5];
            const int bad_d = orc_row_probs_p(drow, dtype, V, T, top_k, top_p, Q, stats) != 0;
            if (p_margin) p_margin[r] = fmin(pm_t, stats[5]);
            if (bad_t || bad_d) {
                /* a row with no finite kept logit defines no distribution */
                fl |= ORC_FLAG_BAD_INPUT;
                beta[r] = NAN;
                terms[3 * r] = terms[3 * r + 1] = terms[3 * r + 2] = NAN;
                continue;
            }
            double bsum = 0.0, zsum = 0.0;
            for (int64_t v = 0; v < V; ++v) {
                bsum += P[v] < Q[v] ? P[v] : Q[v];
                zsum += P[v] > Q[v] ? P[v] - Q[v] : 0.0;
            }
            beta[r] = bsum;
            const int32_t y = tokens[r];
            if (y < 0 || (int64_t)y >= V) {
                fl |= ORC_FLAG_BAD_INPUT;
                terms[3 * r] = terms[3 * r + 1] = terms[3 * r + 2] = NAN;
                continue;
            }
            const double py = P[y], qy = Q[y];
            double acc;
            if (qy > 0.0) {
                const double ratio = py / qy;
                acc = qy * (ratio < 1.0 ? ratio : 1.0);
            } else {
                acc = 0.0;
            }
            const double rdens = py > qy ? py - qy : 0.0;   /* max(0, p - q) at y */
            const double rej = zsum > 0.0 ? (1.0 - bsum) * (rdens / zsum) : 0.0;
            terms[3 * r] = acc;
            terms[3 * r + 1] = rej;
            terms[3 * r + 2] = py;
            s_nll -= log(acc + rej);
        }
        nll[b] = (fl & ORC_FLAG_BAD_INPUT) ? NAN : s_nll;
        flags[b] = fl;
        if (fl & ORC_FLAG_BAD_INPUT) rc_all = -1;
    }
    free(P);
    free(Q);
    return rc_all;
}

/*
 * Greedy argmax-compare: a_k = argmax of target row k; n = the first k with
 * x_k != a_k (K_b when none); tokens x_0..x_{n-1}, a_n, then -1.
 */
int orc_verify_greedy(int32_t B, const int32_t* cu, int64_t V, int32_t dtype,
                      const void* target, int64_t t_stride, const int32_t* ids,
                      int32_t b_begin, int32_t b_end, int32_t* tokens, int32_t* n_acc)
{
    const size_t esz = dtype == ORC_DTYPE_F32 ? 4 : 2;
    for (int32_t b = b_begin; b < b_end && b < B; ++b) {
        int32_t K = cu[b + 1] - cu[b];
        int64_t trow0 = (int64_t)cu[b] + b;
        int64_t drow0 = cu[b];
        for (int32_t j = 0; j <= K; ++j) tokens[trow0 + j] = -1;
        /* a guess outside [0, V) makes the sequence invalid (reported as -1),
           wherever it stands, as in the sampling variant */
        int bad = 0;
        for (int32_t k = 0; k < K; ++k)
            if (ids[drow0 + k] < 0 || (int64_t)ids[drow0 + k] >= V) bad = 1;
        if (bad) {
            n_acc[b] = -1;
            continue;
        }
        int32_t n = K;
        for (int32_t k = 0; k <= K; ++k) {
            const char* row = (const char*)target + (size_t)(trow0 + k) * (size_t)t_stride * esz;
            int64_t a = orc_row_argmax(row, dtype, V);
            if (k == K || ids[drow0 + k] != (int32_t)a) {
                n = k;
                tokens[trow0 + k] = (int32_t)a;
                break;
            }
            tokens[trow0 + k] = ids[drow0 + k];
        }
        n_acc[b] = n;
    }
    return 0;
}
