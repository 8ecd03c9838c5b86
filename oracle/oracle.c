/*
 * oracle.c -- plain fp64 CPU oracle for exact causal grouped-query attention
 * over a K/V history, and for the deterministic K/V page regenerator.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library links, includes or
 * calls this file; only the test suite, the smoke check and the benchmark's
 * CPU-baseline leg load it (through oracle/__init__.py).  It shares no code,
 * header, table or constant generator with the HIP path.
 *
 * What it computes (sources are the three reference pages):
 *
 *  - Attention.  CFR-Atlas README, "Core contract": the folded (paged) result
 *    must equal full_kv_attention(query) over every causal K/V row.  This file
 *    is that full-KV attention written out: for each query row and q-head it
 *    materialises every visible score, takes the maximum, then a second pass
 *    forms exp(s - max), their sum, and the weighted sum of V rows, all in
 *    fp64.  No pages, no online softmax, no blocking.
 *      * query positions: CPUAttn README, "Parallel example" -- with a K/V
 *        cache the queries are the suffix of K/V, so query i sits at position
 *        S_kv - S_q + i.  Callers pass the absolute position of every query
 *        row explicitly.
 *      * GQA/MQA/MHA: an explicit q-head -> K/V-head map (CPUAttn "Operator
 *        model"; CFR-Atlas "Validation and hardening" lists MHA/MQA/GQA
 *        mapping).
 *      * sliding window, attention sinks, logit softcap: ferrox-core crate
 *        index, attention re-exports (causal_gqa_attention_windowed, _sinks,
 *        _softcap, _windowed_softcap).  The pages give names only; the
 *        readings used here are: window W keeps keys j with pos - W < j <= pos;
 *        sink count n keeps keys j < n (still j <= pos) in addition; softcap c
 *        replaces a scaled score s by c * tanh(s / c), applied after the scale
 *        and before masking/softmax.
 *
 *  - Regenerator.  CFR-Atlas README, "Minimal integration": a page is replayed
 *    as row-major K[token][dim] and V[token][dim] for one (layer, K/V head,
 *    token range).  The reference adapter's generator is not shown on the
 *    pages, so this file defines one from published algorithms:
 *      * Philox4x32-10, J. K. Salmon, M. A. Moraes, R. O. Dror, D. E. Shaw,
 *        "Parallel Random Numbers: As Easy as 1, 2, 3", SC'11, the section
 *        defining Philox (S-box, key schedule, multipliers, Weyl constants).
 *      * Box-Muller transform, G. E. P. Box and M. E. Muller, "A Note on the
 *        Generation of Random Normal Deviates", Ann. Math. Stat. 29 (1958).
 *    Counter = (token, dim/4, head | tensor<<30, layer | seq<<16), key = the
 *    64-bit seed split low/high; tensor 0 = Q, 1 = K, 2 = V.  Word x maps to
 *    u = (floor(x / 2^9) + 1/2) * 2^-23, which is exact in fp32 and never 0
 *    or 1.  Words (x0, x1) give dims 4k and 4k+1 as r cos(2 pi u1) and
 *    r sin(2 pi u1) with r = sqrt(-2 ln u0); words (x2, x3) give dims 4k+2
 *    and 4k+3 the same way.  The value is formed in fp64 and rounded to the
 *    storage type (fp32 round-to-nearest-even; bf16 rounds that fp32 value
 *    to nearest-even).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

/* ---------------------------------------------------------------- Philox */

/* Salmon et al. SC'11, Philox section: the Philox-4x32 S-box multipliers and
 * the key-schedule (Weyl sequence) increments. */
#define ORACLE_PHILOX_MUL_A 0xD2511F53u
#define ORACLE_PHILOX_MUL_B 0xCD9E8D57u
#define ORACLE_PHILOX_WEYL_A 0x9E3779B9u
#define ORACLE_PHILOX_WEYL_B 0xBB67AE85u

/* One application of the 10-round Philox4x32 bijection to counter `ctr`
 * under key `key`.  Each round multiplies words 0 and 2 by the two constants
 * (64-bit products split into high/low halves), then outputs
 *   (hi(B*x2) ^ x1 ^ k0, lo(B*x2), hi(A*x0) ^ x3 ^ k1, lo(A*x0));
 * the key is advanced by the Weyl increments between rounds. */
void oracle_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4])
{
    uint32_t x0 = ctr[0], x1 = ctr[1], x2 = ctr[2], x3 = ctr[3];
    uint32_t k0 = key[0], k1 = key[1];
    for (int round = 0; round < 10; ++round) {
        if (round > 0) {
            k0 += ORACLE_PHILOX_WEYL_A;
            k1 += ORACLE_PHILOX_WEYL_B;
        }
        uint64_t prod_a = (uint64_t)ORACLE_PHILOX_MUL_A * (uint64_t)x0;
        uint64_t prod_b = (uint64_t)ORACLE_PHILOX_MUL_B * (uint64_t)x2;
        uint32_t hi_a = (uint32_t)(prod_a >> 32), lo_a = (uint32_t)prod_a;
        uint32_t hi_b = (uint32_t)(prod_b >> 32), lo_b = (uint32_t)prod_b;
        uint32_t n0 = hi_b ^ x1 ^ k0;
        uint32_t n1 = lo_b;
        uint32_t n2 = hi_a ^ x3 ^ k1;
        uint32_t n3 = lo_a;
        x0 = n0; x1 = n1; x2 = n2; x3 = n3;
    }
    out[0] = x0; out[1] = x1; out[2] = x2; out[3] = x3;
}

/* Bulk form for tests: n counters (row-major [n][4]) under one key. */
void oracle_philox4x32_10_batch(int64_t n, const uint32_t *ctrs, const uint32_t key[2], uint32_t *outs)
{
    for (int64_t i = 0; i < n; ++i)
        oracle_philox4x32_10(ctrs + 4 * i, key, outs + 4 * i);
}

/* ------------------------------------------------------ regenerated K/V */

/* Uniform in (0,1): (floor(x / 2^9) + 1/2) * 2^-23. */
static double oracle_uniform(uint32_t x)
{
    return ((double)(x >> 9) + 0.5) * (1.0 / 8388608.0);
}

double oracle_regen_value(uint64_t seed, uint32_t layer, uint32_t seq, uint32_t tensor,
                          uint32_t head, uint32_t token, uint32_t dim)
{
    uint32_t ctr[4] = { token, dim >> 2, head | (tensor << 30), layer | (seq << 16) };
    uint32_t key[2] = { (uint32_t)seed, (uint32_t)(seed >> 32) };
    uint32_t w[4];
    oracle_philox4x32_10(ctr, key, w);
    int pair = (int)((dim >> 1) & 1u);
    double u_radius = oracle_uniform(w[2 * pair]);
    double u_angle = oracle_uniform(w[2 * pair + 1]);
    double r = sqrt(-2.0 * log(u_radius));
    double theta = 2.0 * M_PI * u_angle;
    return (dim & 1u) ? r * sin(theta) : r * cos(theta);
}

/* fp32 -> bf16 bit pattern, round to nearest, ties to even (finite input). */
static uint16_t oracle_f32_to_bf16_bits(float f)
{
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    uint32_t lsb = (u >> 16) & 1u;
    u += 0x7FFFu + lsb;
    return (uint16_t)(u >> 16);
}

/* Rows [t0, t0 + n_tokens) of one (layer, seq, tensor, head) stream, D dims
 * per row, row-major.  out_kind: 0 = fp64, 1 = fp32, 2 = bf16 bit patterns. */
void oracle_regen_rows(uint64_t seed, uint32_t layer, uint32_t seq, uint32_t tensor, uint32_t head,
                       int64_t t0, int64_t n_tokens, int dims, int out_kind, void *out)
{
    #pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < n_tokens; ++t) {
        for (int d = 0; d < dims; ++d) {
            double z = oracle_regen_value(seed, layer, seq, tensor, head, (uint32_t)(t0 + t), (uint32_t)d);
            int64_t idx = t * dims + d;
            if (out_kind == 0) {
                ((double *)out)[idx] = z;
            } else if (out_kind == 1) {
                ((float *)out)[idx] = (float)z;
            } else {
                ((uint16_t *)out)[idx] = oracle_f32_to_bf16_bits((float)z);
            }
        }
    }
}

/* ------------------------------------------------------------ attention */

/* Is key j visible from a query at absolute position pos? */
static int oracle_visible(int64_t j, int64_t pos, int64_t window, int64_t n_sinks)
{
    if (j > pos)
        return 0;
    if (window <= 0)
        return 1;
    if (j > pos - window)
        return 1;
    return j < n_sinks;
}

/*
 * Full-KV attention for one sequence, two-pass fp64 softmax, with the score
 * and mask modifications of the CPUAttn operator model ("Operator model":
 * standard or causal Parallel attention whose score_mod / mask_mod are
 * elementwise expressions; "Parallel lowering": arbitrary masks keep their
 * elementwise meaning).
 *   nq          number of query rows
 *   pos[nq]     absolute position of each query row (0 <= pos < n_kv)
 *   n_kv        number of K/V rows supplied (history length)
 *   q           [nq][hq][dims]          query values (fp32 or bf16-exact)
 *   k, v        [hkv][n_kv][dims]       key / value rows
 *   head_map    [hq] -> K/V head
 *   scale       score scale
 *   window      0 = off, else keys with pos - window < j <= pos (causal only)
 *   n_sinks     keys j < n_sinks stay visible when a window is set
 *   softcap     0 = off, else s -> softcap * tanh(s / softcap)
 *   causal      1: key j needs j <= pos; 0: every key j < n_kv
 *   alibi       [hq] slopes or NULL: the logit gains -slope_h * |pos - j|
 *               after the softcap
 *   mask        [nq][n_kv] bytes or NULL: key j of row i also needs
 *               mask[i][j] != 0
 *   allow_empty 0: a row with no visible key is an error; 1: its output is
 *               NaN and its lse -inf
 *   out         [nq][hq][dims]  fp64
 *   lse         [nq][hq]        fp64, natural log of the softmax denominator
 *                               plus the maximum (i.e. log sum exp s_j)
 * Returns 0, or -1 when a row has no visible key (allow_empty = 0) or a
 * position is out of range.
 */
int oracle_attend_mods(int nq, const int32_t *pos, int64_t n_kv, int hq, int hkv, int dims,
                       const float *q, const float *k, const float *v, const int32_t *head_map,
                       double scale, int64_t window, int64_t n_sinks, double softcap,
                       int causal, const double *alibi, const uint8_t *mask, int allow_empty,
                       double *out, double *lse)
{
    for (int i = 0; i < nq; ++i)
        if (pos[i] < 0 || pos[i] >= n_kv)
            return -1;
    for (int h = 0; h < hq; ++h)
        if (head_map[h] < 0 || head_map[h] >= hkv)
            return -1;

    int failed = 0;
    int64_t rows = (int64_t)nq * hq;
    #pragma omp parallel
    {
        double *score = (double *)malloc(sizeof(double) * (size_t)(n_kv > 0 ? n_kv : 1));
        #pragma omp for schedule(dynamic, 1)
        for (int64_t r = 0; r < rows; ++r) {
            int i = (int)(r / hq), h = (int)(r % hq);
            int g = head_map[h];
            const float *qrow = q + ((int64_t)i * hq + h) * dims;
            const float *kh = k + (int64_t)g * n_kv * dims;
            const float *vh = v + (int64_t)g * n_kv * dims;
            double *orow = out + ((int64_t)i * hq + h) * dims;
            int64_t p = pos[i];
            /* causal: the keys up to the row's position; else the whole history */
            int64_t j_end = causal ? p + 1 : n_kv;

            /* pass 1: scores and their maximum over the visible set */
            double m = -INFINITY;
            int64_t n_visible = 0;
            for (int64_t j = 0; j < j_end; ++j) {
                if (causal && !oracle_visible(j, p, window, n_sinks))
                    continue;
                if (mask && !mask[(int64_t)i * n_kv + j])
                    continue;
                double s = 0.0;
                for (int d = 0; d < dims; ++d)
                    s += (double)qrow[d] * (double)kh[j * dims + d];
                s *= scale;
                if (softcap > 0.0)
                    s = softcap * tanh(s / softcap);
                if (alibi)
                    s -= alibi[h] * (double)(p > j ? p - j : j - p);
                score[j] = s;
                if (s > m)
                    m = s;
                ++n_visible;
            }
            if (n_visible == 0) {
                if (!allow_empty) {
                    #pragma omp atomic write
                    failed = 1;
                } else {
                    for (int d = 0; d < dims; ++d)
                        orow[d] = NAN;
                    lse[(int64_t)i * hq + h] = -INFINITY;
                }
                continue;
            }

            /* pass 2: exp(s - m), their sum, and the weighted V sum */
            double l = 0.0;
            for (int d = 0; d < dims; ++d)
                orow[d] = 0.0;
            for (int64_t j = 0; j < j_end; ++j) {
                if (causal && !oracle_visible(j, p, window, n_sinks))
                    continue;
                if (mask && !mask[(int64_t)i * n_kv + j])
                    continue;
                double w = exp(score[j] - m);
                l += w;
                for (int d = 0; d < dims; ++d)
                    orow[d] += w * (double)vh[j * dims + d];
            }
            for (int d = 0; d < dims; ++d)
                orow[d] /= l;
            lse[(int64_t)i * hq + h] = m + log(l);
        }
        free(score);
    }
    return failed ? -1 : 0;
}

/* Causal attention without mods (the method's plain form). */
int oracle_attend(int nq, const int32_t *pos, int64_t n_kv, int hq, int hkv, int dims,
                  const float *q, const float *k, const float *v, const int32_t *head_map,
                  double scale, int64_t window, int64_t n_sinks, double softcap,
                  double *out, double *lse)
{
    return oracle_attend_mods(nq, pos, n_kv, hq, hkv, dims, q, k, v, head_map, scale, window, n_sinks,
                              softcap, 1, NULL, NULL, 0, out, lse);
}

/* Number of OpenMP threads a parallel region would use (1 without OpenMP). */
int oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
