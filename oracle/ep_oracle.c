/*
 * ep_oracle.c -- the CPU oracle for MoE dispatch / combine (test
 * infrastructure only; see ep_oracle.h for the page key and notation).
 *
 * Build: gcc -std=c11 -O2 -ffp-contract=off (no fast-math), x86-64 SSE, so
 * every float operation below is one correctly rounded binary32 operation and
 * fmaf() is the C library's correctly rounded fused multiply-add.
 *
 * Readings of points the pages leave open (each is listed with its reason in
 * the design notes):
 *  - a (token, slot) pair is one received row; rank r's row count is the number
 *    of pairs routed to its experts, so the counts sum to T*k;
 *  - inside an expert's segment the pairs keep ascending p = t*k + j order;
 *  - slots are numbered expert-major over all ranks, so rank r's rows are the
 *    slot range [roff[r], roff[r+1]) and row = slot - roff[r];
 *  - the same expert may appear twice in a token's top-k row: each pair is its
 *    own row;
 *  - FP8 is OCP E4M3 "fn"; the per-block scale is s = a/448 rounded to binary32,
 *    the code is E4M3(RN32(x/s)) with ties to even and saturation at +-448;
 *    an all-zero block gives s = 0 and codes 0x00; signed zeros keep their sign;
 *    non-finite values follow IEEE binary32: a NaN in a block makes its amax
 *    (and so s and every code) NaN, an infinity makes s = +inf, so finite
 *    values encode as signed zeros and infinities as NaN codes;
 *  - combine accumulates in binary32 with fmaf in ascending j from +0, then
 *    rounds once to bf16 with ties to even.
 */
#include "ep_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------ codecs */

float oracle_bf16_to_f32(uint16_t b)
{
    /* bf16 is the top half of a binary32 pattern: widening is exact. */
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

uint16_t oracle_bf16_rne(float v)
{
    /* Nearest bf16 value, ties to the one whose last kept bit is 0.  The two
     * candidates are the truncation toward zero ("lo") and the next bf16 away
     * from zero ("lo" + one unit in the 16th bit, which carries into the
     * exponent and reaches infinity correctly); the discarded low 16 bits
     * measure the distance to "lo" in units of 2^-16 of the bf16 spacing. */
    uint32_t u;
    memcpy(&u, &v, sizeof u);
    if (isnan(v))
        return (uint16_t)((u >> 16) | 0x0040u); /* quiet NaN, sign kept */
    uint32_t lo = u >> 16;
    uint32_t rem = u & 0xFFFFu;
    if (rem > 0x8000u)
        return (uint16_t)(lo + 1u);
    if (rem < 0x8000u)
        return (uint16_t)lo;
    return (uint16_t)((lo & 1u) ? lo + 1u : lo); /* exact tie: to even */
}

/* Round a non-negative double that holds an exact value to the nearest
 * integer, ties to even. */
static double round_half_even(double n)
{
    double f = floor(n);
    double d = n - f;
    if (d > 0.5)
        return f + 1.0;
    if (d < 0.5)
        return f;
    return (fmod(f, 2.0) == 0.0) ? f : f + 1.0;
}

uint8_t oracle_e4m3_encode(float v)
{
    /* OCP E4M3 "fn": magnitudes (1+m/8)*2^(e) for e in [-6, 8] and m*2^-9
     * below 2^-6; the largest finite value is 1.75*2^8 = 448 (code 0x7E) and
     * S.1111.111 is NaN.  Round to nearest with ties to an even mantissa
     * code, then saturate: every magnitude >= 448 becomes 448, which is the
     * same as "round, then clamp" because (448, 464] already rounds to 448. */
    uint8_t sign = signbit(v) ? 0x80 : 0x00;
    if (isnan(v))
        return (uint8_t)(sign | 0x7F);
    double m = fabs((double)v); /* exact */
    if (m >= 448.0)
        return (uint8_t)(sign | 0x7E);
    if (m < 0.015625) {
        /* subnormal range: spacing 2^-9, code = count of 2^-9 steps; 8 steps
         * is 2^-6, which is exactly code 0x08 (the smallest normal). */
        double n = round_half_even(m * 512.0);
        return (uint8_t)(sign | (uint8_t)n);
    }
    int ex;
    (void)frexp(m, &ex); /* m in [2^(ex-1), 2^ex) */
    int e = ex - 1;
    double n = round_half_even(ldexp(m, 3 - e)); /* m / 2^(e-3) in [8, 16] */
    if (n == 16.0) {                             /* carry into the next binade */
        e += 1;
        n = 8.0;
    }
    int code = ((e + 7) << 3) | ((int)n - 8);
    if (code > 0x7E)
        code = 0x7E;
    return (uint8_t)(sign | code);
}

float oracle_e4m3_decode(uint8_t c)
{
    int S = c >> 7, Ex = (c >> 3) & 15, M = c & 7;
    if (Ex == 15 && M == 7)
        return S ? -NAN : NAN;
    double mag = (Ex == 0) ? M * ldexp(1.0, -9) : (1.0 + M / 8.0) * ldexp(1.0, Ex - 7);
    return (float)(S ? -mag : mag);
}

void oracle_e4m3_encode_n(const float *v, uint8_t *out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = oracle_e4m3_encode(v[i]);
}

void oracle_e4m3_decode_n(const uint8_t *c, float *out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = oracle_e4m3_decode(c[i]);
}

void oracle_bf16_rne_n(const float *v, uint16_t *out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = oracle_bf16_rne(v[i]);
}

/* ------------------------------------------------------------------ layout */

int oracle_validate(int T, int H, int k, int E, int R, int fp8, const int32_t *idx)
{
    if (T < 1 || k < 1 || R < 1 || E < 1 || H < 8)
        return 1;
    if (E % R != 0 || H % 8 != 0)
        return 1;
    if (fp8 && H % 128 != 0)
        return 1;
    int64_t P = (int64_t)T * k;
    if (P > 0x7FFFFFFF)
        return 1;
    for (int64_t p = 0; p < P; ++p)
        if (idx[p] < 0 || idx[p] >= E)
            return 2;
    return 0;
}

int oracle_layout(int T, int k, int E, int R, const int32_t *idx,
                  int32_t *cnt, int32_t *off, int32_t *rcnt, int32_t *roff,
                  int32_t *slot, int32_t *src, int32_t *row)
{
    int rc = oracle_validate(T, 8, k, E, R, 0, idx);
    if (rc)
        return rc;
    const int64_t P = (int64_t)T * k;
    const int El = E / R;

    /* count: cnt[e] = #{p : idx[p] = e} */
    for (int e = 0; e < E; ++e)
        cnt[e] = 0;
    for (int64_t p = 0; p < P; ++p)
        cnt[idx[p]] += 1;

    /* exclusive prefix over experts, then the per-rank ranges */
    off[0] = 0;
    for (int e = 0; e < E; ++e)
        off[e + 1] = off[e] + cnt[e];
    for (int r = 0; r < R; ++r) {
        roff[r] = off[r * El];
        rcnt[r] = off[(r + 1) * El] - off[r * El];
    }
    roff[R] = (int32_t)P;

    /* stable counting sort: visit pairs in ascending p, each takes the next
     * free slot of its expert's segment */
    int32_t *fill = (int32_t *)calloc((size_t)E, sizeof(int32_t));
    if (!fill)
        return 3;
    for (int64_t p = 0; p < P; ++p) {
        int e = idx[p];
        slot[p] = off[e] + fill[e];
        fill[e] += 1;
        src[slot[p]] = (int32_t)p;
        row[p] = slot[p] - roff[e / El];
    }
    free(fill);
    return 0;
}

/* ---------------------------------------------------------------- dispatch */

void oracle_dispatch_bf16(int T, int H, int k, int E, int R, const int32_t *idx,
                          const int32_t *slot, const int32_t *roff,
                          const uint16_t *x, uint16_t *const *recv)
{
    const int El = E / R;
    (void)R;
    for (int t = 0; t < T; ++t)
        for (int j = 0; j < k; ++j) {
            int64_t p = (int64_t)t * k + j;
            int r = idx[p] / El;
            int64_t rrow = slot[p] - roff[r];
            memcpy(recv[r] + rrow * H, x + (int64_t)t * H, (size_t)H * sizeof(uint16_t));
        }
}

void oracle_quantize_row(int H, const uint16_t *xrow, uint8_t *q, float *s)
{
    for (int b = 0; b < H / 128; ++b) {
        const uint16_t *xb = xrow + b * 128;
        float a = 0.0f; /* amax of the block; a NaN value makes it NaN */
        for (int h = 0; h < 128; ++h) {
            float v = fabsf(oracle_bf16_to_f32(xb[h]));
            if (v > a || isnan(v))
                a = v;
        }
        if (a == 0.0f) {
            s[b] = 0.0f;
            for (int h = 0; h < 128; ++h)
                q[b * 128 + h] = 0x00;
            continue;
        }
        float sb = a / 448.0f; /* binary32 division */
        s[b] = sb;
        for (int h = 0; h < 128; ++h) {
            float ratio = oracle_bf16_to_f32(xb[h]) / sb; /* binary32 division */
            q[b * 128 + h] = oracle_e4m3_encode(ratio);
        }
    }
}

void oracle_dispatch_fp8(int T, int H, int k, int E, int R, const int32_t *idx,
                         const int32_t *slot, const int32_t *roff,
                         const uint16_t *x, uint8_t *const *recv_q,
                         float *const *recv_s)
{
    const int El = E / R;
    const int nb = H / 128;
    (void)R;
    uint8_t *q = (uint8_t *)malloc((size_t)H);
    float *s = (float *)malloc((size_t)nb * sizeof(float));
    if (!q || !s) {
        free(q);
        free(s);
        return;
    }
    for (int t = 0; t < T; ++t) {
        oracle_quantize_row(H, x + (int64_t)t * H, q, s);
        for (int j = 0; j < k; ++j) {
            int64_t p = (int64_t)t * k + j;
            int r = idx[p] / El;
            int64_t rrow = slot[p] - roff[r];
            memcpy(recv_q[r] + rrow * H, q, (size_t)H);
            memcpy(recv_s[r] + rrow * nb, s, (size_t)nb * sizeof(float));
        }
    }
    free(q);
    free(s);
}

/* ------------------------------------------------------ unpermute, combine */

void oracle_unpermute(int T, int H, int k, int E, int R, const int32_t *idx,
                      const int32_t *slot, const int32_t *roff,
                      const uint16_t *const *recv_y, uint16_t *u)
{
    const int El = E / R;
    (void)R;
    for (int64_t p = 0; p < (int64_t)T * k; ++p) {
        int r = idx[p] / El;
        int64_t rrow = slot[p] - roff[r];
        memcpy(u + p * H, recv_y[r] + rrow * H, (size_t)H * sizeof(uint16_t));
    }
}

void oracle_combine(int T, int H, int k, int E, int R, const int32_t *idx,
                    const int32_t *slot, const int32_t *roff,
                    const uint16_t *const *recv_y, const float *w, uint16_t *out)
{
    const int El = E / R;
    (void)R;
    const uint16_t **rows = (const uint16_t **)malloc((size_t)k * sizeof(*rows));
    if (!rows)
        return;
    for (int t = 0; t < T; ++t) {
        /* the k received rows of token t, in j order */
        for (int j = 0; j < k; ++j) {
            int64_t p = (int64_t)t * k + j;
            int r = idx[p] / El;
            int64_t rrow = slot[p] - roff[r];
            rows[j] = recv_y[r] + rrow * H;
        }
        for (int h = 0; h < H; ++h) {
            float acc = 0.0f;
            for (int j = 0; j < k; ++j) {
                float wj = w ? w[(int64_t)t * k + j] : 1.0f;
                acc = fmaf(wj, oracle_bf16_to_f32(rows[j][h]), acc);
            }
            out[(int64_t)t * H + h] = oracle_bf16_rne(acc);
        }
    }
    free(rows);
}

void oracle_combine_shared(int T, int H, int k, int E, int R, const int32_t *idx,
                           const int32_t *slot, const int32_t *roff,
                           const uint16_t *const *recv_y, const float *w,
                           const uint16_t *shared, uint16_t *out)
{
    const int El = E / R;
    (void)R;
    const uint16_t **rows = (const uint16_t **)malloc((size_t)k * sizeof(*rows));
    if (!rows)
        return;
    for (int t = 0; t < T; ++t) {
        for (int j = 0; j < k; ++j) {
            int64_t p = (int64_t)t * k + j;
            int r = idx[p] / El;
            rows[j] = recv_y[r] + (int64_t)(slot[p] - roff[r]) * H;
        }
        for (int h = 0; h < H; ++h) {
            float acc = 0.0f;
            for (int j = 0; j < k; ++j) {
                float wj = w ? w[(int64_t)t * k + j] : 1.0f;
                acc = fmaf(wj, oracle_bf16_to_f32(rows[j][h]), acc);
            }
            acc = acc + oracle_bf16_to_f32(shared[(int64_t)t * H + h]);
            out[(int64_t)t * H + h] = oracle_bf16_rne(acc);
        }
    }
    free(rows);
}

void oracle_combine_backward(int T, int H, int k, int E, int R, const int32_t *idx,
                             const int32_t *slot, const int32_t *roff,
                             const uint16_t *grad_out, const float *w,
                             const uint16_t *const *recv_y, uint16_t *const *grad_recv,
                             float *grad_w)
{
    const int El = E / R;
    (void)R;
    for (int t = 0; t < T; ++t) {
        const uint16_t *g = grad_out + (int64_t)t * H;
        for (int j = 0; j < k; ++j) {
            int64_t p = (int64_t)t * k + j;
            int r = idx[p] / El;
            int64_t rrow = slot[p] - roff[r];
            float wj = w ? w[p] : 1.0f;
            uint16_t *dst = grad_recv[r] + rrow * H;
            for (int h = 0; h < H; ++h) {
                float prod = wj * oracle_bf16_to_f32(g[h]); /* one binary32 multiply */
                dst[h] = oracle_bf16_rne(prod);
            }
            if (grad_w) {
                const uint16_t *y = recv_y[r] + rrow * H;
                double dot = 0.0;
                for (int h = 0; h < H; ++h)
                    dot += (double)oracle_bf16_to_f32(g[h]) * (double)oracle_bf16_to_f32(y[h]);
                grad_w[p] = (float)dot;
            }
        }
    }
}

/* ------------------------------------------------- expert-side activation */

void oracle_quantize_f32_row(int n, const float *a, uint8_t *q, float *s)
{
    /* the same steps as oracle_quantize_row, on binary32 activations */
    for (int b = 0; b < n / 128; ++b) {
        const float *ab = a + b * 128;
        float amax = 0.0f; /* a NaN value makes it NaN */
        for (int h = 0; h < 128; ++h) {
            float v = fabsf(ab[h]);
            if (v > amax || isnan(v))
                amax = v;
        }
        if (amax == 0.0f) {
            s[b] = 0.0f;
            for (int h = 0; h < 128; ++h)
                q[b * 128 + h] = 0x00;
            continue;
        }
        float sb = amax / 448.0f;
        s[b] = sb;
        for (int h = 0; h < 128; ++h)
            q[b * 128 + h] = oracle_e4m3_encode(ab[h] / sb);
    }
}

void oracle_silu_mul_row(int I, const uint16_t *row, float *a)
{
    for (int h = 0; h < I; ++h) {
        double g = (double)oracle_bf16_to_f32(row[h]);
        double u = (double)oracle_bf16_to_f32(row[I + h]);
        double silu = g / (1.0 + exp(-g));
        a[h] = (float)(silu * u);
    }
}

void oracle_silu_mul_quant_row(int I, const uint16_t *row, uint8_t *q, float *s)
{
    float *a = (float *)malloc((size_t)I * sizeof(float));
    if (!a)
        return;
    oracle_silu_mul_row(I, row, a);
    oracle_quantize_f32_row(I, a, q, s);
    free(a);
}

/* ------------------------------------------------------------------ router */

/* Expert (or group) a with score sa ranks above b with score sb: the larger
 * score first, equal scores to the lower id.  Scores are compared as their
 * binary32 bit patterns read as unsigned integers, which is numeric order for
 * the non-negative scores a softmax or sigmoid gate gives (+0 < subnormals <
 * normals < +inf) and still a total order when a NaN appears. */
static int ranks_above(float sa, int a, float sb, int b)
{
    uint32_t ua, ub;
    memcpy(&ua, &sa, sizeof ua);
    memcpy(&ub, &sb, sizeof ub);
    if (ua != ub)
        return ua > ub;
    return a < b;
}

/* One token's gate scores s[0..El) from its logits row: the router input is
 * the logit plus the per-expert bias (one binary32 add); the gate is
 * evaluated in binary64 and rounded once to binary32.  Softmax subtracts the
 * maximum input and divides by the binary64 sum of the numerators taken in
 * ascending expert order.  z and ex are scratch rows of El entries. */
static void gate_scores(int El, int gate, const float *lrow, const float *bias, float *z, double *ex,
                        float *s)
{
    for (int e = 0; e < El; ++e)
        z[e] = bias ? lrow[e] + bias[e] : lrow[e];
    if (gate == 0) { /* softmax over the token's experts, max-subtracted */
        float m = z[0];
        for (int e = 1; e < El; ++e)
            if (z[e] > m)
                m = z[e];
        double sum = 0.0;
        for (int e = 0; e < El; ++e) {
            ex[e] = exp((double)z[e] - (double)m);
            sum += ex[e];
        }
        for (int e = 0; e < El; ++e)
            s[e] = (float)(ex[e] / sum);
    } else { /* sigmoid */
        for (int e = 0; e < El; ++e)
            s[e] = (float)(1.0 / (1.0 + exp(-(double)z[e])));
    }
}

int oracle_route_scores(int T, int El, int gate, const float *logits, const float *bias,
                        float *scores)
{
    if (T < 1 || El < 1 || (gate != 0 && gate != 1))
        return 1;
    float *z = malloc(sizeof(float) * (size_t)El);
    double *ex = malloc(sizeof(double) * (size_t)El);
    for (int t = 0; t < T; ++t)
        gate_scores(El, gate, logits + (int64_t)t * El, bias, z, ex, scores + (int64_t)t * El);
    free(z);
    free(ex);
    return 0;
}

int oracle_route(int T, int El, int k, int gate, int G, int TG, int group_topn, int renorm,
                 const float *logits, const float *bias, const int32_t *rep_off,
                 const int32_t *rep_slots, int32_t *idx, float *w)
{
    if (T < 1 || El < 1 || k < 1 || k > El || G < 1 || El % G != 0 || TG < 1 || TG > G ||
        (gate != 0 && gate != 1) || (group_topn != 1 && group_topn != 2))
        return 1;
    const int gs = El / G;
    if (k > TG * gs)
        return 1;
    const int n_top = group_topn < gs ? group_topn : gs;

    float *z = malloc(sizeof(float) * (size_t)El);
    float *s = malloc(sizeof(float) * (size_t)El);
    double *ex = malloc(sizeof(double) * (size_t)El);
    float *gsc = malloc(sizeof(float) * (size_t)G);
    char *kept = malloc((size_t)G);
    char *taken = malloc((size_t)El);
    int *sel = malloc(sizeof(int) * (size_t)k);
    float *ws = malloc(sizeof(float) * (size_t)k);

    for (int t = 0; t < T; ++t) {
        gate_scores(El, gate, logits + (int64_t)t * El, bias, z, ex, s);

        /* group-limited routing: a group's score is its best score, or the
         * binary32 sum of its two best; the TG best groups stay eligible.
         * One group (G = 1) is plain top-k over every expert. */
        for (int c = 0; c < G; ++c) {
            int b1 = -1, b2 = -1;
            for (int e = c * gs; e < (c + 1) * gs; ++e) {
                if (b1 < 0 || ranks_above(s[e], e, s[b1], b1)) {
                    b2 = b1;
                    b1 = e;
                } else if (b2 < 0 || ranks_above(s[e], e, s[b2], b2)) {
                    b2 = e;
                }
            }
            gsc[c] = (n_top == 1) ? s[b1] : s[b1] + s[b2];
            kept[c] = 0;
        }
        for (int r = 0; r < TG; ++r) {
            int best = -1;
            for (int c = 0; c < G; ++c)
                if (!kept[c] && (best < 0 || ranks_above(gsc[c], c, gsc[best], best)))
                    best = c;
            kept[best] = 1;
        }

        /* top-k among the eligible experts, best first */
        memset(taken, 0, (size_t)El);
        for (int j = 0; j < k; ++j) {
            int best = -1;
            for (int e = 0; e < El; ++e)
                if (kept[e / gs] && !taken[e] && (best < 0 || ranks_above(s[e], e, s[best], best)))
                    best = e;
            taken[best] = 1;
            sel[j] = best;
            ws[j] = s[best];
        }

        /* weights: the chosen scores, optionally divided by their binary32
         * sum taken in ascending j (left as they are when that sum is 0) */
        if (renorm) {
            float sum = 0.0f;
            for (int j = 0; j < k; ++j)
                sum += ws[j];
            if (sum > 0.0f)
                for (int j = 0; j < k; ++j)
                    ws[j] = ws[j] / sum;
        }

        /* redundant experts: logical expert l has replicas
         * rep_slots[rep_off[l] .. rep_off[l+1]); token t takes replica
         * t mod (their number); no replica gives -1, an invalid index */
        for (int j = 0; j < k; ++j) {
            const int l = sel[j];
            int32_t phys = l;
            if (rep_off) {
                const int n = rep_off[l + 1] - rep_off[l];
                phys = n > 0 ? rep_slots[rep_off[l] + t % n] : -1;
            }
            idx[(int64_t)t * k + j] = phys;
            w[(int64_t)t * k + j] = ws[j];
        }
    }
    free(z);
    free(s);
    free(ex);
    free(gsc);
    free(kept);
    free(taken);
    free(sel);
    free(ws);
    return 0;
}
