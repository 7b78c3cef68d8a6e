/*
 * rgdr_oracle.c -- plain, slow, fp64 CPU oracle for the recurrent gated-delta-rule
 * decode step and for the linear-attention gate front end.
 *
 * TEST INFRASTRUCTURE. Only the test suite, the smoke check and the benchmark's CPU
 * baseline may load or call this library. The GPU library does not link it, include it or
 * share any code, header, table or constant with it, and this file knows nothing of the
 * GPU library.
 *
 * Sources (cited by page title and section):
 *   [R] MindSpore Lite API page "lite_boost.ops.recurrent_gated_delta_rule":
 *       the algorithm section (four steps, applied token by token to every batch entry),
 *       the parameter list (shapes, dtypes, meaning of each argument) and the returns.
 *   [G] Kernel README "com.microsoft.LinearAttentionGate": the Description paragraph,
 *       the Inputs and Outputs tables and the Type constraints table.
 *
 * Arithmetic is IEEE fp64 throughout, evaluated in the order written, built with
 * -ffp-contract=off and without fast-math. bf16 and fp16 inputs are decoded exactly;
 * outputs are either returned unrounded (fp64) or rounded once to bf16 with
 * round-to-nearest-even directly from fp64, by this file's own codec.
 *
 * Readings taken where the pages leave a step open:
 *   - State pool: the state argument is a pool [N_slots, H_v, D_k, D_v]; batch entry b
 *     reads and commits slot ssm_state_indices[b]; slots no entry names are not written.
 *     With N_slots = B and identity indices this is the page's [B, H_v, D_k, D_v].
 *   - A batch entry whose slot index lies outside [0, N_slots) is skipped: its outputs
 *     are zero and no state is read or written.
 *   - Head sharing: value head h reads query/key head floor(h * H_q / H_v).
 *   - actual_seq_lengths[b] = L is clamped to [0, T]; tokens t >= L are never read and
 *     their output rows are exactly zero.
 *   - num_accepted_tokens[b] = n is clamped to [0, L]; outputs are produced for all L
 *     tokens and the committed state is the state after the first n tokens.
 *   - q is multiplied by scale before step 4 (the scale_value parameter).
 *   - Unit-norm q and k are a precondition of the operator (its query and key parameters).
 *     On request (normalize_qk) the oracle establishes it itself: each token's query and
 *     key head vector is divided by its L2 norm over D_k before the four steps (and before
 *     the scale); an all-zero vector stays zero.
 *   - Step 3's "k^T @ (...)" is the outer product k (x) u, shape [D_k, D_v].
 *   - Gate: softplus(x) = ln(1 + e^x) with no beta/threshold parameters, evaluated in
 *     the overflow-safe form x + log1p(e^-x) for x > 0 and log1p(e^x) otherwise, which
 *     is the same function.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* Element types of the tensors the driver reads. */
enum { TY_BF16 = 0, TY_F32 = 1, TY_F64 = 2, TY_F16 = 3 };

/* ------------------------------------------------------------------------------------ */
/* Number codecs (bf16: 1 sign, 8 exponent, 7 fraction bits; fp16: 1, 5, 10).           */
/* ------------------------------------------------------------------------------------ */

double oracle_bf16_to_f64(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 7) & 0xFF;
    int m = h & 0x7F;
    double x;
    if (e == 0xFF)
        x = m ? NAN : INFINITY;
    else if (e == 0)
        x = ldexp((double)m, -133); /* subnormal: m * 2^-126 / 2^7 */
    else
        x = ldexp((double)(128 + m), e - 134); /* (1 + m/128) * 2^(e-127) */
    return sign ? -x : x;
}

double oracle_f16_to_f64(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1F;
    int m = h & 0x3FF;
    double x;
    if (e == 0x1F)
        x = m ? NAN : INFINITY;
    else if (e == 0)
        x = ldexp((double)m, -24); /* m * 2^-14 / 2^10 */
    else
        x = ldexp((double)(1024 + m), e - 25);
    return sign ? -x : x;
}

/* Round an fp64 value to the nearest bf16, ties to even, in one step (no detour through
 * fp32, so no double rounding). The quantum is 2^(e-7) for a value in [2^e, 2^(e+1)),
 * and 2^-133 below the normal range. Counting quanta from zero gives the encoding
 * directly: ((e + 126) << 7) + n for the normal range, n for subnormals, and both agree
 * at the boundary. A count that reaches the exponent field's all-ones code is infinity. */
uint16_t oracle_f64_to_bf16(double x)
{
    uint16_t sign = signbit(x) ? 0x8000 : 0;
    double a = fabs(x);
    if (isnan(x))
        return (uint16_t)(sign | 0x7FC0);
    if (isinf(a))
        return (uint16_t)(sign | 0x7F80);
    if (a == 0.0)
        return sign;
    int e;
    if (a < ldexp(1.0, -126)) {
        e = -126;
    } else {
        int ex;
        frexp(a, &ex); /* a = f * 2^ex, f in [0.5, 1) */
        e = ex - 1;
    }
    double n = ldexp(a, 7 - e); /* a / quantum, exact (power-of-two scale) */
    double fl = floor(n);
    double frac = n - fl;
    if (frac > 0.5 || (frac == 0.5 && fmod(fl, 2.0) != 0.0))
        fl += 1.0;
    long code = ((long)(e + 126) << 7) + (long)fl;
    if (code >= 0x7F80)
        return (uint16_t)(sign | 0x7F80);
    return (uint16_t)(sign | (uint16_t)code);
}

static double rd(const void *p, int ty, size_t i)
{
    switch (ty) {
    case TY_BF16: return oracle_bf16_to_f64(((const uint16_t *)p)[i]);
    case TY_F16: return oracle_f16_to_f64(((const uint16_t *)p)[i]);
    case TY_F32: return (double)((const float *)p)[i];
    default: return ((const double *)p)[i];
    }
}

/* ------------------------------------------------------------------------------------ */
/* The recurrence for one (batch entry, value head) pair  [R], algorithm section.       */
/* ------------------------------------------------------------------------------------ */

/*
 * S      : D_k x D_v state, row i = key dimension, column j = value dimension; updated in
 *          place through all L tokens.
 * Scommit: receives S as it stands after the first n tokens (n <= L).
 * q, k   : [T][D_k] (this pair's query/key head); v: [T][D_v]; beta, g: [T];
 * gk     : [T][D_k]; out: [T][D_v] (rows t >= L are set to zero).
 * kv, u  : D_v-long scratch.
 * snap   : NULL, or where S after token t (t < L) goes: snap + t * snap_stride.
 */
static void gdr_pair(double *S, double *Scommit, int L, int n, int T, int Dk, int Dv,
                     const double *q, const double *k, const double *v, const double *beta,
                     const double *g, const double *gk, double scale, double *out,
                     double *kv, double *u, double *snap, size_t snap_stride)
{
    size_t nS = (size_t)Dk * Dv;
    if (n == 0)
        memcpy(Scommit, S, nS * sizeof(double));
    for (int t = 0; t < L; ++t) {
        const double *qt = q + (size_t)t * Dk;
        const double *kt = k + (size_t)t * Dk;
        const double *vt = v + (size_t)t * Dv;
        const double *gkt = gk + (size_t)t * Dk;
        double eg = exp(g[t]);
        /* step 1, state decay: S = S * exp(g) * exp(gk), gk scaling row i */
        for (int i = 0; i < Dk; ++i) {
            double egk = exp(gkt[i]);
            for (int j = 0; j < Dv; ++j)
                S[(size_t)i * Dv + j] = S[(size_t)i * Dv + j] * eg * egk;
        }
        /* step 2, memory read: kv_mem = S^T k */
        for (int j = 0; j < Dv; ++j) {
            double acc = 0.0;
            for (int i = 0; i < Dk; ++i)
                acc += S[(size_t)i * Dv + j] * kt[i];
            kv[j] = acc;
        }
        /* step 3, delta update: S = S + k (x) ((v - kv_mem) * beta) */
        for (int j = 0; j < Dv; ++j)
            u[j] = (vt[j] - kv[j]) * beta[t];
        for (int i = 0; i < Dk; ++i)
            for (int j = 0; j < Dv; ++j)
                S[(size_t)i * Dv + j] = S[(size_t)i * Dv + j] + kt[i] * u[j];
        /* step 4, output: o = S^T (q * scale), with the updated S */
        double *ot = out + (size_t)t * Dv;
        for (int j = 0; j < Dv; ++j) {
            double acc = 0.0;
            for (int i = 0; i < Dk; ++i)
                acc += S[(size_t)i * Dv + j] * (qt[i] * scale);
            ot[j] = acc;
        }
        if (t + 1 == n)
            memcpy(Scommit, S, nS * sizeof(double));
        if (snap)
            memcpy(snap + (size_t)t * snap_stride, S, nS * sizeof(double));
    }
    for (int t = L; t < T; ++t)
        for (int j = 0; j < Dv; ++j)
            out[(size_t)t * Dv + j] = 0.0;
}

/* q/k normalisation  [R], parameters query and key (unit L2 norm per head vector):
 * x = x / ||x||_2 over the n elements, the norm the square root of the sum of squares taken
 * in index order; an all-zero vector is left as it is. */
static void l2_normalize(double *x, int n)
{
    double ss = 0.0;
    for (int i = 0; i < n; ++i)
        ss += x[i] * x[i];
    if (ss == 0.0)
        return;
    double nrm = sqrt(ss);
    for (int i = 0; i < n; ++i)
        x[i] = x[i] / nrm;
}

typedef struct {
    const void *q, *k, *v, *beta, *g, *gk; /* inputs, element types below */
    int q_ty, k_ty, v_ty, beta_ty, g_ty, gk_ty;
    const void *pool; int pool_ty;         /* [N_slots, H_v, D_k, D_v] */
    const int32_t *lens, *idx, *nacc;      /* [B] */
    double scale;
    int B, Hq, Hv, T, Dk, Dv, N_slots;
    double *out;                           /* [B, H_v, T, D_v], unrounded */
    void *pool_out; int pool_out_ty;       /* [N_slots, H_v, D_k, D_v]; may alias pool */
    double *rows_out;                      /* optional [B, H_v, D_k, D_v], unrounded */
    int normalize_qk;                      /* nonzero: L2-normalise q and k per token */
    double *snap_out;                      /* optional [B, T, H_v, D_k, D_v], unrounded */
} rgdr_args;

static int clampi(int x, int lo, int hi) { return x < lo ? lo : (x > hi ? hi : x); }

static int rgdr_drive(const rgdr_args *a)
{
    if (!a->q || !a->k || !a->v || !a->beta || !a->g || !a->gk || !a->pool || !a->lens ||
        !a->idx || !a->nacc || !a->out || !a->pool_out)
        return 1;
    if (a->B <= 0 || a->Hq <= 0 || a->Hv <= 0 || a->T <= 0 || a->Dk <= 0 || a->Dv <= 0 ||
        a->N_slots <= 0)
        return 2;
    const int T = a->T, Dk = a->Dk, Dv = a->Dv;
    size_t nS = (size_t)Dk * Dv;
    double *S = malloc(nS * sizeof(double));
    double *Sc = malloc(nS * sizeof(double));
    double *q = malloc((size_t)T * Dk * sizeof(double));
    double *k = malloc((size_t)T * Dk * sizeof(double));
    double *gk = malloc((size_t)T * Dk * sizeof(double));
    double *v = malloc((size_t)T * Dv * sizeof(double));
    double *beta = malloc((size_t)T * sizeof(double));
    double *g = malloc((size_t)T * sizeof(double));
    double *kv = malloc((size_t)Dv * sizeof(double));
    double *u = malloc((size_t)Dv * sizeof(double));
    if (!S || !Sc || !q || !k || !gk || !v || !beta || !g || !kv || !u) {
        free(S); free(Sc); free(q); free(k); free(gk); free(v); free(beta); free(g);
        free(kv); free(u);
        return 3;
    }
    for (int b = 0; b < a->B; ++b) {
        int slot = a->idx[b];
        int L = clampi(a->lens[b], 0, T);
        int n = clampi(a->nacc[b], 0, L);
        int valid = slot >= 0 && slot < a->N_slots;
        for (int h = 0; h < a->Hv; ++h) {
            double *out = a->out + ((size_t)b * a->Hv + h) * T * Dv;
            if (!valid) {
                for (size_t e = 0; e < (size_t)T * Dv; ++e)
                    out[e] = 0.0;
                continue;
            }
            int hq = (int)(((long long)h * a->Hq) / a->Hv);
            size_t qo = ((size_t)b * a->Hq + hq) * T * Dk;
            size_t vo = ((size_t)b * a->Hv + h) * T * Dv;
            size_t go = ((size_t)b * a->Hv + h) * T;
            size_t so = ((size_t)slot * a->Hv + h) * nS;
            /* tokens t >= L are never read */
            for (int t = 0; t < L; ++t) {
                for (int i = 0; i < Dk; ++i) {
                    q[(size_t)t * Dk + i] = rd(a->q, a->q_ty, qo + (size_t)t * Dk + i);
                    k[(size_t)t * Dk + i] = rd(a->k, a->k_ty, qo + (size_t)t * Dk + i);
                    gk[(size_t)t * Dk + i] = rd(a->gk, a->gk_ty, (go + t) * Dk + i);
                }
                for (int j = 0; j < Dv; ++j)
                    v[(size_t)t * Dv + j] = rd(a->v, a->v_ty, vo + (size_t)t * Dv + j);
                beta[t] = rd(a->beta, a->beta_ty, go + t);
                g[t] = rd(a->g, a->g_ty, go + t);
                if (a->normalize_qk) {
                    l2_normalize(q + (size_t)t * Dk, Dk);
                    l2_normalize(k + (size_t)t * Dk, Dk);
                }
            }
            for (size_t e = 0; e < nS; ++e)
                S[e] = rd(a->pool, a->pool_ty, so + e);
            double *snap = a->snap_out ? a->snap_out + ((size_t)b * T * a->Hv + h) * nS : NULL;
            gdr_pair(S, Sc, L, n, T, Dk, Dv, q, k, v, beta, g, gk, a->scale, out, kv, u,
                     snap, (size_t)a->Hv * nS);
            /* commit slot ssm_state_indices[b]; the returned state feeds the next call */
            if (a->pool_out_ty == TY_BF16) {
                uint16_t *po = (uint16_t *)a->pool_out + so;
                for (size_t e = 0; e < nS; ++e)
                    po[e] = oracle_f64_to_bf16(Sc[e]);
            } else {
                double *po = (double *)a->pool_out + so;
                memcpy(po, Sc, nS * sizeof(double));
            }
            if (a->rows_out)
                memcpy(a->rows_out + ((size_t)b * a->Hv + h) * nS, Sc, nS * sizeof(double));
        }
    }
    free(S); free(Sc); free(q); free(k); free(gk); free(v); free(beta); free(g);
    free(kv); free(u);
    return 0;
}

/*
 * Same contract as the operator [R]: bf16 query/key/value/beta/state, fp32 g/gk,
 * int32 index arrays, fp32 scale. out is returned unrounded (fp64); state_out receives
 * the committed bf16 state of every named slot (it may be the same buffer as pool);
 * rows_out, if not NULL, receives each batch entry's committed state unrounded.
 * normalize_qk nonzero: q and k are L2-normalised per token and head first.
 * Returns 0, or nonzero for a NULL pointer or a non-positive size.
 */
int oracle_rgdr_bf16(const uint16_t *query, const uint16_t *key, const uint16_t *value,
                     const uint16_t *beta, const uint16_t *pool, const int32_t *lens,
                     const int32_t *idx, const float *g, const float *gk, const int32_t *nacc,
                     float scale, int B, int Hq, int Hv, int T, int Dk, int Dv, int N_slots,
                     double *out, uint16_t *state_out, double *rows_out, int normalize_qk)
{
    rgdr_args a = {query, key, value, beta, g, gk, TY_BF16, TY_BF16, TY_BF16, TY_BF16,
                   TY_F32, TY_F32, pool, TY_BF16, lens, idx, nacc, (double)scale,
                   B, Hq, Hv, T, Dk, Dv, N_slots, out, state_out, TY_BF16, rows_out,
                   normalize_qk, NULL};
    return rgdr_drive(&a);
}

/*
 * oracle_rgdr_bf16, and the state after each token: snap_out [B, T, H_v, D_k, D_v]
 * receives, for every batch entry b with a valid slot and every t < L_b (the clamped
 * length), the state after its first t + 1 tokens, unrounded; other entries are not
 * written. The page's num_accepted_tokens commits one such state; these are all of them.
 */
int oracle_rgdr_bf16_snapshots(const uint16_t *query, const uint16_t *key,
                               const uint16_t *value, const uint16_t *beta,
                               const uint16_t *pool, const int32_t *lens, const int32_t *idx,
                               const float *g, const float *gk, const int32_t *nacc,
                               float scale, int B, int Hq, int Hv, int T, int Dk, int Dv,
                               int N_slots, double *out, uint16_t *state_out,
                               double *rows_out, double *snap_out)
{
    if (!snap_out)
        return 1;
    rgdr_args a = {query, key, value, beta, g, gk, TY_BF16, TY_BF16, TY_BF16, TY_BF16,
                   TY_F32, TY_F32, pool, TY_BF16, lens, idx, nacc, (double)scale,
                   B, Hq, Hv, T, Dk, Dv, N_slots, out, state_out, TY_BF16, rows_out,
                   0, snap_out};
    return rgdr_drive(&a);
}

/* The same recurrence with every input and the state pool in fp64 and no rounding at
 * all; state_out (fp64 pool, may alias pool) receives the committed state. */
int oracle_rgdr_f64(const double *query, const double *key, const double *value,
                    const double *beta, const double *pool, const int32_t *lens,
                    const int32_t *idx, const double *g, const double *gk,
                    const int32_t *nacc, double scale, int B, int Hq, int Hv, int T, int Dk,
                    int Dv, int N_slots, double *out, double *state_out, int normalize_qk)
{
    rgdr_args a = {query, key, value, beta, g, gk, TY_F64, TY_F64, TY_F64, TY_F64,
                   TY_F64, TY_F64, pool, TY_F64, lens, idx, nacc, scale,
                   B, Hq, Hv, T, Dk, Dv, N_slots, out, state_out, TY_F64, NULL,
                   normalize_qk, NULL};
    return rgdr_drive(&a);
}

/* ------------------------------------------------------------------------------------ */
/* Gate front end  [G], Description and Inputs/Outputs tables.                          */
/* ------------------------------------------------------------------------------------ */

static double softplus(double x)
{
    return x > 0.0 ? x + log1p(exp(-x)) : log1p(exp(x));
}

/*
 * a, b: [n_rows, H] (head axis last, leading axes folded) of element type ab_ty
 * (fp32 or fp16, the pages' T); dt_bias, decay_scale: [H] fp32 (the pages' TF).
 * decay[r,h] = decay_scale[h] * softplus(a[r,h] + dt_bias[h]);
 * beta[r,h]  = sigmoid(b[r,h]) = 1 / (1 + exp(-b[r,h])), only when beta != NULL, which
 * requires b != NULL. Both outputs are fp64 and unrounded.
 * Returns 0, 1 for a missing required pointer, 2 for a bad size, 4 for beta without b.
 */
int oracle_la_gate(const void *a, const float *dt_bias, const float *decay_scale,
                   const void *b, int ab_ty, long long n_rows, int H, double *decay,
                   double *beta)
{
    if (!a || !dt_bias || !decay_scale || !decay)
        return 1;
    if (n_rows < 0 || H <= 0 || (ab_ty != TY_F32 && ab_ty != TY_F16))
        return 2;
    if (beta && !b)
        return 4;
    for (long long r = 0; r < n_rows; ++r)
        for (int h = 0; h < H; ++h) {
            size_t e = (size_t)r * H + h;
            double x = rd(a, ab_ty, e) + (double)dt_bias[h];
            decay[e] = (double)decay_scale[h] * softplus(x);
            if (beta)
                beta[e] = 1.0 / (1.0 + exp(-rd(b, ab_ty, e)));
        }
    return 0;
}

/* Array forms of the codecs. */
void oracle_bf16_to_f64_array(const uint16_t *in, double *out, long long n)
{
    for (long long i = 0; i < n; ++i)
        out[i] = oracle_bf16_to_f64(in[i]);
}

void oracle_f16_to_f64_array(const uint16_t *in, double *out, long long n)
{
    for (long long i = 0; i < n; ++i)
        out[i] = oracle_f16_to_f64(in[i]);
}

void oracle_f64_to_bf16_array(const double *in, uint16_t *out, long long n)
{
    for (long long i = 0; i < n; ++i)
        out[i] = oracle_f64_to_bf16(in[i]);
}
