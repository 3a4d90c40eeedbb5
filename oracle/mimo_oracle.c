/*
 * mimo_oracle.c -- plain, slow, fp64 CPU oracle for MiMo-V2-Flash hybrid attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the CPU
 * baseline leg of the benchmark may load this library.  The GPU library never
 * links, includes or calls anything here, and nothing here comes from the GPU
 * sources: the two share only the documented buffer layouts, which are written
 * out again below from the definitions.
 *
 * What it computes (Hugging Face Transformers model doc "MiMo-V2-Flash"):
 *   - Key features: sliding-window attention (SWA) and global attention (GA)
 *     layers interleaved 5:1, a 128-token window, and a learnable attention
 *     sink bias.
 *   - MiMoV2FlashConfig: num_attention_heads=64, num_key_value_heads=4 (GQA,
 *     heads grouped), head_dim=192 for queries and keys, v_head_dim=128,
 *     sliding_window=129, attention_value_scale=0.707.
 *   - MiMoV2FlashModel.forward, past_key_values: with a cache only the tokens
 *     not yet processed are passed; earlier keys and values come from the cache.
 *   - MiMoV2FlashForCausalLM: a causal decoder, so global attention is causal.
 *
 * For a query token at position p (0-based, within its sequence) and query
 * head h:
 *   g      = h / (Hq / Hkv)                      contiguous GQA groups
 *   J      = { j : lo <= j <= p },  lo = 0 (GA) or max(0, p - (W - 1)) (SWA)
 *   s_j    = scale * sum_d q[p,h,d] * k[j,g,d]
 *   M      = max(max_j s_j, sigma_h)             sigma_h left out when absent
 *   Z      = sum_j exp(s_j - M) + exp(sigma_h - M)   (sink term 0 when absent)
 *   LSE    = M + ln Z
 *   o[e]   = value_scale * sum_j exp(s_j - LSE) * v[j,g,e]
 * The sink only joins the denominator; it contributes no value row.  A sink
 * pointer of NULL, or a sink value of -inf, means "no sink".
 *
 * Inputs are the bf16 bit patterns the GPU receives, widened exactly to double;
 * sink, scale and value_scale are fp32 widened to double.  Everything else is
 * double with libm exp/log.
 *
 * An FP8 GA cache (a storage format of the same cache; the model doc does not
 * define one) holds OCP E4M3 codes with one fp32 scale per KV head: a cached
 * key or value element x is stored as E4M3(clamp(x / scale, -448, 448)), the
 * division done in fp32 and the rounding to nearest-even, and read back as
 * value(code) * scale.  The new token of a decode step is read from k_new /
 * v_new as given (bf16), as for the bf16 cache.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <unistd.h>

#define ORACLE_OK 0
#define ORACLE_EINVAL 1
#define ORACLE_ECAPACITY 2

enum { ORACLE_SWA = 0, ORACLE_GA = 1 };

/* bf16 -> double: a bf16 value is the upper 16 bits of an IEEE binary32. */
static double bf16_to_double(uint16_t bits) {
    uint32_t w = ((uint32_t)bits) << 16;
    float f;
    memcpy(&f, &w, sizeof f);
    return (double)f;
}

/* x rounded once to the nearest bf16 value, ties to the even significand.
 * bf16 keeps 8 significant bits: in the binade [2^b, 2^(b+1)) the grid step is
 * 2^(b-7); below 2^-126 (subnormals) it is 2^-133.  Magnitudes that round past
 * the largest finite value (2 - 2^-7) * 2^127 become infinite. */
static double round_bf16(double x) {
    if (!isfinite(x) || x == 0.0) return x;
    double a = fabs(x);
    int b = -126;
    if (a >= 0x1p-126) {
        frexp(a, &b);
        b -= 1;
    }
    double step = ldexp(1.0, b - 7);
    double r = nearbyint(a / step) * step; /* a / step is exact; nearbyint rounds half to even */
    if (r > 0x1.fep127) r = INFINITY;
    return copysign(r, x);
}

/* OCP 8-bit floating point, E4M3 (OCP "OCP 8-bit Floating Point Specification
 * (OFP8)"): sign bit, 4 exponent bits with bias 7, 3 mantissa bits.  Exponent
 * field 0 holds zero and the subnormals m/8 * 2^-6; fields 1..15 hold
 * (1 + m/8) * 2^(e-7), except S.1111.111, which is NaN.  No infinities; the
 * largest finite magnitude is 448. */
static double e4m3_to_double(uint8_t c) {
    int e = (c >> 3) & 15, m = c & 7;
    double sgn = (c & 0x80) ? -1.0 : 1.0;
    if (e == 15 && m == 7) return NAN;
    if (e == 0) return sgn * ldexp((double)m / 8.0, -6);
    return sgn * ldexp(1.0 + (double)m / 8.0, e - 7);
}

/* E4M3 code nearest to x after clamping |x| to 448, ties to the even code;
 * the sign of x (zero included) is kept.  x must not be NaN. */
static uint8_t e4m3_from_float(float x) {
    uint8_t sgn = signbit(x) ? 0x80 : 0;
    double a = fabs((double)x);
    if (a > 448.0) a = 448.0;
    /* grid step: 2^-9 below 2^-6 (subnormals), else 2^(b-3) in binade [2^b, 2^(b+1)) */
    int b = -6;
    if (a >= 0x1p-6) {
        frexp(a, &b);
        b -= 1;
    }
    double step = ldexp(1.0, b - 3);
    double r = nearbyint(a / step) * step; /* a / step is exact; nearbyint rounds half to even */
    if (r < 0x1p-6) return (uint8_t)(sgn | (uint8_t)(r / 0x1p-9));
    frexp(r, &b);
    b -= 1;
    int m = (int)(r / ldexp(1.0, b) * 8.0) - 8;
    return (uint8_t)(sgn | ((b + 7) << 3) | m);
}

/* Stored code of element x (bf16 bits) of a KV head with the given scale. */
static uint8_t e4m3_quantize(uint16_t x, float scale) {
    uint32_t w = ((uint32_t)x) << 16;
    float f;
    memcpy(&f, &w, sizeof f);
    return e4m3_from_float(f / scale);
}

typedef struct {
    int hq, hkv, dqk, dv, layer_type, window;
    double scale, value_scale;
} dims_t;

/* Rows of an FP8 cache: per key, E4M3 code rows (NULL = take the bf16 row)
 * and the scales that turn codes into values. */
typedef struct {
    const uint8_t* const* k8;
    const uint8_t* const* v8;
    double kscale, vscale;
} fp8_rows_t;

/* One attention row: query vector qrow (length dqk), keys given as arrays of
 * row pointers (one per key in J, in increasing position order).  Writes
 * o[dv] and *lse.  If wkeys is non-NULL it receives exp(s_j - LSE) for each
 * key, and *wsink the sink mass exp(sigma - LSE) (0 without a sink).  With f8
 * non-NULL, a key whose f8 row is set is read from E4M3 codes times the scale. */
static void attend_row(const dims_t* d, const uint16_t* qrow, int nkeys,
                       const uint16_t* const* krows, const uint16_t* const* vrows, const fp8_rows_t* f8,
                       int has_sink, double sigma, double* scores,
                       double* o, double* lse, double* wkeys, double* wsink) {
    double m = -INFINITY;
    for (int j = 0; j < nkeys; ++j) {
        double acc = 0.0;
        if (f8 && f8->k8[j])
            for (int x = 0; x < d->dqk; ++x)
                acc += bf16_to_double(qrow[x]) * (e4m3_to_double(f8->k8[j][x]) * f8->kscale);
        else
            for (int x = 0; x < d->dqk; ++x)
                acc += bf16_to_double(qrow[x]) * bf16_to_double(krows[j][x]);
        scores[j] = d->scale * acc;
        if (scores[j] > m) m = scores[j];
    }
    if (has_sink && sigma > m) m = sigma;
    double z = 0.0;
    for (int j = 0; j < nkeys; ++j) z += exp(scores[j] - m);
    if (has_sink) z += exp(sigma - m);
    double l = m + log(z);
    for (int e = 0; e < d->dv; ++e) o[e] = 0.0;
    for (int j = 0; j < nkeys; ++j) {
        double w = exp(scores[j] - l);
        if (wkeys) wkeys[j] = w;
        if (f8 && f8->v8[j])
            for (int e = 0; e < d->dv; ++e) o[e] += w * (e4m3_to_double(f8->v8[j][e]) * f8->vscale);
        else
            for (int e = 0; e < d->dv; ++e) o[e] += w * bf16_to_double(vrows[j][e]);
    }
    for (int e = 0; e < d->dv; ++e) o[e] *= d->value_scale;
    if (wkeys) *wsink = has_sink ? exp(sigma - l) : 0.0;
    *lse = l;
}

static int sink_present(const float* sink, int h, double* sigma) {
    if (!sink) return 0;
    double s = (double)sink[h];
    if (isinf(s) && s < 0) return 0;
    *sigma = s;
    return 1;
}

/* ------------------------------------------------------------------------ */
/* Prefill: packed variable-length sequences, keys from the same sequence.  */

typedef struct {
    const dims_t* d;
    const uint16_t *q, *k, *v;
    const int32_t* cu;
    int nseq;
    const float* sink;
    const int64_t* rows; /* packed token indices to evaluate, or NULL = all */
    int64_t nrows;
    double *out, *lse, *weights;
    int wstride; /* weights row length (longest sequence + 1) */
    int64_t next;
    pthread_mutex_t mu;
} prefill_job_t;

static int seq_of_token(const int32_t* cu, int nseq, int64_t t) {
    int lo = 0, hi = nseq - 1;
    while (lo < hi) { /* last b with cu[b] <= t */
        int mid = (lo + hi + 1) / 2;
        if (cu[mid] <= t) lo = mid; else hi = mid - 1;
    }
    return lo;
}

/* Rows of the keys and values lo..p of the sequence whose first token is
 * packed row base, KV head g (prefill: keys come from the same sequence);
 * returns their count. */
static int prefill_key_rows(const dims_t* d, const uint16_t* k, const uint16_t* v, int64_t base, int lo, int p, int g,
                            const uint16_t** kr, const uint16_t** vr) {
    int n = 0;
    for (int j = lo; j <= p; ++j, ++n) {
        kr[n] = k + ((size_t)(base + j) * d->hkv + g) * d->dqk;
        vr[n] = v + ((size_t)(base + j) * d->hkv + g) * d->dv;
    }
    return n;
}

static void* prefill_worker(void* arg) {
    prefill_job_t* jb = (prefill_job_t*)arg;
    const dims_t* d = jb->d;
    int maxkeys = 0;
    for (int b = 0; b < jb->nseq; ++b) {
        int L = jb->cu[b + 1] - jb->cu[b];
        if (L > maxkeys) maxkeys = L;
    }
    const uint16_t** kr = malloc(sizeof(*kr) * (size_t)(maxkeys + 1));
    const uint16_t** vr = malloc(sizeof(*vr) * (size_t)(maxkeys + 1));
    double* sc = malloc(sizeof(double) * (size_t)(maxkeys + 1));
    int group = d->hq / d->hkv;
    for (;;) {
        pthread_mutex_lock(&jb->mu);
        int64_t r = jb->next++;
        pthread_mutex_unlock(&jb->mu);
        if (r >= jb->nrows) break;
        int64_t t = jb->rows ? jb->rows[r] : r;
        int b = seq_of_token(jb->cu, jb->nseq, t);
        int64_t base = jb->cu[b];
        int p = (int)(t - base);
        int lo = 0;
        if (d->layer_type == ORACLE_SWA) lo = p - (d->window - 1) > 0 ? p - (d->window - 1) : 0;
        for (int h = 0; h < d->hq; ++h) {
            int g = h / group;
            int n = prefill_key_rows(d, jb->k, jb->v, base, lo, p, g, kr, vr);
            double sigma = 0.0;
            int hs = sink_present(jb->sink, h, &sigma);
            double* w = jb->weights ? jb->weights + ((size_t)r * d->hq + h) * jb->wstride : NULL;
            attend_row(d, jb->q + ((size_t)t * d->hq + h) * d->dqk, n, kr, vr, NULL, hs, sigma, sc,
                       jb->out + ((size_t)r * d->hq + h) * d->dv, jb->lse + (size_t)r * d->hq + h,
                       w ? w + lo : NULL, w ? w + jb->wstride - 1 : NULL);
        }
    }
    free(kr); free(vr); free(sc);
    return NULL;
}

static int check_dims(const dims_t* d) {
    if (d->hq <= 0 || d->hkv <= 0 || d->hq % d->hkv) return 0;
    if (d->dqk <= 0 || d->dv <= 0) return 0;
    if (d->layer_type != ORACLE_SWA && d->layer_type != ORACLE_GA) return 0;
    if (d->layer_type == ORACLE_SWA && d->window < 1) return 0;
    return 1;
}

static int run_threads(void* (*fn)(void*), void* job, int nthreads) {
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 256) nthreads = 256;
    pthread_t th[256];
    int started = 0;
    for (int i = 0; i < nthreads; ++i)
        if (pthread_create(&th[i], NULL, fn, job) == 0) started++; else break;
    if (started == 0) fn(job);
    for (int i = 0; i < started; ++i) pthread_join(th[i], NULL);
    return ORACLE_OK;
}

/* Attention of every packed query token (or of the listed ones) over its own
 * sequence.  out: [rows][hq][dv], lse: [rows][hq]; weights (optional, the
 * post-softmax attention weights of the model doc's `attentions` output):
 * [rows][hq][wstride], entry j = weight of key position j of the sequence
 * (0 outside the key set), last entry = sink mass; wstride must be at least
 * the longest sequence + 1. */
int oracle_prefill(int hq, int hkv, int dqk, int dv, int layer_type, int window,
                   float scale, float value_scale,
                   const uint16_t* q, const uint16_t* k, const uint16_t* v,
                   const int32_t* cu_seqlens, int nseq, const float* sink,
                   const int64_t* rows, int64_t nrows,
                   double* out, double* lse, double* weights, int wstride, int nthreads) {
    dims_t d = {hq, hkv, dqk, dv, layer_type, window, (double)scale, (double)value_scale};
    if (!check_dims(&d) || nseq < 1 || !q || !k || !v || !cu_seqlens || !out || !lse) return ORACLE_EINVAL;
    int64_t T = cu_seqlens[nseq];
    int maxlen = 0;
    for (int b = 0; b < nseq; ++b) {
        if (cu_seqlens[b + 1] < cu_seqlens[b]) return ORACLE_EINVAL;
        if (cu_seqlens[b + 1] - cu_seqlens[b] > maxlen) maxlen = cu_seqlens[b + 1] - cu_seqlens[b];
    }
    if (cu_seqlens[0] != 0) return ORACLE_EINVAL;
    if (!rows) nrows = T;
    for (int64_t r = 0; rows && r < nrows; ++r)
        if (rows[r] < 0 || rows[r] >= T) return ORACLE_EINVAL;
    if (weights) {
        if (wstride < maxlen + 1) return ORACLE_EINVAL;
        memset(weights, 0, sizeof(double) * (size_t)nrows * hq * wstride);
    }
    prefill_job_t jb;
    memset(&jb, 0, sizeof jb);
    jb.d = &d; jb.q = q; jb.k = k; jb.v = v; jb.cu = cu_seqlens; jb.nseq = nseq; jb.sink = sink;
    jb.rows = rows; jb.nrows = nrows; jb.out = out; jb.lse = lse; jb.weights = weights; jb.wstride = wstride;
    pthread_mutex_init(&jb.mu, NULL);
    run_threads(prefill_worker, &jb, nthreads);
    pthread_mutex_destroy(&jb.mu);
    return ORACLE_OK;
}

/* ------------------------------------------------------------------------ */
/* Backward of prefill: the gradient of sum(dO * out) for an upstream dO    */
/* [T][Hq][Dv].  Differentiating o = value_scale * sum_j exp(s_j - LSE) v_j */
/* with LSE = log(sum_j exp(s_j) + exp(sigma)) gives, for one query row     */
/* (position p, head h, group g, key set J, weights P_j = exp(s_j - LSE)):  */
/*   D       = sum_e dO[e] * o[e]                                           */
/*   dP_j    = value_scale * sum_e dO[e] * v[j,g,e]                         */
/*   dS_j    = P_j * (dP_j - D)                    (d sum(dO*o) / d s_j)     */
/*   dq[x]   = scale * sum_j dS_j * k[j,g,x]                                */
/*   dk[j,g,x] += scale * dS_j * q[x]      dv[j,g,e] += value_scale * P_j * dO[e] */
/*   dsink[h] += -exp(sigma_h - LSE) * D   (d o / d sigma = -P_sink * o)    */
/* dk and dv sum over the 16 heads of the group and over every query row    */
/* whose key set holds j; dsink sums over every row of every sequence.      */

typedef struct {
    const dims_t* d;
    const uint16_t *q, *k, *v, *dout;
    const int32_t* cu;
    int nseq;
    const float* sink;
    const int64_t* items; /* packed token indices of this phase */
    int64_t nitems;
    double *lse, *D, *psink; /* per [T][hq] row statistics (phase 0 writes, 2 reads) */
    double *dq, *dk, *dv;    /* phase 1 writes dq [nitems][hq][dqk]; phase 2 dk/dv [nitems][hkv][.] */
    int phase, maxkeys;
    int stored_out;          /* D from the output rounded to bf16 */
    int64_t next;
    pthread_mutex_t mu;
} bwd_job_t;

static void* bwd_worker(void* arg) {
    bwd_job_t* jb = (bwd_job_t*)arg;
    const dims_t* d = jb->d;
    const uint16_t** kr = malloc(sizeof(*kr) * (size_t)(jb->maxkeys + 1));
    const uint16_t** vr = malloc(sizeof(*vr) * (size_t)(jb->maxkeys + 1));
    double* sc = malloc(sizeof(double) * (size_t)(jb->maxkeys + 1));
    double* w = malloc(sizeof(double) * (size_t)(jb->maxkeys + 1));
    double* o = malloc(sizeof(double) * (size_t)d->dv);
    int group = d->hq / d->hkv;
    for (;;) {
        pthread_mutex_lock(&jb->mu);
        int64_t it = jb->next++;
        pthread_mutex_unlock(&jb->mu);
        if (it >= jb->nitems) break;
        int64_t t = jb->items[it];
        int b = seq_of_token(jb->cu, jb->nseq, t);
        int64_t base = jb->cu[b];
        int L = jb->cu[b + 1] - jb->cu[b];
        int p = (int)(t - base);
        if (jb->phase <= 1) { /* a query row: forward, then row statistics or dq */
            int lo = 0;
            if (d->layer_type == ORACLE_SWA) lo = p - (d->window - 1) > 0 ? p - (d->window - 1) : 0;
            for (int h = 0; h < d->hq; ++h) {
                int g = h / group;
                int n = prefill_key_rows(d, jb->k, jb->v, base, lo, p, g, kr, vr);
                double sigma = 0.0, lse, wsink;
                int hs = sink_present(jb->sink, h, &sigma);
                attend_row(d, jb->q + ((size_t)t * d->hq + h) * d->dqk, n, kr, vr, NULL, hs, sigma, sc, o, &lse, w,
                           &wsink);
                const uint16_t* dorow = jb->dout + ((size_t)t * d->hq + h) * d->dv;
                double D = 0.0;
                for (int e = 0; e < d->dv; ++e)
                    D += bf16_to_double(dorow[e]) * (jb->stored_out ? round_bf16(o[e]) : o[e]);
                if (jb->phase == 0) {
                    jb->lse[(size_t)t * d->hq + h] = lse;
                    jb->D[(size_t)t * d->hq + h] = D;
                    jb->psink[(size_t)t * d->hq + h] = wsink;
                    continue;
                }
                double* dq = jb->dq + ((size_t)it * d->hq + h) * d->dqk;
                for (int x = 0; x < d->dqk; ++x) dq[x] = 0.0;
                for (int j = 0; j < n; ++j) {
                    double dp = 0.0;
                    for (int e = 0; e < d->dv; ++e) dp += bf16_to_double(dorow[e]) * bf16_to_double(vr[j][e]);
                    double ds = w[j] * (d->value_scale * dp - D);
                    for (int x = 0; x < d->dqk; ++x) dq[x] += d->scale * ds * bf16_to_double(kr[j][x]);
                }
            }
        } else { /* a key row: dk, dv over every query row that sees it */
            int hi = L - 1;
            if (d->layer_type == ORACLE_SWA && p + d->window - 1 < hi) hi = p + d->window - 1;
            for (int g = 0; g < d->hkv; ++g) {
                const uint16_t* krow = jb->k + ((size_t)t * d->hkv + g) * d->dqk;
                const uint16_t* vrow = jb->v + ((size_t)t * d->hkv + g) * d->dv;
                double* dk = jb->dk + ((size_t)it * d->hkv + g) * d->dqk;
                double* dv = jb->dv + ((size_t)it * d->hkv + g) * d->dv;
                for (int x = 0; x < d->dqk; ++x) dk[x] = 0.0;
                for (int e = 0; e < d->dv; ++e) dv[e] = 0.0;
                for (int h = g * group; h < (g + 1) * group; ++h)
                    for (int i = p; i <= hi; ++i) {
                        size_t row = (size_t)(base + i) * d->hq + h;
                        const uint16_t* qrow = jb->q + row * d->dqk;
                        const uint16_t* dorow = jb->dout + row * d->dv;
                        double acc = 0.0;
                        for (int x = 0; x < d->dqk; ++x) acc += bf16_to_double(qrow[x]) * bf16_to_double(krow[x]);
                        double pw = exp(d->scale * acc - jb->lse[row]);
                        double dp = 0.0;
                        for (int e = 0; e < d->dv; ++e) dp += bf16_to_double(dorow[e]) * bf16_to_double(vrow[e]);
                        double ds = pw * (d->value_scale * dp - jb->D[row]);
                        for (int x = 0; x < d->dqk; ++x) dk[x] += d->scale * ds * bf16_to_double(qrow[x]);
                        for (int e = 0; e < d->dv; ++e) dv[e] += d->value_scale * pw * bf16_to_double(dorow[e]);
                    }
            }
        }
    }
    free(kr); free(vr); free(sc); free(w); free(o);
    return NULL;
}

/* Gradients of sum(dO * out) for a packed prefill batch (layouts as for
 * oracle_prefill; dout [T][hq][dv] bf16 bits).  dq is computed for the packed
 * tokens q_rows [nq] (dq [nq][hq][dqk]), dk/dv for kv_rows [nkv] (dk
 * [nkv][hkv][dqk], dv [nkv][hkv][dv]); dsink [hq] (NULL to skip) sums over
 * every token of the batch and is 0 without a sink.
 *
 * D_t = dO_t . o_t is the one place the forward output enters.  With
 * stored_out = 0 it is the exact output, so the results are the exact
 * gradients.  With stored_out = 1 it is the output as a bf16 forward stores
 * it (each element rounded once to the nearest bf16, ties to even): the
 * gradients a backward computes when it is handed the forward's stored output,
 * as the row-sum step of the flash-attention backward is.  dv does not depend on D. */
int oracle_prefill_backward(int hq, int hkv, int dqk, int dv, int layer_type, int window, float scale,
                            float value_scale, const uint16_t* q, const uint16_t* k, const uint16_t* v,
                            const uint16_t* dout, const int32_t* cu_seqlens, int nseq, const float* sink,
                            const int64_t* q_rows, int64_t nq, const int64_t* kv_rows, int64_t nkv,
                            double* dq, double* dk, double* dvv, double* dsink, int stored_out, int nthreads) {
    dims_t d = {hq, hkv, dqk, dv, layer_type, window, (double)scale, (double)value_scale};
    if (!check_dims(&d) || nseq < 1 || !q || !k || !v || !dout || !cu_seqlens || cu_seqlens[0] != 0)
        return ORACLE_EINVAL;
    if ((nq > 0 && (!q_rows || !dq)) || (nkv > 0 && (!kv_rows || !dk || !dvv)) || nq < 0 || nkv < 0)
        return ORACLE_EINVAL;
    int64_t T = cu_seqlens[nseq];
    int maxkeys = 1;
    for (int b = 0; b < nseq; ++b) {
        int L = cu_seqlens[b + 1] - cu_seqlens[b];
        if (L < 0) return ORACLE_EINVAL;
        if (L > maxkeys) maxkeys = L;
    }
    for (int64_t i = 0; i < nq; ++i) if (q_rows[i] < 0 || q_rows[i] >= T) return ORACLE_EINVAL;
    for (int64_t i = 0; i < nkv; ++i) if (kv_rows[i] < 0 || kv_rows[i] >= T) return ORACLE_EINVAL;
    /* Rows whose statistics are needed: every query row that sees a kv row, and
     * all rows for dsink. */
    uint8_t* need = calloc((size_t)(T > 0 ? T : 1), 1);
    for (int64_t i = 0; i < nkv; ++i) {
        int64_t t = kv_rows[i];
        int b = seq_of_token(cu_seqlens, nseq, t);
        int64_t end = cu_seqlens[b + 1];
        if (layer_type == ORACLE_SWA && t + window < end) end = t + window;
        for (int64_t r = t; r < end; ++r) need[r] = 1;
    }
    if (dsink) memset(need, 1, (size_t)T);
    int64_t nneed = 0;
    for (int64_t r = 0; r < T; ++r) nneed += need[r];
    int64_t* rows = malloc(sizeof(int64_t) * (size_t)(nneed > 0 ? nneed : 1));
    nneed = 0;
    for (int64_t r = 0; r < T; ++r) if (need[r]) rows[nneed++] = r;
    double* lse = calloc((size_t)(T > 0 ? T : 1) * hq, sizeof(double));
    double* D = calloc((size_t)(T > 0 ? T : 1) * hq, sizeof(double));
    double* ps = calloc((size_t)(T > 0 ? T : 1) * hq, sizeof(double));
    bwd_job_t jb;
    memset(&jb, 0, sizeof jb);
    jb.d = &d; jb.q = q; jb.k = k; jb.v = v; jb.dout = dout; jb.cu = cu_seqlens; jb.nseq = nseq; jb.sink = sink;
    jb.lse = lse; jb.D = D; jb.psink = ps; jb.dq = dq; jb.dk = dk; jb.dv = dvv; jb.maxkeys = maxkeys;
    jb.stored_out = stored_out != 0;
    pthread_mutex_init(&jb.mu, NULL);
    const int64_t* phase_items[3] = {rows, q_rows, kv_rows};
    int64_t phase_n[3] = {nneed, nq, nkv};
    for (int ph = 0; ph < 3; ++ph) {
        jb.phase = ph; jb.items = phase_items[ph]; jb.nitems = phase_n[ph]; jb.next = 0;
        if (jb.nitems > 0) run_threads(bwd_worker, &jb, nthreads);
    }
    pthread_mutex_destroy(&jb.mu);
    if (dsink)
        for (int h = 0; h < hq; ++h) {
            double acc = 0.0;
            for (int64_t r = 0; r < T; ++r) acc -= ps[(size_t)r * hq + h] * D[(size_t)r * hq + h];
            dsink[h] = acc;
        }
    free(need); free(rows); free(lse); free(D); free(ps);
    return ORACLE_OK;
}

/* ------------------------------------------------------------------------ */
/* Decode: one new token per sequence at position p = ctx_lens[b].          */
/* Cache readers, written from the layout definitions:                      */
/*   SWA ring  [B][R][Hkv][D], R = W - 1 slots; position j lives in slot j mod R.
 *   GA pool   [N][Hkv][D]; position j of sequence b lives at row base_b + j.
 *   GA paged pool [num_pages * P][Hkv][D], P rows per page: block i of
 *             sequence b (positions i*P .. i*P + P-1) is page table[b][i], so
 *             position j lives at row table[b][j / P] * P + j mod P.  (Paging is
 *             a serving layout of the same cache, not something the model
 *             defines; it changes where rows live, not what is computed.) */

typedef struct {
    const int32_t* table;  /* [batch][max_blocks] */
    int max_blocks, page_size;
    int64_t num_pages;
} pages_t;

typedef struct {
    const dims_t* d;
    const uint16_t *q, *k_new, *v_new, *k_cache, *v_cache;
    const uint8_t *k8, *v8;          /* FP8 GA pool (codes), or NULL */
    const float *k8scale, *v8scale;  /* [hkv] scales of the FP8 pool */
    const int64_t* kv_base;
    const pages_t* pages;
    const int32_t* ctx;
    int batch, ring;
    const float* sink;
    double *out, *lse;
    int64_t next;
    pthread_mutex_t mu;
} decode_job_t;

/* Pool row of position j of sequence b in a paged pool. */
static int64_t paged_row(const pages_t* pg, int b, int64_t j) {
    int64_t page = pg->table[(size_t)b * pg->max_blocks + (size_t)(j / pg->page_size)];
    return page * pg->page_size + j % pg->page_size;
}

/* Row of cached position j of sequence b, KV head g, in the ring, the pool or
 * the paged pool (pages != NULL). */
static const uint16_t* cached_row(const dims_t* d, const uint16_t* cache, int ring, const int64_t* kv_base,
                                  const pages_t* pages, int b, int j, int g, int isv) {
    int D = isv ? d->dv : d->dqk;
    size_t row;
    if (d->layer_type == ORACLE_SWA) row = (size_t)b * ring + (size_t)(j % ring);
    else if (pages) row = (size_t)paged_row(pages, b, j);
    else row = (size_t)(kv_base[b] + j);
    return cache + (row * d->hkv + g) * D;
}

static const uint16_t* cache_row(const decode_job_t* jb, int b, int j, int g, int isv) {
    return cached_row(jb->d, isv ? jb->v_cache : jb->k_cache, jb->ring, jb->kv_base, jb->pages, b, j, g, isv);
}

/* Every block holding a position below npos[b] maps to a page of the pool. */
static int pages_cover(const pages_t* pg, const int32_t* npos, int batch) {
    if (!pg->table || pg->max_blocks < 1 || pg->page_size < 1 || pg->num_pages < 1) return 0;
    for (int b = 0; b < batch; ++b) {
        if (npos[b] > (int64_t)pg->max_blocks * pg->page_size) return 0;
        for (int i = 0; (int64_t)i * pg->page_size < npos[b]; ++i) {
            int32_t page = pg->table[(size_t)b * pg->max_blocks + i];
            if (page < 0 || page >= pg->num_pages) return 0;
        }
    }
    return 1;
}

static void* decode_worker(void* arg) {
    decode_job_t* jb = (decode_job_t*)arg;
    const dims_t* d = jb->d;
    int maxkeys = 1;
    for (int b = 0; b < jb->batch; ++b) if (jb->ctx[b] + 1 > maxkeys) maxkeys = jb->ctx[b] + 1;
    const uint16_t** kr = malloc(sizeof(*kr) * (size_t)maxkeys);
    const uint16_t** vr = malloc(sizeof(*vr) * (size_t)maxkeys);
    const uint8_t** k8r = malloc(sizeof(*k8r) * (size_t)maxkeys);
    const uint8_t** v8r = malloc(sizeof(*v8r) * (size_t)maxkeys);
    double* sc = malloc(sizeof(double) * (size_t)maxkeys);
    int group = d->hq / d->hkv;
    for (;;) {
        pthread_mutex_lock(&jb->mu);
        int64_t item = jb->next++;
        pthread_mutex_unlock(&jb->mu);
        if (item >= (int64_t)jb->batch * d->hq) break;
        int b = (int)(item / d->hq), h = (int)(item % d->hq), g = h / group;
        int p = jb->ctx[b];
        int lo = 0;
        if (d->layer_type == ORACLE_SWA) lo = p - (d->window - 1) > 0 ? p - (d->window - 1) : 0;
        int n = 0;
        for (int j = lo; j < p; ++j, ++n) {
            if (jb->k8) { /* FP8 pool: codes of row kv_base[b] + j, or of the paged row */
                size_t row = jb->pages ? (size_t)paged_row(jb->pages, b, j) : (size_t)(jb->kv_base[b] + j);
                kr[n] = vr[n] = NULL;
                k8r[n] = jb->k8 + (row * d->hkv + g) * d->dqk;
                v8r[n] = jb->v8 + (row * d->hkv + g) * d->dv;
            } else {
                kr[n] = cache_row(jb, b, j, g, 0);
                vr[n] = cache_row(jb, b, j, g, 1);
                k8r[n] = v8r[n] = NULL;
            }
        }
        kr[n] = jb->k_new + ((size_t)b * d->hkv + g) * d->dqk;
        vr[n] = jb->v_new + ((size_t)b * d->hkv + g) * d->dv;
        k8r[n] = v8r[n] = NULL;
        n++;
        double sigma = 0.0;
        int hs = sink_present(jb->sink, h, &sigma);
        fp8_rows_t f8 = {k8r, v8r, jb->k8 ? (double)jb->k8scale[g] : 1.0, jb->k8 ? (double)jb->v8scale[g] : 1.0};
        attend_row(d, jb->q + ((size_t)b * d->hq + h) * d->dqk, n, kr, vr, jb->k8 ? &f8 : NULL, hs, sigma, sc,
                   jb->out + ((size_t)b * d->hq + h) * d->dv, jb->lse + (size_t)b * d->hq + h, NULL, NULL);
    }
    free(kr); free(vr); free(k8r); free(v8r); free(sc);
    return NULL;
}

static int decode_impl(const dims_t* d, const uint16_t* q, const uint16_t* k_new, const uint16_t* v_new,
                       const uint16_t* k_cache, const uint16_t* v_cache, int ring_slots, const int64_t* kv_base,
                       const pages_t* pages, const int32_t* ctx_lens, int batch, const float* sink, double* out,
                       double* lse, int nthreads) {
    if (!check_dims(d) || batch < 1 || !q || !k_new || !v_new || !ctx_lens || !out || !lse) return ORACLE_EINVAL;
    if (d->layer_type == ORACLE_SWA && ring_slots != d->window - 1) return ORACLE_EINVAL;
    if (d->layer_type == ORACLE_GA && !kv_base && !pages) return ORACLE_EINVAL;
    for (int b = 0; b < batch; ++b) {
        if (ctx_lens[b] < 0) return ORACLE_EINVAL;
        if (ctx_lens[b] > 0 && (!k_cache || !v_cache)) return ORACLE_EINVAL;
    }
    if (pages && !pages_cover(pages, ctx_lens, batch)) return ORACLE_EINVAL;
    decode_job_t jb;
    memset(&jb, 0, sizeof jb);
    jb.d = d; jb.q = q; jb.k_new = k_new; jb.v_new = v_new; jb.k_cache = k_cache; jb.v_cache = v_cache;
    jb.kv_base = kv_base; jb.pages = pages; jb.ctx = ctx_lens; jb.batch = batch; jb.ring = ring_slots;
    jb.sink = sink; jb.out = out; jb.lse = lse;
    pthread_mutex_init(&jb.mu, NULL);
    run_threads(decode_worker, &jb, nthreads);
    pthread_mutex_destroy(&jb.mu);
    return ORACLE_OK;
}

/* Decode attention for one new token per sequence.  SWA reads the ring
 * (ring_slots = W - 1 required), GA reads the pool at kv_base[b] + j. */
int oracle_decode(int hq, int hkv, int dqk, int dv, int layer_type, int window,
                  float scale, float value_scale,
                  const uint16_t* q, const uint16_t* k_new, const uint16_t* v_new,
                  const uint16_t* k_cache, const uint16_t* v_cache, int ring_slots,
                  const int64_t* kv_base, const int32_t* ctx_lens, int batch,
                  const float* sink, double* out, double* lse, int nthreads) {
    dims_t d = {hq, hkv, dqk, dv, layer_type, window, (double)scale, (double)value_scale};
    return decode_impl(&d, q, k_new, v_new, k_cache, v_cache, ring_slots, kv_base, NULL, ctx_lens, batch, sink,
                       out, lse, nthreads);
}

/* GA decode over a paged pool: block_table [batch][max_blocks] maps block i
 * of sequence b to a page of page_size rows.  Every block below ctx_lens[b]
 * must map to a page in [0, num_pages) (ORACLE_EINVAL otherwise). */
int oracle_decode_paged(int hq, int hkv, int dqk, int dv, float scale, float value_scale,
                        const uint16_t* q, const uint16_t* k_new, const uint16_t* v_new,
                        const uint16_t* k_cache, const uint16_t* v_cache,
                        const int32_t* block_table, int max_blocks, int page_size, int64_t num_pages,
                        const int32_t* ctx_lens, int batch, const float* sink, double* out, double* lse,
                        int nthreads) {
    dims_t d = {hq, hkv, dqk, dv, ORACLE_GA, 0, (double)scale, (double)value_scale};
    pages_t pg = {block_table, max_blocks, page_size, num_pages};
    return decode_impl(&d, q, k_new, v_new, k_cache, v_cache, 0, NULL, &pg, ctx_lens, batch, sink, out, lse,
                       nthreads);
}

/* ------------------------------------------------------------------------ */
/* Chunked prefill: sequence b has ctx_lens[b] positions cached and brings  */
/* n_b = cu_newlens[b+1] - cu_newlens[b] new tokens, token i at position    */
/* p = ctx_lens[b] + i (model doc, MiMoV2FlashModel.forward: with a cache   */
/* only the tokens not yet processed are passed).  Its key set is lo..p as  */
/* above: positions below ctx_lens[b] are read from the cache (ring or pool,*/
/* as in decode), the others from the chunk's own k/v rows.  The cache is   */
/* read, never written (appending the chunk is a separate call).            */

/* An FP8 GA cache of a chunked prefill: code pools and per-KV-head scales. */
typedef struct {
    const uint8_t *k8, *v8;
    const float *kscale, *vscale;
} chunk_fp8_t;

typedef struct {
    const dims_t* d;
    const uint16_t *q, *k, *v, *k_cache, *v_cache;
    const chunk_fp8_t* f8;  /* cached rows are FP8 codes when set */
    const int32_t* cu;
    const int64_t* kv_base;
    const pages_t* pages;
    const int32_t* ctx;
    int batch, ring, maxkeys;
    const float* sink;
    double *out, *lse;
    int64_t next, total;
    pthread_mutex_t mu;
} chunk_job_t;

static void* chunk_worker(void* arg) {
    chunk_job_t* jb = (chunk_job_t*)arg;
    const dims_t* d = jb->d;
    const uint16_t** kr = malloc(sizeof(*kr) * (size_t)jb->maxkeys);
    const uint16_t** vr = malloc(sizeof(*vr) * (size_t)jb->maxkeys);
    const uint8_t** k8r = malloc(sizeof(*k8r) * (size_t)jb->maxkeys);
    const uint8_t** v8r = malloc(sizeof(*v8r) * (size_t)jb->maxkeys);
    double* sc = malloc(sizeof(double) * (size_t)jb->maxkeys);
    int group = d->hq / d->hkv;
    for (;;) {
        pthread_mutex_lock(&jb->mu);
        int64_t item = jb->next++;
        pthread_mutex_unlock(&jb->mu);
        if (item >= jb->total * d->hq) break;
        int64_t t = item / d->hq;
        int h = (int)(item % d->hq), g = h / group;
        int b = seq_of_token(jb->cu, jb->batch, t);
        int c = jb->ctx[b];
        int p = c + (int)(t - jb->cu[b]);
        int lo = 0;
        if (d->layer_type == ORACLE_SWA) lo = p - (d->window - 1) > 0 ? p - (d->window - 1) : 0;
        int n = 0;
        for (int j = lo; j <= p; ++j, ++n) {
            k8r[n] = v8r[n] = NULL;
            if (j < c && jb->f8) { /* FP8 codes of the GA pool row (contiguous or paged) */
                size_t row = jb->pages ? (size_t)paged_row(jb->pages, b, j) : (size_t)(jb->kv_base[b] + j);
                kr[n] = vr[n] = NULL;
                k8r[n] = jb->f8->k8 + (row * d->hkv + g) * d->dqk;
                v8r[n] = jb->f8->v8 + (row * d->hkv + g) * d->dv;
            } else if (j < c) {
                kr[n] = cached_row(d, jb->k_cache, jb->ring, jb->kv_base, jb->pages, b, j, g, 0);
                vr[n] = cached_row(d, jb->v_cache, jb->ring, jb->kv_base, jb->pages, b, j, g, 1);
            } else {
                size_t row = (size_t)jb->cu[b] + (size_t)(j - c);
                kr[n] = jb->k + (row * d->hkv + g) * d->dqk;
                vr[n] = jb->v + (row * d->hkv + g) * d->dv;
            }
        }
        double sigma = 0.0;
        int hs = sink_present(jb->sink, h, &sigma);
        fp8_rows_t f8 = {k8r, v8r, jb->f8 ? (double)jb->f8->kscale[g] : 1.0, jb->f8 ? (double)jb->f8->vscale[g] : 1.0};
        attend_row(d, jb->q + ((size_t)t * d->hq + h) * d->dqk, n, kr, vr, jb->f8 ? &f8 : NULL, hs, sigma, sc,
                   jb->out + ((size_t)t * d->hq + h) * d->dv, jb->lse + (size_t)t * d->hq + h, NULL, NULL);
    }
    free(kr); free(vr); free(k8r); free(v8r); free(sc);
    return NULL;
}

static int chunk_impl(const dims_t* d, const uint16_t* q, const uint16_t* k, const uint16_t* v,
                      const int32_t* cu_newlens, int batch, const uint16_t* k_cache, const uint16_t* v_cache,
                      int ring_slots, const int64_t* kv_base, const pages_t* pages, const chunk_fp8_t* f8,
                      const int32_t* ctx_lens, const float* sink, double* out, double* lse, int nthreads) {
    if (!check_dims(d) || batch < 1 || !q || !k || !v || !cu_newlens || !ctx_lens || !out || !lse)
        return ORACLE_EINVAL;
    if (d->layer_type == ORACLE_SWA && ring_slots != d->window - 1) return ORACLE_EINVAL;
    if (d->layer_type == ORACLE_GA && !kv_base && !pages) return ORACLE_EINVAL;
    if (cu_newlens[0] != 0) return ORACLE_EINVAL;
    int maxkeys = 1;
    for (int b = 0; b < batch; ++b) {
        int n = cu_newlens[b + 1] - cu_newlens[b];
        if (n < 0 || ctx_lens[b] < 0) return ORACLE_EINVAL;
        if (ctx_lens[b] > 0 && !f8 && (!k_cache || !v_cache)) return ORACLE_EINVAL;
        if (ctx_lens[b] + n > maxkeys) maxkeys = ctx_lens[b] + n;
    }
    if (pages && !pages_cover(pages, ctx_lens, batch)) return ORACLE_EINVAL;
    chunk_job_t jb;
    memset(&jb, 0, sizeof jb);
    jb.d = d; jb.q = q; jb.k = k; jb.v = v; jb.k_cache = k_cache; jb.v_cache = v_cache; jb.f8 = f8;
    jb.cu = cu_newlens; jb.kv_base = kv_base; jb.pages = pages; jb.ctx = ctx_lens; jb.batch = batch;
    jb.ring = ring_slots; jb.maxkeys = maxkeys; jb.sink = sink; jb.out = out; jb.lse = lse;
    jb.total = cu_newlens[batch];
    pthread_mutex_init(&jb.mu, NULL);
    run_threads(chunk_worker, &jb, nthreads);
    pthread_mutex_destroy(&jb.mu);
    return ORACLE_OK;
}

/* q [Tn][hq][dqk], k [Tn][hkv][dqk], v [Tn][hkv][dv] packed by cu_newlens
 * [batch+1]; caches as for decode (SWA ring_slots = W - 1, GA kv_base).
 * out [Tn][hq][dv], lse [Tn][hq]. */
int oracle_prefill_chunk(int hq, int hkv, int dqk, int dv, int layer_type, int window,
                         float scale, float value_scale,
                         const uint16_t* q, const uint16_t* k, const uint16_t* v,
                         const int32_t* cu_newlens, int batch,
                         const uint16_t* k_cache, const uint16_t* v_cache, int ring_slots,
                         const int64_t* kv_base, const int32_t* ctx_lens,
                         const float* sink, double* out, double* lse, int nthreads) {
    dims_t d = {hq, hkv, dqk, dv, layer_type, window, (double)scale, (double)value_scale};
    return chunk_impl(&d, q, k, v, cu_newlens, batch, k_cache, v_cache, ring_slots, kv_base, NULL, NULL, ctx_lens,
                      sink, out, lse, nthreads);
}

/* GA chunked prefill whose cached positions live in a paged pool (as for
 * oracle_decode_paged). */
int oracle_prefill_chunk_paged(int hq, int hkv, int dqk, int dv, float scale, float value_scale,
                               const uint16_t* q, const uint16_t* k, const uint16_t* v,
                               const int32_t* cu_newlens, int batch,
                               const uint16_t* k_cache, const uint16_t* v_cache,
                               const int32_t* block_table, int max_blocks, int page_size, int64_t num_pages,
                               const int32_t* ctx_lens, const float* sink, double* out, double* lse,
                               int nthreads) {
    dims_t d = {hq, hkv, dqk, dv, ORACLE_GA, 0, (double)scale, (double)value_scale};
    pages_t pg = {block_table, max_blocks, page_size, num_pages};
    return chunk_impl(&d, q, k, v, cu_newlens, batch, k_cache, v_cache, 0, NULL, &pg, NULL, ctx_lens, sink, out,
                      lse, nthreads);
}

/* ------------------------------------------------------------------------ */
/* KV append: new token i of sequence b sits at position ctx_lens[b] + i.   */
/* SWA: written, in position order, to slot (position mod R); later writes  */
/* replace earlier ones, so the ring ends with the last R positions.        */
/* GA: written to pool row kv_base[b] + position, which must stay below     */
/* kv_base[b] + kv_capacity[b] (ORACLE_ECAPACITY otherwise, nothing written */
/* for that sequence).                                                      */
int oracle_kv_append(int hkv, int dqk, int dv, int layer_type, int ring_slots,
                     const uint16_t* k, const uint16_t* v, const int32_t* cu_newlens,
                     const int32_t* ctx_lens, int batch,
                     uint16_t* k_cache, uint16_t* v_cache,
                     const int64_t* kv_base, const int64_t* kv_capacity) {
    if (hkv <= 0 || dqk <= 0 || dv <= 0 || batch < 1 || !k || !v || !cu_newlens || !ctx_lens ||
        !k_cache || !v_cache)
        return ORACLE_EINVAL;
    if (layer_type == ORACLE_SWA && ring_slots < 1) return ORACLE_EINVAL;
    if (layer_type == ORACLE_GA && (!kv_base || !kv_capacity)) return ORACLE_EINVAL;
    if (layer_type != ORACLE_SWA && layer_type != ORACLE_GA) return ORACLE_EINVAL;
    int status = ORACLE_OK;
    size_t krow = (size_t)hkv * dqk, vrow = (size_t)hkv * dv;
    for (int b = 0; b < batch; ++b) {
        int n = cu_newlens[b + 1] - cu_newlens[b];
        if (n < 0) return ORACLE_EINVAL;
        if (layer_type == ORACLE_GA && (int64_t)ctx_lens[b] + n > kv_capacity[b]) {
            status = ORACLE_ECAPACITY;
            continue;
        }
        for (int i = 0; i < n; ++i) {
            int64_t pos = (int64_t)ctx_lens[b] + i;
            size_t src = (size_t)cu_newlens[b] + i;
            size_t dst = layer_type == ORACLE_SWA ? (size_t)b * ring_slots + (size_t)(pos % ring_slots)
                                                  : (size_t)(kv_base[b] + pos);
            memcpy(k_cache + dst * krow, k + src * krow, krow * sizeof(uint16_t));
            memcpy(v_cache + dst * vrow, v + src * vrow, vrow * sizeof(uint16_t));
        }
    }
    return status;
}

/* KV append into a paged GA pool: position pos of sequence b goes to row
 * table[b][pos / P] * P + pos mod P.  A sequence whose ctx_lens[b] + n needs
 * more than max_blocks blocks is skipped whole, and a token whose block maps
 * outside [0, num_pages) is not written; either makes the status
 * ORACLE_ECAPACITY. */
int oracle_kv_append_paged(int hkv, int dqk, int dv, const uint16_t* k, const uint16_t* v,
                           const int32_t* cu_newlens, const int32_t* ctx_lens, int batch,
                           uint16_t* k_cache, uint16_t* v_cache,
                           const int32_t* block_table, int max_blocks, int page_size, int64_t num_pages) {
    if (hkv <= 0 || dqk <= 0 || dv <= 0 || batch < 1 || !k || !v || !cu_newlens || !ctx_lens || !k_cache ||
        !v_cache || !block_table || max_blocks < 1 || page_size < 1 || num_pages < 1)
        return ORACLE_EINVAL;
    pages_t pg = {block_table, max_blocks, page_size, num_pages};
    int status = ORACLE_OK;
    size_t krow = (size_t)hkv * dqk, vrow = (size_t)hkv * dv;
    for (int b = 0; b < batch; ++b) {
        int n = cu_newlens[b + 1] - cu_newlens[b];
        if (n < 0) return ORACLE_EINVAL;
        if ((int64_t)ctx_lens[b] + n > (int64_t)max_blocks * page_size) {
            status = ORACLE_ECAPACITY;
            continue;
        }
        for (int i = 0; i < n; ++i) {
            int64_t pos = (int64_t)ctx_lens[b] + i;
            int32_t page = block_table[(size_t)b * max_blocks + (size_t)(pos / page_size)];
            if (page < 0 || page >= num_pages) {
                status = ORACLE_ECAPACITY;
                continue;
            }
            size_t src = (size_t)cu_newlens[b] + i;
            size_t dst = (size_t)paged_row(&pg, b, pos);
            memcpy(k_cache + dst * krow, k + src * krow, krow * sizeof(uint16_t));
            memcpy(v_cache + dst * vrow, v + src * vrow, vrow * sizeof(uint16_t));
        }
    }
    return status;
}

/* ------------------------------------------------------------------------ */
/* Rotary position embedding of queries and keys (model doc,              */
/* MiMoV2FlashConfig, rope_parameters: rope_theta, with the Transformers   */
/* RoPE convention): the first rd = rotary_dim dims of every head vector x  */
/* at position p rotate in pairs (i, i + rd/2), i < rd/2, by the angle       */
/* p * f_i with f_i = theta^(-2i/rd):                                       */
/*   x'[i]        = x[i] cos(p f_i) - x[i + rd/2] sin(p f_i)                  */
/*   x'[i + rd/2] = x[i + rd/2] cos(p f_i) + x[i] sin(p f_i)                  */
/* and dims rd .. d-1 pass through.                                          */
static void rope_row(const uint16_t* x, double* out, int d, int rd, double p, double theta) {
    int half = rd / 2;
    for (int e = 0; e < d; ++e) out[e] = bf16_to_double(x[e]);
    for (int i = 0; i < half; ++i) {
        double f = pow(theta, -2.0 * i / rd);
        double c = cos(p * f), sn = sin(p * f);
        double a = bf16_to_double(x[i]), b = bf16_to_double(x[i + half]);
        out[i] = a * c - b * sn;
        out[i + half] = b * c + a * sn;
    }
}

/* q [T][hq][d], k [T][hkv][d] (bf16 bits; either may be NULL) at positions
 * [T] -> q_out, k_out (double, same shapes). */
int oracle_rope(int hq, int hkv, int d, const uint16_t* q, const uint16_t* k, const int32_t* positions, int64_t T,
                double theta, int rotary_dim, double* q_out, double* k_out) {
    if (hq < 0 || hkv < 0 || d <= 0 || T < 0 || !positions || rotary_dim < 0 || rotary_dim > d || rotary_dim % 2 ||
        !(theta > 0.0))
        return ORACLE_EINVAL;
    if ((q && !q_out) || (k && !k_out)) return ORACLE_EINVAL;
    for (int64_t t = 0; t < T; ++t) {
        if (positions[t] < 0) return ORACLE_EINVAL;
        double p = (double)positions[t];
        if (q)
            for (int h = 0; h < hq; ++h)
                rope_row(q + ((size_t)t * hq + h) * d, q_out + ((size_t)t * hq + h) * d, d, rotary_dim, p, theta);
        if (k)
            for (int h = 0; h < hkv; ++h)
                rope_row(k + ((size_t)t * hkv + h) * d, k_out + ((size_t)t * hkv + h) * d, d, rotary_dim, p, theta);
    }
    return ORACLE_OK;
}

/* ------------------------------------------------------------------------ */
/* FP8 GA cache (see the header): pool [N][Hkv][D] of E4M3 codes, position j */
/* of sequence b at row kv_base[b] + j, one scale per KV head for K and V.   */

static int scales_ok(const float* s, int hkv) {
    if (!s) return 0;
    for (int g = 0; g < hkv; ++g)
        if (!(s[g] > 0.0f) || isinf(s[g])) return 0;
    return 1;
}

static int decode_fp8_impl(const dims_t* d, const uint16_t* q, const uint16_t* k_new, const uint16_t* v_new,
                           const uint8_t* k_cache, const uint8_t* v_cache, const int64_t* kv_base,
                           const pages_t* pages, const float* k_scale, const float* v_scale,
                           const int32_t* ctx_lens, int batch, const float* sink, double* out, double* lse,
                           int nthreads) {
    if (!check_dims(d) || batch < 1 || !q || !k_new || !v_new || !ctx_lens || !out || !lse ||
        (!kv_base && !pages) || !k_cache || !v_cache || !scales_ok(k_scale, d->hkv) || !scales_ok(v_scale, d->hkv))
        return ORACLE_EINVAL;
    for (int b = 0; b < batch; ++b)
        if (ctx_lens[b] < 0) return ORACLE_EINVAL;
    if (pages && !pages_cover(pages, ctx_lens, batch)) return ORACLE_EINVAL;
    decode_job_t jb;
    memset(&jb, 0, sizeof jb);
    jb.d = d; jb.q = q; jb.k_new = k_new; jb.v_new = v_new; jb.k8 = k_cache; jb.v8 = v_cache;
    jb.k8scale = k_scale; jb.v8scale = v_scale; jb.kv_base = kv_base; jb.pages = pages; jb.ctx = ctx_lens;
    jb.batch = batch; jb.sink = sink; jb.out = out; jb.lse = lse;
    pthread_mutex_init(&jb.mu, NULL);
    run_threads(decode_worker, &jb, nthreads);
    pthread_mutex_destroy(&jb.mu);
    return ORACLE_OK;
}

/* GA decode over an FP8 pool: cached positions j < p read as code * scale. */
int oracle_decode_fp8(int hq, int hkv, int dqk, int dv, float scale, float value_scale,
                      const uint16_t* q, const uint16_t* k_new, const uint16_t* v_new,
                      const uint8_t* k_cache, const uint8_t* v_cache, const int64_t* kv_base,
                      const float* k_scale, const float* v_scale, const int32_t* ctx_lens, int batch,
                      const float* sink, double* out, double* lse, int nthreads) {
    dims_t d = {hq, hkv, dqk, dv, ORACLE_GA, 0, (double)scale, (double)value_scale};
    if (!kv_base) return ORACLE_EINVAL;
    return decode_fp8_impl(&d, q, k_new, v_new, k_cache, v_cache, kv_base, NULL, k_scale, v_scale, ctx_lens, batch,
                           sink, out, lse, nthreads);
}

/* GA decode over a paged FP8 pool: the codes of position j of sequence b in
 * the row the block table gives (as oracle_decode_paged), read as code * scale. */
int oracle_decode_fp8_paged(int hq, int hkv, int dqk, int dv, float scale, float value_scale,
                            const uint16_t* q, const uint16_t* k_new, const uint16_t* v_new,
                            const uint8_t* k_cache, const uint8_t* v_cache,
                            const int32_t* block_table, int max_blocks, int page_size, int64_t num_pages,
                            const float* k_scale, const float* v_scale, const int32_t* ctx_lens, int batch,
                            const float* sink, double* out, double* lse, int nthreads) {
    dims_t d = {hq, hkv, dqk, dv, ORACLE_GA, 0, (double)scale, (double)value_scale};
    pages_t pg = {block_table, max_blocks, page_size, num_pages};
    return decode_fp8_impl(&d, q, k_new, v_new, k_cache, v_cache, NULL, &pg, k_scale, v_scale, ctx_lens, batch,
                           sink, out, lse, nthreads);
}

/* GA chunked prefill whose cached positions are FP8 codes (contiguous pool at
 * kv_base[b] + j, or paged when block_table is non-NULL), read as code * scale;
 * the chunk's own keys and values are bf16 as given. */
static int chunk_fp8_impl(int hq, int hkv, int dqk, int dv, float scale, float value_scale,
                          const uint16_t* q, const uint16_t* k, const uint16_t* v,
                          const int32_t* cu_newlens, int batch, const uint8_t* k_cache, const uint8_t* v_cache,
                          const int64_t* kv_base, const pages_t* pages, const float* k_scale, const float* v_scale,
                          const int32_t* ctx_lens, const float* sink, double* out, double* lse, int nthreads) {
    dims_t d = {hq, hkv, dqk, dv, ORACLE_GA, 0, (double)scale, (double)value_scale};
    if (!k_cache || !v_cache || !scales_ok(k_scale, hkv) || !scales_ok(v_scale, hkv)) return ORACLE_EINVAL;
    chunk_fp8_t f8 = {k_cache, v_cache, k_scale, v_scale};
    return chunk_impl(&d, q, k, v, cu_newlens, batch, NULL, NULL, 0, kv_base, pages, &f8, ctx_lens, sink, out, lse,
                      nthreads);
}

int oracle_prefill_chunk_fp8(int hq, int hkv, int dqk, int dv, float scale, float value_scale,
                             const uint16_t* q, const uint16_t* k, const uint16_t* v,
                             const int32_t* cu_newlens, int batch, const uint8_t* k_cache, const uint8_t* v_cache,
                             const int64_t* kv_base, const float* k_scale, const float* v_scale,
                             const int32_t* ctx_lens, const float* sink, double* out, double* lse, int nthreads) {
    if (!kv_base) return ORACLE_EINVAL;
    return chunk_fp8_impl(hq, hkv, dqk, dv, scale, value_scale, q, k, v, cu_newlens, batch, k_cache, v_cache,
                          kv_base, NULL, k_scale, v_scale, ctx_lens, sink, out, lse, nthreads);
}

int oracle_prefill_chunk_fp8_paged(int hq, int hkv, int dqk, int dv, float scale, float value_scale,
                                   const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                   const int32_t* cu_newlens, int batch, const uint8_t* k_cache,
                                   const uint8_t* v_cache, const int32_t* block_table, int max_blocks,
                                   int page_size, int64_t num_pages, const float* k_scale, const float* v_scale,
                                   const int32_t* ctx_lens, const float* sink, double* out, double* lse,
                                   int nthreads) {
    pages_t pg = {block_table, max_blocks, page_size, num_pages};
    return chunk_fp8_impl(hq, hkv, dqk, dv, scale, value_scale, q, k, v, cu_newlens, batch, k_cache, v_cache, NULL,
                          &pg, k_scale, v_scale, ctx_lens, sink, out, lse, nthreads);
}

/* KV append into an FP8 GA pool: as oracle_kv_append for GA (rows kv_base[b]
 * + position, a sequence past its capacity skipped whole with
 * ORACLE_ECAPACITY), each element stored as its E4M3 code under the scale of
 * its KV head. */
static int kv_append_fp8_impl(int hkv, int dqk, int dv, const uint16_t* k, const uint16_t* v,
                              const int32_t* cu_newlens, const int32_t* ctx_lens, int batch,
                              uint8_t* k_cache, uint8_t* v_cache, const int64_t* kv_base, const int64_t* kv_capacity,
                              const pages_t* pages, const float* k_scale, const float* v_scale) {
    if (hkv <= 0 || dqk <= 0 || dv <= 0 || batch < 1 || !k || !v || !cu_newlens || !ctx_lens || !k_cache ||
        !v_cache || !scales_ok(k_scale, hkv) || !scales_ok(v_scale, hkv))
        return ORACLE_EINVAL;
    if (pages ? (!pages->table || pages->max_blocks < 1 || pages->page_size < 1 || pages->num_pages < 1)
              : (!kv_base || !kv_capacity))
        return ORACLE_EINVAL;
    int status = ORACLE_OK;
    for (int b = 0; b < batch; ++b) {
        int n = cu_newlens[b + 1] - cu_newlens[b];
        if (n < 0) return ORACLE_EINVAL;
        int64_t room = pages ? (int64_t)pages->max_blocks * pages->page_size : kv_capacity[b];
        if ((int64_t)ctx_lens[b] + n > room) {
            status = ORACLE_ECAPACITY;
            continue;
        }
        for (int i = 0; i < n; ++i) {
            size_t src = (size_t)cu_newlens[b] + i;
            int64_t pos = (int64_t)ctx_lens[b] + i;
            size_t dst;
            if (pages) {
                int32_t page = pages->table[(size_t)b * pages->max_blocks + (size_t)(pos / pages->page_size)];
                if (page < 0 || page >= pages->num_pages) {
                    status = ORACLE_ECAPACITY;
                    continue;
                }
                dst = (size_t)paged_row(pages, b, pos);
            } else {
                dst = (size_t)(kv_base[b] + pos);
            }
            for (int g = 0; g < hkv; ++g) {
                for (int x = 0; x < dqk; ++x)
                    k_cache[(dst * hkv + g) * dqk + x] = e4m3_quantize(k[(src * hkv + g) * dqk + x], k_scale[g]);
                for (int x = 0; x < dv; ++x)
                    v_cache[(dst * hkv + g) * dv + x] = e4m3_quantize(v[(src * hkv + g) * dv + x], v_scale[g]);
            }
        }
    }
    return status;
}

int oracle_kv_append_fp8(int hkv, int dqk, int dv, const uint16_t* k, const uint16_t* v,
                         const int32_t* cu_newlens, const int32_t* ctx_lens, int batch,
                         uint8_t* k_cache, uint8_t* v_cache, const int64_t* kv_base, const int64_t* kv_capacity,
                         const float* k_scale, const float* v_scale) {
    return kv_append_fp8_impl(hkv, dqk, dv, k, v, cu_newlens, ctx_lens, batch, k_cache, v_cache, kv_base,
                              kv_capacity, NULL, k_scale, v_scale);
}

/* KV append into a paged FP8 GA pool: the codes as oracle_kv_append_fp8, the
 * rows, refusals and ORACLE_ECAPACITY as oracle_kv_append_paged. */
int oracle_kv_append_fp8_paged(int hkv, int dqk, int dv, const uint16_t* k, const uint16_t* v,
                               const int32_t* cu_newlens, const int32_t* ctx_lens, int batch,
                               uint8_t* k_cache, uint8_t* v_cache,
                               const int32_t* block_table, int max_blocks, int page_size, int64_t num_pages,
                               const float* k_scale, const float* v_scale) {
    pages_t pg = {block_table, max_blocks, page_size, num_pages};
    return kv_append_fp8_impl(hkv, dqk, dv, k, v, cu_newlens, ctx_lens, batch, k_cache, v_cache, NULL, NULL, &pg,
                              k_scale, v_scale);
}

/* The E4M3 codec on its own (for the pins): codes of n floats, values of n codes. */
void oracle_e4m3_encode(const float* x, uint8_t* codes, int64_t n) {
    for (int64_t i = 0; i < n; ++i) codes[i] = e4m3_from_float(x[i]);
}

void oracle_e4m3_decode(const uint8_t* codes, double* x, int64_t n) {
    for (int64_t i = 0; i < n; ++i) x[i] = e4m3_to_double(codes[i]);
}

/* Number of oracle worker threads a caller gets with nthreads <= 0. */
int oracle_default_threads(void) {
    long n = 1;
#ifdef _SC_NPROCESSORS_ONLN
    n = sysconf(_SC_NPROCESSORS_ONLN);
#endif
    return n > 0 ? (int)n : 1;
}
