/*
 * ftm_oracle.c -- plain CPU reference for one decode step of masked
 * multi-head attention over a KV cache.  TEST INFRASTRUCTURE ONLY (see the
 * header): only the tests, the smoke check and the benchmark's CPU baseline
 * use it; the GPU library neither links nor calls it.
 *
 * Build: gcc -O2 -fno-fast-math -ffp-contract=off -shared -fPIC -pthread
 * (no contraction of a*b+c into fma, IEEE division, default rounding mode).
 *
 * The method is exact attention computed in a single fused pass; its result
 * has a plain definition, and this file is that definition written out:
 * append, then softmax(q.K^T / sqrt(D)) V per query head, nothing blocked,
 * fused or reordered.
 */
#include "ftm_oracle.h"

#include <math.h>
#include <pthread.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------ */
/* Number formats (IEEE 754 binary16; bfloat16 = top half of binary32). */
/* ------------------------------------------------------------------ */

/* Decode a binary floating-point bit pattern with the given exponent and
 * fraction widths, straight from the definition:
 *   exponent field 0      -> subnormal: (-1)^s * f * 2^(1 - bias - fbits)
 *   exponent field all 1s -> inf (f == 0) or NaN
 *   otherwise             -> (-1)^s * (1 + f / 2^fbits) * 2^(e - bias)     */
static double decode_binary(uint32_t bits, int ebits, int fbits) {
    const uint32_t fmask = (1u << fbits) - 1u;
    const uint32_t emask = (1u << ebits) - 1u;
    const int bias = (1 << (ebits - 1)) - 1;
    const int sign = (bits >> (ebits + fbits)) & 1u;
    const uint32_t e = (bits >> fbits) & emask;
    const uint32_t f = bits & fmask;
    double v;
    if (e == 0) {
        v = ldexp((double)f, 1 - bias - fbits);
    } else if (e == emask) {
        v = (f == 0) ? INFINITY : NAN;
    } else {
        v = ldexp(1.0 + ldexp((double)f, -fbits), (int)e - bias);
    }
    return sign ? -v : v;
}

double orc_f16_bits_to_double(uint16_t bits) { return decode_binary(bits, 5, 10); }
double orc_bf16_bits_to_double(uint16_t bits) { return decode_binary(bits, 8, 7); }

/* Round a finite or infinite value to a binary format of ebits/fbits with
 * round-to-nearest-even, then encode it.  The rounding is done on the exact
 * value: the spacing of representable numbers at |x| is
 * 2^(max(floor(log2|x|), emin) - fbits); x / spacing is an exact double
 * (x has at most 24 significant bits), rint() rounds it half-to-even in the
 * default rounding mode, and anything that rounds to 2^(emax+1) or beyond
 * overflows to infinity.  NaN maps to a quiet NaN with the sign kept. */
static uint32_t encode_binary_rne(double x, int ebits, int fbits) {
    const int bias = (1 << (ebits - 1)) - 1;
    const int emin = 1 - bias;
    const int emax = bias;
    const uint32_t emask = (1u << ebits) - 1u;
    const uint32_t sign = signbit(x) ? 1u : 0u;
    const uint32_t sbit = sign << (ebits + fbits);
    if (isnan(x)) return sbit | (emask << fbits) | (1u << (fbits - 1));
    double a = fabs(x);
    if (isinf(a)) return sbit | (emask << fbits);
    if (a == 0.0) return sbit;
    int e2;
    frexp(a, &e2);          /* a = m * 2^e2, m in [0.5, 1): floor(log2 a) = e2 - 1 */
    int e = e2 - 1;
    if (e < emin) e = emin;
    const double spacing = ldexp(1.0, e - fbits);
    const double r = rint(a / spacing) * spacing;   /* exact, ties to even */
    if (r >= ldexp(1.0, emax + 1)) return sbit | (emask << fbits);
    if (r == 0.0) return sbit;               /* underflow to a signed zero */
    /* encode the representable value r */
    frexp(r, &e2);
    int er = e2 - 1;
    if (er < emin) {                         /* subnormal */
        const uint32_t f = (uint32_t)(r / ldexp(1.0, emin - fbits));
        return sbit | f;
    }
    const uint32_t f = (uint32_t)((r / ldexp(1.0, er) - 1.0) * ldexp(1.0, fbits));
    return sbit | ((uint32_t)(er + bias) << fbits) | f;
}

uint16_t orc_float_to_f16_rne(float x) { return (uint16_t)encode_binary_rne((double)x, 5, 10); }
uint16_t orc_float_to_bf16_rne(float x) { return (uint16_t)encode_binary_rne((double)x, 8, 7); }

/* ------------------------------------------------------------------ */
/* INT8 KV cache ([pptc.cn/news/144085] section 3.1: K and V kept as INT8;
 * [intelliparadigm.com .../2131745] section 2.1: converted back when used).
 * Reading taken: symmetric, one fp32 scale per (K or V, sequence, KV head,
 * position) equal to absmax/127; codes rounded half-to-even and clamped to
 * [-127, 127]; a zero row gets scale 0 and zero codes.  All in fp32.      */
/* ------------------------------------------------------------------ */
float orc_quantize_row_i8(const float* x, int n, int8_t* codes) {
    float amax = 0.0f;
    for (int d = 0; d < n; ++d) {
        const float ax = fabsf(x[d]);
        if (ax > amax) amax = ax;
    }
    const float scale = amax / 127.0f;
    for (int d = 0; d < n; ++d) {
        if (scale == 0.0f) {
            codes[d] = 0;
            continue;
        }
        float c = rintf(x[d] / scale);
        if (c > 127.0f) c = 127.0f;
        if (c < -127.0f) c = -127.0f;
        codes[d] = (int8_t)c;
    }
    return scale;
}

/* ------------------------------------------------------------------ */
/* Element access.                                                      */
/* ------------------------------------------------------------------ */
static size_t elem_size(int dt) {
    switch (dt) {
    case ORC_F32: return 4;
    case ORC_F16: return 2;
    case ORC_BF16: return 2;
    case ORC_I8: return 1;
    default: return 0;
    }
}

/* Activation element i as fp32 (exact: every act type widens exactly). */
static float act_get_f32(const void* base, size_t i, int act_dt) {
    if (act_dt == ORC_F32) return ((const float*)base)[i];
    if (act_dt == ORC_F16) return (float)orc_f16_bits_to_double(((const uint16_t*)base)[i]);
    return (float)orc_bf16_bits_to_double(((const uint16_t*)base)[i]);
}

/* Stored cache element as an exact double (INT8: code times its scale). */
static double cache_get(const void* base, size_t i, int kv_dt, double scale) {
    switch (kv_dt) {
    case ORC_F32: return (double)((const float*)base)[i];
    case ORC_F16: return orc_f16_bits_to_double(((const uint16_t*)base)[i]);
    case ORC_BF16: return orc_bf16_bits_to_double(((const uint16_t*)base)[i]);
    default: return (double)((const int8_t*)base)[i] * scale;
    }
}

/* ------------------------------------------------------------------ */
/* The step.                                                            */
/* ------------------------------------------------------------------ */
typedef struct {
    const void* q;
    const void* k_new;
    const void* v_new;
    const void* bias;
    void* k_cache;
    void* v_cache;
    const int32_t* seq_lens;
    int B, Lmax, step, H, Hkv, D, kv_dt, act_dt;
    float* kv_scales;
    double* out;
    double* probs;
} Problem;

/* Append the biased new row of one (sequence b, KV head j) at position p.
 * [lpnh.cn/news/2765398] section 2.1 (bias added to the split Q/K/V) and
 * section 2.2 (new K/V appended to the pre-allocated cache).
 * x = fl32(new + bias) in fp32; stored as fp32, as the RNE binary16/bfloat16
 * value, or as INT8 codes with their scale. */
static void append_row(const Problem* P, int b, int j, int p, int which /*0 K, 1 V*/) {
    const int D = P->D;
    const void* src = which == 0 ? P->k_new : P->v_new;
    void* cache = which == 0 ? P->k_cache : P->v_cache;
    const size_t src_off = ((size_t)b * P->Hkv + j) * D;
    const size_t bias_off = (size_t)(P->H + which * P->Hkv + j) * D;
    const size_t row = (((size_t)b * P->Hkv + j) * P->Lmax + p) * D;
    float* x = (float*)malloc(sizeof(float) * D);
    for (int d = 0; d < D; ++d) {
        const float a = act_get_f32(src, src_off + d, P->act_dt);
        /* one fp32 rounding; with no bias the row is stored as given */
        x[d] = P->bias ? a + act_get_f32(P->bias, bias_off + d, P->act_dt) : a;
    }
    switch (P->kv_dt) {
    case ORC_F32:
        for (int d = 0; d < D; ++d) ((float*)cache)[row + d] = x[d];
        break;
    case ORC_F16:
        for (int d = 0; d < D; ++d) ((uint16_t*)cache)[row + d] = orc_float_to_f16_rne(x[d]);
        break;
    case ORC_BF16:
        for (int d = 0; d < D; ++d) ((uint16_t*)cache)[row + d] = orc_float_to_bf16_rne(x[d]);
        break;
    default: {
        const float s = orc_quantize_row_i8(x, D, (int8_t*)cache + row);
        const size_t sidx = (((size_t)which * P->B + b) * P->Hkv + j) * P->Lmax + p;
        P->kv_scales[sidx] = s;
        break;
    }
    }
    free(x);
}

/* Attention of query head h of sequence b over positions [0, L).
 * s_i = (q^ . K^_i) / sqrt(D);  m = max s_i;  w_i = exp(s_i - m);
 * p_i = w_i / sum w;  out = sum p_i V^_i.                               */
static void attend_head(const Problem* P, int b, int h, int L) {
    const int D = P->D;
    const int G = P->H / P->Hkv;
    const int j = h / G;   /* contiguous groups: query head h reads KV head floor(h/G) */
    const size_t kv_base = ((size_t)b * P->Hkv + j) * (size_t)P->Lmax;
    double* qh = (double*)malloc(sizeof(double) * D);
    double* s = (double*)malloc(sizeof(double) * L);
    for (int d = 0; d < D; ++d) {
        double v = (double)act_get_f32(P->q, ((size_t)b * P->H + h) * D + d, P->act_dt);
        if (P->bias) v += (double)act_get_f32(P->bias, (size_t)h * D + d, P->act_dt);
        qh[d] = v;
    }
    const double inv_sqrt_d = 1.0 / sqrt((double)D);
    for (int i = 0; i < L; ++i) {
        double ks = 1.0;
        if (P->kv_dt == ORC_I8)
            ks = (double)P->kv_scales[(((size_t)0 * P->B + b) * P->Hkv + j) * P->Lmax + i];
        double acc = 0.0;
        for (int d = 0; d < D; ++d)
            acc += qh[d] * cache_get(P->k_cache, (kv_base + i) * D + d, P->kv_dt, ks);
        s[i] = acc * inv_sqrt_d;
    }
    double m = -INFINITY;
    for (int i = 0; i < L; ++i)
        if (s[i] > m) m = s[i];
    double z = 0.0;
    for (int i = 0; i < L; ++i) {
        s[i] = exp(s[i] - m);
        z += s[i];
    }
    for (int i = 0; i < L; ++i) s[i] /= z;
    double* o = P->out + ((size_t)b * P->H + h) * D;
    for (int d = 0; d < D; ++d) o[d] = 0.0;
    for (int i = 0; i < L; ++i) {
        double vs = 1.0;
        if (P->kv_dt == ORC_I8)
            vs = (double)P->kv_scales[(((size_t)1 * P->B + b) * P->Hkv + j) * P->Lmax + i];
        for (int d = 0; d < D; ++d)
            o[d] += s[i] * cache_get(P->v_cache, (kv_base + i) * D + d, P->kv_dt, vs);
    }
    if (P->probs) {
        double* pr = P->probs + ((size_t)b * P->H + h) * P->step;
        for (int i = 0; i < P->step; ++i) pr[i] = i < L ? s[i] : 0.0;
    }
    free(qh);
    free(s);
}

/* One unit of work: sequence b, KV head j, and the G query heads it serves. */
static void run_unit(const Problem* P, int b, int j) {
    const int G = P->H / P->Hkv;
    const int L = P->seq_lens ? P->seq_lens[b] : P->step;
    if (L < 1 || L > P->step) {
        for (int g = 0; g < G; ++g) {
            const int h = j * G + g;
            double* o = P->out + ((size_t)b * P->H + h) * P->D;
            for (int d = 0; d < P->D; ++d) o[d] = NAN;
            if (P->probs) {
                double* pr = P->probs + ((size_t)b * P->H + h) * P->step;
                for (int i = 0; i < P->step; ++i) pr[i] = NAN;
            }
        }
        return;
    }
    append_row(P, b, j, L - 1, 0);
    append_row(P, b, j, L - 1, 1);
    for (int g = 0; g < G; ++g) attend_head(P, b, j * G + g, L);
}

typedef struct {
    const Problem* P;
    int first, stride;
} Worker;

static void* worker_main(void* arg) {
    const Worker* w = (const Worker*)arg;
    const int units = w->P->B * w->P->Hkv;
    for (int u = w->first; u < units; u += w->stride) run_unit(w->P, u / w->P->Hkv, u % w->P->Hkv);
    return NULL;
}

int orc_decode_mha(const void* q, const void* k_new, const void* v_new,
                   const void* qkv_bias, void* k_cache, void* v_cache,
                   const int32_t* seq_lens, int batch, int max_seq_len, int step,
                   int n_heads, int n_kv_heads, int head_dim, int kv_dtype,
                   float* kv_scales, double* out, double* probs, int n_threads) {
    if (!q || !k_new || !v_new || !k_cache || !v_cache || !out) return -1;
    if (batch < 1 || n_heads < 1 || n_kv_heads < 1 || head_dim < 1) return -1;
    if (n_heads % n_kv_heads != 0) return -1;
    if (step < 1 || step > max_seq_len) return -1;
    if (elem_size(kv_dtype) == 0) return -1;
    if ((kv_dtype == ORC_I8) != (kv_scales != NULL)) return -1;
    Problem P;
    P.q = q;
    P.k_new = k_new;
    P.v_new = v_new;
    P.bias = qkv_bias;
    P.k_cache = k_cache;
    P.v_cache = v_cache;
    P.seq_lens = seq_lens;
    P.B = batch;
    P.Lmax = max_seq_len;
    P.step = step;
    P.H = n_heads;
    P.Hkv = n_kv_heads;
    P.D = head_dim;
    P.kv_dt = kv_dtype;
    P.act_dt = kv_dtype == ORC_I8 ? ORC_F16 : kv_dtype;
    P.kv_scales = kv_scales;
    P.out = out;
    P.probs = probs;

    const int units = batch * n_kv_heads;
    int nt = n_threads < 1 ? 1 : n_threads;
    if (nt > units) nt = units;
    if (nt == 1) {
        Worker w = {&P, 0, 1};
        worker_main(&w);
        return 0;
    }
    pthread_t* th = (pthread_t*)malloc(sizeof(pthread_t) * nt);
    Worker* ws = (Worker*)malloc(sizeof(Worker) * nt);
    int started = 0;
    for (int t = 0; t < nt; ++t) {
        ws[t].P = &P;
        ws[t].first = t;
        ws[t].stride = nt;
        if (pthread_create(&th[t], NULL, worker_main, &ws[t]) != 0) break;
        ++started;
    }
    /* if a thread could not start, the calling thread covers its units */
    for (int t = started; t < nt; ++t) worker_main(&ws[t]);
    for (int t = 0; t < started; ++t) pthread_join(th[t], NULL);
    free(th);
    free(ws);
    return 0;
}
