/*
 * Paged GQA decode attention: plain fp64 CPU oracle.
 *
 * TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check and the
 * benchmark's CPU-baseline leg load this file's library. It shares no code,
 * header or constant with the HIP library, and the HIP library never calls it.
 *
 * What it computes (Loom Kernels home page, "Supported now": paged MQA/GQA
 * decode with GQA packing and local split-K/LSE; the split-K/LSE path is an
 * exact regrouping of the same softmax, so the oracle is the plain
 * definition). For every sequence b and query head h:
 *
 *   g   = h / (Hq / Hkv)                          consecutive GQA grouping
 *   L   = context_lens[b]
 *   for t in [0, L):
 *       blk = block_table[b][t / bs], off = t % bs
 *       k_t = K[blk][off][g][:],  v_t = V[blk][off][g][:]   (exact widening)
 *       s_t = scale * sum_d q[b][h][d] * k_t[d]
 *   m   = max_t s_t,  Z = sum_t exp(s_t - m)
 *   out = sum_t exp(s_t - m) * v_t / Z,   lse = m + ln Z
 *
 * with L = 0 giving out = 0 and lse = -inf. Everything is fp64 over the
 * 16-bit inputs widened exactly; nothing is rounded until pdo_round is
 * asked to. Loops run in plain logical token order; there is no blocking,
 * fusion or reordering.
 *
 * Split-K/LSE (same page, "split-K/LSE"): partition p of a sequence covers
 * tokens [p*P, min((p+1)*P, L)). Each non-empty partition gives its own
 * (o_p, lse_p) from the definition above restricted to its tokens; the merge
 * over the n = ceil(L/P) non-empty partitions is
 *   M = max_p lse_p,  w_p = exp(lse_p - M),  out = sum_p w_p o_p / sum_p w_p
 * taken in order p = 0..n-1.
 *
 * FP8 cache (Loom Kernels home page, "Next boundaries": FP8 KV-cache
 * compression): K and V hold OCP FP8 E4M3FN codes with one float32 scale per
 * tensor; the value of a code c is decode(c) * scale, widened exactly, and
 * everything else is the definition above.
 *
 * Status codes: 0 ok, -1 bad shape, -2 a live block id outside the pool,
 * -3 a context length outside [0, max_blocks_per_seq * block_size],
 * -4 out of memory, -5 bad dtype.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <unistd.h>

enum { PDO_F16 = 0, PDO_BF16 = 1 };

/* IEEE 754 binary16: 1 sign, 5 exponent (bias 15), 10 fraction bits. */
static double widen_f16(uint16_t b) {
    int s = b >> 15, e = (b >> 10) & 0x1f, f = b & 0x3ff;
    double v;
    if (e == 0) v = ldexp((double)f, -24);
    else if (e == 31) v = f ? NAN : INFINITY;
    else v = ldexp((double)(1024 + f), e - 25);
    return s ? -v : v;
}

/* bfloat16: 1 sign, 8 exponent (bias 127), 7 fraction bits. */
static double widen_bf16(uint16_t b) {
    int s = b >> 15, e = (b >> 7) & 0xff, f = b & 0x7f;
    double v;
    if (e == 0) v = ldexp((double)f, -133);
    else if (e == 255) v = f ? NAN : INFINITY;
    else v = ldexp((double)(128 + f), e - 134);
    return s ? -v : v;
}

static double widen(uint16_t b, int dtype) {
    return dtype == PDO_BF16 ? widen_bf16(b) : widen_f16(b);
}

/* OCP 8-bit floating point, E4M3FN: 1 sign, 4 exponent (bias 7), 3 fraction
 * bits; no infinities; exponent and fraction all ones is NaN, so the largest
 * finite magnitude is 1.75 * 2^8 = 448; exponent 0 is subnormal (f * 2^-9). */
static double widen_e4m3(uint8_t b) {
    int s = b >> 7, e = (b >> 3) & 0xf, f = b & 7;
    double v;
    if (e == 15 && f == 7) return NAN;
    if (e == 0) v = ldexp((double)f, -9);
    else v = ldexp((double)(8 + f), e - 10);
    return s ? -v : v;
}

void pdo_widen_fp8(const uint8_t* x, int64_t n, double* out) {
    for (int64_t i = 0; i < n; ++i) out[i] = widen_e4m3(x[i]);
}

void pdo_widen(const uint16_t* x, int64_t n, int32_t dtype, double* out) {
    for (int64_t i = 0; i < n; ++i) out[i] = widen(x[i], dtype);
}

/* Round-to-nearest-even from fp64 straight to the 16-bit format: one rounding.
 * p = significand bits (with the implicit one), emin = least normal exponent,
 * bias = exponent bias, ebits = exponent field width. */
static uint16_t round_one(double x, int dtype) {
    const int p = dtype == PDO_BF16 ? 8 : 11;
    const int emin = dtype == PDO_BF16 ? -126 : -14;
    const int bias = dtype == PDO_BF16 ? 127 : 15;
    const int ebits = dtype == PDO_BF16 ? 8 : 5;
    const int fbits = p - 1;
    const uint16_t sign = signbit(x) ? (uint16_t)(1u << 15) : 0;
    const uint16_t expmax = (uint16_t)((1u << ebits) - 1);
    if (isnan(x)) return (uint16_t)(sign | (expmax << fbits) | (1u << (fbits - 1)));
    double a = fabs(x);
    if (isinf(a)) return (uint16_t)(sign | (expmax << fbits));
    if (a == 0.0) return sign;
    int e = ilogb(a);
    if (e < emin) e = emin;               /* subnormal range: fixed quantum */
    int qe = e - fbits;                   /* exponent of one unit in the last place */
    double r = nearbyint(ldexp(a, -qe));  /* exact scaling; RNE in the default mode */
    if (r >= ldexp(1.0, p)) { r = ldexp(1.0, fbits); qe += 1; }
    uint32_t ir = (uint32_t)r;
    uint32_t field;
    uint32_t frac;
    if (ir < (1u << fbits)) {             /* subnormal (or rounded to zero) */
        field = 0;
        frac = ir;
    } else {
        field = (uint32_t)(qe + fbits + bias);
        frac = ir - (1u << fbits);
        if (field >= expmax) return (uint16_t)(sign | (expmax << fbits));  /* overflow */
    }
    return (uint16_t)(sign | (field << fbits) | frac);
}

void pdo_round(const double* x, int64_t n, int32_t dtype, uint16_t* out) {
    for (int64_t i = 0; i < n; ++i) out[i] = round_one(x[i], dtype);
}

typedef struct {
    const uint16_t *q, *k, *v;
    const uint8_t *k8, *v8;  /* FP8 codes instead of k, v when non-null */
    double k_scale, v_scale;
    const int32_t *bt, *cl;
    int32_t B, Hq, Hkv, D, bs, MB;
    int64_t num_blocks;
    double scale;
    int32_t dtype;
    int32_t P, S;          /* partition tokens and count; P = 0 means one pass */
    double *out, *lse;     /* [B,Hq,D] / [B,Hq], or [B,Hq,S,D] / [B,Hq,S] when P > 0 */
    int32_t nthreads;
    int32_t status;
    pthread_mutex_t lock;
} job_t;

typedef struct { job_t* job; int tid; } worker_t;

/* Attention of query (b, h) over tokens [t0, t1) of its sequence.
 * s is scratch of at least t1 - t0 doubles. Returns 0 or -2. */
static int attend(const job_t* J, int b, int h, int t0, int t1, double* s,
                  double* o, double* lse) {
    const int G = J->Hq / J->Hkv;
    const int g = h / G;
    const int D = J->D;
    const uint16_t* qh = J->q + ((int64_t)b * J->Hq + h) * D;
    if (t1 <= t0) {
        for (int d = 0; d < D; ++d) o[d] = 0.0;
        *lse = -INFINITY;
        return 0;
    }
    /* scores */
    for (int t = t0; t < t1; ++t) {
        int32_t blk = J->bt[(int64_t)b * J->MB + t / J->bs];
        if (blk < 0 || blk >= J->num_blocks) return -2;
        const int64_t row = (((int64_t)blk * J->bs + t % J->bs) * J->Hkv + g) * D;
        double dot = 0.0;
        if (J->k8) {
            for (int d = 0; d < D; ++d)
                dot += widen(qh[d], J->dtype) * (widen_e4m3(J->k8[row + d]) * J->k_scale);
        } else {
            for (int d = 0; d < D; ++d) dot += widen(qh[d], J->dtype) * widen(J->k[row + d], J->dtype);
        }
        s[t - t0] = J->scale * dot;
    }
    double m = -INFINITY;
    for (int t = t0; t < t1; ++t) if (s[t - t0] > m) m = s[t - t0];
    double Z = 0.0;
    for (int t = t0; t < t1; ++t) Z += exp(s[t - t0] - m);
    for (int d = 0; d < D; ++d) o[d] = 0.0;
    for (int t = t0; t < t1; ++t) {
        int32_t blk = J->bt[(int64_t)b * J->MB + t / J->bs];
        const int64_t row = (((int64_t)blk * J->bs + t % J->bs) * J->Hkv + g) * D;
        double w = exp(s[t - t0] - m);
        if (J->v8) {
            for (int d = 0; d < D; ++d) o[d] += w * (widen_e4m3(J->v8[row + d]) * J->v_scale);
        } else {
            for (int d = 0; d < D; ++d) o[d] += w * widen(J->v[row + d], J->dtype);
        }
    }
    for (int d = 0; d < D; ++d) o[d] /= Z;
    *lse = m + log(Z);
    return 0;
}

static void* run_worker(void* arg) {
    worker_t* W = (worker_t*)arg;
    job_t* J = W->job;
    int ctx_cap = J->MB * J->bs;
    double* s = (double*)malloc(sizeof(double) * (size_t)(ctx_cap > 0 ? ctx_cap : 1));
    int err = s ? 0 : -4;
    int64_t pairs = (int64_t)J->B * J->Hq;
    for (int64_t i = W->tid; i < pairs && !err; i += J->nthreads) {
        int b = (int)(i / J->Hq), h = (int)(i % J->Hq);
        int L = J->cl[b];
        if (J->P <= 0) {
            err = attend(J, b, h, 0, L, s, J->out + i * J->D, J->lse + i);
        } else {
            for (int p = 0; p < J->S && !err; ++p) {
                int t0 = p * J->P;
                int t1 = t0 + J->P < L ? t0 + J->P : L;
                int64_t slot = i * J->S + p;
                err = attend(J, b, h, t0, t1, s, J->out + slot * J->D, J->lse + slot);
            }
        }
    }
    free(s);
    if (err) {
        pthread_mutex_lock(&J->lock);
        if (!J->status) J->status = err;
        pthread_mutex_unlock(&J->lock);
    }
    return NULL;
}

static int run(job_t* J) {
    if (J->B < 0 || J->Hq <= 0 || J->Hkv <= 0 || J->D <= 0 || J->bs <= 0 || J->MB < 0 ||
        J->Hq % J->Hkv != 0 || J->num_blocks < 0)
        return -1;
    if (J->dtype != PDO_F16 && J->dtype != PDO_BF16) return -5;
    for (int b = 0; b < J->B; ++b)
        if (J->cl[b] < 0 || (int64_t)J->cl[b] > (int64_t)J->MB * J->bs) return -3;
    if (J->P > 0) {
        for (int b = 0; b < J->B; ++b)
            if ((int64_t)J->S * J->P < J->cl[b]) return -1;
    }
    int nt = J->nthreads;
    if (nt <= 0) nt = (int)sysconf(_SC_NPROCESSORS_ONLN);
    if (nt < 1) nt = 1;
    int64_t pairs = (int64_t)J->B * J->Hq;
    if (nt > pairs) nt = pairs > 0 ? (int)pairs : 1;
    J->nthreads = nt;
    J->status = 0;
    pthread_mutex_init(&J->lock, NULL);
    pthread_t* th = (pthread_t*)malloc(sizeof(pthread_t) * (size_t)nt);
    worker_t* ws = (worker_t*)malloc(sizeof(worker_t) * (size_t)nt);
    if (!th || !ws) { free(th); free(ws); return -4; }
    for (int i = 0; i < nt; ++i) {
        ws[i].job = J;
        ws[i].tid = i;
        if (i > 0) pthread_create(&th[i], NULL, run_worker, &ws[i]);
    }
    run_worker(&ws[0]);
    for (int i = 1; i < nt; ++i) pthread_join(th[i], NULL);
    free(th);
    free(ws);
    pthread_mutex_destroy(&J->lock);
    return J->status;
}

/* Single pass: out [B,Hq,D] and lse [B,Hq] in fp64. nthreads <= 0 uses every
 * online core. Returns the number of threads used (> 0) or a status (< 0). */
int32_t pdo_attention(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                      const int32_t* block_table, const int32_t* context_lens,
                      int32_t B, int32_t Hq, int32_t Hkv, int32_t D, int32_t block_size,
                      int32_t max_blocks_per_seq, int64_t num_blocks, double scale,
                      int32_t dtype, double* out, double* lse, int32_t nthreads) {
    job_t J;
    memset(&J, 0, sizeof J);
    J.q = q; J.k = k; J.v = v; J.bt = block_table; J.cl = context_lens;
    J.B = B; J.Hq = Hq; J.Hkv = Hkv; J.D = D; J.bs = block_size; J.MB = max_blocks_per_seq;
    J.num_blocks = num_blocks; J.scale = scale; J.dtype = dtype;
    J.P = 0; J.S = 1; J.out = out; J.lse = lse; J.nthreads = nthreads;
    int st = run(&J);
    return st ? st : J.nthreads;
}

/* Per-partition results: o_part [B,Hq,S,D] and lse_part [B,Hq,S], partition
 * p covering tokens [p*P, min((p+1)*P, L)); empty partitions give o = 0,
 * lse = -inf. Requires S*P >= every context length. */
int32_t pdo_partials(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                     const int32_t* block_table, const int32_t* context_lens,
                     int32_t B, int32_t Hq, int32_t Hkv, int32_t D, int32_t block_size,
                     int32_t max_blocks_per_seq, int64_t num_blocks, double scale,
                     int32_t dtype, int32_t P, int32_t S,
                     double* o_part, double* lse_part, int32_t nthreads) {
    if (P <= 0 || S <= 0) return -1;
    job_t J;
    memset(&J, 0, sizeof J);
    J.q = q; J.k = k; J.v = v; J.bt = block_table; J.cl = context_lens;
    J.B = B; J.Hq = Hq; J.Hkv = Hkv; J.D = D; J.bs = block_size; J.MB = max_blocks_per_seq;
    J.num_blocks = num_blocks; J.scale = scale; J.dtype = dtype;
    J.P = P; J.S = S; J.out = o_part; J.lse = lse_part; J.nthreads = nthreads;
    int st = run(&J);
    return st ? st : J.nthreads;
}

/* LSE merge of the n = ceil(L/P) non-empty partitions of each (b, h). */
int32_t pdo_merge(const double* o_part, const double* lse_part, const int32_t* context_lens,
                  int32_t B, int32_t Hq, int32_t S, int32_t D, int32_t P, double* out) {
    if (P <= 0 || S <= 0 || B < 0 || Hq <= 0 || D <= 0) return -1;
    for (int b = 0; b < B; ++b) {
        int L = context_lens[b];
        if (L < 0 || (int64_t)S * P < L) return -3;
        int n = (L + P - 1) / P;
        for (int h = 0; h < Hq; ++h) {
            int64_t i = (int64_t)b * Hq + h;
            double* o = out + i * D;
            for (int d = 0; d < D; ++d) o[d] = 0.0;
            if (n == 0) continue;
            double M = -INFINITY;
            for (int p = 0; p < n; ++p) if (lse_part[i * S + p] > M) M = lse_part[i * S + p];
            double W = 0.0;
            for (int p = 0; p < n; ++p) {
                double w = exp(lse_part[i * S + p] - M);
                W += w;
                const double* op = o_part + (i * S + p) * D;
                for (int d = 0; d < D; ++d) o[d] += w * op[d];
            }
            for (int d = 0; d < D; ++d) o[d] /= W;
        }
    }
    return 0;
}

/* pdo_attention / pdo_partials over an FP8 E4M3FN cache: k8, v8 hold byte
 * codes in the same [num_blocks, block_size, Hkv, D] layout; q (and the
 * dtype argument) stay 16-bit. */
int32_t pdo_attention_fp8kv(const uint16_t* q, const uint8_t* k8, const uint8_t* v8,
                            const int32_t* block_table, const int32_t* context_lens,
                            int32_t B, int32_t Hq, int32_t Hkv, int32_t D, int32_t block_size,
                            int32_t max_blocks_per_seq, int64_t num_blocks, double scale,
                            int32_t dtype, double k_scale, double v_scale, double* out,
                            double* lse, int32_t nthreads) {
    job_t J;
    memset(&J, 0, sizeof J);
    J.q = q; J.k8 = k8; J.v8 = v8; J.k_scale = k_scale; J.v_scale = v_scale;
    J.bt = block_table; J.cl = context_lens;
    J.B = B; J.Hq = Hq; J.Hkv = Hkv; J.D = D; J.bs = block_size; J.MB = max_blocks_per_seq;
    J.num_blocks = num_blocks; J.scale = scale; J.dtype = dtype;
    J.P = 0; J.S = 1; J.out = out; J.lse = lse; J.nthreads = nthreads;
    if (!k8 || !v8) return -1;
    int st = run(&J);
    return st ? st : J.nthreads;
}

int32_t pdo_partials_fp8kv(const uint16_t* q, const uint8_t* k8, const uint8_t* v8,
                           const int32_t* block_table, const int32_t* context_lens,
                           int32_t B, int32_t Hq, int32_t Hkv, int32_t D, int32_t block_size,
                           int32_t max_blocks_per_seq, int64_t num_blocks, double scale,
                           int32_t dtype, double k_scale, double v_scale, int32_t P, int32_t S,
                           double* o_part, double* lse_part, int32_t nthreads) {
    if (P <= 0 || S <= 0 || !k8 || !v8) return -1;
    job_t J;
    memset(&J, 0, sizeof J);
    J.q = q; J.k8 = k8; J.v8 = v8; J.k_scale = k_scale; J.v_scale = v_scale;
    J.bt = block_table; J.cl = context_lens;
    J.B = B; J.Hq = Hq; J.Hkv = Hkv; J.D = D; J.bs = block_size; J.MB = max_blocks_per_seq;
    J.num_blocks = num_blocks; J.scale = scale; J.dtype = dtype;
    J.P = P; J.S = S; J.out = o_part; J.lse = lse_part; J.nthreads = nthreads;
    int st = run(&J);
    return st ? st : J.nthreads;
}
