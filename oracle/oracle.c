/*
 * oracle.c -- plain, slow, fp64 CPU oracle for the decode step of one
 * tensor-parallel (TP) shard of a Llama-style decoder block, and for a
 * PaLM-style FFN block held under 2D weight-stationary partitioning.
 *
 * TEST INFRASTRUCTURE. Only the test suite, the package's smoke check and the
 * CPU-baseline leg of the benchmark load this library. The product (the HIP
 * library) never links, calls or includes it, and the two share no source.
 *
 * Build: gcc -O2 -std=c11 -ffp-contract=off -fno-fast-math -fPIC -shared
 * (no FMA contraction, no fast-math: every fp32 step of the int8 codec is one
 * IEEE operation, and fp64 sums are plain left-to-right loops). The same
 * source built with -fopenmp spreads independent output rows, features and
 * heads over the host's threads (the omp pragmas below); every sum keeps its
 * order, so both builds return the same bits. The plain build ignores them.
 *
 * Pages followed (cited by title and the part of the page):
 *  [DL]  distributed-llama issue "[Feature Suggest] Tensor Parallellism for
 *        Accelerating LLM", function buildLlama2Arch: the per-layer task list
 *        of the root node (llamaRmsAttNorm ... llamaMergeFfn2) and of a worker.
 *  [TP]  aiterms.tw "Tensor Parallelism" (張量並行), sections 核心概念 (column /
 *        row / 2D split) and 運作原理 (the two-GPU FFN walk-through: replicated
 *        input, column-split Linear1, elementwise activation, row-split
 *        Linear2, all-reduce of the partial outputs).
 *  [POPE] CS349E lecture 4, 03_pope_partitioning.py: PaLM-540B dims (PALM
 *        record), 2D weight-stationary FFN (demo 1), GQA head sharding note
 *        (demo 3 observations).
 *  [TT]  tt-metal issue "Llama-2 (meta) TT implementation": GQA vs MHA.
 *
 * Where the pages leave a step open, the plainest reading is taken and stated
 * next to the code (eps, RoPE pairing, position of the new token, attention
 * scale, merge = residual + sum of partials, the int8 codec's arithmetic).
 *
 * Parity pins: every function below is checked by the CPU test suite against
 * closed forms, invariants, special cases or float64 library routines.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { ORC_F32 = 0, ORC_BF16 = 1 };
enum { ORC_Q_PARTIALS = 1, ORC_Q_INPUTS = 2 };
#define ORC_QBLOCK 32

/* Threads an OpenMP build uses for its parallel loops (1 for the plain build). */
int orc_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* ---------------------------------------------------------------- storage */

/* exact widening of a stored element (fp32, or bf16 = upper half of an fp32) */
static double ld(const void *p, int dt, int64_t i)
{
    if (dt == ORC_F32)
        return (double)((const float *)p)[i];
    uint32_t u = (uint32_t)((const uint16_t *)p)[i] << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

/* fp32 -> bf16, round to nearest, ties to even (finite values) */
static uint16_t f32_to_bf16(float f)
{
    uint32_t u;
    memcpy(&u, &f, 4);
    if ((u & 0x7f800000u) == 0x7f800000u)            /* inf / nan: keep, quiet nan */
        return (uint16_t)((u >> 16) | ((u & 0xffffu) ? 0x40u : 0u));
    uint32_t lsb = (u >> 16) & 1u;
    return (uint16_t)((u + 0x7fffu + lsb) >> 16);
}

/* store a computed value into a typed buffer: fp64 -> fp32 (C cast, nearest)
 * and, for bf16 buffers, fp32 -> bf16 (nearest-even) */
static void st(void *p, int dt, int64_t i, double v)
{
    float f = (float)v;
    if (dt == ORC_F32)
        ((float *)p)[i] = f;
    else
        ((uint16_t *)p)[i] = f32_to_bf16(f);
}

/* ---------------------------------------------------------------- steps */

/* RMSNorm of one row ([DL] llamaRmsAttNorm / llamaRmfFfn + llamaRmfFfnNorm):
 * y_i = g_i * x_i / sqrt(mean_j x_j^2 + eps). The pages do not give eps; the
 * Llama-2 value 1e-5 is the caller's default. */
void orc_rmsnorm(int64_t D, const double *x, const float *g, double eps, double *y)
{
    double ss = 0.0;
    for (int64_t i = 0; i < D; i++)
        ss += x[i] * x[i];
    double r = 1.0 / sqrt(ss / (double)D + eps);
    for (int64_t i = 0; i < D; i++)
        y[i] = (double)g[i] * x[i] * r;
}

/* Block-wise int8 quantisation of exchanged activations ([DL] llamaQuantize*
 * before each llamaSync*), in fp32 arithmetic, blocks of 32 consecutive
 * elements: scale = max|x| / 127 (one IEEE fp32 division); code =
 * round-half-away-from-zero(x / scale) (one IEEE fp32 division, then roundf),
 * clamped to [-127, 127]; a block whose scale is 0 gets all-zero codes.
 * n must be a multiple of 32. */
void orc_q8_quantize(int64_t n, const float *x, int8_t *codes, float *scales)
{
    for (int64_t b = 0; b < n / ORC_QBLOCK; b++) {
        const float *xb = x + b * ORC_QBLOCK;
        float amax = 0.0f;
        for (int i = 0; i < ORC_QBLOCK; i++) {
            float a = fabsf(xb[i]);
            if (a > amax)
                amax = a;
        }
        float scale = amax / 127.0f;
        scales[b] = scale;
        for (int i = 0; i < ORC_QBLOCK; i++) {
            int8_t q = 0;
            if (scale != 0.0f) {
                float r = roundf(xb[i] / scale);
                if (r > 127.0f)
                    r = 127.0f;
                if (r < -127.0f)
                    r = -127.0f;
                q = (int8_t)r;
            }
            codes[b * ORC_QBLOCK + i] = q;
        }
    }
}

/* Dequantisation ([DL] llamaDequantizeAtt / llamaDequantizeFfn2):
 * y = (float)code * scale, one fp32 multiply. */
void orc_q8_dequantize(int64_t n, const int8_t *codes, const float *scales, float *y)
{
    for (int64_t i = 0; i < n; i++)
        y[i] = (float)codes[i] * scales[i / ORC_QBLOCK];
}

/* y[n] = sum_k W[n*ldw + col0 + k] * x[k]: a block of a stored (out, in)
 * row-major weight times a vector, in fp64. Rows of the block are the output
 * features a column-split shard owns; col0/K select the input features a
 * row-split shard owns ([TP] 核心概念 items 1 and 2). */
void orc_matvec(int64_t N, int64_t K, const void *W, int dt, int64_t ldw, int64_t col0,
                const double *x, double *y)
{
#pragma omp parallel for if (N >= 64) schedule(static)
    for (int64_t n = 0; n < N; n++) {
        double acc = 0.0;
        for (int64_t k = 0; k < K; k++)
            acc += ld(W, dt, n * ldw + col0 + k) * x[k];
        y[n] = acc;
    }
}

/* Rotary position encoding of one head vector at position pos ([DL]
 * llamaMultiheadAtt, whose description names RoPE). The pages name RoPE only; the
 * Llama form is taken: adjacent pairs (u_2i, u_2i+1) rotated by
 * pos * theta^(-2i/hd). */
void orc_rope(int64_t hd, int64_t pos, double theta, double *u)
{
    for (int64_t i = 0; i < hd / 2; i++) {
        double ang = (double)pos * pow(theta, -2.0 * (double)i / (double)hd);
        double c = cos(ang), s = sin(ang);
        double a = u[2 * i], b = u[2 * i + 1];
        u[2 * i] = a * c - b * s;
        u[2 * i + 1] = a * s + b * c;
    }
}

/* softmax(s)_t = exp(s_t - max) / sum_u exp(s_u - max) */
void orc_softmax(int64_t n, const double *s, double *w)
{
    double m = s[0];
    for (int64_t t = 1; t < n; t++)
        if (s[t] > m)
            m = s[t];
    double sum = 0.0;
    for (int64_t t = 0; t < n; t++) {
        w[t] = exp(s[t] - m);
        sum += w[t];
    }
    for (int64_t t = 0; t < n; t++)
        w[t] /= sum;
}

/* One query head attending over n_pos cached positions ([DL]
 * llamaMultiheadAtt: each node attends with its own heads over its own cache):
 * o = sum_t softmax_t(q . K[t] / sqrt(hd)) V[t]. K and V point at n_pos rows
 * of hd stored elements each, ld_kv elements apart. The pages fix no scale or
 * mask; the usual 1/sqrt(hd) is taken, and decode attends to every cached
 * position (no mask beyond the length). */
void orc_attend(int64_t hd, int64_t n_pos, const double *q, const void *K, const void *V,
                int kv_dt, int64_t ld_kv, double *o)
{
    double *s = (double *)malloc(sizeof(double) * (size_t)n_pos);
    double *w = (double *)malloc(sizeof(double) * (size_t)n_pos);
    for (int64_t t = 0; t < n_pos; t++) {
        double acc = 0.0;
        for (int64_t c = 0; c < hd; c++)
            acc += q[c] * ld(K, kv_dt, t * ld_kv + c);
        s[t] = acc / sqrt((double)hd);
    }
    orc_softmax(n_pos, s, w);
    for (int64_t c = 0; c < hd; c++) {
        double acc = 0.0;
        for (int64_t t = 0; t < n_pos; t++)
            acc += w[t] * ld(V, kv_dt, t * ld_kv + c);
        o[c] = acc;
    }
    free(s);
    free(w);
}

/* silu(z) = z * sigmoid(z) = z / (1 + exp(-z)) (SwiGLU's gate, [DL] llamaFfn) */
double orc_silu(double z)
{
    return z / (1.0 + exp(-z));
}

/* ---------------------------------------------------------------- one shard */

typedef struct {
    int32_t dim, n_heads, n_kv_heads, head_dim, ffn_hidden, tp_size, batch, max_ctx;
    int32_t w_dtype, kv_dtype, quant, pad_;
    double rope_theta, norm_eps;
} orc_llama_cfg;

typedef struct {
    const void *wq, *wk, *wv, *wo, *w1, *w3, *w2; /* full tensors, (out, in) row-major */
    const float *g_att, *g_ffn;
} orc_llama_weights;

/* Q8 round trip of a normalised vector ([DL] llamaQuantizeRmsAtt /
 * llamaQuantizeRmfFfn, then each consumer's dequantisation): the vector is
 * taken to fp32 (the type it is stored in), quantised and dequantised. */
static void q8_round_trip(int64_t D, double *v, int8_t *codes_out, float *scales_out)
{
    float *f = (float *)malloc(sizeof(float) * (size_t)D);
    int8_t *q = (int8_t *)malloc((size_t)D);
    float *sc = (float *)malloc(sizeof(float) * (size_t)(D / ORC_QBLOCK));
    for (int64_t i = 0; i < D; i++)
        f[i] = (float)v[i];
    orc_q8_quantize(D, f, q, sc);
    orc_q8_dequantize(D, q, sc, f);
    for (int64_t i = 0; i < D; i++)
        v[i] = (double)f[i];
    if (codes_out)
        memcpy(codes_out, q, (size_t)D);
    if (scales_out)
        memcpy(scales_out, sc, sizeof(float) * (size_t)(D / ORC_QBLOCK));
    free(f);
    free(q);
    free(sc);
}

/* Attention stage of shard s ([DL] root tasks llamaRmsAttNorm,
 * llamaQuantizeRmsAtt, llamaQkv, llamaMultiheadAtt, llamaAttOutput; the same
 * tasks a worker runs after receiving the normalised input).
 *
 *  x      [B][D]      stage input (residual stream)
 *  lens   [B]         cached positions per sequence; the new token is
 *                     appended at index lens[b] and attention covers
 *                     lens[b] + 1 positions (the cache is read back after the
 *                     append, so the new K/V are used as stored)
 *  kc, vc [B][Hkv][max_ctx][hd] full caches (cache dtype); the shard's kv
 *                     heads get the new entry appended in place
 * outputs (any may be NULL except p):
 *  xn  [B][D]          normalised input (after the optional Q8 round trip)
 *  q   [B][Hq_s*hd]    rotated queries of the shard's heads
 *  k,v [B][Hkv_s*hd]   rotated keys, values of the shard's kv heads
 *  att [B][Hq_s*hd]    attention outputs of the shard's heads
 *  p   [B][D]          row-split W_O partial sum ([TP] 運作原理 step 3)
 *
 * Heads: shard s owns q heads [s*Hq/T, (s+1)*Hq/T) and kv heads
 * [s*Hkv/T, (s+1)*Hkv/T); q head hq reads kv head hq / (Hq/Hkv) (contiguous
 * groups, so the shard's q heads only read its own kv heads: no KV
 * replication while T divides Hkv, [POPE] demo 3 observations).
 */
int orc_attn_shard(const orc_llama_cfg *c, const orc_llama_weights *w, int32_t s,
                   const double *x, const int32_t *lens, void *kc, void *vc,
                   double *xn_out, double *q_out, double *k_out, double *v_out,
                   double *att_out, double *p)
{
    const int64_t D = c->dim, hd = c->head_dim, T = c->tp_size, B = c->batch;
    const int64_t Hq = c->n_heads, Hkv = c->n_kv_heads, G = Hq / Hkv;
    const int64_t Hq_s = Hq / T, Hkv_s = Hkv / T, C = c->max_ctx;
    if (Hq % Hkv || Hq % T || Hkv % T || hd % 2 || s < 0 || s >= T)
        return -1;
    for (int64_t b = 0; b < B; b++)
        if (lens[b] < 0 || lens[b] >= C)
            return -2;
    double *xn = (double *)malloc(sizeof(double) * (size_t)D);
    double *q = (double *)malloc(sizeof(double) * (size_t)(Hq_s * hd));
    double *kv = (double *)malloc(sizeof(double) * (size_t)hd);
    double *att = (double *)malloc(sizeof(double) * (size_t)(Hq_s * hd));
    for (int64_t b = 0; b < B; b++) {
        const int64_t L = lens[b];
        orc_rmsnorm(D, x + b * D, w->g_att, c->norm_eps, xn);
        if (c->quant & ORC_Q_INPUTS)
            q8_round_trip(D, xn, NULL, NULL);
        if (xn_out)
            memcpy(xn_out + b * D, xn, sizeof(double) * (size_t)D);
        /* column-split Q, K, V ([DL] llamaQkv): the rows of the shard's heads
         * (selected by offsetting the weight pointer), then RoPE at position L */
        for (int64_t h = 0; h < Hq_s; h++) {
            const int64_t hq = s * Hq_s + h;
            const int64_t esz = c->w_dtype == ORC_F32 ? 4 : 2;
            orc_matvec(hd, D, (const char *)w->wq + hq * hd * D * esz, c->w_dtype, D, 0, xn,
                       q + h * hd);
            orc_rope(hd, L, c->rope_theta, q + h * hd);
        }
        for (int64_t g = 0; g < Hkv_s; g++) {
            const int64_t hk = s * Hkv_s + g;
            const int64_t esz = c->w_dtype == ORC_F32 ? 4 : 2;
            const int64_t slot = ((b * Hkv + hk) * C + L) * hd;
            orc_matvec(hd, D, (const char *)w->wk + hk * hd * D * esz, c->w_dtype, D, 0, xn, kv);
            orc_rope(hd, L, c->rope_theta, kv);
            if (k_out)
                memcpy(k_out + (b * Hkv_s + g) * hd, kv, sizeof(double) * (size_t)hd);
            for (int64_t e = 0; e < hd; e++) /* append to the cache ([DL] llamaMultiheadAtt) */
                st(kc, c->kv_dtype, slot + e, kv[e]);
            orc_matvec(hd, D, (const char *)w->wv + hk * hd * D * esz, c->w_dtype, D, 0, xn, kv);
            if (v_out)
                memcpy(v_out + (b * Hkv_s + g) * hd, kv, sizeof(double) * (size_t)hd);
            for (int64_t e = 0; e < hd; e++)
                st(vc, c->kv_dtype, slot + e, kv[e]);
        }
        /* attention of each local q head over its kv head's L + 1 positions */
#pragma omp parallel for if (Hq_s > 1) schedule(static)
        for (int64_t h = 0; h < Hq_s; h++) {
            const int64_t hk = (s * Hq_s + h) / G;
            const int64_t esz = c->kv_dtype == ORC_F32 ? 4 : 2;
            const int64_t base = (b * Hkv + hk) * C * hd;
            orc_attend(hd, L + 1, q + h * hd, (const char *)kc + base * esz,
                       (const char *)vc + base * esz, c->kv_dtype, hd, att + h * hd);
        }
        if (q_out)
            memcpy(q_out + b * Hq_s * hd, q, sizeof(double) * (size_t)(Hq_s * hd));
        if (att_out)
            memcpy(att_out + b * Hq_s * hd, att, sizeof(double) * (size_t)(Hq_s * hd));
        /* row-split W_O ([DL] llamaAttOutput): the shard's columns of W_O */
        orc_matvec(D, Hq_s * hd, w->wo, c->w_dtype, Hq * hd, s * Hq_s * hd, att, p + b * D);
    }
    free(xn);
    free(q);
    free(kv);
    free(att);
    return 0;
}

/* FFN stage of shard s ([DL] llamaRmfFfn, llamaRmfFfnNorm,
 * llamaQuantizeRmfFfn, llamaFfn (SwiGLU), llamaFfn2; [TP] 運作原理):
 *  h   [B][D]      stage input (residual after the attention merge)
 * outputs (any may be NULL except p):
 *  hn  [B][D]      normalised input (after the optional Q8 round trip)
 *  a   [B][F_s]    silu(W1_f . hn) * (W3_f . hn) for the shard's columns f
 *  p   [B][D]      row-split W2 partial sum
 * Shard s owns FFN features [s*F/T, (s+1)*F/T). */
int orc_ffn_shard(const orc_llama_cfg *c, const orc_llama_weights *w, int32_t s,
                  const double *h, double *hn_out, double *a_out, double *p)
{
    const int64_t D = c->dim, T = c->tp_size, B = c->batch, F = c->ffn_hidden;
    const int64_t Fs = F / T;
    const int64_t esz = c->w_dtype == ORC_F32 ? 4 : 2;
    if (F % T || s < 0 || s >= T)
        return -1;
    double *hn = (double *)malloc(sizeof(double) * (size_t)D);
    double *a = (double *)malloc(sizeof(double) * (size_t)Fs);
    for (int64_t b = 0; b < B; b++) {
        orc_rmsnorm(D, h + b * D, w->g_ffn, c->norm_eps, hn);
        if (c->quant & ORC_Q_INPUTS)
            q8_round_trip(D, hn, NULL, NULL);
        if (hn_out)
            memcpy(hn_out + b * D, hn, sizeof(double) * (size_t)D);
#pragma omp parallel for schedule(static)
        for (int64_t f = 0; f < Fs; f++) {
            const int64_t row = s * Fs + f;
            double g1, g3;
            orc_matvec(1, D, (const char *)w->w1 + row * D * esz, c->w_dtype, D, 0, hn, &g1);
            orc_matvec(1, D, (const char *)w->w3 + row * D * esz, c->w_dtype, D, 0, hn, &g3);
            a[f] = orc_silu(g1) * g3;
        }
        if (a_out)
            memcpy(a_out + b * Fs, a, sizeof(double) * (size_t)Fs);
        orc_matvec(D, Fs, w->w2, c->w_dtype, F, s * Fs, a, p + b * D);
    }
    free(hn);
    free(a);
    return 0;
}

/* What travels for one shard's partial ([DL] llamaQuantizeAtt -> llamaSyncAtt
 * -> llamaDequantizeAtt, and the Ffn2 counterparts): with partial
 * quantisation the fp32 partial is quantised per row in blocks of 32 and the
 * receiver uses the dequantised values; otherwise the partial itself.
 *  p [B][D] -> d [B][D]; codes [B][D], scales [B][D/32] (may be NULL). */
void orc_wire(int64_t B, int64_t D, int32_t quant, const double *p, double *d, int8_t *codes,
              float *scales)
{
    if (!(quant & ORC_Q_PARTIALS)) {
        memcpy(d, p, sizeof(double) * (size_t)(B * D));
        return;
    }
    float *f = (float *)malloc(sizeof(float) * (size_t)D);
    int8_t *q = (int8_t *)malloc((size_t)D);
    float *sc = (float *)malloc(sizeof(float) * (size_t)(D / ORC_QBLOCK));
    for (int64_t b = 0; b < B; b++) {
        for (int64_t i = 0; i < D; i++)
            f[i] = (float)p[b * D + i];
        orc_q8_quantize(D, f, q, sc);
        if (codes)
            memcpy(codes + b * D, q, (size_t)D);
        if (scales)
            memcpy(scales + b * (D / ORC_QBLOCK), sc, sizeof(float) * (size_t)(D / ORC_QBLOCK));
        orc_q8_dequantize(D, q, sc, f);
        for (int64_t i = 0; i < D; i++)
            d[b * D + i] = (double)f[i];
    }
    free(f);
    free(q);
    free(sc);
}

/* Merge ([DL] llamaMergeAtt / llamaMergeFfn2; [TP] 運作原理 step 3's
 * all-reduce): out = residual + sum over shards, in shard order. The page
 * says only "merge"; the block's residual connection is the plain reading. */
void orc_merge(int64_t n, int32_t T, const double *residual, const double *d, double *out)
{
    for (int64_t i = 0; i < n; i++) {
        double acc = residual[i];
        for (int32_t s = 0; s < T; s++)
            acc += d[(int64_t)s * n + i];
        out[i] = acc;
    }
}

/* The whole layer step, every shard in turn ([DL] buildLlama2Arch, one
 * iteration of the layer loop). Per-shard outputs are laid out [T][...].
 * Nullable outputs as in the stage functions; h and out are required. */
typedef struct {
    double *xn;        /* [T][B][D] */
    double *q;         /* [T][B][Hq_s*hd] */
    double *k, *v;     /* [T][B][Hkv_s*hd] */
    double *att;       /* [T][B][Hq_s*hd] */
    double *p_att;     /* [T][B][D] */
    int8_t *codes_att; /* [T][B][D] */
    float *scales_att; /* [T][B][D/32] */
    double *h;         /* [B][D] */
    double *hn;        /* [T][B][D] */
    double *a;         /* [T][B][F_s] */
    double *p_ffn;     /* [T][B][D] */
    int8_t *codes_ffn;
    float *scales_ffn;
    double *out;       /* [B][D] */
} orc_layer_out;

int orc_llama_layer(const orc_llama_cfg *c, const orc_llama_weights *w, const double *x,
                    const int32_t *lens, void *kc, void *vc, orc_layer_out *o)
{
    const int64_t D = c->dim, T = c->tp_size, B = c->batch, hd = c->head_dim;
    const int64_t Hq_s = c->n_heads / T, Hkv_s = c->n_kv_heads / T, Fs = c->ffn_hidden / T;
    const int64_t BD = B * D;
    double *p = (double *)malloc(sizeof(double) * (size_t)(T * BD));
    double *d = (double *)malloc(sizeof(double) * (size_t)(T * BD));
    int rc = 0;
#define OFS(ptr, n) ((ptr) ? (ptr) + (int64_t)s * (n) : NULL)
    for (int32_t s = 0; s < T && !rc; s++) {
        rc = orc_attn_shard(c, w, s, x, lens, kc, vc, OFS(o->xn, BD), OFS(o->q, B * Hq_s * hd),
                            OFS(o->k, B * Hkv_s * hd), OFS(o->v, B * Hkv_s * hd),
                            OFS(o->att, B * Hq_s * hd), p + s * BD);
        if (o->p_att)
            memcpy(o->p_att + s * BD, p + s * BD, sizeof(double) * (size_t)BD);
        orc_wire(B, D, c->quant, p + s * BD, d + s * BD, OFS(o->codes_att, BD),
                 OFS(o->scales_att, BD / ORC_QBLOCK));
    }
    if (!rc)
        orc_merge(BD, (int32_t)T, x, d, o->h);
    for (int32_t s = 0; s < T && !rc; s++) {
        rc = orc_ffn_shard(c, w, s, o->h, OFS(o->hn, BD), OFS(o->a, B * Fs), p + s * BD);
        if (o->p_ffn)
            memcpy(o->p_ffn + s * BD, p + s * BD, sizeof(double) * (size_t)BD);
        orc_wire(B, D, c->quant, p + s * BD, d + s * BD, OFS(o->codes_ffn, BD),
                 OFS(o->scales_ffn, BD / ORC_QBLOCK));
    }
    if (!rc)
        orc_merge(BD, (int32_t)T, o->h, d, o->out);
#undef OFS
    free(p);
    free(d);
    return rc;
}

/* ---------------------------------------------------------------- 2D FFN block */

/* PaLM-style FFN on the block one chip holds under 2D weight-stationary
 * partitioning ([POPE] demo 1 and the PALM record; [TP] 核心概念 item 3):
 * Y = (silu(X W_gate^T) * (X W_in^T)) W_out^T with X bf16 [B][E],
 * W_gate, W_in bf16 [F][E], W_out bf16 [E][F], for rows [row0, row0+nrows)
 * of X; Y fp64 [nrows][E]. No intermediate rounding. The page's cross-chip
 * reduce-scatter / all-gather of the block's activations is not part of a
 * single chip's computation and is left out. */
void orc_ffn2d(int64_t E, int64_t F, const uint16_t *X, const uint16_t *Wgate,
               const uint16_t *Win, const uint16_t *Wout, int64_t row0, int64_t nrows, double *Y)
{
    double *x = (double *)malloc(sizeof(double) * (size_t)E);
    double *hgt = (double *)malloc(sizeof(double) * (size_t)F);
    for (int64_t r = 0; r < nrows; r++) {
        for (int64_t e = 0; e < E; e++)
            x[e] = ld(X, ORC_BF16, (row0 + r) * E + e);
#pragma omp parallel for schedule(static)
        for (int64_t f = 0; f < F; f++) {
            double g, u;
            orc_matvec(1, E, Wgate + f * E, ORC_BF16, E, 0, x, &g);
            orc_matvec(1, E, Win + f * E, ORC_BF16, E, 0, x, &u);
            hgt[f] = orc_silu(g) * u;
        }
        orc_matvec(E, F, Wout, ORC_BF16, F, 0, hgt, Y + r * E);
    }
    free(x);
    free(hgt);
}

/* ---------------------------------------------------------------- final stage */

/* Logits of shard s of T ([DL] root tasks llamaRmsFinal, llamaRmsFinalNorm,
 * llamaLogits; a worker runs llamaLogits): RMSNorm of the last layer's
 * merged output with the final gain g, then the shard's rows
 * [s*V/T, (s+1)*V/T) of the classifier W_cls [V][D] (stored type dt) times
 * the normalised row. The pages split the vocabulary between the nodes (the
 * workers compute logits too) but give no split rule; the column split of
 * [TP] 核心概念 item 1 over the vocabulary is the plain reading: each shard
 * owns whole logits. The page lists no quantise / sync task between the
 * final norm and the logits, so the normalised row is used unquantised.
 *  x [B][D]; xn_out [B][D] (may be NULL); z [B][V/T]. */
int orc_logits_shard(int64_t B, int64_t D, int64_t V, int32_t T, int32_t s, const void *Wcls,
                     int dt, const float *g, double eps, const double *x, double *xn_out,
                     double *z)
{
    if (T < 1 || V % T || s < 0 || s >= T)
        return -1;
    const int64_t Vs = V / T;
    const int64_t esz = dt == ORC_F32 ? 4 : 2;
    double *xn = (double *)malloc(sizeof(double) * (size_t)D);
    for (int64_t b = 0; b < B; b++) {
        orc_rmsnorm(D, x + b * D, g, eps, xn);
        if (xn_out)
            memcpy(xn_out + b * D, xn, sizeof(double) * (size_t)D);
        orc_matvec(Vs, D, (const char *)Wcls + s * Vs * D * esz, dt, D, 0, xn, z + b * Vs);
    }
    free(xn);
    return 0;
}

/* Merge of the shards' logits ([DL] llamaSyncLogits, llamaDequantizeLogits,
 * llamaMergeLogits): shard i's (dequantised) slice d[i] [B][Vs] becomes
 * columns [i*Vs, (i+1)*Vs) of the full logits rows, out [B][T*Vs]. With a
 * vocabulary split the slices are disjoint, so the merge places them and
 * adds nothing. */
void orc_merge_logits(int64_t B, int64_t Vs, int32_t T, const double *d, double *out)
{
    for (int32_t i = 0; i < T; i++)
        for (int64_t b = 0; b < B; b++)
            for (int64_t j = 0; j < Vs; j++)
                out[b * T * Vs + i * Vs + j] = d[(i * B + b) * Vs + j];
}

/* ---------------------------------------------------------------- batch-sharded attention */

/* Batch-sharded attention ([POPE] demo 3 observations: with fewer KV heads
 * than shards, sharding attention by head would store a KV head on several
 * chips; sharding by sequence stores each sequence's KV once, on the shard
 * that owns the sequence with every head local, and the queries and outputs
 * cross an all-to-all instead). One batch shard: for each of its nb
 * sequences (rows of qkv: the raw q of every q head, then the raw k and v of
 * every kv head), RoPE at position lens[b] on q and k, the new k / v
 * appended at slot lens[b] of the shard's caches, then every q head attends
 * over its kv head's lens[b] + 1 positions, exactly as in the head-sharded
 * stage (same rotation, append, scale and kv-head map).
 *  qkv [nb][(Hq + 2 Hkv) hd]; kc, vc [nb][Hkv][C][hd] (cache dtype kv_dt);
 *  att [nb][Hq hd]. Returns -2 (nothing written) if a length is outside
 *  [0, C). */
int orc_attn_batch_shard(int64_t nb, int64_t Hq, int64_t Hkv, int64_t hd, int64_t C, double theta,
                         int kv_dt, const double *qkv, const int32_t *lens, void *kc, void *vc,
                         double *att)
{
    if (Hq % Hkv || hd % 2)
        return -1;
    for (int64_t b = 0; b < nb; b++)
        if (lens[b] < 0 || lens[b] >= C)
            return -2;
    const int64_t G = Hq / Hkv, ld = (Hq + 2 * Hkv) * hd;
    const int64_t esz = kv_dt == ORC_F32 ? 4 : 2;
    double *u = (double *)malloc(sizeof(double) * (size_t)hd);
    for (int64_t b = 0; b < nb; b++) {
        const int64_t L = lens[b];
        const double *row = qkv + b * ld;
        for (int64_t hk = 0; hk < Hkv; hk++) {
            const int64_t slot = (b * Hkv + hk) * C * hd + L * hd; /* row L of the head's cache */
            memcpy(u, row + (Hq + hk) * hd, sizeof(double) * (size_t)hd);
            orc_rope(hd, L, theta, u);
            for (int64_t e = 0; e < hd; e++)
                st(kc, kv_dt, slot + e, u[e]);
            for (int64_t e = 0; e < hd; e++)
                st(vc, kv_dt, slot + e, row[(Hq + Hkv + hk) * hd + e]);
        }
        for (int64_t h = 0; h < Hq; h++) {
            const int64_t base = (b * Hkv + h / G) * C * hd;
            memcpy(u, row + h * hd, sizeof(double) * (size_t)hd);
            orc_rope(hd, L, theta, u);
            const int64_t n_pos = L + 1; /* the cached positions and the new one */
            orc_attend(hd, n_pos, u, (const char *)kc + base * esz, (const char *)vc + base * esz,
                       kv_dt, hd, att + (b * Hq + h) * hd);
        }
    }
    free(u);
    return 0;
}

/* The two all-to-alls around batch-sharded attention, seen from shard r of
 * T with B sequences in all (nb = B / T per shard) and C = (Hq / T) hd
 * columns of one head shard:
 *  heads -> batch: src [T][B][C] (shard i's head-sharded rows: its q heads
 *    [i Hq/T, (i+1) Hq/T) for every sequence) -> dst [nb][T C]: shard r's
 *    sequences [r nb, (r+1) nb) with every head, head shard i's columns at
 *    [i C, (i+1) C);
 *  batch -> heads: src [T][nb][T C] (shard i's batch-sharded rows) -> dst
 *    [B][C]: every sequence b (from shard b / nb, row b % nb) with shard r's
 *    heads, columns [r C, (r+1) C) of that row.
 * Pure placement: every value is copied unchanged. */
void orc_a2a_heads_to_batch(int64_t B, int32_t T, int32_t r, int64_t C, const double *src,
                            double *dst)
{
    const int64_t nb = B / T;
    for (int64_t b = 0; b < nb; b++)
        for (int32_t i = 0; i < T; i++)
            for (int64_t c = 0; c < C; c++)
                dst[b * T * C + i * C + c] = src[((int64_t)i * B + r * nb + b) * C + c];
}

void orc_a2a_batch_to_heads(int64_t B, int32_t T, int32_t r, int64_t C, const double *src,
                            double *dst)
{
    const int64_t nb = B / T;
    for (int64_t b = 0; b < B; b++)
        for (int64_t c = 0; c < C; c++)
            dst[b * C + c] = src[((b / nb) * nb + b % nb) * T * C + r * C + c];
}
