/*
 * oracle.c -- plain CPU oracle for the Llama-2 decoder forward pass.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test-suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  The product path (the
 * HIP library under llama_decoder_forward_amd/) never calls it, shares no code
 * with it, and includes none of its headers.
 *
 * What it computes follows the pages collected for this project:
 *   P1 = "Meta Llama 源码深度剖析与生产应用教程" (juejin.cn walkthrough of the
 *        meta-llama/llama reference implementation),
 *   P2 = course notes on the generate loop (wiki.maxwellmou.com),
 *   P3 = "nano-vllm 学习笔记-Llama" reading notes,
 *   P4 = the llama2.zig CPU engine article (cyqw.cn).
 * Each function names the section it follows.  Every floating-point step is
 * plain fp32 (or fp64 when acc64 is set) with the fp16 rounding points that
 * the reference's casts imply (fp16 default tensor type, P1 section 4.1;
 * `.float()` / `.type_as()` in RMSNorm and softmax, P1 sections 3.2 and 3.5).
 * No blocking, fusion or reordering beyond the definition: the layer is
 * computed exactly in the order written in P1 sections 3.5-3.7.
 *
 * Parity status: every component is pinned by tests under tests/ (closed
 * forms, invariants, brute force, library routines).  The composed model
 * (all layers together) has no printed values on the pages and is pinned
 * only through its components plus an fp64-accumulation self-consistency
 * check: the composed logits are "parity unpinned" by the pages themselves.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <stdio.h>

#ifdef _OPENMP
#include <omp.h>
#endif

#define ORC_F32 0
#define ORC_F16 1

/* ------------------------------------------------------------------------ */
/* Model hyper-parameters: the fields of ModelArgs (P1 section 3.1) plus the  */
/* RoPE base (P1 section 3.3) and the storage dtype.                          */
/* ------------------------------------------------------------------------ */
typedef struct {
    int32_t n_layers, dim, n_heads, n_kv_heads, vocab_size, multiple_of;
    float ffn_dim_multiplier; /* <= 0 means None */
    float norm_eps, rope_theta;
    int32_t max_batch_size, max_seq_len, dtype;
} orc_params;

/* ------------------------------------------------------------------------ */
/* IEEE binary16 conversion, written out from the format's definition       */
/* (1 sign bit, 5 exponent bits with bias 15, 10 fraction bits, subnormals  */
/* below 2^-14, round to nearest with ties to even).                         */
/* ------------------------------------------------------------------------ */
uint16_t orc_f64_to_f16(double v)
{
    uint64_t bits;
    memcpy(&bits, &v, 8);
    uint16_t sign = (uint16_t)((bits >> 48) & 0x8000u);
    if (isnan(v)) return (uint16_t)(sign | 0x7e00u);
    double a = fabs(v);
    if (isinf(v) || a >= 65520.0) return (uint16_t)(sign | 0x7c00u); /* overflow */
    if (a == 0.0) return sign;
    int e2;
    frexp(a, &e2);              /* a = m * 2^e2 with m in [0.5, 1) */
    int E = e2 - 1;             /* floor(log2(a)) */
    if (E < -14) E = -14;       /* subnormal range shares the 2^-24 quantum */
    double scaled = ldexp(a, 10 - E);      /* exact: power-of-two scaling */
    double r = nearbyint(scaled);          /* ties to even (default mode) */
    uint32_t ir = (uint32_t)r;
    if (E == -14 && ir < 1024u) return (uint16_t)(sign | ir); /* subnormal */
    if (ir == 2048u) { ir = 1024u; E += 1; }
    return (uint16_t)(sign | (uint32_t)((E + 15) << 10) | (ir - 1024u));
}

uint16_t orc_f32_to_f16(float f) { return orc_f64_to_f16((double)f); }

static float f16_decode(uint16_t h)
{
    int sign = (h >> 15) & 1, ex = (h >> 10) & 31, fr = h & 1023;
    double v;
    if (ex == 31) v = fr ? NAN : INFINITY;
    else if (ex == 0) v = ldexp((double)fr, -24);
    else v = ldexp((double)(1024 + fr), ex - 25);
    return (float)(sign ? -v : v);
}

/* All 65536 decoded values, filled once when the library loads. */
static float f16_table[65536];

__attribute__((constructor)) static void f16_table_init(void)
{
    for (uint32_t h = 0; h < 65536u; h++) f16_table[h] = f16_decode((uint16_t)h);
}

float orc_f16_to_f32(uint16_t h) { return f16_table[h]; }

/* Round an fp32 value to the storage precision: fp16 for half models,     */
/* identity for fp32 models.                                                 */
static inline float rnd(float x, int dtype)
{
    return dtype == ORC_F16 ? orc_f16_to_f32(orc_f32_to_f16(x)) : x;
}

/* ------------------------------------------------------------------------ */
/* Seeded synthetic weights.  The pages load trained checkpoints (P1 4.1);   */
/* none exist here, so weights are drawn from a counter-based generator:     */
/* SplitMix64 (Steele, Lea & Flood, "Fast splittable pseudorandom number     */
/* generators", OOPSLA 2014).  Output n of the generator started at state s  */
/* is mix(s + (n+1)*gamma).  Tensor t of a model with seed S uses the stream */
/* state s_t = output t of the generator started at S; element e (row-major  */
/* index over the logical [out][in] shape) uses output e of stream s_t.      */
/* The 64 output bits are four 16-bit uniforms whose sum (Irwin-Hall, n=4)   */
/* is centred and scaled to standard deviation 0.02, the initializer range   */
/* printed in the TinyLlama config (P3), then rounded once to the storage    */
/* type.                                                                     */
/* ------------------------------------------------------------------------ */
#define SM64_GAMMA 0x9E3779B97F4A7C15ULL
#define WEIGHT_SCALE 0x1.1bc779ef0d4e8p-21 /* nearest double to 0.02*sqrt(3)/2^16 */

static uint64_t sm64_mix(uint64_t z)
{
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
    return z ^ (z >> 31);
}

uint64_t orc_splitmix64_at(uint64_t state, uint64_t n)
{
    return sm64_mix(state + (n + 1) * SM64_GAMMA);
}

/* Tensor ids: 0 = tok_embeddings, 1 = output head, layer l uses
 * 16 + 8l + {0 wq, 1 wk, 2 wv, 3 wo, 4 w1, 5 w2, 6 w3}. */
enum { T_WQ = 0, T_WK = 1, T_WV = 2, T_WO = 3, T_W1 = 4, T_W2 = 5, T_W3 = 6 };
static int tensor_id(int layer, int which) { return 16 + 8 * layer + which; }

double orc_weight_value(uint64_t seed, int32_t tid, uint64_t e)
{
    uint64_t st = orc_splitmix64_at(seed, (uint64_t)tid);
    uint64_t h = orc_splitmix64_at(st, e);
    int64_t s = (int64_t)(h & 0xffffu) + (int64_t)((h >> 16) & 0xffffu) +
                (int64_t)((h >> 32) & 0xffffu) + (int64_t)(h >> 48);
    return (double)(s - 131070) * WEIGHT_SCALE;
}

/* Fill `count` stored elements [first, first+count) of tensor `tid`.
 * dtype f16 writes uint16 bit patterns, f32 writes floats. */
void orc_gen_tensor(uint64_t seed, int32_t tid, uint64_t first, uint64_t count,
                    int32_t dtype, void *out)
{
    int64_t n = (int64_t)count;
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; i++) {
        double w = orc_weight_value(seed, tid, first + (uint64_t)i);
        if (dtype == ORC_F16) ((uint16_t *)out)[i] = orc_f64_to_f16(w);
        else ((float *)out)[i] = (float)w;
    }
}

/* ------------------------------------------------------------------------ */
/* FFN width (P1 section 3.6): start from 4*dim, take int(2/3 of it), apply  */
/* the optional multiplier with int(), round up to multiple_of.              */
/* ------------------------------------------------------------------------ */
int32_t orc_ffn_hidden(int32_t dim, int32_t multiple_of, float mult)
{
    int64_t h = 4 * (int64_t)dim;
    h = (int64_t)(2.0 * (double)h / 3.0);
    if (mult > 0.0f) h = (int64_t)((double)mult * (double)h);
    return (int32_t)(multiple_of * ((h + multiple_of - 1) / multiple_of));
}

/* ------------------------------------------------------------------------ */
/* RoPE table (P1 section 3.3 precompute_freqs_cis): theta_i = base^(-2i/d)  */
/* for i < d/2, angle = m * theta_i in fp32, cos/sin of that angle in fp32   */
/* (complex64).  theta_i is evaluated in double and rounded once; cos/sin of */
/* the fp32 angle are evaluated in double and rounded once.                  */
/* ------------------------------------------------------------------------ */
void orc_rope_table(int32_t head_dim, int32_t n_pos, float base, float *cos_t, float *sin_t)
{
    int half = head_dim / 2;
    for (int i = 0; i < half; i++) {
        float th = (float)(1.0 / pow((double)base, (double)(2 * i) / (double)head_dim));
        for (int m = 0; m < n_pos; m++) {
            float ang = (float)m * th;
            cos_t[(size_t)m * half + i] = (float)cos((double)ang);
            sin_t[(size_t)m * half + i] = (float)sin((double)ang);
        }
    }
}

/* ------------------------------------------------------------------------ */
/* Dot product with fp32 (or fp64) accumulation: the plain sum of the        */
/* products in index order, one rounding per addition.  The pages fix no     */
/* summation order, so the oracle takes the definition as written.           */
/* ------------------------------------------------------------------------ */
static float dot_f32(const float *a, const float *b, int n, int acc64)
{
    if (acc64) {
        double s = 0.0;
        for (int k = 0; k < n; k++) s += (double)a[k] * (double)b[k];
        return (float)s;
    }
    float s = 0.0f;
    for (int k = 0; k < n; k++) s += a[k] * b[k];
    return s;
}

/* A weight matrix W[rows][cols] (logical out x in, row-major). */
typedef struct {
    int32_t rows, cols, dtype;
    void *data;
} orc_tensor;

static void tensor_row_f32(const orc_tensor *t, int r, float *out)
{
    if (t->dtype == ORC_F16) {
        const uint16_t *s = (const uint16_t *)t->data + (size_t)r * t->cols;
        for (int k = 0; k < t->cols; k++) out[k] = orc_f16_to_f32(s[k]);
    } else {
        memcpy(out, (const float *)t->data + (size_t)r * t->cols, sizeof(float) * t->cols);
    }
}

static int tensor_alloc_gen(orc_tensor *t, int rows, int cols, int dtype, uint64_t seed, int tid)
{
    size_t n = (size_t)rows * cols;
    t->rows = rows; t->cols = cols; t->dtype = dtype;
    t->data = malloc(n * (dtype == ORC_F16 ? 2 : 4));
    if (!t->data) return -1;
    orc_gen_tensor(seed, tid, 0, n, dtype, t->data);
    return 0;
}

static void tensor_free(orc_tensor *t) { free(t->data); t->data = NULL; }

/* Linear layer without bias (P1 section 2: all bias=False):
 * Y[m][n] = round(sum_k W[n][k] * X[m][k]) for m < M, n < N. */
static void linear(const orc_tensor *W, const float *X, int M, float *Y, int dtype, int acc64)
{
    int N = W->rows, K = W->cols;
#pragma omp parallel
    {
        float *row = (float *)malloc(sizeof(float) * K);
#pragma omp for schedule(static)
        for (int n = 0; n < N; n++) {
            tensor_row_f32(W, n, row);
            for (int m = 0; m < M; m++)
                Y[(size_t)m * N + n] = rnd(dot_f32(row, X + (size_t)m * K, K, acc64), dtype);
        }
        free(row);
    }
}

/* ------------------------------------------------------------------------ */
/* RMSNorm (P1 section 3.2): x * rsqrt(mean(x^2) + eps) computed in fp32 on  */
/* x.float(), cast back to the model dtype, then multiplied by the weight    */
/* (initialised to 1) with one more rounding.  rsqrt is 1/sqrt in fp32.      */
/* ------------------------------------------------------------------------ */
void orc_rmsnorm(const float *x, const float *w, int32_t D, float eps, int32_t dtype,
                 int32_t acc64, float *y)
{
    float r;
    if (acc64) {
        double s = 0.0;
        for (int i = 0; i < D; i++) s += (double)x[i] * (double)x[i];
        r = (float)(1.0 / sqrt(s / D + (double)eps));
    } else {
        float s = 0.0f;
        for (int i = 0; i < D; i++) s += x[i] * x[i];
        r = 1.0f / sqrtf(s / (float)D + eps);
    }
    for (int i = 0; i < D; i++) {
        float n = rnd(x[i] * r, dtype);
        y[i] = rnd(n * (w ? w[i] : 1.0f), dtype);
    }
}

/* ------------------------------------------------------------------------ */
/* Rotary embedding on one head vector at position m (P1 sections 3.3 and    */
/* 9): adjacent pairs (x_2i, x_2i+1) are complex numbers multiplied by       */
/* cos + i sin of the table entry, in fp32, rounded back to the dtype.       */
/* ------------------------------------------------------------------------ */
void orc_rope_apply(float *v, int32_t head_dim, const float *cos_row, const float *sin_row,
                    int32_t dtype)
{
    for (int i = 0; i < head_dim / 2; i++) {
        float a = v[2 * i], b = v[2 * i + 1], c = cos_row[i], s = sin_row[i];
        float re = a * c - b * s;
        float im = a * s + b * c;
        v[2 * i] = rnd(re, dtype);
        v[2 * i + 1] = rnd(im, dtype);
    }
}

/* ------------------------------------------------------------------------ */
/* Scaled dot-product attention of one query against keys 0..L-1 (P1         */
/* section 3.5 step 5; the causal mask of P1 section 3.8 / P2 section 2 is   */
/* applied by the caller choosing L = position + 1).  Scores q.k / sqrt(d),  */
/* softmax with the maximum subtracted (P4 section 5.4) in fp32, weighted    */
/* sum of values in fp32, output rounded to the dtype.  K and V rows are     */
/* `stride` floats apart.                                                    */
/* ------------------------------------------------------------------------ */
void orc_attention_row(const float *q, const float *K, const float *V, int32_t L, int32_t d,
                       int64_t stride, int32_t dtype, int32_t acc64, float *out)
{
    float scale = (float)(1.0 / sqrt((double)d));
    float *s = (float *)malloc(sizeof(float) * (L > 0 ? L : 1));
    float mx = -INFINITY;
    for (int j = 0; j < L; j++) {
        s[j] = dot_f32(q, K + (size_t)j * stride, d, acc64) * scale;
        if (s[j] > mx) mx = s[j];
    }
    if (acc64) {
        double sum = 0.0;
        for (int j = 0; j < L; j++) sum += exp((double)s[j] - (double)mx);
        for (int c = 0; c < d; c++) {
            double o = 0.0;
            for (int j = 0; j < L; j++)
                o += exp((double)s[j] - (double)mx) / sum * (double)V[(size_t)j * stride + c];
            out[c] = rnd((float)o, dtype);
        }
    } else {
        float sum = 0.0f;
        for (int j = 0; j < L; j++) { s[j] = expf(s[j] - mx); sum += s[j]; }
        for (int j = 0; j < L; j++) s[j] = s[j] / sum;
        for (int c = 0; c < d; c++) {
            float o = 0.0f;
            for (int j = 0; j < L; j++) o += s[j] * V[(size_t)j * stride + c];
            out[c] = rnd(o, dtype);
        }
    }
    free(s);
}

/* SiLU (P1 section 3.6): x * sigmoid(x) = x / (1 + exp(-x)), fp32. */
float orc_silu(float x) { return x / (1.0f + expf(-x)); }

/* ------------------------------------------------------------------------ */
/* One decoder layer                                                        */
/* ------------------------------------------------------------------------ */
typedef struct {
    orc_tensor w[7]; /* wq wk wv wo w1 w2 w3 */
} orc_layer;

typedef struct {
    int32_t D, H, Hkv, hd, F, V, NL, S, dtype;
    float eps;
} orc_dims;

static void dims_from_params(const orc_params *p, orc_dims *d)
{
    d->D = p->dim; d->H = p->n_heads;
    d->Hkv = p->n_kv_heads > 0 ? p->n_kv_heads : p->n_heads;
    d->hd = p->dim / p->n_heads;
    d->F = orc_ffn_hidden(p->dim, p->multiple_of, p->ffn_dim_multiplier);
    d->V = p->vocab_size; d->NL = p->n_layers; d->S = p->max_seq_len;
    d->dtype = p->dtype; d->eps = p->norm_eps;
}

static int layer_gen(orc_layer *L, const orc_dims *d, uint64_t seed, int l)
{
    int shape[7][2] = {{d->H * d->hd, d->D}, {d->Hkv * d->hd, d->D}, {d->Hkv * d->hd, d->D},
                       {d->D, d->H * d->hd}, {d->F, d->D},           {d->D, d->F},
                       {d->F, d->D}};
    for (int i = 0; i < 7; i++)
        if (tensor_alloc_gen(&L->w[i], shape[i][0], shape[i][1], d->dtype, seed, tensor_id(l, i)))
            return -1;
    return 0;
}

static void layer_free(orc_layer *L)
{
    for (int i = 0; i < 7; i++) tensor_free(&L->w[i]);
}

/* TransformerBlock (P1 section 3.7): h = x + attention(attention_norm(x)),
 * out = h + feed_forward(ffn_norm(h)).  x holds B*T rows of D values for
 * positions start_pos .. start_pos+T-1 of each batch row.  kc / vc are this
 * layer's caches laid out [B][S][Hkv][hd] like the reference's cache_k
 * (P1 section 3.1).  Keys visible to position p are 0..p (P1 section 3.8). */
static void layer_forward(const orc_layer *Lw, const orc_dims *d, float *x, int B, int T,
                          int start_pos, float *kc, float *vc, const float *cos_t,
                          const float *sin_t, int acc64)
{
    const int D = d->D, H = d->H, Hkv = d->Hkv, hd = d->hd, F = d->F, M = B * T;
    const int n_rep = H / Hkv, half = hd / 2, dt = d->dtype;
    float *xn = (float *)malloc(sizeof(float) * (size_t)M * D);
    float *q = (float *)malloc(sizeof(float) * (size_t)M * H * hd);
    float *k = (float *)malloc(sizeof(float) * (size_t)M * Hkv * hd);
    float *v = (float *)malloc(sizeof(float) * (size_t)M * Hkv * hd);
    float *o = (float *)malloc(sizeof(float) * (size_t)M * H * hd);
    float *t = (float *)malloc(sizeof(float) * (size_t)M * D);
    float *a = (float *)malloc(sizeof(float) * (size_t)M * F);
    float *b = (float *)malloc(sizeof(float) * (size_t)M * F);

    /* attention_norm */
#pragma omp parallel for schedule(static)
    for (int m = 0; m < M; m++) orc_rmsnorm(x + (size_t)m * D, NULL, D, d->eps, dt, acc64, xn + (size_t)m * D);
    /* wq, wk, wv (P1 section 3.5 step 1) */
    linear(&Lw->w[T_WQ], xn, M, q, dt, acc64);
    linear(&Lw->w[T_WK], xn, M, k, dt, acc64);
    linear(&Lw->w[T_WV], xn, M, v, dt, acc64);
    /* RoPE on q and k, not v (step 2); cache write at start_pos.. (step 3) */
    for (int bb = 0; bb < B; bb++)
        for (int tt = 0; tt < T; tt++) {
            int m = bb * T + tt, pos = start_pos + tt;
            for (int h = 0; h < H; h++)
                orc_rope_apply(q + ((size_t)m * H + h) * hd, hd, cos_t + (size_t)pos * half,
                               sin_t + (size_t)pos * half, dt);
            for (int h = 0; h < Hkv; h++) {
                float *kk = k + ((size_t)m * Hkv + h) * hd;
                orc_rope_apply(kk, hd, cos_t + (size_t)pos * half, sin_t + (size_t)pos * half, dt);
                size_t slot = (((size_t)bb * d->S + pos) * Hkv + h) * hd;
                memcpy(kc + slot, kk, sizeof(float) * hd);
                memcpy(vc + slot, v + ((size_t)m * Hkv + h) * hd, sizeof(float) * hd);
            }
        }
    /* attention: query head h reads KV head h / n_rep (repeat_kv, P1
     * section 3.4), keys 0..pos (causal mask, P1 section 3.8) */
#pragma omp parallel for collapse(2) schedule(static)
    for (int m = 0; m < M; m++)
        for (int h = 0; h < H; h++) {
            int bb = m / T, pos = start_pos + m % T, g = h / n_rep;
            const float *Kb = kc + ((size_t)bb * d->S * Hkv + g) * hd;
            const float *Vb = vc + ((size_t)bb * d->S * Hkv + g) * hd;
            orc_attention_row(q + ((size_t)m * H + h) * hd, Kb, Vb, pos + 1, hd,
                              (int64_t)Hkv * hd, dt, acc64, o + ((size_t)m * H + h) * hd);
        }
    /* wo and residual (step 6; P1 section 3.7) */
    linear(&Lw->w[T_WO], o, M, t, dt, acc64);
    for (size_t i = 0; i < (size_t)M * D; i++) x[i] = rnd(x[i] + t[i], dt);
    /* ffn_norm, SwiGLU w2(silu(w1 x) * w3 x) (P1 section 3.6), residual */
#pragma omp parallel for schedule(static)
    for (int m = 0; m < M; m++) orc_rmsnorm(x + (size_t)m * D, NULL, D, d->eps, dt, acc64, xn + (size_t)m * D);
    linear(&Lw->w[T_W1], xn, M, a, dt, acc64);
    linear(&Lw->w[T_W3], xn, M, b, dt, acc64);
    for (size_t i = 0; i < (size_t)M * F; i++) a[i] = rnd(rnd(orc_silu(a[i]), dt) * b[i], dt);
    linear(&Lw->w[T_W2], a, M, t, dt, acc64);
    for (size_t i = 0; i < (size_t)M * D; i++) x[i] = rnd(x[i] + t[i], dt);

    free(xn); free(q); free(k); free(v); free(o); free(t); free(a); free(b);
}

/* Final RMSNorm and output head on one row, logits promoted to fp32 (P1
 * section 2 data flow; only the last position is needed, P3 lm_head). */
static void head_forward(const orc_tensor *out_w, const orc_dims *d, const float *h, int rows,
                         float *logits, int acc64)
{
    float *xn = (float *)malloc(sizeof(float) * (size_t)rows * d->D);
    for (int r = 0; r < rows; r++)
        orc_rmsnorm(h + (size_t)r * d->D, NULL, d->D, d->eps, d->dtype, acc64, xn + (size_t)r * d->D);
    linear(out_w, xn, rows, logits, d->dtype, acc64);
    free(xn);
}

/* Embedding lookup (P1 section 2): an exact copy of row tok. */
static void embed(const orc_tensor *E, const int32_t *tok, int M, float *x)
{
    for (int m = 0; m < M; m++) tensor_row_f32(E, tok[m], x + (size_t)m * E->cols);
}

/* ------------------------------------------------------------------------ */
/* Resident model: all weights in host memory plus a static KV cache of      */
/* max_batch_size rows (P1 section 3.1).                                     */
/* ------------------------------------------------------------------------ */
typedef struct {
    orc_params p;
    orc_dims d;
    int acc64;
    orc_tensor emb, out;
    orc_layer *layers;
    float *kc, *vc; /* [NL][B][S][Hkv][hd] */
    float *cos_t, *sin_t;
} orc_model;

void orc_model_destroy(orc_model *m);

orc_model *orc_model_create(const orc_params *p, uint64_t seed, int32_t acc64)
{
    orc_model *m = (orc_model *)calloc(1, sizeof(orc_model));
    if (!m) return NULL;
    m->p = *p; m->acc64 = acc64;
    dims_from_params(p, &m->d);
    orc_dims *d = &m->d;
    m->layers = (orc_layer *)calloc((size_t)d->NL, sizeof(orc_layer));
    if (!m->layers) { free(m); return NULL; }
    if (tensor_alloc_gen(&m->emb, d->V, d->D, d->dtype, seed, 0) ||
        tensor_alloc_gen(&m->out, d->V, d->D, d->dtype, seed, 1)) { orc_model_destroy(m); return NULL; }
    for (int l = 0; l < d->NL; l++)
        if (layer_gen(&m->layers[l], d, seed, l)) { orc_model_destroy(m); return NULL; }
    size_t cache = (size_t)d->NL * p->max_batch_size * d->S * d->Hkv * d->hd;
    m->kc = (float *)calloc(cache, sizeof(float));
    m->vc = (float *)calloc(cache, sizeof(float));
    m->cos_t = (float *)malloc(sizeof(float) * (size_t)d->S * (d->hd / 2));
    m->sin_t = (float *)malloc(sizeof(float) * (size_t)d->S * (d->hd / 2));
    if (!m->kc || !m->vc || !m->cos_t || !m->sin_t) { orc_model_destroy(m); return NULL; }
    orc_rope_table(d->hd, d->S, p->rope_theta, m->cos_t, m->sin_t);
    return m;
}

void orc_model_destroy(orc_model *m)
{
    if (!m) return;
    tensor_free(&m->emb); tensor_free(&m->out);
    if (m->layers) for (int l = 0; l < m->d.NL; l++) layer_free(&m->layers[l]);
    free(m->layers); free(m->kc); free(m->vc); free(m->cos_t); free(m->sin_t);
    free(m);
}

/* Transformer.forward(tokens, start_pos) (P1 sections 2 and 3.8): B rows of
 * T tokens at positions start_pos..start_pos+T-1, KV cache updated, and the
 * fp32 logits of the last position of each row written to logits[B][V].
 * With T=1 this is a decode step (P2 section 3).  When resid is not NULL it
 * receives the residual stream at every layer boundary, resid[l][B*T][D]
 * for l = 0..NL: entry 0 is the embedding rows, entry l + 1 the output of
 * layer l (the input of the next TransformerBlock, P1 section 3.7).
 * Returns 0 or -1. */
int orc_model_forward_resid(orc_model *m, const int32_t *tokens, int32_t B, int32_t T,
                            int32_t start_pos, float *logits, float *resid)
{
    orc_dims *d = &m->d;
    if (B < 1 || B > m->p.max_batch_size || T < 1 || start_pos < 0 || start_pos + T > d->S) return -1;
    for (int i = 0; i < B * T; i++) if (tokens[i] < 0 || tokens[i] >= d->V) return -1;
    size_t M = (size_t)B * T;
    float *x = (float *)malloc(sizeof(float) * M * d->D);
    float *last = (float *)malloc(sizeof(float) * (size_t)B * d->D);
    embed(&m->emb, tokens, (int)M, x);
    if (resid) memcpy(resid, x, sizeof(float) * M * d->D);
    size_t per_layer = (size_t)m->p.max_batch_size * d->S * d->Hkv * d->hd;
    for (int l = 0; l < d->NL; l++) {
        layer_forward(&m->layers[l], d, x, B, T, start_pos, m->kc + l * per_layer,
                      m->vc + l * per_layer, m->cos_t, m->sin_t, m->acc64);
        if (resid) memcpy(resid + (size_t)(l + 1) * M * d->D, x, sizeof(float) * M * d->D);
    }
    for (int bb = 0; bb < B; bb++)
        memcpy(last + (size_t)bb * d->D, x + ((size_t)bb * T + T - 1) * d->D, sizeof(float) * d->D);
    head_forward(&m->out, d, last, B, logits, m->acc64);
    free(x); free(last);
    return 0;
}

int orc_model_forward(orc_model *m, const int32_t *tokens, int32_t B, int32_t T,
                      int32_t start_pos, float *logits)
{
    return orc_model_forward_resid(m, tokens, B, T, start_pos, logits, NULL);
}

/* Read back stored weights of the resident model (for generator checks). */
int orc_model_weights(const orc_model *m, int32_t tid, uint64_t first, uint64_t count, void *out)
{
    const orc_tensor *t = NULL;
    if (tid == 0) t = &m->emb;
    else if (tid == 1) t = &m->out;
    else if (tid >= 16 && (tid - 16) / 8 < m->d.NL && (tid - 16) % 8 < 7)
        t = &m->layers[(tid - 16) / 8].w[(tid - 16) % 8];
    if (!t || first + count > (uint64_t)t->rows * t->cols) return -1;
    size_t es = t->dtype == ORC_F16 ? 2 : 4;
    memcpy(out, (const char *)t->data + first * es, count * es);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Layer-major full-sequence forward for models too large to keep resident.  */
/* Runs the whole token sequence tokens[B][N] through one layer at a time    */
/* (weights generated, used, freed) and writes the fp32 logits of positions  */
/* first_pos..N-1 of each row to logits[B][N-first_pos][V].  Because every   */
/* query attends to keys 0..p with the same arithmetic, each position's      */
/* logits equal those of incremental prefill + decode over the same tokens.  */
/* When resid is not NULL it receives the residual stream at every layer     */
/* boundary, resid[l][B][N][D] for l = 0..NL (entry 0: the embedding rows,   */
/* entry l + 1: the output of layer l).                                      */
/* ------------------------------------------------------------------------ */
int orc_forward_stream_resid(const orc_params *p, uint64_t seed, int32_t acc64,
                             const int32_t *tokens, int32_t B, int32_t N, int32_t first_pos,
                             float *logits, float *resid)
{
    orc_dims d;
    dims_from_params(p, &d);
    if (B < 1 || N < 1 || N > d.S || first_pos < 0 || first_pos >= N) return -1;
    for (int i = 0; i < B * N; i++) if (tokens[i] < 0 || tokens[i] >= d.V) return -1;
    size_t M = (size_t)B * N;
    float *x = (float *)malloc(sizeof(float) * M * d.D);
    float *cos_t = (float *)malloc(sizeof(float) * (size_t)d.S * (d.hd / 2));
    float *sin_t = (float *)malloc(sizeof(float) * (size_t)d.S * (d.hd / 2));
    size_t cache = (size_t)B * d.S * d.Hkv * d.hd;
    float *kc = (float *)calloc(cache, sizeof(float));
    float *vc = (float *)calloc(cache, sizeof(float));
    if (!x || !cos_t || !sin_t || !kc || !vc) return -1;
    orc_rope_table(d.hd, d.S, p->rope_theta, cos_t, sin_t);
    orc_tensor t;
    if (tensor_alloc_gen(&t, d.V, d.D, d.dtype, seed, 0)) return -1;
    embed(&t, tokens, (int)M, x);
    tensor_free(&t);
    if (resid) memcpy(resid, x, sizeof(float) * M * d.D);
    for (int l = 0; l < d.NL; l++) {
        orc_layer L;
        if (layer_gen(&L, &d, seed, l)) return -1;
        layer_forward(&L, &d, x, B, N, 0, kc, vc, cos_t, sin_t, acc64);
        layer_free(&L);
        if (resid) memcpy(resid + (size_t)(l + 1) * M * d.D, x, sizeof(float) * M * d.D);
    }
    if (tensor_alloc_gen(&t, d.V, d.D, d.dtype, seed, 1)) return -1;
    int R = N - first_pos;
    float *rows = (float *)malloc(sizeof(float) * (size_t)B * R * d.D);
    for (int bb = 0; bb < B; bb++)
        memcpy(rows + (size_t)bb * R * d.D, x + ((size_t)bb * N + first_pos) * d.D,
               sizeof(float) * (size_t)R * d.D);
    head_forward(&t, &d, rows, B * R, logits, acc64);
    tensor_free(&t);
    free(rows); free(x); free(cos_t); free(sin_t); free(kc); free(vc);
    return 0;
}

int orc_forward_stream(const orc_params *p, uint64_t seed, int32_t acc64, const int32_t *tokens,
                       int32_t B, int32_t N, int32_t first_pos, float *logits)
{
    return orc_forward_stream_resid(p, seed, acc64, tokens, B, N, first_pos, logits, NULL);
}

/* One TransformerBlock (P1 section 3.7) of a model too large to keep       */
/* resident, applied to caller rows: x[B][N][D] holds the residual entering  */
/* layer `layer` at positions 0..N-1 of each row (causal over those N, P1    */
/* section 3.8) and receives the residual leaving it.  The layer's weights   */
/* are generated for the call and freed.  Returns 0 or -1.                   */
int orc_layer_apply(const orc_params *p, uint64_t seed, int32_t layer, int32_t acc64, float *x,
                    int32_t B, int32_t N)
{
    orc_dims d;
    dims_from_params(p, &d);
    if (layer < 0 || layer >= d.NL || B < 1 || N < 1 || N > d.S) return -1;
    float *cos_t = (float *)malloc(sizeof(float) * (size_t)d.S * (d.hd / 2));
    float *sin_t = (float *)malloc(sizeof(float) * (size_t)d.S * (d.hd / 2));
    size_t cache = (size_t)B * d.S * d.Hkv * d.hd;
    float *kc = (float *)calloc(cache, sizeof(float));
    float *vc = (float *)calloc(cache, sizeof(float));
    orc_layer L;
    if (!cos_t || !sin_t || !kc || !vc || layer_gen(&L, &d, seed, layer)) return -1;
    orc_rope_table(d.hd, d.S, p->rope_theta, cos_t, sin_t);
    layer_forward(&L, &d, x, B, N, 0, kc, vc, cos_t, sin_t, acc64);
    layer_free(&L);
    free(cos_t); free(sin_t); free(kc); free(vc);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Sampling (P1 section 4.2 / 4.3, P2 section 4)                            */
/* ------------------------------------------------------------------------ */

/* Greedy: argmax of the last-position logits; among equal maxima the
 * lowest token id (the pages do not say; this is the fixed reading). */
int32_t orc_argmax(const float *logits, int32_t V)
{
    int32_t best = 0;
    for (int32_t i = 1; i < V; i++) if (logits[i] > logits[best]) best = i;
    return best;
}

/* Temperature softmax in fp32: P_i = exp(z_i/t - max) / sum (P2 section 4,
 * formula for p_i(T); P1 section 4.2 divides the logits by t; maximum
 * subtracted per P4 section 5.4).  The pages fix neither the exp routine nor
 * the order of the normaliser's sum, and either changes the last bits of P
 * and so, at the nucleus edge, the drawn token.  The oracle therefore takes
 * each term and the normaliser as their correctly rounded fp32 values: the
 * exp of the fp32 argument evaluated in double and rounded once, and the sum
 * of the fp32 terms accumulated in double (relative error below V 2^-53,
 * under 2^-31 for V <= 2^22, far below one fp32 step) and rounded once.
 * z_i/t and P_i = e_i/s are fp32 divisions. */
void orc_softmax_temp(const float *logits, int32_t V, float temperature, float *probs)
{
    float mx = -INFINITY;
    for (int i = 0; i < V; i++) {
        probs[i] = logits[i] / temperature;
        if (probs[i] > mx) mx = probs[i];
    }
    double sd = 0.0;
    for (int i = 0; i < V; i++) {
        probs[i] = (float)exp((double)(probs[i] - mx));
        sd += (double)probs[i];
    }
    float s = (float)sd;
    for (int i = 0; i < V; i++) probs[i] = probs[i] / s;
}

typedef struct { float p; int32_t idx; } pi_pair;

static int cmp_desc(const void *a, const void *b)
{
    const pi_pair *x = (const pi_pair *)a, *y = (const pi_pair *)b;
    if (x->p > y->p) return -1;
    if (x->p < y->p) return 1;
    return (x->idx > y->idx) - (x->idx < y->idx);
}

/* Top-p (nucleus) sampling, sample_top_p of P1 section 4.3, made exact:
 *  1. sort probabilities descending (ties: lower token id first);
 *  2. Q_i = floor(P_(i) * 2^48), E_i = Q_0 + ... + Q_{i-1} (exact integers);
 *  3. keep i while E_i <= floor(top_p * 2^48): the reference's mask
 *     "cumsum - p_sorted > p" drops exactly the others, and i = 0 is always
 *     kept (P1 section 4.3 note);
 *  4. renormalise and draw by inverse CDF on the kept prefix: with S = E_k
 *     and U = floor(u * 2^24), target t = floor(U * S / 2^24), the drawn
 *     element is the first i < k with E_{i+1} > t.
 * Returns the token id.  *n_kept receives k when non-NULL. */
int32_t orc_top_p(const float *probs, int32_t V, float top_p, float u, int32_t *n_kept)
{
    pi_pair *s = (pi_pair *)malloc(sizeof(pi_pair) * V);
    for (int i = 0; i < V; i++) { s[i].p = probs[i]; s[i].idx = i; }
    qsort(s, V, sizeof(pi_pair), cmp_desc);
    const double two48 = 281474976710656.0;
    uint64_t thr = (uint64_t)floor((double)top_p * two48);
    uint64_t E = 0;
    int k = 0;
    uint64_t *Ei = (uint64_t *)malloc(sizeof(uint64_t) * (V + 1));
    for (int i = 0; i < V; i++) {
        if (E > thr) break;
        Ei[i] = E;
        E += (uint64_t)((double)s[i].p * two48);
        k = i + 1;
    }
    Ei[k] = E; /* S */
    uint64_t U = (uint64_t)floor((double)u * 16777216.0);
    uint64_t t = (uint64_t)(((unsigned __int128)U * E) >> 24);
    int32_t pick = s[0].idx;
    for (int i = 0; i < k; i++)
        if (Ei[i + 1] > t) { pick = s[i].idx; break; }
    if (n_kept) *n_kept = k;
    free(Ei); free(s);
    return pick;
}

int32_t orc_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Overwrite one whole tensor of the resident model (used by tests that build
 * models with related weights, e.g. GQA against replicated MHA). */
int orc_model_set_weights(orc_model *m, int32_t tid, const void *data)
{
    orc_tensor *t = NULL;
    if (tid == 0) t = &m->emb;
    else if (tid == 1) t = &m->out;
    else if (tid >= 16 && (tid - 16) / 8 < m->d.NL && (tid - 16) % 8 < 7)
        t = &m->layers[(tid - 16) / 8].w[(tid - 16) % 8];
    if (!t) return -1;
    memcpy(t->data, data, (size_t)t->rows * t->cols * (t->dtype == ORC_F16 ? 2 : 4));
    return 0;
}

/* Array forms of the binary16 conversions. */
void orc_f64_to_f16_vec(const double *x, int64_t n, uint16_t *out)
{
    for (int64_t i = 0; i < n; i++) out[i] = orc_f64_to_f16(x[i]);
}

void orc_f32_to_f16_vec(const float *x, int64_t n, uint16_t *out)
{
    for (int64_t i = 0; i < n; i++) out[i] = orc_f32_to_f16(x[i]);
}

void orc_f16_to_f32_vec(const uint16_t *h, int64_t n, float *out)
{
    for (int64_t i = 0; i < n; i++) out[i] = orc_f16_to_f32(h[i]);
}

/* Bias-free linear layer on caller-supplied weights W[N][K] (stored dtype
 * wdtype: uint16 binary16 or float) and rows X[M][K]: Y[m][n] =
 * round_out(sum_k W[n][k] X[m][k]) with out_dtype's rounding. */
void orc_linear(const void *W, int32_t wdtype, int32_t N, int32_t K, const float *X, int32_t M,
                int32_t out_dtype, int32_t acc64, float *Y)
{
    orc_tensor t;
    t.rows = N; t.cols = K; t.dtype = wdtype; t.data = (void *)W;
    linear(&t, X, M, Y, out_dtype, acc64);
}
