/*
 * CPU oracle for the guarded W8A8 linear layer and padded-row compaction.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the slow, plain reference that the
 * GPU library is checked against.  Only the tests, the smoke check and the
 * benchmark's CPU-baseline leg may load it; the product path never does.
 * It shares no code, header, table or helper with the HIP library.
 *
 * Source of the method: TurboT2VA, page "音视频生成提速54倍！浙大等团队开源联合
 * 蒸馏方案TurboT2VA" (智猩猩), section 01.3 "量化策略": linear layers use W8A8 —
 * weights statically quantised to INT8 per output channel, activations
 * dynamically quantised to INT8 per row, the matrix product accumulated in
 * INT32, scale and bias applied once after the whole accumulation, and
 * branches whose shapes the optimised operator cannot serve run in native BF16.
 * The same section's closing paragraph, and the paperlayer.ai summary (section
 * "C. Fused Multimodal Transformer Operations"), describe removing padded text
 * positions with the shared text mask while keeping every valid token.
 *
 * Readings where the pages are silent:
 *   Q  symmetric per-row scale s = absmax/127 in fp32, codes rne(x * (127/absmax))
 *      clamped to [-127,127]; rows with absmax < 2^-100 get s = 0, q = 0.
 *   E  epilogue in fp32: v = fma(float(acc), fl(sa*sw), float(bias)); y = bf16_rne(v).
 *   GELU (tanh form, only for the FFN up-projection) applied to the bf16 output,
 *      evaluated in float64 and rounded once to bf16.
 *   F  BF16 fallback: sum of exact products in float64, rounded once to bf16.
 *   G  guard: K % 128 == 0, 128 <= K <= 131072, N % 64 == 0, N >= 64.
 *   C  mask nonzero = valid; output keeps (sample, position) order.
 *   QB attention Q / K: blocks of `block` tokens of one sample and one head of
 *      a token-row matrix [B x S x H*D], each quantised as in Q over the block.
 *   NM normalisation + modulation ahead of a linear layer (the fused operators
 *      of the paperlayer.ai summary, section C): per row, LayerNorm without
 *      affine (mean and variance over the row) or RMSNorm (mean square), then
 *      z = y * (1 + scale) + shift with the modulation vectors of the row's
 *      conditioning group; the real-valued formula evaluated in binary64 and
 *      rounded once to bf16 (the page gives no precision); the fused variant
 *      quantises that bf16 row as in Q.
 *
 * Build: gcc -O2 -ffp-contract=off -fno-fast-math -shared -fPIC -pthread.
 */
#include <fenv.h>
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ---------------------------------------------------------------------- */
/* bf16 <-> binary32 / binary64 (IEEE definitions, round to nearest even)  */
/* ---------------------------------------------------------------------- */

/* bf16 is the top 16 bits of a binary32; widening is exact. */
static float bf16_to_f32(uint16_t h) {
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

/* Round a finite binary32 to the nearest bf16, ties to even.  Works on the
 * bit pattern: add 0x7fff plus the lowest kept bit, then truncate. */
static uint16_t f32_to_bf16(float f) {
    uint32_t u;
    memcpy(&u, &f, 4);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u); /* NaN stays NaN */
    uint32_t lsb = (u >> 16) & 1u;
    u += 0x7fffu + lsb;
    return (uint16_t)(u >> 16);
}

/* Round a binary64 directly to the nearest bf16 (ties to even), with no
 * intermediate binary32 rounding.  bf16 has 8 significant bits, exponent
 * range of binary32, subnormal spacing 2^-133. */
static uint16_t f64_to_bf16(double v) {
    if (v == 0.0) return signbit(v) ? 0x8000u : 0x0000u;
    if (isnan(v)) return 0x7fc0u;
    uint16_t sign = signbit(v) ? 0x8000u : 0x0000u;
    double a = fabs(v);
    if (isinf(a)) return sign | 0x7f80u;
    int e;
    (void)frexp(a, &e);                 /* a = m * 2^e, m in [0.5, 1) */
    /* Exponent of the leading bit is e-1; normal bf16 needs e-1 >= -126. */
    int lsb_exp = (e - 1 >= -126) ? (e - 8) : -133;
    double scaled = ldexp(a, -lsb_exp); /* exact: power-of-two scaling      */
    double r = nearbyint(scaled);       /* ties to even (FE_TONEAREST)      */
    double out = ldexp(r, lsb_exp);     /* exact                            */
    if (out > 3.3895313892515355e38) return sign | 0x7f80u; /* past bf16 max -> inf */
    float of = (float)out;              /* exact: out has <= 8 significant bits */
    uint32_t u;
    memcpy(&u, &of, 4);
    return (uint16_t)(sign | ((u >> 16) & 0x7fffu));
}

/* Exported so the tests can pin the conversions against library routines. */
float oracle_bf16_to_f32(uint16_t h) { return bf16_to_f32(h); }
uint16_t oracle_f32_to_bf16(float f) { return f32_to_bf16(f); }
uint16_t oracle_f64_to_bf16(double v) { return f64_to_bf16(v); }

/* ---------------------------------------------------------------------- */
/* Row-parallel helper: plain static partition of [0, n) over threads.     */
/* ---------------------------------------------------------------------- */

typedef void (*row_fn)(void* ctx, int64_t r0, int64_t r1);
typedef struct { row_fn fn; void* ctx; int64_t r0, r1; } row_task;

static void* run_task(void* p) {
    row_task* t = (row_task*)p;
    t->fn(t->ctx, t->r0, t->r1);
    return NULL;
}

static void parallel_rows(row_fn fn, void* ctx, int64_t n, int nthreads) {
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 256) nthreads = 256;
    if ((int64_t)nthreads > n) nthreads = (int)(n > 0 ? n : 1);
    if (nthreads == 1) { fn(ctx, 0, n); return; }
    pthread_t th[256];
    row_task task[256];
    for (int i = 0; i < nthreads; ++i) {
        task[i].fn = fn;
        task[i].ctx = ctx;
        task[i].r0 = n * i / nthreads;
        task[i].r1 = n * (i + 1) / nthreads;
        pthread_create(&th[i], NULL, run_task, &task[i]);
    }
    for (int i = 0; i < nthreads; ++i) pthread_join(th[i], NULL);
}

/* ---------------------------------------------------------------------- */
/* Q: per-row symmetric INT8 quantisation (weights per output channel =    */
/*    rows of W[N x K]; activations per token row = rows of X[M x K]).     */
/* ---------------------------------------------------------------------- */

typedef struct { const uint16_t* x; int64_t cols; int8_t* q; float* s; } quant_ctx;

static void quant_rows(void* p, int64_t r0, int64_t r1) {
    quant_ctx* c = (quant_ctx*)p;
    for (int64_t r = r0; r < r1; ++r) {
        const uint16_t* xr = c->x + r * c->cols;
        int8_t* qr = c->q + r * c->cols;
        /* 1. absolute maximum of the row (exact in binary32) */
        float a = 0.0f;
        for (int64_t k = 0; k < c->cols; ++k) {
            float v = fabsf(bf16_to_f32(xr[k]));
            if (v > a) a = v;
        }
        /* 2. degenerate rows: scale 0, all codes 0 */
        if (!(a >= 0x1p-100f)) {
            c->s[r] = 0.0f;
            for (int64_t k = 0; k < c->cols; ++k) qr[k] = 0;
            continue;
        }
        /* 3. scale and its reciprocal, each one correctly rounded division */
        float s = a / 127.0f;
        float inv = 127.0f / a;
        c->s[r] = s;
        /* 4. code = round-half-even(x * inv), clamped to the symmetric range */
        for (int64_t k = 0; k < c->cols; ++k) {
            float p = bf16_to_f32(xr[k]) * inv;
            float n = nearbyintf(p);
            if (n > 127.0f) n = 127.0f;
            if (n < -127.0f) n = -127.0f;
            qr[k] = (int8_t)(int)n;
        }
    }
}

int oracle_quantize_rows(const uint16_t* x, int64_t rows, int64_t cols, int8_t* q, float* scale,
                         int nthreads) {
    if (fegetround() != FE_TONEAREST) return -1;
    if (rows < 0 || cols < 0) return -1;
    quant_ctx c = {x, cols, q, scale};
    parallel_rows(quant_rows, &c, rows, nthreads);
    return 0;
}

/* ---------------------------------------------------------------------- */
/* QB: per-block symmetric INT8 quantisation of attention Query / Key.     */
/*    The pages (智猩猩 article, section 01.3, the attention paragraph)    */
/*    state only that Query and Key are quantised to INT8 for the sparse  */
/*    attention; block size and granularity are a reading: x holds token  */
/*    rows [B x S x H*D] (a projection's output, head h in columns        */
/*    h*D .. h*D+D-1), and one block is `block` consecutive tokens of one */
/*    sample and one head (the last block of a sample may be shorter).    */
/*    Each block is quantised with the steps of Q above, the absolute     */
/*    maximum taken over the whole block.  scale[(b*nblk + j)*H + h].     */
/* ---------------------------------------------------------------------- */

typedef struct {
    const uint16_t* x; int64_t S, H, D, block, nblk; int8_t* q; float* s;
} qblk_ctx;

static void quant_blocks(void* p, int64_t i0, int64_t i1) {
    qblk_ctx* c = (qblk_ctx*)p;
    const int64_t C = c->H * c->D;
    for (int64_t i = i0; i < i1; ++i) {          /* i = b * nblk + j: one token block */
        const int64_t b = i / c->nblk, j = i % c->nblk;
        const int64_t t0 = j * c->block;
        const int64_t t1 = t0 + c->block < c->S ? t0 + c->block : c->S;
        for (int64_t h = 0; h < c->H; ++h) {
            /* 1. absolute maximum over the block's tokens and the head's columns */
            float a = 0.0f;
            for (int64_t t = t0; t < t1; ++t)
                for (int64_t d = 0; d < c->D; ++d) {
                    float v = fabsf(bf16_to_f32(c->x[(b * c->S + t) * C + h * c->D + d]));
                    if (v > a) a = v;
                }
            float* sp = &c->s[i * c->H + h];
            /* 2. degenerate blocks: scale 0, all codes 0 */
            if (!(a >= 0x1p-100f)) {
                *sp = 0.0f;
                for (int64_t t = t0; t < t1; ++t)
                    for (int64_t d = 0; d < c->D; ++d) c->q[(b * c->S + t) * C + h * c->D + d] = 0;
                continue;
            }
            /* 3. scale and reciprocal, one correctly rounded division each */
            float s = a / 127.0f;
            float inv = 127.0f / a;
            *sp = s;
            /* 4. codes: round-half-even(x * inv), clamped */
            for (int64_t t = t0; t < t1; ++t)
                for (int64_t d = 0; d < c->D; ++d) {
                    const int64_t e = (b * c->S + t) * C + h * c->D + d;
                    float n = nearbyintf(bf16_to_f32(c->x[e]) * inv);
                    if (n > 127.0f) n = 127.0f;
                    if (n < -127.0f) n = -127.0f;
                    c->q[e] = (int8_t)(int)n;
                }
        }
    }
}

int oracle_quantize_blocks(const uint16_t* x, int64_t B, int64_t S, int64_t H, int64_t D,
                           int64_t block, int8_t* q, float* scale, int nthreads) {
    if (fegetround() != FE_TONEAREST) return -1;
    if (B < 0 || S < 0 || H < 0 || D < 0 || block < 1) return -1;
    const int64_t nblk = (S + block - 1) / block;
    qblk_ctx c = {x, S, H, D, block, nblk, q, scale};
    parallel_rows(quant_blocks, &c, B * nblk, nthreads);
    return 0;
}

/* ---------------------------------------------------------------------- */
/* I: INT8 x INT8 -> INT32 product, acc[i][j] = sum_k qa[i][k] * qw[j][k]. */
/* ---------------------------------------------------------------------- */

typedef struct { const int8_t* a; const int8_t* w; int64_t N, K; int32_t* acc; } gemm_ctx;

static void gemm_rows(void* p, int64_t r0, int64_t r1) {
    gemm_ctx* c = (gemm_ctx*)p;
    for (int64_t i = r0; i < r1; ++i) {
        const int8_t* ai = c->a + i * c->K;
        for (int64_t j = 0; j < c->N; ++j) {
            const int8_t* wj = c->w + j * c->K;
            int64_t s = 0;
            for (int64_t k = 0; k < c->K; ++k) s += (int64_t)ai[k] * (int64_t)wj[k];
            c->acc[i * c->N + j] = (int32_t)s; /* |s| <= 127*127*K fits for K <= 131072 */
        }
    }
}

int oracle_gemm_i32(const int8_t* qa, int64_t M, const int8_t* qw, int64_t N, int64_t K,
                    int32_t* acc, int nthreads) {
    if (M < 0 || N < 0 || K < 0 || K > 131072) return -1;
    gemm_ctx c = {qa, qw, N, K, acc};
    parallel_rows(gemm_rows, &c, M, nthreads);
    return 0;
}

/* ---------------------------------------------------------------------- */
/* GELU, tanh approximation: g(z) = z/2 * (1 + tanh(sqrt(2/pi)(z + 0.044715 z^3))) */
/* evaluated in binary64 on the bf16 value z, rounded once to bf16.        */
/* 1 + tanh(u) = 2 / (1 + exp(-2u)) is used so the z << 0 tail keeps its   */
/* relative accuracy instead of cancelling to zero.                        */
/* ---------------------------------------------------------------------- */

double oracle_gelu_tanh_f64(double z) {
    const double c = 0.79788456080286535587989211986876; /* sqrt(2/pi) */
    double u = c * (z + 0.044715 * z * z * z);
    return z / (1.0 + exp(-2.0 * u));
}

uint16_t oracle_gelu_bf16(uint16_t y) {
    return f64_to_bf16(oracle_gelu_tanh_f64((double)bf16_to_f32(y)));
}

/* Elementwise GELU over an array of bf16 values (h[i] = oracle_gelu_bf16(y[i])). */
typedef struct { const uint16_t* y; uint16_t* h; } gelu_ctx;

static void gelu_range(void* p, int64_t i0, int64_t i1) {
    gelu_ctx* c = (gelu_ctx*)p;
    for (int64_t i = i0; i < i1; ++i) c->h[i] = oracle_gelu_bf16(c->y[i]);
}

int oracle_gelu_rows(const uint16_t* y, int64_t n, uint16_t* h, int nthreads) {
    if (n < 0) return -1;
    gelu_ctx c = {y, h};
    parallel_rows(gelu_range, &c, n, nthreads);
    return 0;
}

/* ---------------------------------------------------------------------- */
/* E: the epilogue, once per output after the whole accumulation.          */
/* ---------------------------------------------------------------------- */

enum { ACT_NONE = 0, ACT_GELU_TANH = 1 };

typedef struct {
    const int32_t* acc; const float* sa; const float* sw; const uint16_t* bias;
    int64_t N; int act; uint16_t* y;
} epi_ctx;

static void epi_rows(void* p, int64_t r0, int64_t r1) {
    epi_ctx* c = (epi_ctx*)p;
    for (int64_t i = r0; i < r1; ++i) {
        for (int64_t j = 0; j < c->N; ++j) {
            float t = (float)c->acc[i * c->N + j]; /* int32 -> binary32, nearest even */
            float u = c->sa[i] * c->sw[j];         /* combined scale, one rounding     */
            float v = c->bias ? fmaf(t, u, bf16_to_f32(c->bias[j])) : t * u;
            uint16_t h = f32_to_bf16(v);
            if (c->act == ACT_GELU_TANH) h = oracle_gelu_bf16(h);
            c->y[i * c->N + j] = h;
        }
    }
}

int oracle_epilogue(const int32_t* acc, const float* sa, int64_t M, const float* sw, int64_t N,
                    const uint16_t* bias, int act, uint16_t* y, int nthreads) {
    if (M < 0 || N < 0 || (act != ACT_NONE && act != ACT_GELU_TANH)) return -1;
    epi_ctx c = {acc, sa, sw, bias, N, act, y};
    parallel_rows(epi_rows, &c, M, nthreads);
    return 0;
}

/* ---------------------------------------------------------------------- */
/* F: native BF16 linear (the fallback): y = bf16(sum_k x*w + b).          */
/* ---------------------------------------------------------------------- */

typedef struct {
    const uint16_t* x; const uint16_t* w; const uint16_t* bias; int64_t N, K; int act; uint16_t* y;
} bf16_ctx;

static void bf16_rows(void* p, int64_t r0, int64_t r1) {
    bf16_ctx* c = (bf16_ctx*)p;
    for (int64_t i = r0; i < r1; ++i) {
        const uint16_t* xi = c->x + i * c->K;
        for (int64_t j = 0; j < c->N; ++j) {
            const uint16_t* wj = c->w + j * c->K;
            double s = 0.0;
            for (int64_t k = 0; k < c->K; ++k)
                s += (double)bf16_to_f32(xi[k]) * (double)bf16_to_f32(wj[k]); /* exact product */
            if (c->bias) s += (double)bf16_to_f32(c->bias[j]);
            uint16_t h = f64_to_bf16(s);
            if (c->act == ACT_GELU_TANH) h = oracle_gelu_bf16(h);
            c->y[i * c->N + j] = h;
        }
    }
}

int oracle_linear_bf16(const uint16_t* x, int64_t M, int64_t K, const uint16_t* w, int64_t N,
                       const uint16_t* bias, int act, uint16_t* y, int nthreads) {
    if (M < 0 || N < 0 || K < 0 || (act != ACT_NONE && act != ACT_GELU_TANH)) return -1;
    bf16_ctx c = {x, w, bias, N, K, act, y};
    parallel_rows(bf16_rows, &c, M, nthreads);
    return 0;
}

/* ---------------------------------------------------------------------- */
/* G: the shape guard of the INT8 path.                                    */
/* ---------------------------------------------------------------------- */

int oracle_guard(int64_t N, int64_t K) {
    return (K >= 128 && K <= 131072 && K % 128 == 0 && N >= 64 && N % 64 == 0) ? 1 : 0;
}

/* ---------------------------------------------------------------------- */
/* The whole guarded linear: route by the guard, then either               */
/* quantise W (static) and X (dynamic) -> INT32 product -> epilogue, or    */
/* the BF16 fallback.  Returns the path taken (0 INT8, 1 BF16), <0 error.  */
/* ---------------------------------------------------------------------- */

int oracle_w8a8_linear(const uint16_t* x, int64_t M, int64_t K, const uint16_t* w, int64_t N,
                       const uint16_t* bias, int act, uint16_t* y, int nthreads) {
    if (M < 0 || N < 0 || K < 0) return -1;
    if (!oracle_guard(N, K)) {
        int rc = oracle_linear_bf16(x, M, K, w, N, bias, act, y, nthreads);
        return rc < 0 ? rc : 1;
    }
    int8_t* qw = (int8_t*)malloc((size_t)(N * K > 0 ? N * K : 1));
    float* sw = (float*)malloc((size_t)(N > 0 ? N : 1) * sizeof(float));
    int8_t* qx = (int8_t*)malloc((size_t)(M * K > 0 ? M * K : 1));
    float* sx = (float*)malloc((size_t)(M > 0 ? M : 1) * sizeof(float));
    int32_t* acc = (int32_t*)malloc((size_t)(M * N > 0 ? M * N : 1) * sizeof(int32_t));
    int rc = -1;
    if (qw && sw && qx && sx && acc) {
        rc = oracle_quantize_rows(w, N, K, qw, sw, nthreads);
        if (rc == 0) rc = oracle_quantize_rows(x, M, K, qx, sx, nthreads);
        if (rc == 0) rc = oracle_gemm_i32(qx, M, qw, N, K, acc, nthreads);
        if (rc == 0) rc = oracle_epilogue(acc, sx, M, sw, N, bias, act, y, nthreads);
    }
    free(qw); free(sw); free(qx); free(sx); free(acc);
    return rc < 0 ? rc : 0;
}

/* ---------------------------------------------------------------------- */
/* C: padded-row compaction.  Keeps row (b, t) of X[B x L x D] iff         */
/* mask[b*L + t] != 0, in (b, t) order; records its flat source index.     */
/* ---------------------------------------------------------------------- */

int oracle_compact_rows(const uint16_t* x, const uint8_t* mask, int64_t B, int64_t L, int64_t D,
                        uint16_t* out, int32_t* src_row, int32_t* count) {
    if (B < 0 || L < 0 || D < 0) return -1;
    int64_t m = 0;
    for (int64_t b = 0; b < B; ++b) {
        for (int64_t t = 0; t < L; ++t) {
            int64_t r = b * L + t;
            if (mask[r] != 0) {
                memcpy(out + m * D, x + r * D, (size_t)D * sizeof(uint16_t));
                src_row[m] = (int32_t)r;
                ++m;
            }
        }
    }
    *count = (int32_t)m;
    return 0;
}

/* ---------------------------------------------------------------------- */
/* NM: normalisation and modulation of each row, rounded once to bf16.     */
/*   LayerNorm (norm 0): mu = sum(x)/D, var = sum((x - mu)^2)/D            */
/*     (Ba, Kiros & Hinton 2016, without the elementwise affine);          */
/*   RMSNorm (norm 1): mu = 0, var = sum(x^2)/D (Zhang & Sennrich 2019);   */
/*   rstd = 1/sqrt(var + eps), 0 where var + eps is 0;                    */
/*   z = (x - mu) * rstd * (1 + scale[g]) + shift[g], g = row / rpc        */
/*     (adaptive-norm modulation as in DiT, Peebles & Xie 2023); NULL      */
/*     scale or shift reads as 0.                                          */
/* Every step in binary64, sums in index order; z is rounded once, from    */
/* binary64, to the nearest bf16 (ties to even).                           */
/* ---------------------------------------------------------------------- */

typedef struct {
    const uint16_t *x, *shift, *scale; int64_t cols, rpc; int norm; double eps; uint16_t* y;
} nm_ctx;

static void nm_rows(void* p, int64_t r0, int64_t r1) {
    nm_ctx* c = (nm_ctx*)p;
    const int64_t D = c->cols;
    for (int64_t r = r0; r < r1; ++r) {
        const uint16_t* xr = c->x + r * D;
        const int64_t g = r / c->rpc;
        /* 1. the row's statistics */
        double mu = 0.0;
        if (c->norm == 0) {
            double s1 = 0.0;
            for (int64_t j = 0; j < D; ++j) s1 += (double)bf16_to_f32(xr[j]);
            mu = s1 / (double)D;
        }
        double s2 = 0.0;
        for (int64_t j = 0; j < D; ++j) {
            const double d = (double)bf16_to_f32(xr[j]) - mu;
            s2 += d * d;
        }
        const double v = s2 / (double)D + c->eps;
        const double rstd = v > 0.0 ? 1.0 / sqrt(v) : 0.0;
        /* 2. normalise, modulate, round once */
        for (int64_t j = 0; j < D; ++j) {
            const double y = ((double)bf16_to_f32(xr[j]) - mu) * rstd;
            const double sc = c->scale ? (double)bf16_to_f32(c->scale[g * D + j]) : 0.0;
            const double sh = c->shift ? (double)bf16_to_f32(c->shift[g * D + j]) : 0.0;
            c->y[r * D + j] = f64_to_bf16(y * (1.0 + sc) + sh);
        }
    }
}

int oracle_norm_mod(const uint16_t* x, int64_t rows, int64_t cols, const uint16_t* shift,
                    const uint16_t* scale, int64_t rows_per_cond, int norm, double eps,
                    uint16_t* y, int nthreads) {
    if (fegetround() != FE_TONEAREST) return -1;
    if (rows < 0 || cols < 1 || rows_per_cond < 1 || (norm != 0 && norm != 1) || !(eps >= 0.0))
        return -1;
    nm_ctx c = {x, shift, scale, cols, rows_per_cond, norm, eps, y};
    parallel_rows(nm_rows, &c, rows, nthreads);
    return 0;
}
