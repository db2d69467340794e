/*
 * Runs the CPU oracle (oracle/oracle.c) under AddressSanitizer and
 * UndefinedBehaviorSanitizer: the hand-worked fixtures of tests/golden/, then
 * every entry point on ragged shapes with exact-size heap buffers (so any read
 * or write past an array is reported), one and several threads, degenerate
 * sizes and rejected arguments.  Built and run by tests/test_oracle_sanitize.py:
 *
 *   gcc -O1 -g -fsanitize=address,undefined -fno-sanitize-recover=all
 *       -ffp-contract=off -pthread oracle/oracle.c tests/c/oracle_sanitize.c -lm
 *   ./a.out tests/golden
 *
 * Exit status 0 when every check holds; a sanitizer report aborts the run.
 * The fixtures' formats are described in their own headers.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int oracle_quantize_rows(const uint16_t* x, int64_t rows, int64_t cols, int8_t* q, float* scale,
                         int nthreads);
int oracle_quantize_blocks(const uint16_t* x, int64_t B, int64_t S, int64_t H, int64_t D,
                           int64_t block, int8_t* q, float* scale, int nthreads);
int oracle_gemm_i32(const int8_t* qa, int64_t M, const int8_t* qw, int64_t N, int64_t K,
                    int32_t* acc, int nthreads);
int oracle_epilogue(const int32_t* acc, const float* sa, int64_t M, const float* sw, int64_t N,
                    const uint16_t* bias, int act, uint16_t* y, int nthreads);
int oracle_linear_bf16(const uint16_t* x, int64_t M, int64_t K, const uint16_t* w, int64_t N,
                       const uint16_t* bias, int act, uint16_t* y, int nthreads);
int oracle_w8a8_linear(const uint16_t* x, int64_t M, int64_t K, const uint16_t* w, int64_t N,
                       const uint16_t* bias, int act, uint16_t* y, int nthreads);
int oracle_compact_rows(const uint16_t* x, const uint8_t* mask, int64_t B, int64_t L, int64_t D,
                        uint16_t* out, int32_t* src_row, int32_t* count);
int oracle_norm_mod(const uint16_t* x, int64_t rows, int64_t cols, const uint16_t* shift,
                    const uint16_t* scale, int64_t rows_per_cond, int norm, double eps,
                    uint16_t* y, int nthreads);
int oracle_gelu_rows(const uint16_t* y, int64_t n, uint16_t* h, int nthreads);
int oracle_guard(int64_t N, int64_t K);
float oracle_bf16_to_f32(uint16_t h);
uint16_t oracle_f32_to_bf16(float f);
uint16_t oracle_f64_to_bf16(double v);
uint16_t oracle_gelu_bf16(uint16_t y);

static int failures = 0;
static int checks = 0;

#define CHECK(cond, ...)                                   \
    do {                                                   \
        ++checks;                                          \
        if (!(cond)) {                                     \
            fprintf(stderr, "FAIL %s:%d: ", __FILE__, __LINE__); \
            fprintf(stderr, __VA_ARGS__);                  \
            fputc('\n', stderr);                           \
            ++failures;                                    \
        }                                                  \
    } while (0)

/* exact-size heap buffer (never zero bytes, so malloc never returns NULL on 0) */
static void* xalloc(size_t n) {
    void* p = malloc(n ? n : 1);
    if (!p) {
        fprintf(stderr, "out of memory\n");
        exit(2);
    }
    return p;
}

/* ---- fixture parsing ---- */

#define MAXV 4096
#define MAXF 8

/* Splits a line at ';' into at most MAXF trimmed fields; returns the count. */
static int split_fields(char* line, char** f) {
    int n = 0;
    char* p = line;
    while (n < MAXF) {
        f[n++] = p;
        char* s = strchr(p, ';');
        if (!s) break;
        *s = 0;
        p = s + 1;
    }
    return n;
}

/* Parses whitespace-separated numbers (C syntax, hex floats included; "v*n"
 * repeats v n times) into out; returns the count, -1 for "-" or "none". */
static int parse_vals(const char* field, double* out) {
    char buf[65536];
    strncpy(buf, field, sizeof buf - 1);
    buf[sizeof buf - 1] = 0;
    int n = 0;
    for (char* t = strtok(buf, " \t\r\n"); t; t = strtok(NULL, " \t\r\n")) {
        if (!strcmp(t, "-") || !strcmp(t, "none")) return -1;
        char* star = strchr(t, '*');
        long rep = 1;
        if (star) {
            *star = 0;
            rep = strtol(star + 1, NULL, 10);
        }
        double v = strtod(t, NULL);
        for (long i = 0; i < rep && n < MAXV; ++i) out[n++] = v;
    }
    return n;
}

/* bf16 bits of a value that must be exactly a bf16 number */
static uint16_t exact_bf16(double v) {
    float f = (float)v;
    uint32_t u;
    memcpy(&u, &f, 4);
    CHECK((double)f == v && (u & 0xffffu) == 0, "fixture value %.17g is not a bf16 number", v);
    return (uint16_t)(u >> 16);
}

static FILE* open_golden(const char* dir, const char* name) {
    char path[4096];
    snprintf(path, sizeof path, "%s/%s", dir, name);
    FILE* f = fopen(path, "r");
    if (!f) {
        fprintf(stderr, "cannot open %s\n", path);
        exit(2);
    }
    return f;
}

static int next_case(FILE* f, char* line, size_t cap) {
    while (fgets(line, (int)cap, f)) {
        char* p = line;
        while (*p == ' ' || *p == '\t') ++p;
        if (*p == '#' || *p == '\n' || *p == '\r' || *p == 0) continue;
        return 1;
    }
    return 0;
}

static float scale_of(double absmax) {
    return absmax >= 0x1p-100 ? (float)absmax / 127.0f : 0.0f;
}

static void golden_quantize_rows(const char* dir) {
    FILE* f = open_golden(dir, "quantize_rows.txt");
    static char line[1 << 17];
    static double xs[MAXV], qs[MAXV], am[MAXV];
    int cases = 0;
    while (next_case(f, line, sizeof line)) {
        char* fl[MAXF];
        if (split_fields(line, fl) != 3) continue;
        int n = parse_vals(fl[0], xs), nq = parse_vals(fl[1], qs);
        parse_vals(fl[2], am);
        CHECK(n == nq && n > 0, "quantize_rows fixture %d: %d values, %d codes", cases, n, nq);
        uint16_t* x = xalloc((size_t)n * 2);
        int8_t* q = xalloc((size_t)n);
        float* s = xalloc(4);
        for (int i = 0; i < n; ++i) x[i] = exact_bf16(xs[i]);
        CHECK(oracle_quantize_rows(x, 1, n, q, s, 1) == 0, "quantize_rows rc");
        for (int i = 0; i < n; ++i)
            CHECK(q[i] == (int)qs[i], "quantize_rows fixture %d code %d: %d != %g", cases, i, q[i], qs[i]);
        CHECK(s[0] == scale_of(am[0]), "quantize_rows fixture %d scale", cases);
        free(x), free(q), free(s);
        ++cases;
    }
    fclose(f);
    CHECK(cases >= 5, "quantize_rows: only %d fixtures", cases);
}

static void golden_quantize_blocks(const char* dir) {
    FILE* f = open_golden(dir, "quantize_blocks.txt");
    static char line[1 << 17];
    static double hd[8], xs[MAXV], qs[MAXV], am[MAXV];
    int cases = 0;
    while (next_case(f, line, sizeof line)) {
        char* fl[MAXF];
        if (split_fields(line, fl) != 4) continue;
        parse_vals(fl[0], hd);
        const int64_t B = (int64_t)hd[0], S = (int64_t)hd[1], H = (int64_t)hd[2], D = (int64_t)hd[3],
                      blk = (int64_t)hd[4];
        const int64_t nblk = (S + blk - 1) / blk, n = B * S * H * D;
        int nx = parse_vals(fl[1], xs), nq = parse_vals(fl[2], qs), na = parse_vals(fl[3], am);
        CHECK(nx == n && nq == n && na == B * nblk * H, "quantize_blocks fixture %d sizes", cases);
        if (nx != n || nq != n || na != B * nblk * H) continue;
        uint16_t* x = xalloc((size_t)n * 2);
        int8_t* q = xalloc((size_t)n);
        float* s = xalloc((size_t)(B * nblk * H) * 4);
        for (int64_t i = 0; i < n; ++i) x[i] = exact_bf16(xs[i]);
        CHECK(oracle_quantize_blocks(x, B, S, H, D, blk, q, s, 2) == 0, "quantize_blocks rc");
        for (int64_t i = 0; i < n; ++i)
            CHECK(q[i] == (int)qs[i], "quantize_blocks fixture %d code %ld", cases, (long)i);
        for (int64_t i = 0; i < B * nblk * H; ++i)
            CHECK(s[i] == scale_of(am[i]), "quantize_blocks fixture %d scale %ld", cases, (long)i);
        free(x), free(q), free(s);
        ++cases;
    }
    fclose(f);
    CHECK(cases >= 1, "quantize_blocks: no fixtures");
}

static void golden_epilogue(const char* dir) {
    FILE* f = open_golden(dir, "epilogue.txt");
    static char line[1 << 16];
    static double v[5][MAXV];
    int cases = 0;
    while (next_case(f, line, sizeof line)) {
        char* fl[MAXF];
        if (split_fields(line, fl) != 5) continue;
        int nb = 0;
        for (int i = 0; i < 5; ++i) {
            int c = parse_vals(fl[i], v[i]);
            if (i == 3) nb = c;
        }
        int32_t acc = (int32_t)v[0][0];
        float sa = (float)v[1][0], sw = (float)v[2][0];
        uint16_t b = nb > 0 ? exact_bf16(v[3][0]) : 0;
        uint16_t y = 0, want = exact_bf16(v[4][0]);
        CHECK(oracle_epilogue(&acc, &sa, 1, &sw, 1, nb > 0 ? &b : NULL, 0, &y, 1) == 0, "epilogue rc");
        CHECK(y == want, "epilogue fixture %d: %04x != %04x", cases, y, want);
        ++cases;
    }
    fclose(f);
    CHECK(cases >= 5, "epilogue: only %d fixtures", cases);
}

static void golden_norm_mod(const char* dir) {
    FILE* f = open_golden(dir, "norm_mod.txt");
    static char line[1 << 17];
    static double xs[MAXV], sc[MAXV], sh[MAXV], ys[MAXV];
    int cases = 0;
    while (next_case(f, line, sizeof line)) {
        char* fl[MAXF];
        if (split_fields(line, fl) != 5) continue;
        char norm[8] = {0};
        double eps = 0;
        long rpc = 0, D = 0;
        if (sscanf(fl[0], "%7s %lf %ld %ld", norm, &eps, &rpc, &D) != 4) continue;
        int nx = parse_vals(fl[1], xs), ns = parse_vals(fl[2], sc), nh = parse_vals(fl[3], sh),
            ny = parse_vals(fl[4], ys);
        CHECK(nx == ny && nx % D == 0, "norm_mod fixture %d sizes", cases);
        const int64_t R = nx / D;
        uint16_t* x = xalloc((size_t)nx * 2);
        uint16_t* y = xalloc((size_t)nx * 2);
        uint16_t* s = ns > 0 ? xalloc((size_t)ns * 2) : NULL;
        uint16_t* h = nh > 0 ? xalloc((size_t)nh * 2) : NULL;
        for (int i = 0; i < nx; ++i) x[i] = exact_bf16(xs[i]);
        for (int i = 0; i < ns; ++i) s[i] = exact_bf16(sc[i]);
        for (int i = 0; i < nh; ++i) h[i] = exact_bf16(sh[i]);
        CHECK(oracle_norm_mod(x, R, D, h, s, rpc, strcmp(norm, "RMS") == 0, eps, y, 1) == 0,
              "norm_mod rc");
        for (int i = 0; i < nx; ++i)
            CHECK(y[i] == exact_bf16(ys[i]), "norm_mod fixture %d value %d", cases, i);
        free(x), free(y), free(s), free(h);
        ++cases;
    }
    fclose(f);
    CHECK(cases >= 5, "norm_mod: only %d fixtures", cases);
}

/* ---- every entry point on ragged shapes ---- */

static uint64_t rng_state = 0x9E3779B97F4A7C15ull;
static uint64_t next_u64(void) { /* splitmix64 */
    uint64_t z = (rng_state += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}
static double uniform(void) { return (double)(next_u64() >> 11) * 0x1p-53; }
static uint16_t rand_bf16(double scale) {
    double v = (uniform() * 2.0 - 1.0) * scale;
    return oracle_f32_to_bf16((float)v);
}

static void exercise(void) {
    static const int64_t shapes[][3] = {{1, 1, 1}, {3, 7, 5}, {7, 13, 64}, {16, 64, 130}, {5, 129, 257}};
    for (size_t si = 0; si < sizeof shapes / sizeof shapes[0]; ++si) {
        const int64_t M = shapes[si][0], N = shapes[si][1], K = shapes[si][2];
        uint16_t* x = xalloc((size_t)(M * K) * 2);
        uint16_t* w = xalloc((size_t)(N * K) * 2);
        uint16_t* b = xalloc((size_t)N * 2);
        for (int64_t i = 0; i < M * K; ++i) x[i] = rand_bf16(3.0);
        for (int64_t i = 0; i < N * K; ++i) w[i] = rand_bf16(0.05);
        for (int64_t i = 0; i < N; ++i) b[i] = rand_bf16(0.1);
        int8_t* qx = xalloc((size_t)(M * K));
        int8_t* qw = xalloc((size_t)(N * K));
        float* sx = xalloc((size_t)M * 4);
        float* sw = xalloc((size_t)N * 4);
        int32_t* acc = xalloc((size_t)(M * N) * 4);
        uint16_t* y = xalloc((size_t)(M * N) * 2);
        for (int th = 1; th <= 3; th += 2) {
            CHECK(oracle_quantize_rows(x, M, K, qx, sx, th) == 0, "quantize_rows");
            CHECK(oracle_quantize_rows(w, N, K, qw, sw, th) == 0, "quantize_rows w");
            for (int64_t i = 0; i < M * K; ++i) CHECK(qx[i] >= -127 && qx[i] <= 127, "code range");
            CHECK(oracle_gemm_i32(qx, M, qw, N, K, acc, th) == 0, "gemm_i32");
            for (int act = 0; act <= 1; ++act) {
                CHECK(oracle_epilogue(acc, sx, M, sw, N, b, act, y, th) == 0, "epilogue");
                CHECK(oracle_epilogue(acc, sx, M, sw, N, NULL, act, y, th) == 0, "epilogue no bias");
                CHECK(oracle_linear_bf16(x, M, K, w, N, b, act, y, th) == 0, "linear_bf16");
                CHECK(oracle_w8a8_linear(x, M, K, w, N, b, act, y, th) >= 0, "w8a8_linear");
            }
            uint16_t* g = xalloc((size_t)(M * K) * 2);
            CHECK(oracle_gelu_rows(x, M * K, g, th) == 0, "gelu_rows");
            for (int norm = 0; norm <= 1; ++norm) {
                const int64_t rpc = M > 1 ? M - 1 : 1, G = (M + rpc - 1) / rpc;
                uint16_t* sh = xalloc((size_t)(G * K) * 2);
                uint16_t* sc = xalloc((size_t)(G * K) * 2);
                for (int64_t i = 0; i < G * K; ++i) sh[i] = rand_bf16(0.3), sc[i] = rand_bf16(0.3);
                CHECK(oracle_norm_mod(x, M, K, sh, sc, rpc, norm, 1e-6, g, th) == 0, "norm_mod");
                CHECK(oracle_norm_mod(x, M, K, NULL, NULL, rpc, norm, 0.0, g, th) == 0, "norm_mod");
                free(sh), free(sc);
            }
            free(g);
            /* quantize_blocks: the rows as [B x S x H*D] token rows */
            if (K % 2 == 0) {
                const int64_t H = 2, D = K / 2;
                for (int64_t blk = 1; blk <= 4; blk += 3) {
                    const int64_t nblk = (M + blk - 1) / blk;
                    float* sb = xalloc((size_t)(nblk * H) * 4);
                    CHECK(oracle_quantize_blocks(x, 1, M, H, D, blk, qx, sb, th) == 0, "blocks");
                    free(sb);
                }
            }
        }
        /* compaction: random, all-valid and empty masks over [M x N x K] */
        for (int kind = 0; kind < 3; ++kind) {
            const int64_t B = M, L = N, D = K;
            uint16_t* xc = xalloc((size_t)(B * L * D) * 2);
            uint8_t* mask = xalloc((size_t)(B * L));
            uint16_t* out = xalloc((size_t)(B * L * D) * 2);
            int32_t* src = xalloc((size_t)(B * L) * 4);
            int32_t cnt = -1;
            int64_t want = 0;
            for (int64_t i = 0; i < B * L * D; ++i) xc[i] = (uint16_t)next_u64();
            for (int64_t i = 0; i < B * L; ++i) {
                mask[i] = kind == 0 ? (uint8_t)(next_u64() & 1) * (uint8_t)(1 + (next_u64() % 255))
                                    : (kind == 1 ? 1 : 0);
                want += mask[i] != 0;
            }
            CHECK(oracle_compact_rows(xc, mask, B, L, D, out, src, &cnt) == 0, "compact");
            CHECK(cnt == want, "compact count %d != %ld", cnt, (long)want);
            for (int32_t m = 0; m < cnt; ++m) {
                CHECK(mask[src[m]] != 0 && (m == 0 || src[m] > src[m - 1]), "compact order");
                CHECK(!memcmp(out + (int64_t)m * D, xc + (int64_t)src[m] * D, (size_t)D * 2),
                      "compact copy");
            }
            free(xc), free(mask), free(out), free(src);
        }
        free(x), free(w), free(b), free(qx), free(qw), free(sx), free(sw), free(acc), free(y);
    }
    /* degenerate sizes */
    int32_t cnt = -1;
    CHECK(oracle_compact_rows(NULL, NULL, 0, 5, 3, NULL, NULL, &cnt) == 0 && cnt == 0, "empty compact");
    CHECK(oracle_quantize_rows(NULL, 0, 8, NULL, NULL, 2) == 0, "zero rows");
    CHECK(oracle_gemm_i32(NULL, 0, NULL, 0, 0, NULL, 2) == 0, "empty gemm");
    /* rejected arguments: nothing is touched */
    CHECK(oracle_quantize_rows(NULL, -1, 8, NULL, NULL, 1) < 0, "negative rows");
    CHECK(oracle_gemm_i32(NULL, 1, NULL, 1, 131072 + 128, NULL, 1) < 0, "K beyond the bound");
    CHECK(oracle_norm_mod(NULL, 1, 0, NULL, NULL, 1, 0, 0.0, NULL, 1) < 0, "zero cols");
    CHECK(oracle_norm_mod(NULL, 1, 4, NULL, NULL, 1, 0, -1.0, NULL, 1) < 0, "negative eps");
    CHECK(oracle_epilogue(NULL, NULL, 1, NULL, 1, NULL, 7, NULL, 1) < 0, "bad act");
    CHECK(oracle_guard(4096, 4096) == 1 && oracle_guard(4100, 4096) == 0 &&
          oracle_guard(2048, 2050) == 0, "guard");
    /* conversions over every bf16 pattern: widening then narrowing is the identity
     * on finite values; GELU of every pattern runs */
    for (uint32_t hbits = 0; hbits < 0x10000u; ++hbits) {
        const float f = oracle_bf16_to_f32((uint16_t)hbits);
        if (isfinite(f)) {
            CHECK(oracle_f32_to_bf16(f) == hbits, "f32 round trip %04x", hbits);
            CHECK(oracle_f64_to_bf16((double)f) == hbits, "f64 round trip %04x", hbits);
            (void)oracle_gelu_bf16((uint16_t)hbits);
        }
    }
}

int main(int argc, char** argv) {
    if (argc != 2) {
        fprintf(stderr, "usage: %s GOLDEN_DIR\n", argv[0]);
        return 2;
    }
    golden_quantize_rows(argv[1]);
    golden_quantize_blocks(argv[1]);
    golden_epilogue(argv[1]);
    golden_norm_mod(argv[1]);
    exercise();
    printf("%d checks, %d failures\n", checks, failures);
    return failures ? 1 : 0;
}
