/*
 * w8a8.h — guarded W8A8 linear layer for AMD Instinct MI355X (gfx950).
 *
 * C ABI of libw8a8.so.  The method is TurboT2VA's W8A8 linear (page "音视频
 * 生成提速54倍！浙大等团队开源联合蒸馏方案TurboT2VA", 智猩猩, section 01.3
 * "量化策略"): weights quantised statically to INT8 per output channel,
 * activations dynamically to INT8 per row, the product accumulated in INT32,
 * scale and bias applied once after the whole accumulation, and shapes the
 * INT8 kernel cannot serve falling back to native BF16.  Padded-row compaction
 * follows the closing paragraph of that section and the paperlayer.ai summary
 * (section "C. Fused Multimodal Transformer Operations"): padded text
 * positions are removed with the shared mask, every valid row kept unchanged.
 *
 * Conventions for every call:
 *   - Tensors are device pointers on the current HIP device, dense row-major.
 *     bf16 values are passed as uint16_t bit patterns.  The caller owns all
 *     memory; nothing is allocated, freed or synchronised inside the library.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Work is enqueued
 *     asynchronously; device faults surface at the caller's next sync.
 *   - Outputs must not alias inputs.  Inputs must be finite.
 *   - All argument checks run on the host before anything is launched; a
 *     failed check returns W8A8_EINVAL and launches nothing.
 *   - Zero-sized work (rows == 0, M == 0, ...) is a valid no-op returning W8A8_OK,
 *     except compact_padded_rows, which still writes *count = 0.
 */
#ifndef W8A8_H
#define W8A8_H

#include <stddef.h>
#include <stdint.h>

#if defined(__GNUC__)
#define W8A8_API __attribute__((visibility("default")))
#else
#define W8A8_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    W8A8_OK = 0,
    W8A8_EINVAL = -1,       /* bad argument: NULL, negative size, misalignment, combo */
    W8A8_EUNSUPPORTED = -2, /* shape the INT8 GEMM does not serve (see w8a8_guard)     */
    W8A8_EHIP = -3,         /* a HIP launch failed                                     */
    W8A8_ESCRATCH = -4      /* input beyond the static scratch of w8a8_linear_noalloc  */
} w8a8_status;

typedef enum { W8A8_OUT_BF16 = 0, W8A8_OUT_I32 = 1 } w8a8_out;
typedef enum { W8A8_ACT_NONE = 0, W8A8_ACT_GELU_TANH = 1 } w8a8_act;
typedef enum { W8A8_PATH_INT8 = 0, W8A8_PATH_BF16 = 1 } w8a8_path;

/* Largest K the INT8 path admits: with codes in [-127, 127] (all that
 * w8a8_quantize_rows produces), |acc| <= 127*127*K stays below 2^31. */
#define W8A8_MAX_K 131072

/*
 * Per-row symmetric INT8 quantisation (section 01.3: weights per output
 * channel — the rows of W[N x K] — statically, activations per token row
 * dynamically; the same routine serves both).
 *
 *   x     [rows x cols] bf16 input
 *   q     [rows x cols] int8 codes out
 *   scale [rows]        fp32 scale out
 *
 * For each row: a = max|x|; if a < 2^-100 then scale = 0 and every code is 0;
 * else scale = RN32(a/127), inv = RN32(127/a), q = RNE(RN32(x*inv)) clamped to
 * [-127, 127].  Dequantisation is q*scale.
 * Alignment: 2-byte for x, 1-byte for q, 4-byte for scale; 16-byte x and
 * 8-byte q with cols % 8 == 0 take the vector path.
 */
W8A8_API int w8a8_quantize_rows(const uint16_t* x, int64_t rows, int64_t cols, int8_t* q, float* scale,
                       void* stream);

/* Largest block (tokens x head_dim values) w8a8_quantize_blocks holds in registers. */
#define W8A8_MAX_BLOCK_VALUES 32768

/*
 * Per-block symmetric INT8 quantisation of attention Query / Key (section
 * 01.3, attention paragraph: the sparse attention quantises Query and Key to
 * INT8; the page gives no block size or layout, so those are the caller's).
 *
 *   x     [batch x seq x heads*head_dim] bf16 token rows (a projection's output;
 *         head h in columns h*head_dim .. h*head_dim + head_dim - 1)
 *   q     [batch x seq x heads*head_dim] int8 codes out, same layout
 *   scale [batch x ceil(seq/block) x heads] fp32 out, index (b*nblk + j)*heads + h
 *
 * A block is `block` consecutive tokens (the last block of each sample may be
 * shorter) of one sample and one head: block x head_dim values with one
 * scale, computed exactly as w8a8_quantize_rows computes a row's (a = max|x|
 * over the block; a < 2^-100 gives scale 0 and zero codes).  With block = 1
 * and heads = 1 it is w8a8_quantize_rows.
 * Requirements (W8A8_EINVAL otherwise): head_dim % 8 == 0, head_dim >= 8;
 * min(block, seq) * head_dim <= W8A8_MAX_BLOCK_VALUES; fewer than 2^31 blocks
 * (batch * ceil(seq/block) * heads); x 16-byte, q 8-byte, scale 4-byte
 * aligned.  batch, seq or heads = 0 is a no-op.
 */
W8A8_API int w8a8_quantize_blocks(const uint16_t* x, int64_t batch, int64_t seq, int64_t heads,
                                  int64_t head_dim, int64_t block, int8_t* q, float* scale,
                                  void* stream);

typedef enum { W8A8_NORM_LAYER = 0, W8A8_NORM_RMS = 1 } w8a8_norm;

/*
 * Normalisation + modulation of rows ahead of a linear layer: the
 * normalisation and modulation that the fused operators of the joint
 * Transformer take over (paperlayer.ai summary, section C).  The page names the
 * operations only; the formulas are the textbook ones:
 *
 *   x      [rows x cols] bf16 input rows
 *   shift, scale [G x cols] bf16 modulation rows, G = ceil(rows / rows_per_cond);
 *          row r takes row g = r / rows_per_cond of each (a sample's tokens share
 *          its conditioning); either may be NULL (read as 0)
 *   norm   W8A8_NORM_LAYER: mu = mean(x), var = mean((x - mu)^2) (LayerNorm
 *          without its elementwise affine);  W8A8_NORM_RMS: mu = 0,
 *          var = mean(x^2) (RMSNorm)
 *   eps    >= 0, added to var: rstd = 1/sqrt(var + eps), 0 if var + eps == 0
 *   y      [rows x cols] bf16 out: z = (x - mu) * rstd * (1 + scale[g]) + shift[g]
 *          rounded to bf16
 *
 * Precision: the value defined is z evaluated in binary64 and rounded once to
 * bf16 (nearest, ties to even).  The kernels take mu, var and rstd in binary64
 * (sums in no fixed order) and the elementwise steps in binary32:
 * d = RN32(x - mu), y' = RN32(d * RN32(rstd)), z' = fmaf(y', RN32(1 + scale[g]),
 * shift[g]), then z' to bf16.  Each output is within 1 bf16 ulp of the defined
 * value, or, where the shift cancels most of the product, within
 * ulp + 2^-21 (|P| + |shift|) of it, P = (x - mu) rstd (1 + scale).
 * Alignment: 2-byte for every bf16 pointer; 16-byte x,
 * shift, scale and y with cols % 8 == 0 and cols <= 32768 take the vector
 * path.  rows = 0 is a no-op; cols >= 1, rows_per_cond >= 1 and fewer than
 * 2^31 rows are required (W8A8_EINVAL otherwise).  y must not overlap x.
 */
W8A8_API int w8a8_norm_mod_bf16(const uint16_t* x, int64_t rows, int64_t cols,
                                const uint16_t* shift, const uint16_t* scale,
                                int64_t rows_per_cond, int norm, double eps, uint16_t* y,
                                void* stream);

/*
 * The same normalisation and modulation fused with the per-row INT8
 * quantisation of the following W8A8 linear's activations (section 01.3):
 * q [rows x cols] int8 codes and qscale [rows] fp32 are exactly
 * w8a8_quantize_rows applied to the bf16 rows w8a8_norm_mod_bf16 writes for
 * the same arguments (the same arithmetic, bit for bit); those rows themselves
 * are not written.  Requirements as w8a8_norm_mod_bf16,
 * plus qscale 4-byte aligned (8-byte q with the vector path's conditions takes
 * the vector path).
 */
W8A8_API int w8a8_norm_mod_quantize_rows(const uint16_t* x, int64_t rows, int64_t cols,
                                         const uint16_t* shift, const uint16_t* scale,
                                         int64_t rows_per_cond, int norm, double eps, int8_t* q,
                                         float* qscale, void* stream);

/*
 * Fused GELU + per-row INT8 quantisation: the input of a linear that follows a
 * GELU-tanh (the FFN down projection, whose input is the up projection's
 * output passed through GELU; the quantisation is the per-row dynamic
 * activation quantisation of section 01.3).
 *
 *   y     [rows x cols] bf16 pre-activation
 *   q     [rows x cols] int8 codes of h, scale [rows] fp32
 *
 * h = GELU-tanh(y) rounded to bf16 (the same value w8a8_gemm's
 * W8A8_ACT_GELU_TANH epilogue produces), then exactly w8a8_quantize_rows(h).
 * h itself is not written.  Same alignment rules as w8a8_quantize_rows.
 */
W8A8_API int w8a8_gelu_quantize_rows(const uint16_t* y, int64_t rows, int64_t cols, int8_t* q,
                                     float* scale, void* stream);

/*
 * Elementwise GELU-tanh on bf16 values: the activation between the halves of
 * an FFN, on its own.
 *
 *   x [n] bf16 in, y [n] bf16 out (2-byte aligned, not overlapping)
 *
 * y[i] = g(x[i]) rounded to bf16 exactly as the W8A8_ACT_GELU_TANH epilogue of
 * w8a8_gemm does (one table lookup per element).
 */
W8A8_API int w8a8_gelu_bf16(const uint16_t* x, int64_t n, uint16_t* y, void* stream);

/*
 * INT8 GEMM with INT32 accumulation and the epilogue after full accumulation
 * (section 01.3).
 *
 *   qa [M x K] int8, sa [M] fp32    quantised activations and their row scales
 *   qw [N x K] int8, sw [N] fp32    quantised weights and their channel scales
 *   bias [N] bf16 or NULL
 *   out [M x N]: out_kind == W8A8_OUT_BF16 -> bf16
 *                  y = bf16_RNE(fma(float(acc), RN32(sa[i]*sw[j]), bias[j]))
 *                  (no bias: bf16_RNE(float(acc) * RN32(sa[i]*sw[j])));
 *                  act == W8A8_ACT_GELU_TANH then applies
 *                  g(z) = z/2 (1 + tanh(sqrt(2/pi)(z + 0.044715 z^3))) to the bf16 y
 *                  and rounds g(y) once to bf16 from its binary64 value (round to
 *                  nearest even).  That is the correctly rounded value except for
 *                  |y| < 2^-125, where the binary64 value is the exact midpoint
 *                  y/2 and goes to the even neighbour.
 *                out_kind == W8A8_OUT_I32 -> the raw int32 accumulator
 *                  acc[i][j] = sum_k qa[i][k]*qw[j][k] (act must be NONE; sa, sw,
 *                  bias are ignored and may be NULL).
 * Shapes: w8a8_guard(N, K) must hold, else W8A8_EUNSUPPORTED (never a silent
 * fallback).  M is unrestricted.  qa, qw, out must be 16-byte aligned.
 * Codes: every code in qa and qw must lie in [-127, 127], the range
 * w8a8_quantize_rows produces; then the INT32 accumulator is exact for every K
 * the guard admits.  The codes are not checked: a -128 code can take |acc| to
 * 128*128*K, which for K = W8A8_MAX_K is 2^31 and wraps.
 */
W8A8_API int w8a8_gemm(const int8_t* qa, const float* sa, int64_t M, const int8_t* qw, const float* sw,
              int64_t N, int64_t K, const uint16_t* bias, int act, int out_kind, void* out,
              void* stream);

/*
 * w8a8_gemm with the K loop split across workgroups, for shapes whose tiles
 * leave most compute units idle (few rows and columns, long K: a short
 * sequence through a down projection, say).  Section 01.3 applies the scale
 * and bias once after the whole INT32 accumulation, so the accumulation may be
 * cut into K slices whose INT32 partial sums are added exactly before the
 * epilogue: the result is w8a8_gemm's, bit for bit, for every shape.
 *
 *   Arguments as w8a8_gemm, plus
 *   workspace [workspace_bytes] device memory, 16-byte aligned, at least
 *             w8a8_gemm_splitk_workspace_bytes(M, N, K) bytes; it holds the
 *             slices' INT32 partial sums (S x M x N) and is overwritten.
 * When that size is 0 the shape is not split: the call is w8a8_gemm and the
 * workspace may be NULL.  Errors as w8a8_gemm, and W8A8_EINVAL for a missing,
 * misaligned or too small workspace.
 */
W8A8_API int w8a8_gemm_splitk(const int8_t* qa, const float* sa, int64_t M, const int8_t* qw,
                              const float* sw, int64_t N, int64_t K, const uint16_t* bias, int act,
                              int out_kind, void* out, void* workspace, size_t workspace_bytes,
                              void* stream);

/* Workspace bytes w8a8_gemm_splitk needs: S * M * N * 4 for a shape cut into S
 * K slices (S = 2 .. 8: when the 128 x 128 tiles fill fewer than half of the
 * 256 compute units, as many slices as fill them, each of at least 8 K stages
 * of 128 bytes), 0 for a shape that is not split or not served.  Host only. */
W8A8_API size_t w8a8_gemm_splitk_workspace_bytes(int64_t M, int64_t N, int64_t K);

/*
 * The guarded W8A8 linear y = X W^T + b (section 01.3; paperlayer.ai section C,
 * "guarded acceleration according to architectural role and shape").
 *
 *   x [M x K] bf16, y [M x N] bf16, bias [N] bf16 or NULL
 *   If w8a8_guard(N, K): INT8 path.  qw [N x K] int8 and sw [N] fp32 (the
 *     weight prepared once with w8a8_quantize_rows) are required; x is
 *     quantised per row into the workspace, then w8a8_gemm runs.  The
 *     workspace needs w8a8_linear_workspace_bytes(M, K) bytes, 256-byte aligned.
 *   Else: BF16 path (w8a8_linear_bf16); w [N x K] bf16 is required and the
 *     workspace is unused (may be NULL).
 *   path_taken (host pointer, may be NULL) receives W8A8_PATH_INT8 or _BF16.
 */
W8A8_API int w8a8_linear(const uint16_t* x, int64_t M, int64_t K, int64_t N, const int8_t* qw,
                const float* sw, const uint16_t* w, const uint16_t* bias, int act, uint16_t* y,
                void* workspace, size_t workspace_bytes, int* path_taken, void* stream);

/* Size of the device scratch array of w8a8_linear_noalloc (64 MiB per GPU). */
#define W8A8_NOALLOC_SCRATCH_BYTES (64u << 20)

/*
 * w8a8_linear without a workspace argument, for callers that cannot allocate
 * device memory: code being captured into a HIP graph, tight serving loops,
 * harnesses that forbid hipMalloc.  Arguments, result and routing are those of
 * w8a8_linear.  The INT8 path's workspace (x's codes and row scales) is a
 * static device array of W8A8_NOALLOC_SCRATCH_BYTES in the library, one per
 * GPU, held from the first call on that GPU until the process ends; its device
 * address is looked up on that first call (hipGetSymbolAddress).  No call
 * allocates or frees anything.
 *
 * Limits: w8a8_linear_workspace_bytes(M, K) must not exceed
 * W8A8_NOALLOC_SCRATCH_BYTES (returns W8A8_ESCRATCH and launches nothing).
 * Every call on one GPU uses that GPU's array, and it keeps what the last call
 * wrote (each call writes all it reads, so nothing needs clearing): calls that
 * overlap on one GPU (on two streams, or two threads) race and must be
 * serialised by the caller.  The BF16 path uses no scratch.
 */
W8A8_API int w8a8_linear_noalloc(const uint16_t* x, int64_t M, int64_t K, int64_t N,
                                 const int8_t* qw, const float* sw, const uint16_t* w,
                                 const uint16_t* bias, int act, uint16_t* y, int* path_taken,
                                 void* stream);

/*
 * Native BF16 linear, the fallback of the guarded layer (section 01.3: branches
 * the optimised operator cannot serve run in native BF16):
 *   y = bf16_RNE(sum_k x[i][k] w[j][k] + b[j]) with fp32 accumulation, optional
 *   GELU-tanh as in w8a8_gemm.  Any M, N, K >= 0; x, w, y, bias need 2-byte
 *   alignment only (rows of any K, e.g. 2050, are allowed).
 */
W8A8_API int w8a8_linear_bf16(const uint16_t* x, int64_t M, int64_t K, const uint16_t* w, int64_t N,
                     const uint16_t* bias, int act, uint16_t* y, void* stream);

/*
 * Padded-row compaction (section 01.3 closing paragraph; paperlayer.ai section C:
 * only invalid prompt positions are removed, every valid token kept unchanged).
 *
 *   x    [B x L x D] bf16, mask [B x L] uint8 (nonzero = valid; any pattern)
 *   out  [capacity B*L x D] bf16: the valid rows, in (b, t) order, copied bit-exactly
 *   src_row [capacity B*L] int32: src_row[m] = b*L + t of output row m
 *   count   [1] int32, device memory: number of valid rows (always written)
 * The caller synchronises if it needs the count on the host.  B*L < 2^31.
 */
W8A8_API int compact_padded_rows(const uint16_t* x, const uint8_t* mask, int64_t B, int64_t L, int64_t D,
                        uint16_t* out, int32_t* src_row, int32_t* count, void* stream);

/*
 * Compaction fused with the per-row activation quantisation (section 01.3:
 * padded positions are dropped with the shared text mask, and activations are
 * quantised to INT8 per row at run time): one pass over the valid rows, which
 * are never written back in bf16.
 *
 *   x    [B x L x D] bf16, mask [B x L] uint8 (nonzero = valid; any pattern)
 *   q    [capacity B*L x D] int8, scale [capacity B*L] fp32: the valid rows, in
 *        (b, t) order, quantised exactly as w8a8_quantize_rows does
 *   src_row [capacity B*L] int32, count [1] int32 (device): as compact_padded_rows
 *
 * Equal to compact_padded_rows followed by w8a8_quantize_rows on the first
 * count rows.  Rows of q and scale past count are not written.  The INT8 GEMM
 * then runs on them (w8a8_gemm with M = count, read after a synchronisation).
 * Alignment: 2-byte x, 4-byte scale, src_row, count; 16-byte x with 8-byte q
 * and D % 8 == 0 take the vector path.  B*L < 2^31.
 */
W8A8_API int w8a8_compact_quantize_rows(const uint16_t* x, const uint8_t* mask, int64_t B,
                                        int64_t L, int64_t D, int8_t* q, float* scale,
                                        int32_t* src_row, int32_t* count, void* stream);

/* ---- host-only helpers: no GPU is touched ---- */

/* 1 if the INT8 GEMM serves (N, K): K % 128 == 0, 128 <= K <= W8A8_MAX_K,
 * N % 64 == 0, N >= 64.  0 otherwise (the linear then takes the BF16 path). */
W8A8_API int w8a8_guard(int64_t N, int64_t K);

/* Workspace bytes w8a8_linear needs on the INT8 path: M*K int8 codes rounded
 * up to 256 bytes, then M fp32 scales.  0 for M <= 0 or K <= 0. */
W8A8_API size_t w8a8_linear_workspace_bytes(int64_t M, int64_t K);

/* Static string for a status code. */
W8A8_API const char* w8a8_status_str(int status);

#ifdef __cplusplus
}
#endif
#endif /* W8A8_H */
