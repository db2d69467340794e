// Internal helpers shared by the gfx950 kernels of libw8a8.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

namespace w8a8 {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

// bf16 bit pattern -> binary32 (exact).
__device__ __forceinline__ float bf16_bits_to_float(uint32_t h) {
    return __uint_as_float(h << 16);
}

// binary32 -> bf16 bit pattern, round to nearest even (finite inputs; NaN kept NaN).
__device__ __forceinline__ uint32_t float_to_bf16_bits(float f) {
    uint32_t u = __float_as_uint(f);
    uint32_t r = (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
    return ((u & 0x7fffffffu) > 0x7f800000u) ? ((u >> 16) | 0x40u) : r;
}

// GELU, tanh approximation, g(z) = z/2 (1 + tanh(sqrt(2/pi) (z + 0.044715 z^3))),
// evaluated on a bf16 input and rounded once to bf16 from its binary64 value:
// the correctly rounded result, except for |z| < 2^-125, where the binary64
// value is the exact midpoint z/2 and the tie goes to even.
//
// 1 + tanh(u) = 2 / (1 + exp(-2u)), so g(z) = z / (1 + 2^w) with
// w = -2 log2(e) sqrt(2/pi) (z + 0.044715 z^3), which keeps relative accuracy
// for z << 0.  Fast path in binary32: w from z^2 and two constants, 2^w with
// v_exp_f32 and the reciprocal with v_rcp_f32 (1 ulp each).  Its error is at
// most 2.8|w| + 3 binary32 ulps of g; when the low 16 bits of the binary32
// result are within 16 + 4|w| ulps of the bf16 rounding midpoint (0x8000),
// or w > 100 (results near the bottom of the exponent range), the value is
// recomputed in binary64 and rounded directly to bf16.
__device__ __forceinline__ uint32_t f64_to_bf16_bits(double v) {
    const uint64_t u = __double_as_longlong(v);
    const uint32_t sign = (uint32_t)(u >> 48) & 0x8000u;
    const double a = fabs(v);
    if (!(a < 3.4e38)) return sign | (a == a ? 0x7f80u : 0x7fc0u);  // inf / NaN
    if (a >= 0x1p-126) {
        // keep 8 significant bits: round the binary64 mantissa at bit 45, ties to even
        uint64_t m = u & 0x7fffffffffffffffull;
        m += ((1ull << 44) - 1) + ((m >> 45) & 1);
        m &= ~((1ull << 45) - 1);
        const float f = (float)__longlong_as_double((long long)m);  // exact
        const uint32_t fb = __float_as_uint(f);
        return sign | ((fb >> 16) & 0x7fffu);  // 0x7f80 if it rounded past the max
    }
    // bf16 subnormal: spacing 2^-133; the integer multiple is the encoding
    const double r = rint(a * 0x1p133);
    return sign | (uint32_t)r;
}

__device__ __forceinline__ uint32_t gelu_bf16_rn(uint32_t hbits) {
    const float z = __uint_as_float(hbits << 16);
    // -2 log2(e) sqrt(2/pi) * {1, 0.044715}
    const float B = -2.3022082f, A = -0.10294324f;
    const float t = __fmul_rn(z, z);
    const float p = __builtin_fmaf(t, A, B);
    const float w = __fmul_rn(p, z);
    const float e = __builtin_amdgcn_exp2f(w);
    const float r = __builtin_amdgcn_rcpf(__fadd_rn(1.0f, e));
    const float g = __fmul_rn(z, r);
    const uint32_t gb = __float_as_uint(g);
    const int dist = abs((int)(gb & 0xffffu) - 0x8000);
    const float margin = 16.0f + 4.0f * fabsf(w);
    if (w > 100.0f || !((float)dist > margin)) {
        const double zd = (double)z;
        const double u = 0.79788456080286535588 * (zd + 0.044715 * zd * zd * zd);
        return f64_to_bf16_bits(zd / (1.0 + exp(-2.0 * u)));
    }
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    bf16x2 v = {(__bf16)g, (__bf16)0.0f};
    return __builtin_bit_cast(uint32_t, v) & 0xffffu;
}

// Two binary32 values -> two bf16 (round to nearest even) packed low/high in a
// dword; gfx950 does this in one v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    bf16x2 v = {(__bf16)lo, (__bf16)hi};
    return __builtin_bit_cast(uint32_t, v);
}

}  // namespace w8a8

// Host-side launchers (defined in the .hip files, called by the C-ABI layer).
namespace w8a8 {
// Compute units of the current device, queried once per device (-1 on error).
inline int cu_count() {
    constexpr int kMaxDevices = 64;
    static std::atomic<int> cached[kMaxDevices];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return -1;
    if (dev < kMaxDevices) {
        const int v = cached[dev].load(std::memory_order_relaxed);
        if (v > 0) return v;
    }
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        cus <= 0)
        return -1;
    if (dev < kMaxDevices) cached[dev].store(cus, std::memory_order_relaxed);
    return cus;
}
int launch_gelu_bf16(const uint16_t* x, int64_t n, uint16_t* y, hipStream_t stream);
int launch_quantize_rows(const uint16_t* x, int64_t rows, int64_t cols, int8_t* q, float* scale,
                         hipStream_t stream, bool gelu = false);
int launch_quantize_blocks(const uint16_t* x, int64_t B, int64_t S, int64_t H, int64_t D,
                           int64_t block, int8_t* q, float* scale, hipStream_t stream);
// Normalisation + modulation of rows; q != NULL: fused with the per-row
// quantisation (codes q, scales qscale), else the bf16 rows y.
int launch_norm_mod(const uint16_t* x, int64_t rows, int64_t cols, const uint16_t* shift,
                    const uint16_t* scale, int64_t rows_per_cond, int norm, double eps, int8_t* q,
                    float* qscale, uint16_t* y, hipStream_t stream);
int launch_compact_rows(const uint16_t* x, const uint8_t* mask, int64_t R, int64_t D,
                        uint16_t* out, int32_t* src_row, int32_t* count, hipStream_t stream);
// Compaction up to this many rows takes one launch (its per-block prefix
// rescans at most that many mask bytes); more rows take the linear-time path.
bool compact_single_pass(int64_t R);
// The linear-time path's scan: src_row and *count from the mask, with up to
// scratch_ints int32 of scratch for the chunk counts (memory of an output that
// only a later launch writes).
int launch_compact_scan(const uint8_t* mask, int64_t R, int32_t* scratch, int64_t scratch_ints,
                        int32_t* src_row, int32_t* count, hipStream_t stream);
int launch_compact_quantize_rows(const uint16_t* x, const uint8_t* mask, int64_t R, int64_t D,
                                 int8_t* q, float* scale, int32_t* src_row, int32_t* count,
                                 hipStream_t stream);
int launch_gemm_i8(const int8_t* qa, const float* sa, int64_t M, const int8_t* qw,
                   const float* sw, int64_t N, int64_t K, const uint16_t* bias, int act,
                   int out_kind, void* out, hipStream_t stream);
// Split-K of the INT8 GEMM across workgroups (K slices of 128 x 128 tiles, exact
// INT32 sum of the slices, then the epilogue): slices for a shape (1: not
// split), the workspace it needs, and the launch (falls back to
// launch_gemm_i8 when the shape is not split).
int splitk_slices(int64_t M, int64_t N, int64_t K);
size_t splitk_workspace_bytes(int64_t M, int64_t N, int64_t K);
int launch_gemm_i8_splitk(const int8_t* qa, const float* sa, int64_t M, const int8_t* qw,
                          const float* sw, int64_t N, int64_t K, const uint16_t* bias, int act,
                          int out_kind, void* out, void* workspace, hipStream_t stream);
int launch_gemm_bf16(const uint16_t* x, int64_t M, int64_t K, const uint16_t* w, int64_t N,
                     const uint16_t* bias, int act, uint16_t* y, hipStream_t stream);
// The tiled MFMA path for BF16 operands (gemm_tiled.hip) and the shapes it serves.
bool gemm_bf16_tiled_ok(const uint16_t* x, int64_t K, const uint16_t* w);
int launch_gemm_bf16_tiled(const uint16_t* x, int64_t M, int64_t K, const uint16_t* w, int64_t N,
                           const uint16_t* bias, int act, uint16_t* y, hipStream_t stream);
}  // namespace w8a8
