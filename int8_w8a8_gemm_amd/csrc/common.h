// Internal helpers shared by the gfx950 kernels of libw8a8.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

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

// GELU, tanh approximation, on a binary32 input; returns binary32.
// 1 + tanh(t) is evaluated as 2 / (1 + exp(-2t)) so large negative inputs keep
// their relative accuracy.
__device__ __forceinline__ float gelu_tanh(float z) {
    const float c = 0.7978845608028654f;  // sqrt(2/pi)
    float z3 = __fmul_rn(__fmul_rn(z, z), z);
    float t = __fmul_rn(c, __fadd_rn(z, __fmul_rn(0.044715f, z3)));
    float e = expf(-2.0f * t);
    return __fdiv_rn(z, __fadd_rn(1.0f, e));
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
int launch_quantize_rows(const uint16_t* x, int64_t rows, int64_t cols, int8_t* q, float* scale,
                         hipStream_t stream);
int launch_compact_rows(const uint16_t* x, const uint8_t* mask, int64_t R, int64_t D,
                        uint16_t* out, int32_t* src_row, int32_t* count, hipStream_t stream);
int launch_gemm_i8(const int8_t* qa, const float* sa, int64_t M, const int8_t* qw,
                   const float* sw, int64_t N, int64_t K, const uint16_t* bias, int act,
                   int out_kind, void* out, hipStream_t stream);
int launch_gemm_bf16(const uint16_t* x, int64_t M, int64_t K, const uint16_t* w, int64_t N,
                     const uint16_t* bias, int act, uint16_t* y, hipStream_t stream);
}  // namespace w8a8
