// Per-row symmetric INT8 quantisation for gfx950.
//
// TurboT2VA (智猩猩 article, section 01.3 "量化策略"): activations are quantised
// to INT8 per row at run time and weights per output channel ahead of time;
// the same per-row routine serves both.  For each row
//     a = max|x|,  scale = RN32(a/127),  inv = RN32(127/a),
//     q = RNE(RN32(x * inv)) clamped to [-127, 127],
// and rows with a < 2^-100 get scale 0 and all-zero codes.
//
// The GELU variant quantises h = GELU-tanh(x) (correctly rounded to bf16) in
// the same pass: the input of an FFN down projection, straight from the
// up projection's bf16 output, without writing h to memory.
//
// The kernel is HBM-bound (2 bytes read + 1 byte written per element).  The
// vector path keeps a whole row in registers so each element is read from HBM
// once: 16-byte loads (8 bf16 per lane per chunk, a wave moves 1 KB per
// instruction), the absmax as an integer max over sign-cleared bf16 bit
// patterns (monotone for non-negative values), a cross-lane butterfly (and an
// LDS step when several waves share a row), then 8-byte packed int8 stores.
#include "common.h"

namespace w8a8 {

namespace {

constexpr int kBlock = 256;  // 4 waves
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint32_t absmax_bits(u32x4 v) {
    // Each dword holds two bf16; clear both sign bits and take the packed
    // unsigned 16-bit maximum.
    typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
    u16x2 p0 = __builtin_bit_cast(u16x2, v.x & 0x7fff7fffu);
    u16x2 p1 = __builtin_bit_cast(u16x2, v.y & 0x7fff7fffu);
    u16x2 p2 = __builtin_bit_cast(u16x2, v.z & 0x7fff7fffu);
    u16x2 p3 = __builtin_bit_cast(u16x2, v.w & 0x7fff7fffu);
    u16x2 r = __builtin_elementwise_max(__builtin_elementwise_max(p0, p1),
                                        __builtin_elementwise_max(p2, p3));
    return max((uint32_t)r.x, (uint32_t)r.y);
}

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v = max(v, (uint32_t)__shfl_xor((int)v, off, 64));
    return v;
}

__device__ __forceinline__ int quant1(float x, float inv) {
    float r = __builtin_rintf(__fmul_rn(x, inv));  // v_rndne_f32: ties to even
    r = __builtin_fminf(__builtin_fmaxf(r, -127.0f), 127.0f);
    return (int)r;
}

// 8 bf16 -> 8 int8 packed in a uint2.
__device__ __forceinline__ uint2 quant8(u32x4 v, float inv) {
    uint32_t w[4] = {v.x, v.y, v.z, v.w};
    uint32_t o[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        int q0 = quant1(__uint_as_float(w[2 * h] << 16), inv);
        int q1 = quant1(__uint_as_float(w[2 * h] & 0xffff0000u), inv);
        int q2 = quant1(__uint_as_float(w[2 * h + 1] << 16), inv);
        int q3 = quant1(__uint_as_float(w[2 * h + 1] & 0xffff0000u), inv);
        o[h] = (uint32_t)(q0 & 0xff) | ((uint32_t)(q1 & 0xff) << 8) |
               ((uint32_t)(q2 & 0xff) << 16) | ((uint32_t)(q3 & 0xff) << 24);
    }
    return make_uint2(o[0], o[1]);
}

// GELU applied to the 8 bf16 of one chunk.
__device__ __forceinline__ u32x4 gelu8(u32x4 v) {
    u32x4 o;
#pragma unroll
    for (int i = 0; i < 4; ++i)
        o[i] = gelu_bf16_rn(v[i] & 0xffffu) | (gelu_bf16_rn(v[i] >> 16) << 16);
    return o;
}

// WPR waves cooperate on one row; each lane holds CPL 16-byte chunks.  Serves
// rows of up to WPR*64*CPL*8 elements with cols % 8 == 0.
template <int WPR, int CPL, bool GELU>
__global__ __launch_bounds__(kBlock) void quantize_rows_vec(const uint16_t* __restrict__ x,
                                                            int64_t rows, int64_t cols,
                                                            int8_t* __restrict__ q,
                                                            float* __restrict__ scale) {
    constexpr int RPB = (kBlock / 64) / WPR;  // rows per block
    __shared__ uint32_t red[kBlock / 64];
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int wr = wave % WPR;
    const int64_t row = (int64_t)blockIdx.x * RPB + wave / WPR;
    const bool live = row < rows;
    const int64_t nchunk = cols >> 3;
    const u32x4* xr = reinterpret_cast<const u32x4*>(x + (live ? row : 0) * cols);

    u32x4 v[CPL];
    uint32_t amax = 0;
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
        const int64_t ch = (int64_t)(c * WPR + wr) * 64 + lane;
        if (live && ch < nchunk) {
            v[c] = __builtin_nontemporal_load(xr + ch);
            if (GELU) v[c] = gelu8(v[c]);
        } else {
            v[c] = (u32x4){0u, 0u, 0u, 0u};
        }
        amax = max(amax, absmax_bits(v[c]));
    }
    amax = wave_max_u32(amax);
    if (WPR > 1) {
        if (lane == 0) red[wave] = amax;
        __syncthreads();
        const int w0 = wave - wr;
#pragma unroll
        for (int i = 0; i < WPR; ++i) amax = max(amax, red[w0 + i]);
    }
    if (!live) return;

    const float a = __uint_as_float(amax << 16);
    int8_t* qr = q + row * cols;
    if (!(a >= 0x1p-100f)) {
        if (wr == 0 && lane == 0) scale[row] = 0.0f;
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
            const int64_t ch = (int64_t)(c * WPR + wr) * 64 + lane;
            if (ch < nchunk) reinterpret_cast<uint2*>(qr)[ch] = make_uint2(0, 0);
        }
        return;
    }
    const float inv = __fdiv_rn(127.0f, a);
    if (wr == 0 && lane == 0) scale[row] = __fdiv_rn(a, 127.0f);
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
        const int64_t ch = (int64_t)(c * WPR + wr) * 64 + lane;
        if (ch < nchunk) {
            uint2 o = quant8(v[c], inv);
            __builtin_nontemporal_store(o.x, reinterpret_cast<uint32_t*>(qr) + 2 * ch);
            __builtin_nontemporal_store(o.y, reinterpret_cast<uint32_t*>(qr) + 2 * ch + 1);
        }
    }
}

// Any cols, any alignment: one block per row, two passes over the row.
template <bool GELU>
__global__ __launch_bounds__(kBlock) void quantize_rows_generic(const uint16_t* __restrict__ x,
                                                                int64_t rows, int64_t cols,
                                                                int8_t* __restrict__ q,
                                                                float* __restrict__ scale) {
    __shared__ uint32_t red[kBlock / 64];
    const int64_t row = blockIdx.x;
    if (row >= rows) return;
    const uint16_t* xr = x + row * cols;
    int8_t* qr = q + row * cols;
    uint32_t amax = 0;
    for (int64_t k = threadIdx.x; k < cols; k += kBlock) {
        const uint32_t h = GELU ? gelu_bf16_rn(xr[k]) : (uint32_t)xr[k];
        amax = max(amax, h & 0x7fffu);
    }
    amax = wave_max_u32(amax);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = amax;
    __syncthreads();
    amax = max(max(red[0], red[1]), max(red[2], red[3]));
    const float a = __uint_as_float(amax << 16);
    if (!(a >= 0x1p-100f)) {
        if (threadIdx.x == 0) scale[row] = 0.0f;
        for (int64_t k = threadIdx.x; k < cols; k += kBlock) qr[k] = 0;
        return;
    }
    const float inv = __fdiv_rn(127.0f, a);
    if (threadIdx.x == 0) scale[row] = __fdiv_rn(a, 127.0f);
    for (int64_t k = threadIdx.x; k < cols; k += kBlock) {
        const uint32_t h = GELU ? gelu_bf16_rn(xr[k]) : (uint32_t)xr[k];
        qr[k] = (int8_t)quant1(__uint_as_float(h << 16), inv);
    }
}

template <int WPR, int CPL>
hipError_t launch_vec(const uint16_t* x, int64_t rows, int64_t cols, int8_t* q, float* scale,
                      hipStream_t stream, bool gelu) {
    constexpr int RPB = (kBlock / 64) / WPR;
    const int64_t blocks = (rows + RPB - 1) / RPB;
    if (gelu)
        hipLaunchKernelGGL((quantize_rows_vec<WPR, CPL, true>), dim3((unsigned)blocks), dim3(kBlock),
                           0, stream, x, rows, cols, q, scale);
    else
        hipLaunchKernelGGL((quantize_rows_vec<WPR, CPL, false>), dim3((unsigned)blocks),
                           dim3(kBlock), 0, stream, x, rows, cols, q, scale);
    return hipGetLastError();
}

}  // namespace

int launch_quantize_rows(const uint16_t* x, int64_t rows, int64_t cols, int8_t* q, float* scale,
                         hipStream_t stream, bool gelu) {
    if (rows == 0) return 0;
    const bool vec = (cols % 8 == 0) && (reinterpret_cast<uintptr_t>(x) % 16 == 0) &&
                     (reinterpret_cast<uintptr_t>(q) % 8 == 0) && cols > 0;
    const int64_t nchunk = cols / 8;
    hipError_t e;
    if (vec && nchunk <= 64) e = launch_vec<1, 1>(x, rows, cols, q, scale, stream, gelu);
    else if (vec && nchunk <= 128) e = launch_vec<1, 2>(x, rows, cols, q, scale, stream, gelu);
    else if (vec && nchunk <= 256) e = launch_vec<1, 4>(x, rows, cols, q, scale, stream, gelu);
    else if (vec && nchunk <= 512) e = launch_vec<1, 8>(x, rows, cols, q, scale, stream, gelu);
    else if (vec && nchunk <= 1024) e = launch_vec<2, 8>(x, rows, cols, q, scale, stream, gelu);
    else if (vec && nchunk <= 2048) e = launch_vec<4, 8>(x, rows, cols, q, scale, stream, gelu);
    else if (vec && nchunk <= 4096) e = launch_vec<4, 16>(x, rows, cols, q, scale, stream, gelu);
    else {
        if (gelu)
            hipLaunchKernelGGL(quantize_rows_generic<true>, dim3((unsigned)rows), dim3(kBlock), 0,
                               stream, x, rows, cols, q, scale);
        else
            hipLaunchKernelGGL(quantize_rows_generic<false>, dim3((unsigned)rows), dim3(kBlock), 0,
                               stream, x, rows, cols, q, scale);
        e = hipGetLastError();
    }
    return e == hipSuccess ? 0 : -1;
}

}  // namespace w8a8
