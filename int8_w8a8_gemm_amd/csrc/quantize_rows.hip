// Per-row symmetric INT8 quantisation for gfx950.
//
// TurboT2VA (智猩猩 article, section 01.3 "量化策略"): activations are quantised
// to INT8 per row at run time and weights per output channel ahead of time;
// the same per-row routine serves both.  For each row
//     a = max|x|,  scale = RN32(a/127),  inv = RN32(127/a),
//     q = RNE(RN32(x * inv)) clamped to [-127, 127],
// and rows with a < 2^-100 get scale 0 and all-zero codes.
//
// The GELU variant quantises h = GELU-tanh(x) (rounded once to bf16 from its
// binary64 value) in the same pass: the input of an FFN down projection,
// straight from the up projection's bf16 output, without writing h to memory.
// Large inputs take a table-driven kernel: GELU of a bf16 input has only 65536
// possible values, so a 128 KB table (built with the library, see
// gen_gelu_table.c) sits in each CU's LDS and GELU becomes one LDS lookup per
// element instead of ~20 VALU instructions; that kernel is HBM-bound.
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
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

// 16 bytes at byte offset off of a row of `bytes` bytes at p, read through a
// buffer resource: zeros past the row's end, and for p == NULL, with no branch
// (AUX: cache policy bits).  p must be wave-uniform.
#if defined(__HIP_DEVICE_COMPILE__)
typedef __amdgpu_buffer_rsrc_t rsrc_t;
#endif
template <int AUX>
__device__ __forceinline__ u32x4 load16_row(const void* p, int bytes, int off) {
#if defined(__HIP_DEVICE_COMPILE__)
    const rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0,
                                                      p ? bytes : 0, 0x00020000);
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, AUX));
#else
    (void)p; (void)bytes; (void)off;
    return (u32x4){0u, 0u, 0u, 0u};
#endif
}

// GELU-tanh of every bf16 bit pattern, as bf16 bits (generated at build time).
__device__ __attribute__((aligned(16))) const uint16_t kGeluTable[65536] = {
#include "gelu_table.inc"
};

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

// GELU applied to the 8 bf16 of one chunk.
__device__ __forceinline__ u32x4 gelu8(u32x4 v) {
    u32x4 o;
#pragma unroll
    for (int i = 0; i < 4; ++i)
        o[i] = gelu_bf16_rn(v[i] & 0xffffu) | (gelu_bf16_rn(v[i] >> 16) << 16);
    return o;
}

// 8 bf16 (one chunk) -> 8 int8, without the clamp of quant1: for |x| <= a,
// |x * RN(127/a)| <= 127 (1 + 2^-24) rounds to at most 127, so the clamp never
// acts.  rint(x * inv) + 128 lies in [1, 255] and v_cvt_pk_u8_f32 packs it
// exactly; flipping bit 7 of each byte gives the two's complement code.
__device__ __forceinline__ uint2 quant8_pk(u32x4 v, float inv) {
    uint32_t o[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const uint32_t w0 = v[2 * h], w1 = v[2 * h + 1];
        uint32_t r = __builtin_amdgcn_cvt_pk_u8_f32(
            __builtin_rintf(__fmul_rn(__uint_as_float(w0 << 16), inv)) + 128.0f, 0, 0);
        r = __builtin_amdgcn_cvt_pk_u8_f32(
            __builtin_rintf(__fmul_rn(__uint_as_float(w0 & 0xffff0000u), inv)) + 128.0f, 1, r);
        r = __builtin_amdgcn_cvt_pk_u8_f32(
            __builtin_rintf(__fmul_rn(__uint_as_float(w1 << 16), inv)) + 128.0f, 2, r);
        r = __builtin_amdgcn_cvt_pk_u8_f32(
            __builtin_rintf(__fmul_rn(__uint_as_float(w1 & 0xffff0000u), inv)) + 128.0f, 3, r);
        o[h] = r ^ 0x80808080u;
    }
    return make_uint2(o[0], o[1]);
}

// GELU of the 8 bf16 of one chunk by table lookup (lut: the table in LDS).
__device__ __forceinline__ u32x4 gelu8_lut(u32x4 v, const uint16_t* lut) {
    u32x4 o;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        u16x2 p;
        p.x = lut[v[i] & 0xffffu];
        p.y = lut[v[i] >> 16];
        o[i] = __builtin_bit_cast(uint32_t, p);
    }
    return o;
}

// Workgroup barrier for LDS only: global loads in flight (the next rows'
// prefetch) stay in flight.  The empty asm statements keep the compiler from
// moving memory accesses across it.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0); vmcnt, expcnt left free
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
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
            uint2 o = quant8_pk(v[c], inv);
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

// Table-driven GELU + quantise.  One 16-wave workgroup per CU copies the GELU
// table into LDS once and then walks row groups (16/WPR rows at a time, WPR
// waves per row as in quantize_rows_vec); the chunks of the next row group
// are loaded while the current one is processed.  Same constraints as
// quantize_rows_vec.
constexpr int kLutBlock = 1024;
constexpr int kLutWaves = kLutBlock / 64;

template <int WPR, int CPL>
__global__ __launch_bounds__(kLutBlock) void gelu_quantize_rows_lut(const uint16_t* __restrict__ x,
                                                                   int64_t rows, int64_t cols,
                                                                   int8_t* __restrict__ q,
                                                                   float* __restrict__ scale) {
    constexpr int RPB = kLutWaves / WPR;  // rows per workgroup per step
    __shared__ __attribute__((aligned(16))) uint16_t lut[65536];
    __shared__ uint32_t red[2][kLutWaves];
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int wr = wave % WPR, w0 = wave - wr;
    const int64_t nchunk = cols >> 3;
    const int64_t step = (int64_t)gridDim.x * RPB;

    auto load_row = [&](int64_t row, u32x4 (&v)[CPL]) {
        const bool live = row < rows;
        const u32x4* xr = reinterpret_cast<const u32x4*>(x + (live ? row : 0) * cols);
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
            const int64_t ch = (int64_t)(c * WPR + wr) * 64 + lane;
            v[c] = (live && ch < nchunk) ? __builtin_nontemporal_load(xr + ch)
                                          : (u32x4){0u, 0u, 0u, 0u};
        }
    };

    int64_t row = (int64_t)blockIdx.x * RPB + wave / WPR;
    u32x4 v[CPL];
    load_row(row, v);
    {
        const u32x4* src = reinterpret_cast<const u32x4*>(kGeluTable);
        u32x4* dst = reinterpret_cast<u32x4*>(lut);
        for (int i = threadIdx.x; i < 65536 / 8; i += kLutBlock) dst[i] = src[i];
    }
    __syncthreads();

    int it = 0;
    for (int64_t base = (int64_t)blockIdx.x * RPB; base < rows; base += step, ++it) {
        u32x4 nv[CPL];
        load_row(row + step, nv);
        uint32_t amax = 0;
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
            v[c] = gelu8_lut(v[c], lut);
            amax = max(amax, absmax_bits(v[c]));
        }
        amax = wave_max_u32(amax);
        if (WPR > 1) {
            // red[it & 1]: a wave rewrites its slot two steps later, after the
            // barrier of the step in between, so no reader is still using it
            if (lane == 0) red[it & 1][wave] = amax;
            lds_barrier();
#pragma unroll
            for (int i = 0; i < WPR; ++i) amax = max(amax, red[it & 1][w0 + i]);
        }
        if (row < rows) {
            const float a = __uint_as_float(amax << 16);
            int8_t* qr = q + row * cols;
            const bool zero = !(a >= 0x1p-100f);
            const float inv = zero ? 0.0f : __fdiv_rn(127.0f, a);
            if (wr == 0 && lane == 0) scale[row] = zero ? 0.0f : __fdiv_rn(a, 127.0f);
#pragma unroll
            for (int c = 0; c < CPL; ++c) {
                const int64_t ch = (int64_t)(c * WPR + wr) * 64 + lane;
                if (ch < nchunk) {
                    const uint2 o = zero ? make_uint2(0, 0) : quant8_pk(v[c], inv);
                    __builtin_nontemporal_store(o.x, reinterpret_cast<uint32_t*>(qr) + 2 * ch);
                    __builtin_nontemporal_store(o.y, reinterpret_cast<uint32_t*>(qr) + 2 * ch + 1);
                }
            }
        }
#pragma unroll
        for (int c = 0; c < CPL; ++c) v[c] = nv[c];
        row += step;
    }
}

// Elementwise GELU by table lookup (the table is read through the caches).
__global__ __launch_bounds__(kBlock) void gelu_bf16_kernel(const uint16_t* __restrict__ x, int64_t n,
                                                           uint16_t* __restrict__ y) {
    const int64_t stride = (int64_t)gridDim.x * kBlock;
    for (int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x; i < n; i += stride)
        y[i] = kGeluTable[x[i]];
}

template <int WPR, int CPL>
hipError_t launch_lut(const uint16_t* x, int64_t rows, int64_t cols, int8_t* q, float* scale,
                      hipStream_t stream) {
    constexpr int RPB = kLutWaves / WPR;
    const int cus = cu_count();
    if (cus <= 0) return hipErrorInvalidDevice;
    const int64_t groups = (rows + RPB - 1) / RPB;
    const int64_t grid = groups < cus ? groups : cus;
    hipLaunchKernelGGL((gelu_quantize_rows_lut<WPR, CPL>), dim3((unsigned)grid), dim3(kLutBlock), 0,
                       stream, x, rows, cols, q, scale);
    return hipGetLastError();
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

// ---------------------------------------------------------------------------
// Compaction fused with the per-row quantisation: the valid rows of a padded
// [B*L x D] batch (mask != 0) are quantised straight into dense rows of q, in
// increasing source order, with src_row and the count as for compaction.  The
// result equals compaction followed by quantize_rows; the compacted bf16 rows
// are never written.  Block i owns source rows [8i, 8i+8), one wave each: the
// block counts the valid mask bytes before its first row (four per load when
// the mask is 4-byte aligned), ranks its rows with a ballot, and every wave
// with a valid row quantises it as quantize_rows_vec does (row in registers).
constexpr int kCqRows = 8;
constexpr int kCqBlock = kCqRows * 64;

// Nonzero bytes in a 32-bit word.
__device__ __forceinline__ int nonzero_bytes(uint32_t w) {
    const uint32_t hi = ((w & 0x7f7f7f7fu) + 0x7f7f7f7fu) | w;  // bit 7 of each byte: byte != 0
    return __builtin_popcount(hi & 0x80808080u);
}

// Valid rows before r0, the rank of this wave's row among the block's valid
// rows, and the block's count.  Every wave of the block calls it (it holds a
// barrier).
__device__ __forceinline__ void cq_rank(const uint8_t* __restrict__ mask, int64_t R, int64_t r0,
                                        int mask_words, int* red, int& base, int& rank,
                                        int& nvalid, bool& valid) {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    int local = 0;
    if (mask_words) {
        const uint32_t* mw = reinterpret_cast<const uint32_t*>(mask);
        for (int64_t i = threadIdx.x; i < r0 / 4; i += kCqBlock) local += nonzero_bytes(mw[i]);
    } else {
        for (int64_t i = threadIdx.x; i < r0; i += kCqBlock) local += (mask[i] != 0);
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) local += __shfl_xor(local, off, 64);
    if (lane == 0) red[wave] = local;
    __syncthreads();
    base = 0;
#pragma unroll
    for (int i = 0; i < kCqRows; ++i) base += red[i];
    const int64_t rl = r0 + lane;
    const uint64_t bal = __ballot(lane < kCqRows && rl < R && mask[rl] != 0);
    valid = (bal >> wave) & 1;
    rank = __builtin_popcountll(bal & ((1ull << wave) - 1));
    nvalid = __builtin_popcountll(bal);
}

// One wave quantises source row r of x [* x D] into output row m of q and
// scale (the row held in registers, CPL 16-byte chunks per lane): cq_load_row
// issues the row's loads, cq_store_row quantises and stores it.
template <int CPL>
__device__ __forceinline__ void cq_load_row(const uint16_t* __restrict__ x, int64_t D, int64_t r,
                                            int lane, u32x4 (&v)[CPL]) {
    const int64_t nchunk = D >> 3;
    const u32x4* xr = reinterpret_cast<const u32x4*>(x + r * D);
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
        const int64_t ch = (int64_t)c * 64 + lane;
        v[c] = ch < nchunk ? __builtin_nontemporal_load(xr + ch) : (u32x4){0u, 0u, 0u, 0u};
    }
}

template <int CPL>
__device__ __forceinline__ void cq_store_row(const u32x4 (&v)[CPL], int64_t D, int64_t m,
                                             int8_t* __restrict__ q, float* __restrict__ scale,
                                             int lane) {
    const int64_t nchunk = D >> 3;
    uint32_t amax = 0;
#pragma unroll
    for (int c = 0; c < CPL; ++c) amax = max(amax, absmax_bits(v[c]));
    amax = wave_max_u32(amax);
    const float a = __uint_as_float(amax << 16);
    const bool zero = !(a >= 0x1p-100f);
    const float inv = zero ? 0.0f : __fdiv_rn(127.0f, a);
    if (lane == 0) scale[m] = zero ? 0.0f : __fdiv_rn(a, 127.0f);
    int8_t* qr = q + m * D;
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
        const int64_t ch = (int64_t)c * 64 + lane;
        if (ch < nchunk) {
            const uint2 o = zero ? make_uint2(0, 0) : quant8_pk(v[c], inv);
            __builtin_nontemporal_store(o.x, reinterpret_cast<uint32_t*>(qr) + 2 * ch);
            __builtin_nontemporal_store(o.y, reinterpret_cast<uint32_t*>(qr) + 2 * ch + 1);
        }
    }
}

template <int CPL>
__device__ __forceinline__ void cq_quantize_row_vec(const uint16_t* __restrict__ x, int64_t D,
                                                    int64_t r, int64_t m, int8_t* __restrict__ q,
                                                    float* __restrict__ scale, int lane) {
    u32x4 v[CPL];
    cq_load_row<CPL>(x, D, r, lane, v);
    cq_store_row<CPL>(v, D, m, q, scale, lane);
}

template <int CPL>
__global__ __launch_bounds__(kCqBlock) void compact_quantize_rows_vec(
    const uint16_t* __restrict__ x, const uint8_t* __restrict__ mask, int64_t R, int64_t D,
    int8_t* __restrict__ q, float* __restrict__ scale, int32_t* __restrict__ src_row,
    int32_t* __restrict__ count, int mask_words) {
    __shared__ int red[kCqRows];
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int64_t r0 = (int64_t)blockIdx.x * kCqRows;
    const int64_t r = r0 + wave;
    // the wave's row is loaded first: it is in flight while the block counts
    // the valid rows before r0, which only its output position needs
    u32x4 v[CPL];
    if (r < R && mask[r] != 0) cq_load_row<CPL>(x, D, r, lane, v);
    int base, rank, nvalid;
    bool valid;
    cq_rank(mask, R, r0, mask_words, red, base, rank, nvalid, valid);
    if (blockIdx.x == gridDim.x - 1 && threadIdx.x == 0) *count = base + nvalid;
    if (!valid) return;
    const int64_t m = base + rank;
    if (lane == 0) src_row[m] = (int32_t)r;
    cq_store_row<CPL>(v, D, m, q, scale, lane);
}

// The linear-time path's last step: output rows m < *count quantised from
// source rows src_row[m], one wave per row in a grid-stride loop.
template <int CPL>
__global__ __launch_bounds__(kCqBlock) void gather_quantize_rows_vec(
    const uint16_t* __restrict__ x, int64_t D, const int32_t* __restrict__ src_row,
    const int32_t* __restrict__ count, int8_t* __restrict__ q, float* __restrict__ scale) {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int64_t n = *count;
    for (int64_t m = (int64_t)blockIdx.x * kCqRows + wave; m < n;
         m += (int64_t)gridDim.x * kCqRows)
        cq_quantize_row_vec<CPL>(x, D, (int64_t)src_row[m], m, q, scale, lane);
}

// Any D and alignment: each wave reads its row twice, element by element.
__device__ __forceinline__ void cq_quantize_row_generic(const uint16_t* __restrict__ x, int64_t D,
                                                        int64_t r, int64_t m,
                                                        int8_t* __restrict__ q,
                                                        float* __restrict__ scale, int lane) {
    const uint16_t* xr = x + r * D;
    int8_t* qr = q + m * D;
    uint32_t amax = 0;
    for (int64_t k = lane; k < D; k += 64) amax = max(amax, (uint32_t)xr[k] & 0x7fffu);
    amax = wave_max_u32(amax);
    const float a = __uint_as_float(amax << 16);
    if (!(a >= 0x1p-100f)) {
        if (lane == 0) scale[m] = 0.0f;
        for (int64_t k = lane; k < D; k += 64) qr[k] = 0;
        return;
    }
    const float inv = __fdiv_rn(127.0f, a);
    if (lane == 0) scale[m] = __fdiv_rn(a, 127.0f);
    for (int64_t k = lane; k < D; k += 64)
        qr[k] = (int8_t)quant1(__uint_as_float((uint32_t)xr[k] << 16), inv);
}

__global__ __launch_bounds__(kCqBlock) void compact_quantize_rows_generic(
    const uint16_t* __restrict__ x, const uint8_t* __restrict__ mask, int64_t R, int64_t D,
    int8_t* __restrict__ q, float* __restrict__ scale, int32_t* __restrict__ src_row,
    int32_t* __restrict__ count, int mask_words) {
    __shared__ int red[kCqRows];
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int64_t r0 = (int64_t)blockIdx.x * kCqRows;
    int base, rank, nvalid;
    bool valid;
    cq_rank(mask, R, r0, mask_words, red, base, rank, nvalid, valid);
    if (blockIdx.x == gridDim.x - 1 && threadIdx.x == 0) *count = base + nvalid;
    if (!valid) return;
    const int64_t r = r0 + wave, m = base + rank;
    if (lane == 0) src_row[m] = (int32_t)r;
    cq_quantize_row_generic(x, D, r, m, q, scale, lane);
}

__global__ __launch_bounds__(kCqBlock) void gather_quantize_rows_generic(
    const uint16_t* __restrict__ x, int64_t D, const int32_t* __restrict__ src_row,
    const int32_t* __restrict__ count, int8_t* __restrict__ q, float* __restrict__ scale) {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int64_t n = *count;
    for (int64_t m = (int64_t)blockIdx.x * kCqRows + wave; m < n;
         m += (int64_t)gridDim.x * kCqRows)
        cq_quantize_row_generic(x, D, (int64_t)src_row[m], m, q, scale, lane);
}

template <int CPL>
hipError_t launch_cq(const uint16_t* x, const uint8_t* mask, int64_t R, int64_t D, int8_t* q,
                     float* scale, int32_t* src_row, int32_t* count, int mask_words,
                     int64_t blocks, bool gather, hipStream_t stream) {
    if (gather)
        hipLaunchKernelGGL(gather_quantize_rows_vec<CPL>, dim3((unsigned)blocks), dim3(kCqBlock), 0,
                           stream, x, D, src_row, count, q, scale);
    else
        hipLaunchKernelGGL(compact_quantize_rows_vec<CPL>, dim3((unsigned)blocks), dim3(kCqBlock),
                           0, stream, x, mask, R, D, q, scale, src_row, count, mask_words);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Per-block quantisation of attention Query / Key (w8a8_quantize_blocks).
// x holds token rows [B x S x H*D]; one block is up to `block` consecutive
// tokens of one sample and one head, and gets one scale, with the arithmetic of
// the per-row routine above (absmax over the block).  One workgroup per block
// (blockIdx.x = (b * nblk + j) * H + h, the scale's index) of NT threads:
// each thread loads its KPT 16-byte chunks of the block (a head's row of D
// values is D/8 chunks; consecutive threads take consecutive chunks, so a wave
// reads whole 128-byte lines), keeps them in registers through the absmax
// reduction and writes their codes, so every element is read from HBM once.
// ---------------------------------------------------------------------------
template <int KPT, int NT>
__global__ __launch_bounds__(NT) void quantize_blocks_vec(const uint16_t* __restrict__ x,
                                                          int64_t S, int64_t H, int64_t D,
                                                          int64_t block, int64_t nblk,
                                                          int8_t* __restrict__ q,
                                                          float* __restrict__ scale) {
    __shared__ uint32_t red[NT / 64];
    // the grid holds fewer than 2^31 blocks (checked by the caller): 32-bit index arithmetic
    const uint32_t i = blockIdx.x, h32 = (uint32_t)H, nb32 = (uint32_t)nblk;
    const uint32_t bj = i / h32, h = i - bj * h32;
    const uint32_t b = bj / nb32, j = bj - b * nb32;
    const int64_t t0 = (int64_t)j * block;
    const int64_t ntok = (S - t0) < block ? (S - t0) : block;
    const uint32_t cpt = (uint32_t)(D >> 3);  // chunks per token row of the head
    const uint32_t n = (uint32_t)ntok * cpt;  // chunks in the block (<= NT * KPT)
    const int64_t C = H * D;
    const int64_t origin = ((int64_t)b * S + t0) * C + (int64_t)h * D;  // the block's first value
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;

    u32x4 v[KPT];
    int64_t off[KPT];
    uint32_t amax = 0;
#pragma unroll
    for (int k = 0; k < KPT; ++k) {
        const uint32_t c = threadIdx.x + (uint32_t)k * NT;
        const uint32_t tok = c / cpt;
        off[k] = origin + (int64_t)tok * C + (int64_t)(c - tok * cpt) * 8;
        if (c < n) v[k] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(x + off[k]));
        else v[k] = (u32x4){0u, 0u, 0u, 0u};
        amax = max(amax, absmax_bits(v[k]));
    }
    amax = wave_max_u32(amax);
    if (lane == 0) red[wave] = amax;
    __syncthreads();
#pragma unroll
    for (int w = 0; w < NT / 64; ++w) amax = max(amax, red[w]);
    const float a = __uint_as_float(amax << 16);
    const bool zero = !(a >= 0x1p-100f);  // degenerate block: scale 0, all codes 0
    const float inv = zero ? 0.0f : __fdiv_rn(127.0f, a);
    if (threadIdx.x == 0) scale[i] = zero ? 0.0f : __fdiv_rn(a, 127.0f);
#pragma unroll
    for (int k = 0; k < KPT; ++k) {
        const uint32_t c = threadIdx.x + (uint32_t)k * NT;
        if (c < n) {
            const uint2 o = zero ? make_uint2(0u, 0u) : quant8_pk(v[k], inv);
            uint32_t* qp = reinterpret_cast<uint32_t*>(q + off[k]);
            __builtin_nontemporal_store(o.x, qp);
            __builtin_nontemporal_store(o.y, qp + 1);
        }
    }
}

template <int KPT, int NT = kBlock>
hipError_t launch_blocks(const uint16_t* x, int64_t B, int64_t S, int64_t H, int64_t D,
                         int64_t block, int8_t* q, float* scale, hipStream_t stream) {
    const int64_t nblk = (S + block - 1) / block;
    hipLaunchKernelGGL((quantize_blocks_vec<KPT, NT>), dim3((unsigned)(B * nblk * H)), dim3(NT), 0,
                       stream, x, S, H, D, block, nblk, q, scale);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Normalisation + modulation ahead of a linear layer, alone (bf16 out) or fused
// with the per-row quantisation (the fused operators of the paperlayer.ai
// summary, section C; the formulas are readings).  Per row of D elements:
//     LayerNorm:  mu = sum(x) / D,  var = sum((x - mu)^2) / D
//     RMSNorm:    mu = 0,           var = sum(x^2) / D
//     rstd = 1 / sqrt(var + eps), 0 where var + eps = 0       (binary64)
//     z = (x - mu) * rstd * (1 + scale[g]) + shift[g],  g = row / rows_per_cond
// The value defined is z in binary64 rounded once to bf16.  Here the
// statistics are binary64 (sums in the order the reduction takes) and the
// elementwise steps binary32, d = RN32(x - mu), y = RN32(d * RN32(rstd)),
// z' = fmaf(y, RN32(1 + scale[g]), shift[g]), then z' to bf16: z' is within
// 2^-24 |z| + 4.01 * 2^-24 |(x - mu) rstd (1 + scale)| of z, so the bf16 result
// is within one bf16 ulp of the defined value except where the shift cancels
// most of the product.  The fused variant quantises the bf16 row it computes
// exactly as quantize_rows does.  The vector kernel keeps the row in registers
// (as quantize_rows_vec), so each element is read from HBM once; the binary64
// work is two or three operations per element in the statistics, the rest is
// binary32 (binary64 elementwise would double the VALU work of a kernel that
// is already bound by VALU issue).

__device__ __forceinline__ double wave_sum_f64(double v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
    return v;
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// binary32 -> bf16 bits, nearest even (finite values)
__device__ __forceinline__ uint32_t f32_bf16_rn(float f) {
    const uint32_t u = __float_as_uint(f);
    return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

// The 8 values of a chunk as binary32 (exact).
__device__ __forceinline__ void unpack8(u32x4 v, float (&f)[8]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        f[2 * i] = bf16_lo(v[i]);
        f[2 * i + 1] = bf16_hi(v[i]);
    }
}

// Their binary64 sum.
__device__ __forceinline__ double sum8(const float (&f)[8]) {
    double t[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) t[i] = (double)f[2 * i] + (double)f[2 * i + 1];
    return (t[0] + t[1]) + (t[2] + t[3]);
}

// Deviations from mu of a chunk's values (in place, rounded to binary32); their
// squares, in binary64, are added to t.
__device__ __forceinline__ void dev8(float (&f)[8], double mu, double& t) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const double a = (double)f[e] - mu;
        t = __builtin_fma(a, a, t);
        f[e] = (float)a;
    }
}

// z of one chunk from its deviations, as bf16 bits
__device__ __forceinline__ u32x4 mod8(const float (&d)[8], float r, u32x4 sc, u32x4 sh) {
    u32x4 o;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float z0 = __builtin_fmaf(__fmul_rn(d[2 * i], r), __fadd_rn(1.0f, bf16_lo(sc[i])),
                                        bf16_lo(sh[i]));
        const float z1 = __builtin_fmaf(__fmul_rn(d[2 * i + 1], r),
                                        __fadd_rn(1.0f, bf16_hi(sc[i])), bf16_hi(sh[i]));
        o[i] = pack_bf16x2(z0, z1);
    }
    return o;
}

__device__ __forceinline__ double rstd_of(double var, double eps) {
    const double v = var + eps;
    return v > 0.0 ? 1.0 / __builtin_sqrt(v) : 0.0;
}

// WPR waves per row, CPL 16-byte chunks per lane (cols % 8 == 0, rows of up to
// WPR*64*CPL*8 elements); QUANT: codes and scale out, else the bf16 z.
template <int WPR, int CPL, bool QUANT>
__global__ __launch_bounds__(kBlock) void norm_mod_rows_vec(
    const uint16_t* __restrict__ x, int64_t rows, int64_t cols, const uint16_t* __restrict__ shift,
    const uint16_t* __restrict__ scale, int64_t rpc, int norm, double eps, int8_t* __restrict__ q,
    float* __restrict__ qscale, uint16_t* __restrict__ y) {
    constexpr int RPB = (kBlock / 64) / WPR;  // rows per block
    __shared__ double red64[2][kBlock / 64];
    __shared__ uint32_t red[kBlock / 64];
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int wr = wave % WPR, w0 = wave - wr;
    const int64_t row = (int64_t)blockIdx.x * RPB + wave / WPR;
    const bool live = row < rows;
    const int64_t nchunk = cols >> 3;
    const int rbytes = (int)cols * 2;  // <= 65536 on this path
    const double D = (double)cols;
    auto chunk = [&](int c) { return (int64_t)(c * WPR + wr) * 64 + lane; };
    // sum over the row's WPR waves (every thread of the block takes part)
    auto row_sum = [&](double t, int slot) {
        t = wave_sum_f64(t);
        if (WPR > 1) {
            if (lane == 0) red64[slot][wave] = t;
            __syncthreads();
            t = 0.0;
#pragma unroll
            for (int i = 0; i < WPR; ++i) t += red64[slot][w0 + i];
        }
        return t;
    };

    // the row, zero past its end (and for a row past the last): nontemporal
    u32x4 v[CPL];
    const uint16_t* xrow = live ? x + row * cols : nullptr;
#pragma unroll
    for (int c = 0; c < CPL; ++c) v[c] = load16_row<2>(xrow, rbytes, (int)chunk(c) * 16);
    float d[CPL][8];  // the values, then their deviations from the mean
#pragma unroll
    for (int c = 0; c < CPL; ++c) unpack8(v[c], d[c]);
    double mu = 0.0;
    if (norm == 0) {
        double t = 0.0;
#pragma unroll
        for (int c = 0; c < CPL; ++c) t += sum8(d[c]);  // padding adds 0
        mu = row_sum(t, 0) / D;
    }
    double ta = 0.0, tb = 0.0;  // two chains of the sum of squared deviations
#pragma unroll
    for (int c = 0; c < CPL; ++c)
        if (chunk(c) < nchunk) dev8(d[c], mu, (c & 1) ? tb : ta);  // padding is not in the row
    const float r = (float)rstd_of(row_sum(ta + tb, 1) / D, eps);

    const int64_t g = (live ? row : 0) / rpc;
    const uint16_t* scr = scale ? scale + g * cols : nullptr;
    const uint16_t* shr = shift ? shift + g * cols : nullptr;
    uint32_t amax = 0;
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
        const int64_t ch = chunk(c);
        v[c] = mod8(d[c], r, load16_row<0>(scr, rbytes, (int)ch * 16),
                    load16_row<0>(shr, rbytes, (int)ch * 16));
        if (ch < nchunk) {
            if (QUANT) amax = max(amax, absmax_bits(v[c]));
            else if (live) __builtin_nontemporal_store(v[c], reinterpret_cast<u32x4*>(y + row * cols) + ch);
        }
    }
    if constexpr (!QUANT) return;

    amax = wave_max_u32(amax);
    if (WPR > 1) {
        if (lane == 0) red[wave] = amax;
        __syncthreads();
#pragma unroll
        for (int i = 0; i < WPR; ++i) amax = max(amax, red[w0 + i]);
    }
    if (!live) return;
    const float a = __uint_as_float(amax << 16);
    int8_t* qr = q + row * cols;
    if (!(a >= 0x1p-100f)) {
        if (wr == 0 && lane == 0) qscale[row] = 0.0f;
#pragma unroll
        for (int c = 0; c < CPL; ++c)
            if (chunk(c) < nchunk) reinterpret_cast<uint2*>(qr)[chunk(c)] = make_uint2(0, 0);
        return;
    }
    const float inv = __fdiv_rn(127.0f, a);
    if (wr == 0 && lane == 0) qscale[row] = __fdiv_rn(a, 127.0f);
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
        const int64_t ch = chunk(c);
        if (ch < nchunk) {
            const uint2 o = quant8_pk(v[c], inv);
            __builtin_nontemporal_store(o.x, reinterpret_cast<uint32_t*>(qr) + 2 * ch);
            __builtin_nontemporal_store(o.y, reinterpret_cast<uint32_t*>(qr) + 2 * ch + 1);
        }
    }
}

// Any cols, any alignment: one block per row, passes over the row in memory
// (z is recomputed where it is needed again).
template <bool QUANT>
__global__ __launch_bounds__(kBlock) void norm_mod_rows_generic(
    const uint16_t* __restrict__ x, int64_t rows, int64_t cols, const uint16_t* __restrict__ shift,
    const uint16_t* __restrict__ scale, int64_t rpc, int norm, double eps, int8_t* __restrict__ q,
    float* __restrict__ qscale, uint16_t* __restrict__ y) {
    __shared__ double red64[kBlock / 64];
    __shared__ uint32_t red[kBlock / 64];
    const int64_t row = blockIdx.x;
    if (row >= rows) return;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const uint16_t* xr = x + row * cols;
    const int64_t g = row / rpc;
    const double D = (double)cols;
    auto block_sum = [&](double t) {
        t = wave_sum_f64(t);
        if (lane == 0) red64[wave] = t;
        __syncthreads();
        t = (red64[0] + red64[1]) + (red64[2] + red64[3]);
        __syncthreads();
        return t;
    };
    double mu = 0.0;
    if (norm == 0) {
        double t = 0.0;
        for (int64_t k = threadIdx.x; k < cols; k += kBlock) t += (double)bf16_lo(xr[k]);
        mu = block_sum(t) / D;
    }
    double t2 = 0.0;
    for (int64_t k = threadIdx.x; k < cols; k += kBlock) {
        const double dv = (double)bf16_lo(xr[k]) - mu;
        t2 = __builtin_fma(dv, dv, t2);
    }
    const float r = (float)rstd_of(block_sum(t2) / D, eps);
    auto z = [&](int64_t k) {
        const float dk = (float)((double)bf16_lo(xr[k]) - mu);
        const float sc = scale ? bf16_lo(scale[g * cols + k]) : 0.0f;
        const float sh = shift ? bf16_lo(shift[g * cols + k]) : 0.0f;
        return f32_bf16_rn(__builtin_fmaf(__fmul_rn(dk, r), __fadd_rn(1.0f, sc), sh));
    };
    if constexpr (!QUANT) {
        for (int64_t k = threadIdx.x; k < cols; k += kBlock) y[row * cols + k] = (uint16_t)z(k);
        return;
    }
    uint32_t amax = 0;
    for (int64_t k = threadIdx.x; k < cols; k += kBlock) amax = max(amax, z(k) & 0x7fffu);
    amax = wave_max_u32(amax);
    if (lane == 0) red[wave] = amax;
    __syncthreads();
    amax = max(max(red[0], red[1]), max(red[2], red[3]));
    const float a = __uint_as_float(amax << 16);
    int8_t* qr = q + row * cols;
    if (!(a >= 0x1p-100f)) {
        if (threadIdx.x == 0) qscale[row] = 0.0f;
        for (int64_t k = threadIdx.x; k < cols; k += kBlock) qr[k] = 0;
        return;
    }
    const float inv = __fdiv_rn(127.0f, a);
    if (threadIdx.x == 0) qscale[row] = __fdiv_rn(a, 127.0f);
    for (int64_t k = threadIdx.x; k < cols; k += kBlock)
        qr[k] = (int8_t)quant1(__uint_as_float(z(k) << 16), inv);
}

template <int WPR, int CPL, bool QUANT>
hipError_t launch_nm(const uint16_t* x, int64_t rows, int64_t cols, const uint16_t* shift,
                     const uint16_t* scale, int64_t rpc, int norm, double eps, int8_t* q,
                     float* qscale, uint16_t* y, hipStream_t stream) {
    constexpr int RPB = (kBlock / 64) / WPR;
    const int64_t blocks = (rows + RPB - 1) / RPB;
    hipLaunchKernelGGL((norm_mod_rows_vec<WPR, CPL, QUANT>), dim3((unsigned)blocks), dim3(kBlock), 0,
                       stream, x, rows, cols, shift, scale, rpc, norm, eps, q, qscale, y);
    return hipGetLastError();
}

template <bool QUANT>
hipError_t launch_nm_any(const uint16_t* x, int64_t rows, int64_t cols, const uint16_t* shift,
                         const uint16_t* scale, int64_t rpc, int norm, double eps, int8_t* q,
                         float* qscale, uint16_t* y, hipStream_t stream) {
    const bool a16 = reinterpret_cast<uintptr_t>(x) % 16 == 0 &&
                     reinterpret_cast<uintptr_t>(shift) % 16 == 0 &&
                     reinterpret_cast<uintptr_t>(scale) % 16 == 0 &&
                     (QUANT ? reinterpret_cast<uintptr_t>(q) % 8 == 0
                            : reinterpret_cast<uintptr_t>(y) % 16 == 0);
    const int64_t nchunk = cols / 8;
    const bool vec = cols % 8 == 0 && a16;
#define W8A8_NM(W, C) launch_nm<W, C, QUANT>(x, rows, cols, shift, scale, rpc, norm, eps, q, qscale, y, stream)
    // at most 4 chunks (32 values) per lane where the row allows: the values and
    // their deviations stay in registers, and with 8 chunks per lane the
    // occupancy falls to 3 waves per SIMD (24576 x 4096: 90 us with 2 waves of
    // 4 chunks per row, 135 us with 1 wave of 8)
    if (vec && nchunk <= 64) return W8A8_NM(1, 1);
    if (vec && nchunk <= 128) return W8A8_NM(1, 2);
    if (vec && nchunk <= 256) return W8A8_NM(1, 4);
    if (vec && nchunk <= 512) return W8A8_NM(2, 4);
    if (vec && nchunk <= 1024) return W8A8_NM(4, 4);
    if (vec && nchunk <= 2048) return W8A8_NM(4, 8);
    if (vec && nchunk <= 4096) return W8A8_NM(4, 16);
#undef W8A8_NM
    hipLaunchKernelGGL(norm_mod_rows_generic<QUANT>, dim3((unsigned)rows), dim3(kBlock), 0, stream,
                       x, rows, cols, shift, scale, rpc, norm, eps, q, qscale, y);
    return hipGetLastError();
}

}  // namespace

int launch_compact_quantize_rows(const uint16_t* x, const uint8_t* mask, int64_t R, int64_t D,
                                 int8_t* q, float* scale, int32_t* src_row, int32_t* count,
                                 hipStream_t stream) {
    int64_t blocks = R > 0 ? (R + kCqRows - 1) / kCqRows : 1;
    const int mask_words = reinterpret_cast<uintptr_t>(mask) % 4 == 0 ? 1 : 0;
    const bool gather = !compact_single_pass(R);
    if (gather) {
        // the linear-time path: src_row and *count first (the chunk counts kept
        // in scale, which only the quantisation below writes), then the rows
        // they list are quantised in a grid-stride loop
        if (launch_compact_scan(mask, R, reinterpret_cast<int32_t*>(scale), R, src_row, count,
                                stream) != 0)
            return -1;
        const int cus = cu_count();
        if (cus <= 0) return -1;
        if (blocks > (int64_t)cus * 16) blocks = (int64_t)cus * 16;
    }
    const bool vec = D > 0 && D % 8 == 0 && reinterpret_cast<uintptr_t>(x) % 16 == 0 &&
                     reinterpret_cast<uintptr_t>(q) % 8 == 0;
    const int64_t nchunk = D / 8;
    hipError_t e;
    if (vec && nchunk <= 64) e = launch_cq<1>(x, mask, R, D, q, scale, src_row, count, mask_words, blocks, gather, stream);
    else if (vec && nchunk <= 128) e = launch_cq<2>(x, mask, R, D, q, scale, src_row, count, mask_words, blocks, gather, stream);
    else if (vec && nchunk <= 256) e = launch_cq<4>(x, mask, R, D, q, scale, src_row, count, mask_words, blocks, gather, stream);
    else if (vec && nchunk <= 512) e = launch_cq<8>(x, mask, R, D, q, scale, src_row, count, mask_words, blocks, gather, stream);
    else if (vec && nchunk <= 1024) e = launch_cq<16>(x, mask, R, D, q, scale, src_row, count, mask_words, blocks, gather, stream);
    else {
        if (gather)
            hipLaunchKernelGGL(gather_quantize_rows_generic, dim3((unsigned)blocks), dim3(kCqBlock),
                               0, stream, x, D, src_row, count, q, scale);
        else
            hipLaunchKernelGGL(compact_quantize_rows_generic, dim3((unsigned)blocks),
                               dim3(kCqBlock), 0, stream, x, mask, R, D, q, scale, src_row, count,
                               mask_words);
        e = hipGetLastError();
    }
    return e == hipSuccess ? 0 : -1;
}

int launch_quantize_rows(const uint16_t* x, int64_t rows, int64_t cols, int8_t* q, float* scale,
                         hipStream_t stream, bool gelu) {
    if (rows == 0) return 0;
    const bool vec = (cols % 8 == 0) && (reinterpret_cast<uintptr_t>(x) % 16 == 0) &&
                     (reinterpret_cast<uintptr_t>(q) % 8 == 0) && cols > 0;
    const int64_t nchunk = cols / 8;
    hipError_t e;
    // the table kernel pays a 128 KB table copy per CU: worth it from about
    // 2^24 elements on
    if (gelu && vec && rows * cols >= ((int64_t)1 << 24) && nchunk <= 4096) {
        if (nchunk <= 512) e = launch_lut<1, 8>(x, rows, cols, q, scale, stream);
        else if (nchunk <= 1024) e = launch_lut<2, 8>(x, rows, cols, q, scale, stream);
        // 16384-wide rows: 8 waves of 4 chunks per row ran 198 us where 4 waves of 8
        // ran 207 (24576 rows)
        else if (nchunk <= 2048) e = launch_lut<8, 4>(x, rows, cols, q, scale, stream);
        else e = launch_lut<8, 8>(x, rows, cols, q, scale, stream);
        return e == hipSuccess ? 0 : -1;
    }
    if (vec && nchunk <= 64) e = launch_vec<1, 1>(x, rows, cols, q, scale, stream, gelu);
    else if (vec && nchunk <= 128) e = launch_vec<1, 2>(x, rows, cols, q, scale, stream, gelu);
    else if (vec && nchunk <= 256) e = launch_vec<1, 4>(x, rows, cols, q, scale, stream, gelu);
    // 4096-wide rows: 2 waves of 4 chunks per row, 47.7 us on 24576 rows against
    // 48.6 us for 1 wave of 8
    else if (vec && nchunk <= 512) e = launch_vec<2, 4>(x, rows, cols, q, scale, stream, gelu);
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

int launch_quantize_blocks(const uint16_t* x, int64_t B, int64_t S, int64_t H, int64_t D,
                           int64_t block, int8_t* q, float* scale, hipStream_t stream) {
    if (B == 0 || S == 0 || H == 0) return 0;
    const int64_t chunks = (S < block ? S : block) * (D / 8);  // of the largest block
    hipError_t e;
    // blocks of more than 4 x 256 chunks take 8-wave workgroups: 128 tokens x
    // 128 values ran 6% faster than with 4 waves of 8 chunks per thread
    if (chunks <= kBlock) e = launch_blocks<1>(x, B, S, H, D, block, q, scale, stream);
    else if (chunks <= 2 * kBlock) e = launch_blocks<2>(x, B, S, H, D, block, q, scale, stream);
    else if (chunks <= 4 * kBlock) e = launch_blocks<4>(x, B, S, H, D, block, q, scale, stream);
    else if (chunks <= 8 * kBlock)
        e = launch_blocks<4, 2 * kBlock>(x, B, S, H, D, block, q, scale, stream);
    else if (chunks <= 16 * kBlock)
        e = launch_blocks<8, 2 * kBlock>(x, B, S, H, D, block, q, scale, stream);
    else return -1;
    return e == hipSuccess ? 0 : -1;
}

int launch_norm_mod(const uint16_t* x, int64_t rows, int64_t cols, const uint16_t* shift,
                    const uint16_t* scale, int64_t rows_per_cond, int norm, double eps, int8_t* q,
                    float* qscale, uint16_t* y, hipStream_t stream) {
    if (rows == 0) return 0;
    const hipError_t e =
        q ? launch_nm_any<true>(x, rows, cols, shift, scale, rows_per_cond, norm, eps, q, qscale,
                                nullptr, stream)
          : launch_nm_any<false>(x, rows, cols, shift, scale, rows_per_cond, norm, eps, nullptr,
                                 nullptr, y, stream);
    return e == hipSuccess ? 0 : -1;
}

int launch_gelu_bf16(const uint16_t* x, int64_t n, uint16_t* y, hipStream_t stream) {
    if (n == 0) return 0;
    const int64_t blocks = (n + kBlock - 1) / kBlock;
    const int64_t grid = blocks < 65536 ? blocks : 65536;
    hipLaunchKernelGGL(gelu_bf16_kernel, dim3((unsigned)grid), dim3(kBlock), 0, stream, x, n, y);
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace w8a8
