// Padded-row compaction for gfx950.
//
// TurboT2VA (智猩猩 article, section 01.3, closing paragraph; paperlayer.ai
// summary, section "C. Fused Multimodal Transformer Operations"): padded text
// positions are dropped using the shared text mask, and every valid row is
// kept unchanged.  Row r = b*L + t of X[B*L x D] is kept iff mask[r] != 0; kept
// rows are written densely in increasing r, with src_row[m] = r and the total
// in *count.
//
// One launch.  Block i owns source rows [i*RPB, (i+1)*RPB).  It first counts the
// valid mask bytes before its first row (a block-wide reduction over at most
// B*L bytes, served from L2), then ranks its own rows and copies each valid row
// with 16-byte loads and stores (2-byte when D or the pointers do not allow).
// The last block writes *count.  Pure data movement: HBM-bound.
#include "common.h"

namespace w8a8 {

namespace {

constexpr int kBlock = 256;
constexpr int kRowsPerBlock = 8;

__device__ __forceinline__ int block_sum(int v, int* red) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
    const int wave = threadIdx.x >> 6;
    __syncthreads();  // red may still be read from a previous call
    if ((threadIdx.x & 63) == 0) red[wave] = v;
    __syncthreads();
    return red[0] + red[1] + red[2] + red[3];
}

__global__ __launch_bounds__(kBlock) void compact_rows_kernel(
    const uint16_t* __restrict__ x, const uint8_t* __restrict__ mask, int64_t R, int64_t D,
    uint16_t* __restrict__ out, int32_t* __restrict__ src_row, int32_t* __restrict__ count,
    int vec16) {
    __shared__ int red[kBlock / 64];
    __shared__ int rank[kRowsPerBlock];
    __shared__ int nvalid;
    const int64_t r0 = (int64_t)blockIdx.x * kRowsPerBlock;

    // 1. valid rows before r0
    int local = 0;
    for (int64_t i = threadIdx.x; i < r0 && i < R; i += kBlock) local += (mask[i] != 0);
    const int base = block_sum(local, red);

    // 2. rank of this block's rows
    if (threadIdx.x == 0) {
        int n = 0;
        for (int j = 0; j < kRowsPerBlock; ++j) {
            const int64_t r = r0 + j;
            if (r < R && mask[r] != 0) rank[j] = n++;
            else rank[j] = -1;
        }
        nvalid = n;
    }
    __syncthreads();
    if (blockIdx.x == gridDim.x - 1 && threadIdx.x == 0) *count = base + nvalid;

    // 3. copy valid rows
    for (int j = 0; j < kRowsPerBlock; ++j) {
        const int rk = rank[j];
        if (rk < 0) continue;
        const int64_t r = r0 + j;
        const int64_t m = base + rk;
        if (threadIdx.x == 0) src_row[m] = (int32_t)r;
        if (vec16) {
            typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
            const u32x4* s = reinterpret_cast<const u32x4*>(x + r * D);
            u32x4* d = reinterpret_cast<u32x4*>(out + m * D);
            for (int64_t c = threadIdx.x; c < D / 8; c += kBlock)
                __builtin_nontemporal_store(__builtin_nontemporal_load(s + c), d + c);
        } else {
            const uint16_t* s = x + r * D;
            uint16_t* d = out + m * D;
            for (int64_t c = threadIdx.x; c < D; c += kBlock) d[c] = s[c];
        }
    }
}

}  // namespace

int launch_compact_rows(const uint16_t* x, const uint8_t* mask, int64_t R, int64_t D,
                        uint16_t* out, int32_t* src_row, int32_t* count, hipStream_t stream) {
    const int64_t blocks = R > 0 ? (R + kRowsPerBlock - 1) / kRowsPerBlock : 1;
    const int vec16 = (D % 8 == 0) && (reinterpret_cast<uintptr_t>(x) % 16 == 0) &&
                      (reinterpret_cast<uintptr_t>(out) % 16 == 0);
    hipLaunchKernelGGL(compact_rows_kernel, dim3((unsigned)blocks), dim3(kBlock), 0, stream, x,
                       mask, R, D, out, src_row, count, vec16);
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace w8a8
