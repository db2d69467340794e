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
// B*L bytes, four mask bytes per load when the mask is 4-byte aligned, served
// from L2), ranks its own rows with a ballot, then copies its valid rows.  The
// (valid row, 16-byte chunk) pairs of the block form one index space that the
// threads walk in batches of kBatch loads issued before any store, so a block
// waits about one memory latency per batch rather than one per row.  The last
// block writes *count.  Pure data movement: HBM-bound.
#include "common.h"

namespace w8a8 {

namespace {

constexpr int kBlock = 256;
constexpr int kRowsPerBlock = 8;
constexpr int kBatch = 16;  // loads in flight per thread
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ int block_sum(int v, int* red) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
    const int wave = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) red[wave] = v;
    __syncthreads();
    return red[0] + red[1] + red[2] + red[3];
}

// Nonzero bytes in a 32-bit word.
__device__ __forceinline__ int nonzero_bytes(uint32_t w) {
    const uint32_t hi = ((w & 0x7f7f7f7fu) + 0x7f7f7f7fu) | w;  // bit 7 of each byte: byte != 0
    return __builtin_popcount(hi & 0x80808080u);
}

template <bool VEC16>
__global__ __launch_bounds__(kBlock) void compact_rows_kernel(
    const uint16_t* __restrict__ x, const uint8_t* __restrict__ mask, int64_t R, int64_t D,
    uint16_t* __restrict__ out, int32_t* __restrict__ src_row, int32_t* __restrict__ count,
    int mask_words) {
    __shared__ int red[kBlock / 64];
    __shared__ int64_t rowsrc[kRowsPerBlock];
    __shared__ int nvalid_s;
    const int64_t r0 = (int64_t)blockIdx.x * kRowsPerBlock;
    const int tid = threadIdx.x;

    // 1. valid rows before r0 (r0 is a multiple of 8, so whole words)
    int local = 0;
    if (mask_words) {
        const uint32_t* mw = reinterpret_cast<const uint32_t*>(mask);
        for (int64_t i = tid; i < r0 / 4; i += kBlock) local += nonzero_bytes(mw[i]);
    } else {
        for (int64_t i = tid; i < r0; i += kBlock) local += (mask[i] != 0);
    }
    const int base = block_sum(local, red);

    // 2. rank of this block's rows: a ballot over the first kRowsPerBlock lanes
    if (tid < 64) {
        const int64_t r = r0 + tid;
        const bool valid = tid < kRowsPerBlock && r < R && mask[r] != 0;
        const uint64_t bal = __ballot(valid);
        if (valid) rowsrc[__builtin_popcountll(bal & ((1ull << tid) - 1))] = r;
        if (tid == 0) nvalid_s = __builtin_popcountll(bal);
    }
    __syncthreads();
    const int nvalid = nvalid_s;
    if (blockIdx.x == gridDim.x - 1 && tid == 0) *count = base + nvalid;
    if (tid < nvalid) src_row[base + tid] = (int32_t)rowsrc[tid];

    // 3. copy: item i is chunk i % nch of valid row i / nch; a thread's items
    // are tid, tid + kBlock, ..., walked as (row, chunk) pairs without division
    if (VEC16) {
        const int64_t nch = D / 8;
        const int64_t step_j = kBlock / nch, step_c = kBlock % nch;
        int64_t j = tid / nch, c = tid % nch;
        while (j < nvalid) {
            u32x4 v[kBatch];
            int64_t jj = j, cc = c;
#pragma unroll
            for (int k = 0; k < kBatch; ++k) {
                if (jj < nvalid)
                    v[k] = __builtin_nontemporal_load(
                        reinterpret_cast<const u32x4*>(x + rowsrc[jj] * D) + cc);
                jj += step_j;
                cc += step_c;
                if (cc >= nch) { cc -= nch; ++jj; }
            }
#pragma unroll
            for (int k = 0; k < kBatch; ++k) {
                if (j < nvalid)
                    __builtin_nontemporal_store(v[k],
                                                reinterpret_cast<u32x4*>(out + (base + j) * D) + c);
                j += step_j;
                c += step_c;
                if (c >= nch) { c -= nch; ++j; }
            }
        }
    } else {
        for (int j = 0; j < nvalid; ++j) {
            const uint16_t* s = x + rowsrc[j] * D;
            uint16_t* d = out + (base + j) * D;
            for (int64_t c = tid; c < D; c += kBlock) d[c] = s[c];
        }
    }
}

}  // namespace

int launch_compact_rows(const uint16_t* x, const uint8_t* mask, int64_t R, int64_t D,
                        uint16_t* out, int32_t* src_row, int32_t* count, hipStream_t stream) {
    const int64_t blocks = R > 0 ? (R + kRowsPerBlock - 1) / kRowsPerBlock : 1;
    const bool vec16 = D > 0 && (D % 8 == 0) && (reinterpret_cast<uintptr_t>(x) % 16 == 0) &&
                       (reinterpret_cast<uintptr_t>(out) % 16 == 0);
    const int mask_words = reinterpret_cast<uintptr_t>(mask) % 4 == 0 ? 1 : 0;
    if (vec16)
        hipLaunchKernelGGL(compact_rows_kernel<true>, dim3((unsigned)blocks), dim3(kBlock), 0,
                           stream, x, mask, R, D, out, src_row, count, mask_words);
    else
        hipLaunchKernelGGL(compact_rows_kernel<false>, dim3((unsigned)blocks), dim3(kBlock), 0,
                           stream, x, mask, R, D, out, src_row, count, mask_words);
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace w8a8
