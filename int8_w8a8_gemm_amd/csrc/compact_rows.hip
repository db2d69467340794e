// Padded-row compaction for gfx950.
//
// TurboT2VA (智猩猩 article, section 01.3, closing paragraph; paperlayer.ai
// summary, section "C. Fused Multimodal Transformer Operations"): padded text
// positions are dropped using the shared text mask, and every valid row is
// kept unchanged.  Row r = b*L + t of X[B*L x D] is kept iff mask[r] != 0; kept
// rows are written densely in increasing r, with src_row[m] = r and the total
// in *count.
//
// Up to kSinglePassRows rows: one launch.  Block i owns source rows
// [i*RPB, (i+1)*RPB).  It ranks its own rows with a ballot, issues the loads
// of its valid rows, and while they are in flight counts the valid mask bytes
// before its first row (a block-wide reduction over fewer than
// kSinglePassRows bytes, four mask bytes per load when the mask is 4-byte
// aligned, served from L2), which places its rows in the output.  The (valid row, 16-byte
// chunk) pairs of the block form one index space that the threads walk in
// batches of kBatch loads issued before any store, so a block waits about one
// memory latency per batch rather than one per row.  The last block writes
// *count.  Pure data movement: HBM-bound.
//
// More rows: three launches, each linear in B*L, and no memory beyond the
// outputs.  (1) compact_count_chunks: workgroup g counts the valid rows of
// chunk g (at most kMaxChunks chunks of whole 16-byte mask groups) into an
// int32 array kept in the first bytes of an output that is written only by
// step 3.  (2) compact_index_chunks: workgroup g adds the counts of the chunks
// before it, walks its chunk 4 KB of mask at a time with a block-wide scan, and
// writes src_row for its valid rows; the last one writes *count.  (3) the rows
// listed in src_row are gathered (here, or quantised on the way in the fused
// variant) by a grid-stride loop that stops at *count.
#include "common.h"

namespace w8a8 {

namespace {

constexpr int kBlock = 256;
constexpr int kRowsPerBlock = 8;
constexpr int kBatch = 16;  // loads in flight per thread
constexpr int64_t kSinglePassRows = 8192;  // above: the linear-time path
constexpr int64_t kMaxChunks = 1024;        // chunks of the linear-time scan
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

// Copies nvalid rows x + rowsrc[j] * D (j < nvalid) to out + (base + j) * D,
// the block's (row, 16-byte chunk) pairs walked in batches of kBatch loads per
// thread (VEC16: D % 8 == 0 and 16-byte aligned rows), else element by
// element.  base = get_base(), which every thread of the block calls once (it
// may hold a barrier): with LATE (and VEC16) after the first batch's loads are
// issued, so that the rows are in flight while the block works out where they
// go, else before any load.
template <bool VEC16, bool LATE, class GetBase>
__device__ __forceinline__ void copy_rows(const uint16_t* __restrict__ x, int64_t D,
                                          const int64_t* rowsrc, int nvalid,
                                          uint16_t* __restrict__ out, GetBase get_base) {
    const int tid = threadIdx.x;
    if (VEC16) {
        const int64_t nch = D / 8;
        const int64_t step_j = kBlock / nch, step_c = kBlock % nch;
        int64_t j = tid / nch, c = tid % nch;
        uint16_t* dst = LATE ? nullptr : out + get_base() * D;
        bool first = LATE;
        for (;;) {
            // every thread takes the first batch (loads guarded), so that all
            // of them reach get_base
            if (!first && j >= nvalid) break;
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
            if (LATE && first) {
                dst = out + get_base() * D;
                first = false;
            }
#pragma unroll
            for (int k = 0; k < kBatch; ++k) {
                if (j < nvalid)
                    __builtin_nontemporal_store(v[k], reinterpret_cast<u32x4*>(dst + j * D) + c);
                j += step_j;
                c += step_c;
                if (c >= nch) { c -= nch; ++j; }
            }
        }
    } else {
        uint16_t* dst = out + get_base() * D;
        for (int j = 0; j < nvalid; ++j) {
            const uint16_t* src = x + rowsrc[j] * D;
            uint16_t* d = dst + j * D;
            for (int64_t c = tid; c < D; c += kBlock) d[c] = src[c];
        }
    }
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

    // 1. rank of this block's rows: a ballot over the first kRowsPerBlock lanes
    if (tid < 64) {
        const int64_t r = r0 + tid;
        const bool valid = tid < kRowsPerBlock && r < R && mask[r] != 0;
        const uint64_t bal = __ballot(valid);
        if (valid) rowsrc[__builtin_popcountll(bal & ((1ull << tid) - 1))] = r;
        if (tid == 0) nvalid_s = __builtin_popcountll(bal);
    }
    __syncthreads();
    const int nvalid = nvalid_s;

    // 2. copy (item i is chunk i % nch of valid row i / nch); the valid rows
    // before r0 (r0 is a multiple of 8, so whole words) are counted while the
    // first loads are in flight
    auto get_base = [&]() -> int64_t {
        int local = 0;
        if (mask_words) {
            const uint32_t* mw = reinterpret_cast<const uint32_t*>(mask);
            for (int64_t i = tid; i < r0 / 4; i += kBlock) local += nonzero_bytes(mw[i]);
        } else {
            for (int64_t i = tid; i < r0; i += kBlock) local += (mask[i] != 0);
        }
        const int base = block_sum(local, red);
        if (blockIdx.x == gridDim.x - 1 && tid == 0) *count = base + nvalid;
        if (tid < nvalid) src_row[base + tid] = (int32_t)rowsrc[tid];
        return base;
    };
    copy_rows<VEC16, true>(x, D, rowsrc, nvalid, out, get_base);
}

// ---- the linear-time path ----

// Flags (bit b) of the nonzero bytes among mask[i .. i+15], bytes at or past
// `end` reading as zero.  VEC: the mask is 16-byte aligned (i is a multiple of
// 16), so whole groups are one load.
template <bool VEC>
__device__ __forceinline__ uint32_t mask_flags16(const uint8_t* __restrict__ mask, int64_t i,
                                                 int64_t end) {
    uint32_t f = 0;
    if (VEC && i + 16 <= end) {
        const u32x4 v = *reinterpret_cast<const u32x4*>(mask + i);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const uint32_t w = v[k];
            const uint32_t nz = (((w & 0x7f7f7f7fu) + 0x7f7f7f7fu) | w) & 0x80808080u;
            f |= (((nz >> 7) & 1u) | ((nz >> 14) & 2u) | ((nz >> 21) & 4u) | ((nz >> 28) & 8u))
                 << (4 * k);
        }
    } else {
        for (int b = 0; b < 16; ++b)
            if (i + b < end && mask[i + b] != 0) f |= 1u << b;
    }
    return f;
}

// Exclusive scan of v over the block (kBlock threads); *total gets the sum.
// Every thread of the block calls it.
__device__ __forceinline__ int block_exclusive_scan(int v, int* red, int* total) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    int x = v;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int y = __shfl_up(x, off, 64);
        if (lane >= off) x += y;
    }
    if (lane == 63) red[wave] = x;
    __syncthreads();
    int before = 0;
#pragma unroll
    for (int w = 0; w < kBlock / 64; ++w) before += w < wave ? red[w] : 0;
    *total = red[0] + red[1] + red[2] + red[3];
    __syncthreads();  // red is free for the next call
    return before + x - v;
}

constexpr int kScanTile = kBlock * 16;  // mask bytes a workgroup takes per step

// Step 1: cnt[g] = valid rows of chunk g (rows [g*chunk, min((g+1)*chunk, R))).
template <bool VEC>
__global__ __launch_bounds__(kBlock) void compact_count_chunks(const uint8_t* __restrict__ mask,
                                                               int64_t R, int64_t chunk,
                                                               int32_t* __restrict__ cnt) {
    __shared__ int red[kBlock / 64];
    const int64_t lo = (int64_t)blockIdx.x * chunk;
    const int64_t hi = lo + chunk < R ? lo + chunk : R;
    int local = 0;
    for (int64_t i = lo + 16 * threadIdx.x; i < hi; i += kScanTile)
        local += __builtin_popcount(mask_flags16<VEC>(mask, i, hi));
    const int sum = block_sum(local, red);
    if (threadIdx.x == 0) cnt[blockIdx.x] = sum;
}

// Step 2: src_row of chunk g's valid rows (cnt: the counts of step 1, NULL for
// a single chunk); the last workgroup writes *count.
template <bool VEC>
__global__ __launch_bounds__(kBlock) void compact_index_chunks(
    const uint8_t* __restrict__ mask, int64_t R, int64_t chunk, const int32_t* __restrict__ cnt,
    int32_t* __restrict__ src_row, int32_t* __restrict__ count) {
    __shared__ int red[kBlock / 64];
    const int g = blockIdx.x;
    int p = 0;
    if (cnt)
        for (int h = threadIdx.x; h < g; h += kBlock) p += cnt[h];
    int64_t base = block_sum(p, red);
    __syncthreads();  // red is reused by the scans
    const int64_t lo = (int64_t)g * chunk;
    const int64_t hi = lo + chunk < R ? lo + chunk : R;
    for (int64_t t0 = lo; t0 < hi; t0 += kScanTile) {
        const int64_t i = t0 + 16 * threadIdx.x;
        uint32_t f = i < hi ? mask_flags16<VEC>(mask, i, hi) : 0u;
        int total;
        int64_t m = base + block_exclusive_scan(__builtin_popcount(f), red, &total);
        while (f) {
            src_row[m++] = (int32_t)(i + __builtin_ctz(f));
            f &= f - 1;
        }
        base += total;
    }
    if (g == (int)gridDim.x - 1 && threadIdx.x == 0) *count = (int32_t)base;
}

// Step 3 of plain compaction: out[m] = x[src_row[m]] for m < *count, blocks of
// kRowsPerBlock output rows in a grid-stride loop.
template <bool VEC16>
__global__ __launch_bounds__(kBlock) void compact_gather_rows(
    const uint16_t* __restrict__ x, int64_t D, const int32_t* __restrict__ src_row,
    const int32_t* __restrict__ count, uint16_t* __restrict__ out) {
    __shared__ int64_t rowsrc[kRowsPerBlock];
    const int64_t n = *count;
    for (int64_t m0 = (int64_t)blockIdx.x * kRowsPerBlock; m0 < n;
         m0 += (int64_t)gridDim.x * kRowsPerBlock) {
        const int nvalid = (int)(n - m0 < kRowsPerBlock ? n - m0 : kRowsPerBlock);
        __syncthreads();  // the previous rows' copies are done with rowsrc
        if ((int)threadIdx.x < nvalid) rowsrc[threadIdx.x] = src_row[m0 + threadIdx.x];
        __syncthreads();
        copy_rows<VEC16, false>(x, D, rowsrc, nvalid, out, [&]() -> int64_t { return m0; });
    }
}

}  // namespace

bool compact_single_pass(int64_t R) { return R <= kSinglePassRows; }

int launch_compact_scan(const uint8_t* mask, int64_t R, int32_t* scratch, int64_t scratch_ints,
                        int32_t* src_row, int32_t* count, hipStream_t stream) {
    // chunks of whole 16-byte mask groups, at least kScanTile bytes, at most
    // kMaxChunks of them (and no more than the scratch holds)
    int64_t G = (R + kScanTile - 1) / kScanTile;
    if (G > kMaxChunks) G = kMaxChunks;
    if (G > scratch_ints) G = scratch_ints > 0 ? scratch_ints : 1;
    int64_t chunk = (R + G - 1) / G;
    chunk = (chunk + 15) & ~(int64_t)15;
    G = (R + chunk - 1) / chunk;
    if (G < 1) G = 1;
    const bool vec = reinterpret_cast<uintptr_t>(mask) % 16 == 0;
    const int32_t* cnt = nullptr;
    if (G > 1) {
        if (vec)
            hipLaunchKernelGGL(compact_count_chunks<true>, dim3((unsigned)G), dim3(kBlock), 0,
                               stream, mask, R, chunk, scratch);
        else
            hipLaunchKernelGGL(compact_count_chunks<false>, dim3((unsigned)G), dim3(kBlock), 0,
                               stream, mask, R, chunk, scratch);
        if (hipGetLastError() != hipSuccess) return -1;
        cnt = scratch;
    }
    if (vec)
        hipLaunchKernelGGL(compact_index_chunks<true>, dim3((unsigned)G), dim3(kBlock), 0, stream,
                           mask, R, chunk, cnt, src_row, count);
    else
        hipLaunchKernelGGL(compact_index_chunks<false>, dim3((unsigned)G), dim3(kBlock), 0, stream,
                           mask, R, chunk, cnt, src_row, count);
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

int launch_compact_rows(const uint16_t* x, const uint8_t* mask, int64_t R, int64_t D,
                        uint16_t* out, int32_t* src_row, int32_t* count, hipStream_t stream) {
    const bool vec16 = D > 0 && (D % 8 == 0) && (reinterpret_cast<uintptr_t>(x) % 16 == 0) &&
                       (reinterpret_cast<uintptr_t>(out) % 16 == 0);
    if (compact_single_pass(R)) {
        const int64_t blocks = R > 0 ? (R + kRowsPerBlock - 1) / kRowsPerBlock : 1;
        const int mask_words = reinterpret_cast<uintptr_t>(mask) % 4 == 0 ? 1 : 0;
        if (vec16)
            hipLaunchKernelGGL(compact_rows_kernel<true>, dim3((unsigned)blocks), dim3(kBlock), 0,
                               stream, x, mask, R, D, out, src_row, count, mask_words);
        else
            hipLaunchKernelGGL(compact_rows_kernel<false>, dim3((unsigned)blocks), dim3(kBlock), 0,
                               stream, x, mask, R, D, out, src_row, count, mask_words);
        return hipGetLastError() == hipSuccess ? 0 : -1;
    }
    // the chunk counts live in out's first bytes (4-byte aligned) until the gather
    // overwrites them; D == 0 leaves no room, and one chunk needs none
    int32_t* scratch = reinterpret_cast<int32_t*>(reinterpret_cast<uintptr_t>(out) +
                                                  (reinterpret_cast<uintptr_t>(out) & 2));
    const int64_t room = D > 0 ? (R * D * 2 - 2) / 4 : 0;
    if (launch_compact_scan(mask, R, scratch, room, src_row, count, stream) != 0) return -1;
    if (D == 0) return 0;
    const int cus = cu_count();
    if (cus <= 0) return -1;
    int64_t blocks = (R + kRowsPerBlock - 1) / kRowsPerBlock;
    if (blocks > (int64_t)cus * 16) blocks = (int64_t)cus * 16;
    if (vec16)
        hipLaunchKernelGGL(compact_gather_rows<true>, dim3((unsigned)blocks), dim3(kBlock), 0,
                           stream, x, D, src_row, count, out);
    else
        hipLaunchKernelGGL(compact_gather_rows<false>, dim3((unsigned)blocks), dim3(kBlock), 0,
                           stream, x, D, src_row, count, out);
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace w8a8
