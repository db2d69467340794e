// Measurement probes (not part of the W8A8 library's ABI): how fast the INT8
// matrix cores run on this GPU for a given kind of operand data and LDS
// traffic, and how fast plain streaming kernels move HBM data.
//
// MI355X is power-capped, and the energy of v_mfma_i32_32x32x32_i8 depends on
// how much its operands toggle: the clock the part sustains, and so the
// reachable INT8 rate, falls as operand data gets more random.  This probe runs
// a loop of independent MFMAs (8 accumulators per wave, one wave per SIMD, no
// memory traffic in the loop) on operands of a chosen kind and reports the
// achieved rate and the shader clock (s_memtime against the 100 MHz
// s_memrealtime counter).  It bounds what any INT8 GEMM can reach on such data.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

constexpr int kBlocks = 1024;  // 4 waves x 1024 = one wave per SIMD on 256 CUs
constexpr int kOperands = 4096;

__global__ __launch_bounds__(256) void mfma_loop(const v4i* __restrict__ ops, int* __restrict__ sink,
                                                 long long* __restrict__ clk, int iters) {
    v4i a[4], b[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        a[i] = ops[(threadIdx.x + i * 256) % kOperands];
        b[i] = ops[(threadIdx.x * 7 + i * 911 + 5) % kOperands];
    }
    v16i c[8] = {};
    const long long t0 = __builtin_readcyclecounter();
    const long long r0 = __builtin_amdgcn_s_memrealtime();
    for (int it = 0; it < iters; ++it) {
        // operand registers chosen at compile time: consecutive MFMAs see
        // different data, and no instruction between them rewrites an operand
#pragma unroll
        for (int j = 0; j < 8; ++j)
            c[j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a[j & 3], b[(j >> 1) & 3], c[j], 0, 0, 0);
    }
    const long long t1 = __builtin_readcyclecounter();
    const long long r1 = __builtin_amdgcn_s_memrealtime();
    int s = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) s += c[j][e];
    sink[blockIdx.x * 256 + threadIdx.x] = s;
    if (threadIdx.x == 0 && blockIdx.x == 0) {
        clk[0] = t1 - t0;
        clk[1] = r1 - r0;
    }
}

// The same MFMA loop at two waves per SIMD (8 waves, one workgroup per CU),
// either with operands fixed in registers (READS = 0) or with READS of the 6
// fragment registers refreshed from LDS by ds_read_b128 per 8 MFMAs, interleaved
// with them like a GEMM's K loop (6 per 8 is the 256 x 256 GEMM tile's rate).
// LDS holds 64 KB of the operand data; every read stays inside it.
constexpr int kLdsBytes = 96 * 1024;  // more than half the CU's LDS: one workgroup per CU

template <int READS>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
void mfma_lds_loop(const v4i* __restrict__ ops, int* __restrict__ sink, long long* __restrict__ clk,
                   int iters) {
    __shared__ __attribute__((aligned(1024))) char lds[kLdsBytes];
    for (int i = threadIdx.x; i < kOperands; i += 512) reinterpret_cast<v4i*>(lds)[i] = ops[i];
    __syncthreads();
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    v4i fa[2], fb[4];
#pragma unroll
    for (int q = 0; q < 2; ++q) fa[q] = ops[(threadIdx.x + q * 512) % kOperands];
#pragma unroll
    for (int q = 0; q < 4; ++q) fb[q] = ops[(threadIdx.x * 7 + q * 911 + 5) % kOperands];
    // never true (iters > 0): keeps the LDS array, and so one workgroup per CU,
    // in the variant without reads
    if (iters < 0) fa[0] = *reinterpret_cast<const v4i*>(lds + lane * 16);
    v16i c[8] = {};
    const long long t0 = __builtin_readcyclecounter();
    const long long r0 = __builtin_amdgcn_s_memrealtime();
    for (int it = 0; it < iters; ++it) {
        v4i nf[6];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            c[j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(fb[j >> 1], fa[j & 1], c[j], 0, 0, 0);
            if (j < READS) {
                // 1 KB-aligned slot ((..) & 63) of the 64 KB, 16 bytes per lane
                const int off = (((it * 6 + j + wave * 5) & 63) << 10) + lane * 16;
                nf[j] = *reinterpret_cast<const v4i*>(lds + off);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int j = 0; j < READS; ++j) {
            if (j < 2) fa[j] = nf[j];
            else fb[j - 2] = nf[j];
        }
    }
    const long long t1 = __builtin_readcyclecounter();
    const long long r1 = __builtin_amdgcn_s_memrealtime();
    int s = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) s += c[j][e];
    sink[blockIdx.x * 512 + threadIdx.x] = s;
    if (threadIdx.x == 0 && blockIdx.x == 0) {
        clk[0] = t1 - t0;
        clk[1] = r1 - r0;
    }
}

template <int READS>
hipError_t run_lds(const void* ops, int* sink, long long* clk, int iters, int cus, hipStream_t s) {
    hipLaunchKernelGGL(mfma_lds_loop<READS>, dim3((unsigned)cus), dim3(512), 0, s,
                       (const v4i*)ops, sink, clk, iters);
    return hipGetLastError();
}

// Streaming kernels for the practical HBM ceiling: 16-byte nontemporal loads
// and stores, grid-stride over n16 chunks (every index below n16).
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

__global__ __launch_bounds__(256) void stream_read(const u32x4* __restrict__ a, size_t n16,
                                                   unsigned* __restrict__ sink) {
    unsigned acc = 0;
    for (size_t i = blockIdx.x * 256ull + threadIdx.x; i < n16; i += (size_t)gridDim.x * 256) {
        const u32x4 v = __builtin_nontemporal_load(a + i);
        acc ^= v.x ^ v.y ^ v.z ^ v.w;
    }
    if (acc == 0x9e3779b9u) sink[0] = acc;  // keeps the loads
}

__global__ __launch_bounds__(256) void stream_write(u32x4* __restrict__ b, size_t n16) {
    for (size_t i = blockIdx.x * 256ull + threadIdx.x; i < n16; i += (size_t)gridDim.x * 256)
        __builtin_nontemporal_store((u32x4){1u, 2u, 3u, (unsigned)i}, b + i);
}

__global__ __launch_bounds__(256) void stream_copy(const u32x4* __restrict__ a,
                                                   u32x4* __restrict__ b, size_t n16) {
    for (size_t i = blockIdx.x * 256ull + threadIdx.x; i < n16; i += (size_t)gridDim.x * 256)
        __builtin_nontemporal_store(__builtin_nontemporal_load(a + i), b + i);
}

// 16 bytes read, 8 written: the 2:1 mix of the quantisers (bf16 in, int8 out)
__global__ __launch_bounds__(256) void stream_half(const u32x4* __restrict__ a,
                                                   u32x2* __restrict__ b, size_t n16) {
    for (size_t i = blockIdx.x * 256ull + threadIdx.x; i < n16; i += (size_t)gridDim.x * 256) {
        const u32x4 v = __builtin_nontemporal_load(a + i);
        __builtin_nontemporal_store((u32x2){v.x ^ v.y, v.z ^ v.w}, b + i);
    }
}

}  // namespace

extern "C" __attribute__((visibility("default")))
// Practical HBM streaming rate.  kind 0: read n16 x 16 bytes of src; 1: write
// them to dst; 2: copy src -> dst; 3: read 16 bytes and write 8 per chunk
// (dst needs n16 x 8 bytes).  nbuf source / destination buffers (src[i],
// dst[i], each n16 x 16 bytes) are used in turn so that caches cannot hold the
// data; grid workgroups of 256 threads.  Runs `iters` untimed then `iters`
// timed launches and returns the average time of one in *ms.
int w8a8_probe_stream(int kind, void* const* src, void* const* dst, int nbuf, size_t n16, int grid,
                      int iters, unsigned* sink, float* ms, void* stream) {
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    if (kind < 0 || kind > 3 || nbuf <= 0 || grid <= 0 || iters <= 0) return -1;
    auto launch = [&](int i) {
        const u32x4* a = static_cast<const u32x4*>(src[i % nbuf]);
        void* b = dst[i % nbuf];
        if (kind == 0)
            hipLaunchKernelGGL(stream_read, dim3(grid), dim3(256), 0, s, a, n16, sink);
        else if (kind == 1)
            hipLaunchKernelGGL(stream_write, dim3(grid), dim3(256), 0, s, (u32x4*)b, n16);
        else if (kind == 2)
            hipLaunchKernelGGL(stream_copy, dim3(grid), dim3(256), 0, s, a, (u32x4*)b, n16);
        else
            hipLaunchKernelGGL(stream_half, dim3(grid), dim3(256), 0, s, a, (u32x2*)b, n16);
    };
    hipEvent_t e0, e1;
    if (hipEventCreate(&e0) != hipSuccess || hipEventCreate(&e1) != hipSuccess) return -3;
    for (int i = 0; i < iters; ++i) launch(i);
    bool ok = hipEventRecord(e0, s) == hipSuccess;
    for (int i = 0; i < iters; ++i) launch(i);
    ok = ok && hipEventRecord(e1, s) == hipSuccess;
    ok = ok && hipEventSynchronize(e1) == hipSuccess;
    ok = ok && hipEventElapsedTime(ms, e0, e1) == hipSuccess;
    if (ok) *ms /= (float)iters;
    ok = (hipEventDestroy(e0) == hipSuccess) && ok;
    ok = (hipEventDestroy(e1) == hipSuccess) && ok;
    return ok && hipGetLastError() == hipSuccess ? 0 : -3;
}

extern "C" __attribute__((visibility("default")))
// As w8a8_probe_mfma, at two waves per SIMD (one 8-wave workgroup on each of
// `cus` CUs; sink holds cus*512 ints) with `reads` (0, 3 or 6) fragment
// registers refreshed from LDS per 8 MFMAs.
int w8a8_probe_mfma_lds(const void* ops, int* sink, long long* clk, int iters, int reads, int cus,
                        float* ms, void* stream) {
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    if (reads != 0 && reads != 3 && reads != 6) return -1;
    if (cus <= 0 || iters <= 0) return -1;
    auto launch = [&]() {
        return reads == 0 ? run_lds<0>(ops, sink, clk, iters, cus, s)
               : reads == 3 ? run_lds<3>(ops, sink, clk, iters, cus, s)
                            : run_lds<6>(ops, sink, clk, iters, cus, s);
    };
    hipEvent_t e0, e1;
    if (hipEventCreate(&e0) != hipSuccess || hipEventCreate(&e1) != hipSuccess) return -3;
    bool ok = launch() == hipSuccess;
    ok = ok && hipEventRecord(e0, s) == hipSuccess;
    ok = ok && launch() == hipSuccess;
    ok = ok && hipEventRecord(e1, s) == hipSuccess;
    ok = ok && hipEventSynchronize(e1) == hipSuccess;
    ok = ok && hipEventElapsedTime(ms, e0, e1) == hipSuccess;
    ok = (hipEventDestroy(e0) == hipSuccess) && ok;
    ok = (hipEventDestroy(e1) == hipSuccess) && ok;
    return ok ? 0 : -3;
}

extern "C" __attribute__((visibility("default")))
// ops: device buffer of 4096 x 16 bytes of int8 operand data; sink: device int
// buffer of 1024*256; clk: device int64[2].  Runs the loop twice (the first is
// a warm-up) and returns the second run's time in *ms plus the cycle counts.
int w8a8_probe_mfma(const void* ops, int* sink, long long* clk, int iters, float* ms,
                    void* stream) {
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    hipEvent_t e0, e1;
    if (hipEventCreate(&e0) != hipSuccess || hipEventCreate(&e1) != hipSuccess) return -3;
    hipLaunchKernelGGL(mfma_loop, dim3(kBlocks), dim3(256), 0, s, (const v4i*)ops, sink, clk, iters);
    bool ok = hipEventRecord(e0, s) == hipSuccess;
    hipLaunchKernelGGL(mfma_loop, dim3(kBlocks), dim3(256), 0, s, (const v4i*)ops, sink, clk, iters);
    ok = ok && hipEventRecord(e1, s) == hipSuccess;
    ok = ok && hipEventSynchronize(e1) == hipSuccess;
    ok = ok && hipEventElapsedTime(ms, e0, e1) == hipSuccess;
    ok = (hipEventDestroy(e0) == hipSuccess) && ok;
    ok = (hipEventDestroy(e1) == hipSuccess) && ok;
    return ok && hipGetLastError() == hipSuccess ? 0 : -3;
}
