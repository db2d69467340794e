// Measurement probe (not part of the W8A8 library's ABI): how fast the INT8
// matrix cores run on this GPU for a given kind of operand data.
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

}  // namespace

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
