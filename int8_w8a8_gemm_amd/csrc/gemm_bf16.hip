// Native BF16 linear, the fallback of the guarded W8A8 layer, for gfx950.
//
// TurboT2VA (智猩猩 article, section 01.3 "量化策略"): branches whose matrix
// shapes the optimised INT8 operator cannot serve run in native BF16.
//     y[i][j] = bf16_RNE(sum_k x[i][k] * w[j][k] + b[j])
// with fp32 accumulation and an optional GELU-tanh on the bf16 result.
// Operands with K even and 4-byte aligned rows take the tiled MFMA kernel
// shared with the INT8 path (gemm_tiled.hip, any M and N; the K tail of the
// last stage is masked).  Everything else (K odd or 2-byte aligned operands)
// takes the kernel below: v_mfma_f32_16x16x32_bf16 on 128 x 128 tiles with
// every edge masked, operands read element by element.
#include "common.h"

namespace w8a8 {

namespace {

constexpr int F_BM = 128, F_BN = 128, F_BK = 32, F_PITCH = F_BK + 8;  // bf16 elements

// Loads a 128 x 32 bf16 tile (rows r0.., cols k0..) into LDS with zero fill
// outside [0, R) x [0, K).  PAIRS: rows hold an even number of elements and are
// 4-byte aligned, so pairs are loaded as one dword.
template <int PAIRS>
__device__ __forceinline__ void load_tile(const uint16_t* __restrict__ g, int64_t R, int64_t K,
                                          int64_t r0, int64_t k0, uint16_t* __restrict__ s) {
    const int tid = threadIdx.x;
    if (PAIRS) {
        // 128 rows x 16 pairs = 2048 dwords, 8 per thread
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int idx = tid + i * 256;
            const int row = idx >> 4, pc = idx & 15;
            const int64_t gr = r0 + row, gk = k0 + 2 * pc;
            uint32_t v = 0;
            if (gr < R && gk < K) v = *reinterpret_cast<const uint32_t*>(g + gr * K + gk);
            *reinterpret_cast<uint32_t*>(s + row * F_PITCH + 2 * pc) = v;
        }
    } else {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int idx = tid + i * 256;
            const int row = idx >> 5, c = idx & 31;
            const int64_t gr = r0 + row, gk = k0 + c;
            uint16_t v = 0;
            if (gr < R && gk < K) v = g[gr * K + gk];
            s[row * F_PITCH + c] = v;
        }
    }
}

template <int PAIRS, int ACT>
__global__ __launch_bounds__(256) void gemm_bf16_kernel(const uint16_t* __restrict__ x, int64_t M,
                                                        int64_t K, const uint16_t* __restrict__ w,
                                                        int64_t N, const uint16_t* __restrict__ bias,
                                                        uint16_t* __restrict__ y) {
    __shared__ __attribute__((aligned(16))) uint16_t As[F_BM * F_PITCH];
    __shared__ __attribute__((aligned(16))) uint16_t Bs[F_BN * F_PITCH];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int64_t ntn = (N + F_BN - 1) / F_BN;
    const int64_t m0 = ((int64_t)blockIdx.x / ntn) * F_BM, n0 = ((int64_t)blockIdx.x % ntn) * F_BN;

    v4f acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = (v4f){0.f, 0.f, 0.f, 0.f};

    for (int64_t k0 = 0; k0 < K; k0 += F_BK) {
        __syncthreads();
        load_tile<PAIRS>(x, M, K, m0, k0, As);
        load_tile<PAIRS>(w, N, K, n0, k0, Bs);
        __syncthreads();
        v8bf fa[4], fb[4];
        // 16x16x32 bf16 operand: lane l feeds row (l & 15), 8 consecutive K at 8*(l >> 4)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            fa[i] = *reinterpret_cast<const v8bf*>(As + (wm * 64 + i * 16 + (lane & 15)) * F_PITCH +
                                                   (lane >> 4) * 8);
            fb[i] = *reinterpret_cast<const v8bf*>(Bs + (wn * 64 + i * 16 + (lane & 15)) * F_PITCH +
                                                   (lane >> 4) * 8);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0);
    }

#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int64_t col = n0 + wn * 64 + j * 16 + (lane & 15);
            if (col >= N) continue;
            const float bj = bias ? bf16_bits_to_float(bias[col]) : 0.f;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int64_t row = m0 + wm * 64 + i * 16 + (lane >> 4) * 4 + r;
                if (row >= M) continue;
                uint32_t h = float_to_bf16_bits(__fadd_rn(acc[i][j][r], bj));
                if (ACT == 1) h = gelu_bf16_rn(h);
                y[row * N + col] = (uint16_t)h;
            }
        }
    }
}

template <int PAIRS, int ACT>
hipError_t launch(const uint16_t* x, int64_t M, int64_t K, const uint16_t* w, int64_t N,
                  const uint16_t* bias, uint16_t* y, hipStream_t stream) {
    const int64_t tiles = ((N + F_BN - 1) / F_BN) * ((M + F_BM - 1) / F_BM);
    hipLaunchKernelGGL((gemm_bf16_kernel<PAIRS, ACT>), dim3((unsigned)tiles), dim3(256), 0, stream, x, M, K, w, N,
                       bias, y);
    return hipGetLastError();
}

}  // namespace

int launch_gemm_bf16(const uint16_t* x, int64_t M, int64_t K, const uint16_t* w, int64_t N,
                     const uint16_t* bias, int act, uint16_t* y, hipStream_t stream) {
    if (M == 0 || N == 0) return 0;
    if (gemm_bf16_tiled_ok(x, K, w)) return launch_gemm_bf16_tiled(x, M, K, w, N, bias, act, y, stream);
    const bool pairs = (K % 2 == 0) && (reinterpret_cast<uintptr_t>(x) % 4 == 0) &&
                       (reinterpret_cast<uintptr_t>(w) % 4 == 0);
    hipError_t e;
    if (pairs) e = act ? launch<1, 1>(x, M, K, w, N, bias, y, stream)
                       : launch<1, 0>(x, M, K, w, N, bias, y, stream);
    else e = act ? launch<0, 1>(x, M, K, w, N, bias, y, stream)
                 : launch<0, 0>(x, M, K, w, N, bias, y, stream);
    return e == hipSuccess ? 0 : -1;
}

}  // namespace w8a8
