// INT8 x INT8 -> INT32 GEMM with the once-after-accumulation epilogue, gfx950.
//
// TurboT2VA (智猩猩 article, section 01.3 "量化策略"): the W8A8 product is
// accumulated in INT32 and the scales and bias are applied once, after the
// whole accumulation, never per K block.  Here
//     acc[i][j] = sum_k qa[i][k] * qw[j][k]              (exact int32)
//     y[i][j]   = bf16_RNE(fma(float(acc), RN32(sa[i]*sw[j]), bias[j]))
// with an optional GELU-tanh on the bf16 y, or the raw acc in int32 mode.
//
// Both operands are K-contiguous (qa [M x K], qw [N x K]), the layout the MFMA
// A/B operands want: every lane feeds 16 consecutive K bytes of one row.
#include "common.h"

namespace w8a8 {

namespace {

// ---------------------------------------------------------------------------
// Simple tiled kernel: 128x128 macro tile, BK = 64, 4 waves each 64x64, single
// LDS buffer.  v_mfma_i32_16x16x64_i8; used for every shape the guard admits.
// ---------------------------------------------------------------------------
constexpr int S_BM = 128, S_BN = 128, S_BK = 64, S_PITCH = S_BK + 16;

template <int OUT_I32, int ACT>
__global__ __launch_bounds__(256) void gemm_i8_simple(const int8_t* __restrict__ qa,
                                                      const float* __restrict__ sa, int64_t M,
                                                      const int8_t* __restrict__ qw,
                                                      const float* __restrict__ sw, int64_t N,
                                                      int64_t K, const uint16_t* __restrict__ bias,
                                                      void* __restrict__ out) {
    __shared__ __attribute__((aligned(16))) int8_t As[S_BM * S_PITCH];
    __shared__ __attribute__((aligned(16))) int8_t Bs[S_BN * S_PITCH];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int64_t ntn = (N + S_BN - 1) / S_BN;
    const int64_t m0 = ((int64_t)blockIdx.x / ntn) * S_BM, n0 = ((int64_t)blockIdx.x % ntn) * S_BN;

    v4i acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = (v4i){0, 0, 0, 0};

    // each thread moves 2 chunks of 16 bytes of A and of B per K step
    int lrow[2], lcol[2];
    const int8_t* ga[2];
    const int8_t* gb[2];
#pragma unroll
    for (int c = 0; c < 2; ++c) {
        const int chunk = tid + c * 256;
        lrow[c] = chunk >> 2;
        lcol[c] = (chunk & 3) * 16;
        int64_t gm = m0 + lrow[c];
        if (gm > M - 1) gm = M - 1;
        int64_t gn = n0 + lrow[c];
        if (gn > N - 1) gn = N - 1;
        ga[c] = qa + gm * K + lcol[c];
        gb[c] = qw + gn * K + lcol[c];
    }

    for (int64_t k0 = 0; k0 < K; k0 += S_BK) {
        v4i ra[2], rb[2];
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            ra[c] = *reinterpret_cast<const v4i*>(ga[c] + k0);
            rb[c] = *reinterpret_cast<const v4i*>(gb[c] + k0);
        }
        __syncthreads();
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            *reinterpret_cast<v4i*>(As + lrow[c] * S_PITCH + lcol[c]) = ra[c];
            *reinterpret_cast<v4i*>(Bs + lrow[c] * S_PITCH + lcol[c]) = rb[c];
        }
        __syncthreads();
        v4i fa[4], fb[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            fa[i] = *reinterpret_cast<const v4i*>(As + (wm * 64 + i * 16 + (lane & 15)) * S_PITCH +
                                                  (lane >> 4) * 16);
            fb[i] = *reinterpret_cast<const v4i*>(Bs + (wn * 64 + i * 16 + (lane & 15)) * S_PITCH +
                                                  (lane >> 4) * 16);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(fa[i], fb[j], acc[i][j], 0, 0, 0);
    }

    // C layout of a 16x16 MFMA tile: lane l holds column (l & 15), rows 4*(l >> 4) + r.
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int64_t col = n0 + wn * 64 + j * 16 + (lane & 15);
            if (col >= N) continue;
            float swj = 0.f, bj = 0.f;
            if (!OUT_I32) {
                swj = sw[col];
                bj = bias ? bf16_bits_to_float(bias[col]) : 0.f;
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int64_t row = m0 + wm * 64 + i * 16 + (lane >> 4) * 4 + r;
                if (row >= M) continue;
                if (OUT_I32) {
                    reinterpret_cast<int32_t*>(out)[row * N + col] = acc[i][j][r];
                } else {
                    reinterpret_cast<uint16_t*>(out)[row * N + col] =
                        (uint16_t)epilogue_bf16<ACT>(acc[i][j][r], sa[row], swj, bj, bias != nullptr);
                }
            }
        }
    }
}

template <int OUT_I32, int ACT>
hipError_t launch_simple(const int8_t* qa, const float* sa, int64_t M, const int8_t* qw,
                         const float* sw, int64_t N, int64_t K, const uint16_t* bias, void* out,
                         hipStream_t stream) {
    const int64_t tiles = ((N + S_BN - 1) / S_BN) * ((M + S_BM - 1) / S_BM);
    hipLaunchKernelGGL((gemm_i8_simple<OUT_I32, ACT>), dim3((unsigned)tiles), dim3(256), 0, stream, qa, sa, M, qw,
                       sw, N, K, bias, out);
    return hipGetLastError();
}

}  // namespace

int launch_gemm_i8(const int8_t* qa, const float* sa, int64_t M, const int8_t* qw,
                   const float* sw, int64_t N, int64_t K, const uint16_t* bias, int act,
                   int out_kind, void* out, hipStream_t stream) {
    if (M == 0 || N == 0) return 0;
    hipError_t e;
    if (out_kind == 1) e = launch_simple<1, 0>(qa, sa, M, qw, sw, N, K, bias, out, stream);
    else if (act == 1) e = launch_simple<0, 1>(qa, sa, M, qw, sw, N, K, bias, out, stream);
    else e = launch_simple<0, 0>(qa, sa, M, qw, sw, N, K, bias, out, stream);
    return e == hipSuccess ? 0 : -1;
}

}  // namespace w8a8
