// C ABI of libw8a8: argument checks, the shape guard and routing.
//
// Every check runs on the host before any launch; a failed check returns
// W8A8_EINVAL and enqueues nothing.  Work goes onto the caller's stream; the
// library allocates, frees and synchronises nothing.
#include "../../include/w8a8.h"
#include "common.h"

#include <atomic>

namespace {

constexpr int64_t kMaxRows = (int64_t)1 << 31;  // grid limits of the row-wise kernels

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }
bool act_ok(int act) { return act == W8A8_ACT_NONE || act == W8A8_ACT_GELU_TANH; }
hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }
int launched(int rc) { return rc == 0 ? W8A8_OK : W8A8_EHIP; }

}  // namespace

extern "C" {

int w8a8_guard(int64_t N, int64_t K) {
    // INT8 kernel requirements: whole 128-byte K steps (no K tail), N in
    // multiples of 64, and K small enough that |acc| <= 127*127*K < 2^31.
    return (K >= 128 && K <= W8A8_MAX_K && K % 128 == 0 && N >= 64 && N % 64 == 0) ? 1 : 0;
}

size_t w8a8_linear_workspace_bytes(int64_t M, int64_t K) {
    if (M <= 0 || K <= 0) return 0;
    const size_t codes = ((size_t)M * (size_t)K + 255) & ~(size_t)255;
    return codes + (size_t)M * sizeof(float);
}

const char* w8a8_status_str(int status) {
    switch (status) {
        case W8A8_OK: return "ok";
        case W8A8_EINVAL: return "invalid argument";
        case W8A8_EUNSUPPORTED: return "shape not supported by the INT8 GEMM";
        case W8A8_EHIP: return "HIP launch failed";
        case W8A8_ESCRATCH: return "input larger than the no-allocation scratch";
        default: return "unknown status";
    }
}

int w8a8_quantize_rows(const uint16_t* x, int64_t rows, int64_t cols, int8_t* q, float* scale,
                       void* stream) {
    if (rows < 0 || cols < 0 || rows >= kMaxRows) return W8A8_EINVAL;
    if (rows == 0) return W8A8_OK;
    if (!scale || !aligned(scale, 4)) return W8A8_EINVAL;
    if (cols > 0 && (!x || !q || !aligned(x, 2))) return W8A8_EINVAL;
    return launched(w8a8::launch_quantize_rows(x, rows, cols, q, scale, as_stream(stream)));
}

int w8a8_quantize_blocks(const uint16_t* x, int64_t batch, int64_t seq, int64_t heads,
                         int64_t head_dim, int64_t block, int8_t* q, float* scale, void* stream) {
    if (batch < 0 || seq < 0 || heads < 0 || head_dim < 0 || block < 1) return W8A8_EINVAL;
    if (batch == 0 || seq == 0 || heads == 0) return W8A8_OK;
    if (head_dim < 8 || head_dim % 8 != 0) return W8A8_EINVAL;
    // the block is held in registers: at most 256 threads x 16 chunks of 8 values
    if ((seq < block ? seq : block) > W8A8_MAX_BLOCK_VALUES / head_dim) return W8A8_EINVAL;
    const int64_t nblk = (seq + block - 1) / block;
    if (heads > (kMaxRows - 1) / head_dim || nblk > (kMaxRows - 1) / heads ||
        batch > (kMaxRows - 1) / (nblk * heads))
        return W8A8_EINVAL;  // grid of batch * nblk * heads workgroups
    if (seq > INT64_MAX / (heads * head_dim) / batch) return W8A8_EINVAL;
    if (!x || !q || !scale || !aligned(x, 16) || !aligned(q, 8) || !aligned(scale, 4))
        return W8A8_EINVAL;
    return launched(w8a8::launch_quantize_blocks(x, batch, seq, heads, head_dim, block, q, scale,
                                                 as_stream(stream)));
}

namespace {
int norm_mod_args(const uint16_t* x, int64_t rows, int64_t cols, const uint16_t* shift,
                  const uint16_t* scale, int64_t rows_per_cond, int norm, double eps) {
    if (rows < 0 || cols < 1 || rows >= kMaxRows || rows_per_cond < 1) return W8A8_EINVAL;
    if (norm != W8A8_NORM_LAYER && norm != W8A8_NORM_RMS) return W8A8_EINVAL;
    if (!(eps >= 0.0) || !(eps < 1.0e300)) return W8A8_EINVAL;
    if (rows > 0 && (!x || !aligned(x, 2))) return W8A8_EINVAL;
    if ((shift && !aligned(shift, 2)) || (scale && !aligned(scale, 2))) return W8A8_EINVAL;
    if (rows > INT64_MAX / cols) return W8A8_EINVAL;
    return W8A8_OK;
}
}  // namespace

int w8a8_norm_mod_bf16(const uint16_t* x, int64_t rows, int64_t cols, const uint16_t* shift,
                       const uint16_t* scale, int64_t rows_per_cond, int norm, double eps,
                       uint16_t* y, void* stream) {
    const int st = norm_mod_args(x, rows, cols, shift, scale, rows_per_cond, norm, eps);
    if (st != W8A8_OK) return st;
    if (rows == 0) return W8A8_OK;
    if (!y || !aligned(y, 2)) return W8A8_EINVAL;
    return launched(w8a8::launch_norm_mod(x, rows, cols, shift, scale, rows_per_cond, norm, eps,
                                          nullptr, nullptr, y, as_stream(stream)));
}

int w8a8_norm_mod_quantize_rows(const uint16_t* x, int64_t rows, int64_t cols,
                                const uint16_t* shift, const uint16_t* scale,
                                int64_t rows_per_cond, int norm, double eps, int8_t* q,
                                float* qscale, void* stream) {
    const int st = norm_mod_args(x, rows, cols, shift, scale, rows_per_cond, norm, eps);
    if (st != W8A8_OK) return st;
    if (rows == 0) return W8A8_OK;
    if (!q || !qscale || !aligned(qscale, 4)) return W8A8_EINVAL;
    return launched(w8a8::launch_norm_mod(x, rows, cols, shift, scale, rows_per_cond, norm, eps, q,
                                          qscale, nullptr, as_stream(stream)));
}

int w8a8_gelu_quantize_rows(const uint16_t* y, int64_t rows, int64_t cols, int8_t* q,
                            float* scale, void* stream) {
    if (rows < 0 || cols < 0 || rows >= kMaxRows) return W8A8_EINVAL;
    if (rows == 0) return W8A8_OK;
    if (!scale || !aligned(scale, 4)) return W8A8_EINVAL;
    if (cols > 0 && (!y || !q || !aligned(y, 2))) return W8A8_EINVAL;
    return launched(w8a8::launch_quantize_rows(y, rows, cols, q, scale, as_stream(stream), true));
}

int w8a8_gelu_bf16(const uint16_t* x, int64_t n, uint16_t* y, void* stream) {
    if (n < 0) return W8A8_EINVAL;
    if (n == 0) return W8A8_OK;
    if (!x || !y || !aligned(x, 2) || !aligned(y, 2)) return W8A8_EINVAL;
    return launched(w8a8::launch_gelu_bf16(x, n, y, as_stream(stream)));
}

}  // extern "C"

namespace {
// The checks of w8a8_gemm's arguments; W8A8_OK if they pass.
int gemm_args(const int8_t* qa, const float* sa, int64_t M, const int8_t* qw, const float* sw,
              int64_t N, int64_t K, const uint16_t* bias, int act, int out_kind, void* out) {
    if (M < 0 || N < 0 || K < 0) return W8A8_EINVAL;
    if (!act_ok(act)) return W8A8_EINVAL;
    if (out_kind != W8A8_OUT_BF16 && out_kind != W8A8_OUT_I32) return W8A8_EINVAL;
    if (out_kind == W8A8_OUT_I32 && act != W8A8_ACT_NONE) return W8A8_EINVAL;
    if (!w8a8_guard(N, K)) return W8A8_EUNSUPPORTED;
    if (M >= kMaxRows) return W8A8_EINVAL;
    if (M == 0) return W8A8_OK;
    if (!qa || !qw || !out) return W8A8_EINVAL;
    if (!aligned(qa, 16) || !aligned(qw, 16) || !aligned(out, 16)) return W8A8_EINVAL;
    if (out_kind == W8A8_OUT_BF16) {
        if (!sa || !sw || !aligned(sa, 4) || !aligned(sw, 4)) return W8A8_EINVAL;
        if (bias && !aligned(bias, 2)) return W8A8_EINVAL;
    }
    return W8A8_OK;
}
}  // namespace

extern "C" {

int w8a8_gemm(const int8_t* qa, const float* sa, int64_t M, const int8_t* qw, const float* sw,
              int64_t N, int64_t K, const uint16_t* bias, int act, int out_kind, void* out,
              void* stream) {
    const int st = gemm_args(qa, sa, M, qw, sw, N, K, bias, act, out_kind, out);
    if (st != W8A8_OK || M == 0) return st;
    return launched(w8a8::launch_gemm_i8(qa, sa, M, qw, sw, N, K, bias, act, out_kind, out,
                                         as_stream(stream)));
}

size_t w8a8_gemm_splitk_workspace_bytes(int64_t M, int64_t N, int64_t K) {
    if (M <= 0 || N <= 0 || K <= 0 || M >= kMaxRows || !w8a8_guard(N, K)) return 0;
    return w8a8::splitk_workspace_bytes(M, N, K);
}

int w8a8_gemm_splitk(const int8_t* qa, const float* sa, int64_t M, const int8_t* qw,
                     const float* sw, int64_t N, int64_t K, const uint16_t* bias, int act,
                     int out_kind, void* out, void* workspace, size_t workspace_bytes,
                     void* stream) {
    const int st = gemm_args(qa, sa, M, qw, sw, N, K, bias, act, out_kind, out);
    if (st != W8A8_OK || M == 0) return st;
    const size_t need = w8a8_gemm_splitk_workspace_bytes(M, N, K);
    if (need > 0 && (!workspace || !aligned(workspace, 16) || workspace_bytes < need))
        return W8A8_EINVAL;
    return launched(w8a8::launch_gemm_i8_splitk(qa, sa, M, qw, sw, N, K, bias, act, out_kind, out,
                                                workspace, as_stream(stream)));
}

int w8a8_linear_bf16(const uint16_t* x, int64_t M, int64_t K, const uint16_t* w, int64_t N,
                     const uint16_t* bias, int act, uint16_t* y, void* stream) {
    if (M < 0 || N < 0 || K < 0 || M >= kMaxRows || N >= kMaxRows) return W8A8_EINVAL;
    if (!act_ok(act)) return W8A8_EINVAL;
    if (M == 0 || N == 0) return W8A8_OK;
    if (!y || !aligned(y, 2)) return W8A8_EINVAL;
    if (K > 0 && (!x || !w || !aligned(x, 2) || !aligned(w, 2))) return W8A8_EINVAL;
    if (bias && !aligned(bias, 2)) return W8A8_EINVAL;
    return launched(w8a8::launch_gemm_bf16(x, M, K, w, N, bias, act, y, as_stream(stream)));
}

}  // extern "C"

namespace {
// The checks of the guarded linear's arguments other than the workspace, for
// the path the guard picks (int8); W8A8_OK if they pass.
int linear_args(const uint16_t* x, int64_t M, int64_t K, int64_t N, const int8_t* qw,
                const float* sw, const uint16_t* w, const uint16_t* bias, int act, uint16_t* y,
                bool int8) {
    if (M < 0 || N < 0 || K < 0 || M >= kMaxRows) return W8A8_EINVAL;
    if (!act_ok(act)) return W8A8_EINVAL;
    if (int8) {
        if (!qw || !sw) return W8A8_EINVAL;
        if (M > 0) {
            if (!x || !y || !aligned(x, 2) || !aligned(y, 16)) return W8A8_EINVAL;
            if (!aligned(qw, 16) || !aligned(sw, 4) || (bias && !aligned(bias, 2)))
                return W8A8_EINVAL;
        }
        return W8A8_OK;
    }
    if (!w && M > 0 && N > 0 && K > 0) return W8A8_EINVAL;
    if (M > 0 && N > 0) {
        if (!y || !aligned(y, 2)) return W8A8_EINVAL;
        if (K > 0 && (!x || !aligned(x, 2) || !aligned(w, 2))) return W8A8_EINVAL;
        if (bias && !aligned(bias, 2)) return W8A8_EINVAL;
        if (N >= kMaxRows) return W8A8_EINVAL;
    }
    return W8A8_OK;
}
}  // namespace

extern "C" {

int w8a8_linear(const uint16_t* x, int64_t M, int64_t K, int64_t N, const int8_t* qw,
                const float* sw, const uint16_t* w, const uint16_t* bias, int act, uint16_t* y,
                void* workspace, size_t workspace_bytes, int* path_taken, void* stream) {
    const bool int8 = w8a8_guard(N, K) != 0;
    const int st = linear_args(x, M, K, N, qw, sw, w, bias, act, y, int8);
    if (st != W8A8_OK) return st;
    if (int8) {
        if (M > 0 && (!workspace || !aligned(workspace, 256) ||
                      workspace_bytes < w8a8_linear_workspace_bytes(M, K)))
            return W8A8_EINVAL;
        if (path_taken) *path_taken = W8A8_PATH_INT8;
        if (M == 0) return W8A8_OK;
        int8_t* qx = static_cast<int8_t*>(workspace);
        float* sx = reinterpret_cast<float*>(static_cast<char*>(workspace) +
                                             (w8a8_linear_workspace_bytes(M, K) - M * sizeof(float)));
        hipStream_t s = as_stream(stream);
        if (w8a8::launch_quantize_rows(x, M, K, qx, sx, s) != 0) return W8A8_EHIP;
        return launched(w8a8::launch_gemm_i8(qx, sx, M, qw, sw, N, K, bias, act, W8A8_OUT_BF16, y, s));
    }
    if (path_taken) *path_taken = W8A8_PATH_BF16;
    if (M == 0 || N == 0) return W8A8_OK;
    return launched(w8a8::launch_gemm_bf16(x, M, K, w, N, bias, act, y, as_stream(stream)));
}

}  // extern "C"

// ---- the no-allocation variant of w8a8_linear ----
// The INT8 path's workspace in a static device array: each GPU the library
// runs on holds its own copy, at its own address, until the process ends.
// Host code never uses the array's name as an address (on the host it is only
// a stand-in for the symbol); it uses the device address looked up below.
static __device__ __align__(256) unsigned char scratch[W8A8_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::atomic<void*> scratch_address[kMaxDevices];

// Device address of the current device's scratch, looked up on the first call
// on that device (with it current) and kept; NULL on failure.
void* device_scratch() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    void* p = scratch_address[dev].load(std::memory_order_acquire);
    if (p) return p;
    void* q = nullptr;
    if (hipGetSymbolAddress(&q, HIP_SYMBOL(scratch)) != hipSuccess || q == nullptr) return nullptr;
    scratch_address[dev].store(q, std::memory_order_release);
    return q;
}
}  // namespace

extern "C" {

int w8a8_linear_noalloc(const uint16_t* x, int64_t M, int64_t K, int64_t N, const int8_t* qw,
                        const float* sw, const uint16_t* w, const uint16_t* bias, int act,
                        uint16_t* y, int* path_taken, void* stream) {
    const bool int8 = w8a8_guard(N, K) != 0;
    const int st = linear_args(x, M, K, N, qw, sw, w, bias, act, y, int8);
    if (st != W8A8_OK) return st;
    if (!int8 || M == 0)  // BF16 path or nothing to do: no scratch
        return w8a8_linear(x, M, K, N, qw, sw, w, bias, act, y, nullptr, 0, path_taken, stream);
    const size_t need = w8a8_linear_workspace_bytes(M, K);
    if (need > (size_t)W8A8_NOALLOC_SCRATCH_BYTES) return W8A8_ESCRATCH;
    void* ws = device_scratch();
    if (!ws) return W8A8_EHIP;
    return w8a8_linear(x, M, K, N, qw, sw, w, bias, act, y, ws, need, path_taken, stream);
}

int compact_padded_rows(const uint16_t* x, const uint8_t* mask, int64_t B, int64_t L, int64_t D,
                        uint16_t* out, int32_t* src_row, int32_t* count, void* stream) {
    if (B < 0 || L < 0 || D < 0) return W8A8_EINVAL;
    if (L > 0 && B > (kMaxRows - 1) / L) return W8A8_EINVAL;
    if (!count || !aligned(count, 4)) return W8A8_EINVAL;
    const int64_t R = B * L;
    if (R > 0) {
        if (!mask || !src_row || !aligned(src_row, 4)) return W8A8_EINVAL;
        if (D > 0 && (!x || !out || !aligned(x, 2) || !aligned(out, 2))) return W8A8_EINVAL;
    }
    return launched(w8a8::launch_compact_rows(x, mask, R, D, out, src_row, count, as_stream(stream)));
}

int w8a8_compact_quantize_rows(const uint16_t* x, const uint8_t* mask, int64_t B, int64_t L,
                               int64_t D, int8_t* q, float* scale, int32_t* src_row,
                               int32_t* count, void* stream) {
    if (B < 0 || L < 0 || D < 0) return W8A8_EINVAL;
    if (L > 0 && B > (kMaxRows - 1) / L) return W8A8_EINVAL;
    if (!count || !aligned(count, 4)) return W8A8_EINVAL;
    const int64_t R = B * L;
    if (R > 0) {
        if (!mask || !src_row || !aligned(src_row, 4) || !scale || !aligned(scale, 4))
            return W8A8_EINVAL;
        if (D > 0 && (!x || !q || !aligned(x, 2))) return W8A8_EINVAL;
    }
    return launched(w8a8::launch_compact_quantize_rows(x, mask, R, D, q, scale, src_row, count,
                                                       as_stream(stream)));
}

}  // extern "C"
