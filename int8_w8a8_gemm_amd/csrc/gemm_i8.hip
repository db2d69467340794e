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
// Tiled MFMA kernel.  A workgroup of WAVES = 8 waves owns a BM x 256 output
// tile; the waves form a (WAVES/2) x 2 grid, each owning (BM/4) x 128 outputs,
// i.e. MI x 4 tiles of v_mfma_i32_32x32x32_i8 (MI = BM/128) held as int32
// accumulators.  Two waves share each SIMD, so one wave's load issue, LDS waits
// and barrier arrival overlap the other's MFMAs.  K is staged BK bytes at a
// time through an NST-deep ring of LDS buffers.
//
// * Operands go global -> LDS directly (buffer_load_dwordx4 ... lds): a wave
//   instruction moves 1 KB (64 lanes x 16 bytes); lane l lands at LDS offset
//   16*l of that KB and is given the global chunk that belongs there under the
//   swizzle below.  Lane offsets are fixed per tile and the stage's K position
//   is a scalar offset, so the loads of a stage need no address arithmetic.
// * An LDS row r (BK bytes = BK/16 chunks) stores logical K-chunk c at physical
//   chunk c ^ f(r).  A fragment read has lane l on row l % 32 at logical chunk
//   l / 32; with f(r) = (r ^ (r >> 3)) & 7 for 128-byte rows and (r >> 2) & 3
//   for 64-byte rows these reads are free of LDS bank conflicts on gfx950
//   (measured with the SQ_LDS_BANK_CONFLICT counter; LDS serves 256 bytes per
//   clock, so a conflict-free ds_read_b128 takes 4 clocks).
// * MFMA roles are transposed (A-operand = weight rows, B-operand = activation
//   rows) so the accumulator holds D[n][m]: each lane ends with 4 consecutive
//   output columns of one row and writes them as one 8-byte store.
// * One barrier per K stage; the MFMAs of the stage's last K sub-step are
//   issued after it, interleaved with the next stage's first fragment reads and
//   the loads that refill the buffer just released.  The order of MFMAs, LDS
//   reads and loads within a sub-step is fixed with sched_barrier.
// * The tile's row scales, column scales and bias are staged into LDS during
//   the prologue, so the epilogue reads them with LDS latency only.
// * Tile order is XCD-aware: workgroup b runs on XCD b % 8, so each XCD is
//   given a contiguous range of tiles, walked in groups of 1024 rows.
// ---------------------------------------------------------------------------
constexpr int L_BN = 256;
constexpr int NUM_XCD = 8;
#ifndef W8A8_GROUP_ROWS
#define W8A8_GROUP_ROWS 1024
#endif
constexpr int GROUP_ROWS = W8A8_GROUP_ROWS;

typedef __attribute__((address_space(3))) void lds_void;

#ifndef W8A8_WAVES
#define W8A8_WAVES 8
#endif
constexpr int WAVES = W8A8_WAVES;          // waves per workgroup: 2 x (WAVES/2) grid
constexpr int WM = WAVES / 2;              // waves along M
constexpr int THREADS = WAVES * 64;

template <int BM, int BK>
struct Geo {
    static constexpr int MI = BM / WM / 32;            // 32-row MFMA tiles per wave along M
    static constexpr int NI = 4;                       // 32-col MFMA tiles per wave along N
    static constexpr int NQ = MI + NI;                 // fragments per sub-step
    static constexpr int NMFMA = MI * NI;              // MFMAs per sub-step
    static constexpr int CPR = BK / 16;                // 16-byte chunks per LDS row
    static constexpr int RPI = 64 / CPR;               // rows one 1-KB wave instruction fills
    static constexpr int STAGE = (BM + L_BN) * BK;     // bytes per stage (A tile then B tile)
    static constexpr int SUB = BK / 32;                // 32-deep MFMA sub-steps per stage
    static constexpr int LPW_A = BM / WAVES / RPI;     // A load instructions per wave per stage
    static constexpr int LPW_B = L_BN / WAVES / RPI;   // B load instructions per wave per stage
    static constexpr int NLOAD = LPW_A + LPW_B;
    static constexpr int WAVES_PER_SIMD = MI * 4 > 8 ? WAVES / 4 : 2;
};

template <int BK>
__device__ __forceinline__ int swz(int r, int c) {
    if (BK == 128) return c ^ ((r ^ (r >> 3)) & 7);
    return c ^ ((r >> 2) & 3);
}

// Workgroup barrier for the wave's own LDS reads and writes (ds_*) only.
// __syncthreads() also waits for every global load and store in flight, and
// any LDS fence waits for the direct-to-LDS loads; this one leaves both in
// flight (the next tile's prefetch, the output stores), so it must not be
// used where those loads' data is about to be read.  The empty asm statements
// keep the compiler from moving memory accesses across it.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0); vmcnt, expcnt left free
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// s_waitcnt immediate for gfx9: vmcnt(v) lgkmcnt(0), expcnt left free.
template <int V>
__device__ __forceinline__ void wait_vm_lgkm0() {
    static_assert(V >= 0 && V < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((V & 15) | ((V >> 4) << 14) | (7 << 4));
}

// The buffer-resource type exists only when compiling for the GPU; the host
// pass sees a placeholder of the same size (kernels never run on the host).
#if defined(__HIP_DEVICE_COMPILE__)
typedef __amdgpu_buffer_rsrc_t rsrc_t;
#else
struct rsrc_t { int w[4]; };
#endif

#if defined(__HIP_DEVICE_COMPILE__)
constexpr int kRawBufferWord3 = 0x00020000;  // untyped 32-bit buffer access
#endif

// Per-tile addressing.  Each operand is read through a buffer resource based
// at the tile's first row and sized to the rows that exist, so rows past M
// (or N) read as zero.  Every lane keeps fixed byte offsets for its loads; the
// K position of a stage goes in the scalar offset, so issuing a stage's loads
// writes no vector registers.
template <int BM, int BK>
struct Ctx {
    rsrc_t rsrc[2];  // 0: activation panel, 1: weight panel
    uint32_t voff_a[Geo<BM, BK>::LPW_A];
    uint32_t voff_b[Geo<BM, BK>::LPW_B];
    int wave, lane, wm, wn;
};

// Points the context's buffer resources at the operand panels of the tile
// whose first output row is m0 and first output column n0.
template <int BM, int BK>
__device__ __forceinline__ void set_tile(Ctx<BM, BK>& c, const int8_t* qa, const int8_t* qw,
                                         int64_t M, int64_t N, int64_t K, int64_t m0, int64_t n0) {
#if defined(__HIP_DEVICE_COMPILE__)
    const int64_t rows_a = (M - m0) < BM ? (M - m0) : BM;
    const int64_t rows_w = (N - n0) < L_BN ? (N - n0) : L_BN;
    c.rsrc[0] = __builtin_amdgcn_make_buffer_rsrc((void*)(qa + m0 * K), (short)0,
                                                  (int)(rows_a * K), kRawBufferWord3);
    c.rsrc[1] = __builtin_amdgcn_make_buffer_rsrc((void*)(qw + n0 * K), (short)0,
                                                  (int)(rows_w * K), kRawBufferWord3);
#endif
}

// Lane offsets are tile-local, so they are set once per workgroup.
template <int BM, int BK>
__device__ __forceinline__ void make_ctx(Ctx<BM, BK>& c, int64_t K, int wave, int lane) {
    typedef Geo<BM, BK> G;
    const int rsub = lane / G::CPR, pc = lane % G::CPR;
#pragma unroll
    for (int i = 0; i < G::LPW_A; ++i) {
        const int r = wave * (BM / WAVES) + i * G::RPI + rsub;  // tile-local A row
        c.voff_a[i] = (uint32_t)r * (uint32_t)K + 16u * (uint32_t)swz<BK>(r, pc);
    }
#pragma unroll
    for (int i = 0; i < G::LPW_B; ++i) {
        const int r = wave * (L_BN / WAVES) + i * G::RPI + rsub;  // tile-local B row
        c.voff_b[i] = (uint32_t)r * (uint32_t)K + 16u * (uint32_t)swz<BK>(r, pc);
    }
    c.wave = wave;
    c.lane = lane;
    c.wm = wave % WM;
    c.wn = wave / WM;
}

// Load j (0 .. NLOAD-1) of one wave's share of a K stage: j < LPW_A loads A
// rows, the rest B rows.  Lane l lands at LDS byte 16*l of the load's 1 KB.
template <int BM, int BK>
__device__ __forceinline__ void stage_load_one(const Ctx<BM, BK>& c, int k0, char* lds_stage,
                                               int j) {
    typedef Geo<BM, BK> G;
    const bool is_a = j < G::LPW_A;
    const int i = is_a ? j : j - G::LPW_A;
    char* dst = is_a ? lds_stage + (c.wave * (BM / WAVES) + i * G::RPI) * BK
                     : lds_stage + BM * BK + (c.wave * (L_BN / WAVES) + i * G::RPI) * BK;
#if defined(__HIP_DEVICE_COMPILE__)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(c.rsrc[is_a ? 0 : 1], (lds_void*)dst, 16,
                                             is_a ? c.voff_a[i] : c.voff_b[i], k0, 0, 0);
#else
    (void)dst;
#endif
}

template <int BM, int BK>
__device__ __forceinline__ void stage_load(const Ctx<BM, BK>& c, int k0, char* lds_stage) {
#pragma unroll
    for (int j = 0; j < Geo<BM, BK>::NLOAD; ++j) stage_load_one<BM, BK>(c, k0, lds_stage, j);
}

template <int MI>
struct Frags {
    v4i a[MI];  // activation rows (MFMA B-operand), m sub-tiles
    v4i w[4];   // weight rows (MFMA A-operand), n sub-tiles
};

// Fragment q of sub-step ks: q < MI -> activation sub-tile q, else weight
// sub-tile q - MI.  Lane l reads row l % 32 of the sub-tile at K-chunk 2*ks + l/32.
template <int BM, int BK>
__device__ __forceinline__ void read_frag(const char* lds_stage, const Ctx<BM, BK>& c, int ks,
                                          int q, Frags<BM / WM / 32>& f) {
    constexpr int MI = BM / WM / 32;
    const int ch = 2 * ks + (c.lane >> 5);
    if (q < MI) {
        const int ra = c.wm * (BM / WM) + q * 32 + (c.lane & 31);
        f.a[q] = *reinterpret_cast<const v4i*>(lds_stage + ra * BK + 16 * swz<BK>(ra, ch));
    } else {
        const int rw = c.wn * 128 + (q - MI) * 32 + (c.lane & 31);
        f.w[q - MI] =
            *reinterpret_cast<const v4i*>(lds_stage + BM * BK + rw * BK + 16 * swz<BK>(rw, ch));
    }
}

template <int MI>
__device__ __forceinline__ void mfma_one(v16i (&acc)[4][MI], const Frags<MI>& f, int j) {
    const int ni = j / MI, mi = j % MI;
    acc[ni][mi] = __builtin_amdgcn_mfma_i32_32x32x32_i8(f.w[ni], f.a[mi], acc[ni][mi], 0, 0, 0);
}

// One K stage, held in ring buffer kt % NST.
// LOAD: stage kt+NST exists and is loaded into this buffer after the barrier.
// NEXT: stage kt+1 exists.  STEADY: exactly NST-2 newer stages are in flight.
// Each sub-step issues its MFMAs in a fixed order with the next fragment reads
// (one after each of the first NQ MFMAs) and the refill loads (spread evenly)
// placed between them; sched_barrier pins that order.
template <int BM, int BK, int NST, bool LOAD, bool NEXT, bool STEADY>
__device__ __forceinline__ void k_stage(const Ctx<BM, BK>& c, char* smem, int kt,
                                        v16i (&acc)[4][BM / WM / 32], Frags<BM / WM / 32>& cur) {
    typedef Geo<BM, BK> G;
    char* buf = smem + (kt % NST) * G::STAGE;
    Frags<G::MI> nxt;
#pragma unroll
    for (int ks = 0; ks + 1 < G::SUB; ++ks) {
#pragma unroll
        for (int j = 0; j < G::NMFMA; ++j) {
            mfma_one<G::MI>(acc, cur, j);
            if (j < G::NQ) read_frag<BM, BK>(buf, c, ks + 1, j, nxt);
            __builtin_amdgcn_sched_barrier(0);
        }
        cur = nxt;
    }
    char* next_buf = smem + ((kt + 1) % NST) * G::STAGE;
    if (NEXT) {
        // my loads of stage kt+1 have landed and my reads of stage kt are done ...
        if (STEADY) wait_vm_lgkm0<G::NLOAD * (NST - 2)>();
        else wait_vm_lgkm0<0>();
        __syncthreads();  // ... and everyone's: stage kt+1 visible, buffer kt % NST free
        __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int j = 0; j < G::NMFMA; ++j) {
        mfma_one<G::MI>(acc, cur, j);
        if (NEXT && j < G::NQ) read_frag<BM, BK>(next_buf, c, 0, j, nxt);
        if (LOAD) {
            // loads (j * NLOAD / NMFMA) .. ((j+1) * NLOAD / NMFMA) - 1 go after MFMA j
#pragma unroll
            for (int l = (j * G::NLOAD) / G::NMFMA; l < ((j + 1) * G::NLOAD) / G::NMFMA; ++l)
                stage_load_one<BM, BK>(c, (kt + NST) * BK, buf, l);
        }
        __builtin_amdgcn_sched_barrier(0);
    }
    if (NEXT) cur = nxt;
}

// Workgroup id -> (tile row, tile col), XCD-aware.
template <int BM>
__device__ __forceinline__ void tile_of(int64_t bid, int64_t tm, int64_t tn, int64_t& tile_m,
                                        int64_t& tile_n) {
    constexpr int GROUP_M = GROUP_ROWS / BM;
    const int64_t total = tm * tn;
    int64_t t = bid;
    if (total % NUM_XCD == 0) {
        // XCD x (= bid % 8) takes tiles [x * total/8, (x+1) * total/8) in dispatch order
        t = (bid % NUM_XCD) * (total / NUM_XCD) + bid / NUM_XCD;
    }
    // grouped raster: walk GROUP_M tile-rows at a time, column by column
    const int64_t per_group = GROUP_M * tn;
    const int64_t g = t / per_group;
    const int64_t first_m = g * GROUP_M;
    const int64_t gm = (tm - first_m) < GROUP_M ? (tm - first_m) : GROUP_M;
    const int64_t r = t % per_group;
    tile_m = first_m + r % gm;
    tile_n = r / gm;
}

// Epilogue.  acc[ni][mi][i] holds D[n][m] for m = m0 + wm*(BM/WM) + mi*32 +
// (lane & 31) and n = n0 + wn*128 + ni*32 + 8*(i/4) + 4*(lane >> 5) + (i & 3):
// four consecutive columns per group of four registers.
//
// Stored straight from the accumulator layout, one wave instruction would
// touch 32 rows with 16 bytes each.  Instead the bf16 tile goes through LDS,
// in MI passes of BM/MI rows (pass p holds the rows of MFMA sub-tile mi = p),
// and is copied out so that each wave instruction writes two whole 512-byte
// tile rows.  Staged rows are padded to 528 bytes: every LDS address is a
// per-lane base plus a compile-time offset, and the 16-byte row reads are free
// of bank conflicts.  `stage` must not overlap the K buffer that the next
// tile's first stage is being loaded into.
constexpr int OUT_ROW = L_BN * 2 + 16;  // bytes per staged output row

template <int BM>
struct Epi {
    static constexpr int MI = BM / WM / 32;
    static constexpr int SROWS = BM / MI;        // staged rows per pass (= WM * 32)
    static constexpr int RPW = SROWS / WAVES;    // staged rows each wave copies out per pass
    static constexpr int BYTES = SROWS * OUT_ROW;
    static_assert(32 % RPW == 0 && RPW % 2 == 0, "copy-out rows per wave");
};

template <int BM, int ACT, bool HAS_BIAS>
__device__ __forceinline__ void store_bf16(const v16i (&acc)[4][BM / WM / 32], uint16_t* __restrict__ y,
                                           int64_t M, int64_t N, int64_t m0, int64_t n0, int wave,
                                           int wm, int wn, int lane, const float* sa_l,
                                           const float* sw_l, const float* b_l, char* stage) {
    typedef Epi<BM> E;
    const int half = lane >> 5;
    const int ncol = wn * 128 + 4 * half;  // tile-local column of this lane's first group
    char* wbase = stage + (wm * 32 + (lane & 31)) * OUT_ROW + ncol * 2;
    const bool interior = (m0 + BM <= M) && (n0 + L_BN <= N);
    const int c8 = lane & 31;
    // copy-out: staged row s = wave*RPW + 2i + half is tile row (s/32)*(BM/WM) + p*32 + s%32
    const int s0 = wave * E::RPW + half;
    const char* rbase = stage + s0 * OUT_ROW + c8 * 16;
    const int trow0 = (s0 / 32) * (BM / WM) + (s0 % 32);
#pragma unroll
    for (int p = 0; p < E::MI; ++p) {
        const float sam = sa_l[wm * (BM / WM) + p * 32 + (lane & 31)];
#pragma unroll
        for (int ni = 0; ni < 4; ++ni) {
            v4f swv[4], bv[4];
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int cl = ncol + ni * 32 + 8 * g;
                swv[g] = *reinterpret_cast<const v4f*>(sw_l + cl);
                if (HAS_BIAS) bv[g] = *reinterpret_cast<const v4f*>(b_l + cl);
            }
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                float v[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float t = (float)acc[ni][p][4 * g + e];  // nearest even
                    const float u = __fmul_rn(sam, swv[g][e]);
                    v[e] = HAS_BIAS ? __builtin_fmaf(t, u, bv[g][e]) : __fmul_rn(t, u);
                }
                uint2 o = make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
                if (ACT == 1) {
                    // GELU-tanh of the bf16-rounded value, rounded to bf16 (gelu_bf16_rn)
                    o = make_uint2(gelu_bf16_rn(o.x & 0xffffu) | (gelu_bf16_rn(o.x >> 16) << 16),
                                   gelu_bf16_rn(o.y & 0xffffu) | (gelu_bf16_rn(o.y >> 16) << 16));
                }
                *reinterpret_cast<uint2*>(wbase + (ni * 32 + 8 * g) * 2) = o;
            }
        }
        lds_barrier();
        v4i d[E::RPW / 2];
#pragma unroll
        for (int i = 0; i < E::RPW / 2; ++i)
            d[i] = *reinterpret_cast<const v4i*>(rbase + 2 * i * OUT_ROW);
        const int64_t row = m0 + trow0 + p * 32;
        uint16_t* gbase = y + row * N + n0 + 8 * c8;
        if (interior) {
#pragma unroll
            for (int i = 0; i < E::RPW / 2; ++i) *reinterpret_cast<v4i*>(gbase + 2 * i * N) = d[i];
        } else {
#pragma unroll
            for (int i = 0; i < E::RPW / 2; ++i)
                if (row + 2 * i < M && n0 + 8 * c8 < N)
                    *reinterpret_cast<v4i*>(gbase + 2 * i * N) = d[i];
        }
        lds_barrier();  // the staging area is free again
    }
}

template <int BM>
__device__ __forceinline__ void store_i32(const v16i (&acc)[4][BM / WM / 32], int32_t* __restrict__ out,
                                          int64_t M, int64_t N, int64_t m0, int64_t n0, int wm,
                                          int wn, int lane) {
    constexpr int MI = BM / WM / 32;
    const int ncol = wn * 128 + 4 * (lane >> 5);
#pragma unroll
    for (int mi = 0; mi < MI; ++mi) {
        const int ml = wm * (BM / WM) + mi * 32 + (lane & 31);
        if (m0 + ml >= M) continue;
        int32_t* rowp = out + (m0 + ml) * N + n0 + ncol;
#pragma unroll
        for (int ni = 0; ni < 4; ++ni)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                if (n0 + ncol + ni * 32 + 8 * g >= N) continue;
                v4i v = {acc[ni][mi][4 * g], acc[ni][mi][4 * g + 1], acc[ni][mi][4 * g + 2],
                         acc[ni][mi][4 * g + 3]};
                *reinterpret_cast<v4i*>(rowp + ni * 32 + 8 * g) = v;
            }
    }
}

// Persistent kernel (PERSIST): the grid holds one workgroup per CU (or one per
// tile if there are fewer tiles), and workgroup b walks tiles b, b + grid, ...
// While a tile's epilogue runs, the next tile's first K stage is already
// loading into ring buffer 0 and its scales into registers; the output is
// staged in the LDS above buffer 0.  Without PERSIST each workgroup does one
// tile (the GELU epilogue's binary64 slow path needs the registers that the
// tile loop's live state would take).
template <int BM, int BK, int NST, int OUT_I32, int ACT, bool PERSIST>
__global__ __launch_bounds__(THREADS)
__attribute__((amdgpu_waves_per_eu(Geo<BM, BK>::WAVES_PER_SIMD, Geo<BM, BK>::WAVES_PER_SIMD)))
void gemm_i8_tiled(const int8_t* __restrict__ qa, const float* __restrict__ sa, int64_t M,
                   const int8_t* __restrict__ qw, const float* __restrict__ sw, int64_t N, int64_t K,
                   const uint16_t* __restrict__ bias, void* __restrict__ out) {
    typedef Geo<BM, BK> G;
    constexpr int MI = G::MI;
    // K ring (from byte STAGE on, also the output staging area), then the
    // tile's row scales, column scales and bias (as binary32).  All of it is
    // one LDS object: with several, the compiler can no longer tell the
    // fragment reads from the in-flight direct-to-LDS loads and waits for
    // every load.
    constexpr int RING = NST * G::STAGE > G::STAGE + Epi<BM>::BYTES ? NST * G::STAGE
                                                                    : G::STAGE + Epi<BM>::BYTES;
    __shared__ __attribute__((aligned(1024))) char smem[RING + (BM + 2 * L_BN) * 4];
    float* sa_l = reinterpret_cast<float*>(smem + RING);
    float* sw_l = sa_l + BM;
    float* b_l = sw_l + L_BN;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave % WM, wn = wave / WM;
    const int64_t tm = (M + BM - 1) / BM, tn = (N + L_BN - 1) / L_BN, total = tm * tn;
    const int KT = (int)(K / BK);
    int64_t t = blockIdx.x, tile_m, tile_n;
    tile_of<BM>(t, tm, tn, tile_m, tile_n);
    int64_t m0 = tile_m * BM, n0 = tile_n * L_BN;
    Ctx<BM, BK> c;
    make_ctx<BM, BK>(c, K, wave, lane);
    set_tile<BM, BK>(c, qa, qw, M, N, K, m0, n0);

    // first tile: epilogue operands, then fill the ring and wait for stage 0
    // (the bias stays in bf16 bits until it is written: converting it at once
    // would make the wave wait for the load)
    float nsa = 0.f, nsw = 0.f;
    uint32_t nb = 0;
    if (!OUT_I32 && tid < L_BN) {
        const int64_t n = n0 + tid < N ? n0 + tid : N - 1;
        if (tid < BM) nsa = sa[m0 + tid < M ? m0 + tid : M - 1];
        nsw = sw[n];
        if (bias) nb = bias[n];
    }
    for (int s = 0; s < NST; ++s)
        if (s < KT) stage_load<BM, BK>(c, s * BK, smem + s * G::STAGE);
    if (!OUT_I32 && tid < L_BN) {
        if (tid < BM) sa_l[tid] = nsa;
        sw_l[tid] = nsw;
        b_l[tid] = bf16_bits_to_float(nb);
    }
    if (KT >= NST) wait_vm_lgkm0<G::NLOAD * (NST - 1)>();
    else wait_vm_lgkm0<0>();
    __syncthreads();

    for (;;) {
        v16i acc[4][MI];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < MI; ++j) acc[i][j] = (v16i){};
        Frags<MI> cur;
#pragma unroll
        for (int q = 0; q < G::NQ; ++q) read_frag<BM, BK>(smem, c, 0, q, cur);

        int kt = 0;
        for (; kt + NST < KT; ++kt) k_stage<BM, BK, NST, true, true, true>(c, smem, kt, acc, cur);
        if (kt == KT - NST && kt + 1 < KT) {
            k_stage<BM, BK, NST, false, true, true>(c, smem, kt, acc, cur);
            ++kt;
        }
        for (; kt + 1 < KT; ++kt) k_stage<BM, BK, NST, false, true, false>(c, smem, kt, acc, cur);
        k_stage<BM, BK, NST, false, false, false>(c, smem, kt, acc, cur);

        const int64_t t_next = t + gridDim.x;
        const bool has_next = PERSIST && t_next < total;
        int64_t m0n = 0, n0n = 0;
        lds_barrier();  // every wave is done reading the K ring
        if (has_next) {
            tile_of<BM>(t_next, tm, tn, tile_m, tile_n);
            m0n = tile_m * BM;
            n0n = tile_n * L_BN;
            if (!OUT_I32 && tid < L_BN) {
                const int64_t n = n0n + tid < N ? n0n + tid : N - 1;
                if (tid < BM) nsa = sa[m0n + tid < M ? m0n + tid : M - 1];
                nsw = sw[n];
                if (bias) nb = bias[n];
            }
            set_tile<BM, BK>(c, qa, qw, M, N, K, m0n, n0n);
            stage_load<BM, BK>(c, 0, smem);  // next tile's stage 0 -> buffer 0
        }
        // The epilogue's lane addresses depend only on the lane, and hoisted out
        // of the tile loop they would stay live across the K loop; an opaque
        // copy of the lane index keeps them local to the epilogue.
        int elane = lane;
        asm volatile("" : "+v"(elane));
        if (OUT_I32) {
            store_i32<BM>(acc, reinterpret_cast<int32_t*>(out), M, N, m0, n0, wm, wn, elane);
        } else if (bias) {
            store_bf16<BM, ACT, true>(acc, reinterpret_cast<uint16_t*>(out), M, N, m0, n0, wave,
                                      wm, wn, elane, sa_l, sw_l, b_l, smem + G::STAGE);
        } else {
            store_bf16<BM, ACT, false>(acc, reinterpret_cast<uint16_t*>(out), M, N, m0, n0, wave,
                                       wm, wn, elane, sa_l, sw_l, b_l, smem + G::STAGE);
        }
        if (!has_next) break;
        if (!OUT_I32 && tid < L_BN) {  // this tile's epilogue is done with the old values
            if (tid < BM) sa_l[tid] = nsa;
            sw_l[tid] = nsw;
            b_l[tid] = bf16_bits_to_float(nb);
        }
        wait_vm_lgkm0<0>();  // the next tile's stage 0 (and this tile's stores) are done ...
        __syncthreads();     // ... for every wave, and the staging area is free
        for (int s = 1; s < NST; ++s)
            if (s < KT) stage_load<BM, BK>(c, s * BK, smem + s * G::STAGE);
        t = t_next;
        m0 = m0n;
        n0 = n0n;
    }
}

// 256 x 256 tiles (the least data movement per MFMA, which is what sets the
// clock under the power cap), 8 waves (two per SIMD, so one wave's load issue
// and LDS waits overlap the other's MFMAs), 128-byte K stages, 2-deep ring.
#ifndef W8A8_BM
#define W8A8_BM 256
#endif
#ifndef W8A8_BK
#define W8A8_BK 128
#endif
#ifndef W8A8_NST
#define W8A8_NST 2
#endif

template <int OUT_I32, int ACT>
hipError_t launch_large(const int8_t* qa, const float* sa, int64_t M, const int8_t* qw,
                        const float* sw, int64_t N, int64_t K, const uint16_t* bias, void* out,
                        hipStream_t stream) {
    const int64_t tiles = ((N + L_BN - 1) / L_BN) * ((M + W8A8_BM - 1) / W8A8_BM);
    constexpr bool persist = ACT == 0;
    int64_t grid = tiles;
    if (persist) {
        const int cus = cu_count();
        if (cus <= 0) return hipErrorInvalidDevice;
        grid = tiles < cus ? tiles : cus;
    }
    hipLaunchKernelGGL((gemm_i8_tiled<W8A8_BM, W8A8_BK, W8A8_NST, OUT_I32, ACT, persist>),
                       dim3((unsigned)grid), dim3(THREADS), 0, stream, qa, sa, M, qw, sw, N, K, bias,
                       out);
    return hipGetLastError();
}

}  // namespace

int launch_gemm_i8(const int8_t* qa, const float* sa, int64_t M, const int8_t* qw,
                   const float* sw, int64_t N, int64_t K, const uint16_t* bias, int act,
                   int out_kind, void* out, hipStream_t stream) {
    if (M == 0 || N == 0) return 0;
    hipError_t e;
    if (out_kind == 1) e = launch_large<1, 0>(qa, sa, M, qw, sw, N, K, bias, out, stream);
    else if (act == 1) e = launch_large<0, 1>(qa, sa, M, qw, sw, N, K, bias, out, stream);
    else e = launch_large<0, 0>(qa, sa, M, qw, sw, N, K, bias, out, stream);
    return e == hipSuccess ? 0 : -1;
}

}  // namespace w8a8
