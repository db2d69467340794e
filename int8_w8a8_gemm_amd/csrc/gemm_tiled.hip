// Tiled MFMA GEMM for gfx950: the INT8 W8A8 product and the native BF16
// fallback of the guarded layer share one kernel.
//
// TurboT2VA (智猩猩 article, section 01.3 "量化策略"): the W8A8 product is
// accumulated in INT32 and the scales and bias are applied once, after the
// whole accumulation, never per K block; branches the INT8 operator cannot
// serve run in native BF16.  Here, for INT8 operands
//     acc[i][j] = sum_k qa[i][k] * qw[j][k]              (exact int32)
//     y[i][j]   = bf16_RNE(fma(float(acc), RN32(sa[i]*sw[j]), bias[j]))
// (or the raw acc in int32 mode), and for BF16 operands
//     acc[i][j] = sum_k x[i][k] * w[j][k]                (fp32 accumulation)
//     y[i][j]   = bf16_RNE(acc + bias[j])
// each with an optional GELU-tanh on the bf16 y.  Without a bias the same
// code adds -0.0, which leaves every value, and the sign of every zero, as
// the product alone has it (x + -0 = x in round-to-nearest), so there is one
// epilogue, not one per bias/no-bias case competing for registers.
//
// Both operands are K-contiguous ([M x K] and [N x K]), the layout the MFMA
// A/B operands want: every lane feeds 16 consecutive K bytes of one row.
// v_mfma_i32_32x32x32_i8 (32 int8 of K per row) and v_mfma_f32_32x32x16_bf16
// (16 bf16) take their operands in the same byte layout and issue in the same
// 32 cycles, so the whole data path is shared and counts K in bytes.
#include "common.h"

#include <type_traits>
#include <utility>

namespace w8a8 {

namespace {

// ---------------------------------------------------------------------------
// A workgroup of WM x WN waves owns a BM x BN output tile; wave (wm, wn) owns
// (BM/WM) x (BN/WN) outputs, i.e. MI x NI MFMA tiles of MT x MT accumulators.
// K is staged BK bytes at a time through an NST-deep ring of LDS buffers.
// Two MFMA shapes, both 1024 multiply-adds per SIMD per clock:
// v_mfma_i32_32x32x32_i8 / v_mfma_f32_32x32x16_bf16 (MT = 32: 32 bytes of K
// per instruction, 16 accumulator registers per lane) and
// v_mfma_i32_16x16x64_i8 / v_mfma_f32_16x16x32_bf16 (MT = 16: 64 bytes of K,
// 4 registers).  The INT8 GEMM's rate is set by the package power limit, so
// energy per operation is what counts: a loop of MFMAs alone on quantised
// N(0,1)-like codes ran the 16 x 16 shape at 4.08 POPS (0.64 pJ per
// multiply-add) against 3.50 POPS (0.74 pJ) for 32 x 32, on the same GPU.  A
// 16 x 16 sub-step covers 64 bytes of K, so a wave holds twice as many live
// fragments; the tiers whose registers allow it take that shape.
// Four configurations:
//   large: 256 x 256 tile, 4 x 2 waves (two per SIMD, so one wave's load issue,
//          LDS waits and barrier arrival overlap the other's MFMAs), each wave
//          64 x 128; 16 x 16 MFMAs (INT8 and BF16).  The 32 x 32 version of
//          the same tile ran FFN up 24576 x 16384 x 4096 in 1332 us against
//          1243 us, and a 384 x 256 tile of 96 x 128 per wave (17% fewer
//          operand bytes per MFMA, 32 x 32 MFMAs: with 16 x 16 its accumulators
//          and fragments outgrow the 256 registers of a wave at two per SIMD)
//          ran 1280 us, 8192^3 7.7% and 4096^3 8.5% slower than this tile.
//   mid:   192 x 256 tile, 2 x 4 waves of 96 x 64, 16 x 16 MFMAs (INT8 and
//          BF16): three quarters of a large tile's work, for row counts where
//          large tiles leave many CUs idle in their last round (the ~2300-row
//          text projection: 160 large tiles or 208 mid ones on 256 CUs; 16 x 16
//          MFMAs took it from 41.1 to 39.6 us, and the BF16 fallback on the
//          same rows, 2378 x 4096 x 4096, from 76.5 to 70.6 us).
//   small: 128 x 128 tile, 2 x 2 waves of 64 x 64, K split between two groups
//          of waves (a 3-deep K ring for long K loops); 32 x 32 MFMAs (16 x 16
//          ran 2048^3 and 512 x 4096 x 4096 12-15% slower).
//   tiny:  64 x 64 tile, 2 x 2 waves of 32 x 32.
// The launcher takes the largest of large/small/tiny whose tile count covers
// at least half of the CUs (a large tile on a CU still outruns four small
// ones; measured on the 2378-row text projection, the 2048^3 audio GEMM and
// 1024 x 1024 x 4096), then mid instead of large where its rounds of tiles per
// CU cost less (see launch_tiles).
//
// * Operands go global -> LDS directly (buffer_load_dwordx4 ... lds): a wave
//   instruction moves 1 KB (64 lanes x 16 bytes); lane l lands at LDS offset
//   16*l of that KB and is given the global chunk that belongs there under the
//   swizzle below.  A lane's offsets are fixed per tile and the stage's K
//   position is a scalar offset; each load's lane offset is formed from two
//   per-lane values and wave-uniform terms as it is issued (stage_load_one).
// * An LDS row r (BK bytes = BK/16 chunks) stores logical K-chunk c at physical
//   chunk c ^ f(r) (swz below).  A fragment read has lane l on row l % MT at
//   logical chunk l / MT of the sub-step; f(r) = (r ^ (r >> 3)) & 7 (32 x 32
//   MFMAs) or (r ^ (r >> 2)) & 7 (16 x 16) for 128-byte rows, (r >> 1) & 3 for
//   64-byte rows, makes those reads free of bank conflicts (SQ_LDS_BANK_CONFLICT
//   counts only the epilogue's).
// * MFMA roles are transposed (A-operand = weight rows, B-operand = activation
//   rows) so the accumulator holds D[n][m]: each lane ends with 4 consecutive
//   output columns of one row.
// * One barrier per K stage; the MFMAs of the stage's last K sub-step are
//   issued after it, interleaved with the next stage's first fragment reads and
//   the loads that refill the buffer just released.  The order of MFMAs, LDS
//   reads and loads within a sub-step is fixed with sched_barrier.
// * Tile order is XCD-aware: workgroup b runs on XCD b % 8, so each XCD is
//   given a contiguous range of tiles, walked in groups of GROUP_M tile-rows
//   (1024 rows: the 32 large tiles an XCD runs at once form a 4 x 8 block).
// * Epilogue once per tile, after the whole K loop: the scale product, fma
//   with the bias and bf16 packing per output, then 16-byte stores: through a
//   staging area per wave on the INT8 256 x 256 tier (store_perwave), straight
//   from registers after a lane exchange on the INT8 192 x 256 tier
//   (store_direct), through an LDS staging area of whole tile rows otherwise
//   (store_bf16).
// ---------------------------------------------------------------------------
constexpr int NUM_XCD = 8;
// The W8A8_* macros below are the tuned defaults; each can be overridden on
// the compiler command line to measure an alternative.
// rows of output per raster group of the tile order (see tile_of)
#ifndef W8A8_GROUP_ROWS
#define W8A8_GROUP_ROWS 1024
#endif
// 1: weight sub-tiles innermost in a sub-step's MFMA order where a wave has
// more of them than activation sub-tiles (Cfg::N_INNER); 0: always activation
#ifndef W8A8_ORDER_N_INNER
#define W8A8_ORDER_N_INNER 1
#endif
constexpr int GROUP_ROWS = W8A8_GROUP_ROWS;
// Cache policy of the operand loads: sc0 (bit 0).  Each stage's data is used
// once per CU, so nothing is gained by keeping it in the CU's L1; measured
// against no policy bits: FFN up 1.355 -> 1.324 ms, down 1.282 -> 1.267 ms,
// 24576 x 4096 x 4096 1.2% faster; sc1 gained about half as much, and nt
// (which lets L2 evict the operand panels other tiles still read) lost 5-7%.
#ifndef W8A8_LOAD_POLICY
#define W8A8_LOAD_POLICY 1
#endif
// Output tiles leave with non-temporal stores (written once, read by the next
// kernel): 0.5-1% faster on the FFN and attention shapes, 3.6% on 2048^3.
#ifndef W8A8_STORE_NT
#define W8A8_STORE_NT 1
#endif

typedef __attribute__((address_space(3))) void lds_void;

// Operand element types.  Mfma<MT>::run takes 16 bytes of weight row (A
// operand) and activation row (B operand) per lane and accumulates an MT x MT
// tile over 32 bytes of K (MT = 32) or 64 bytes (MT = 16).
struct ElemI8 {
    static constexpr int BYTES = 1;
    template <int MT> struct Mfma;
};
template <> struct ElemI8::Mfma<32> {
    typedef v16i acc_t;
    static __device__ __forceinline__ acc_t run(v4i w, v4i a, acc_t c) {
        return __builtin_amdgcn_mfma_i32_32x32x32_i8(w, a, c, 0, 0, 0);
    }
};
template <> struct ElemI8::Mfma<16> {
    typedef v4i acc_t;
    static __device__ __forceinline__ acc_t run(v4i w, v4i a, acc_t c) {
        return __builtin_amdgcn_mfma_i32_16x16x64_i8(w, a, c, 0, 0, 0);
    }
};

struct ElemBF16 {
    static constexpr int BYTES = 2;
    template <int MT> struct Mfma;
};
template <> struct ElemBF16::Mfma<32> {
    typedef v16f acc_t;
    static __device__ __forceinline__ acc_t run(v4i w, v4i a, acc_t c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(v8bf, w),
                                                       __builtin_bit_cast(v8bf, a), c, 0, 0, 0);
    }
};
template <> struct ElemBF16::Mfma<16> {
    typedef v4f acc_t;
    static __device__ __forceinline__ acc_t run(v4i w, v4i a, acc_t c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, w),
                                                       __builtin_bit_cast(v8bf, a), c, 0, 0, 0);
    }
};

template <int BM_, int BN_, int WM_, int WN_, int BK_, int NST_, int GROUP_ROWS_ = GROUP_ROWS,
          int KS_ = 1, bool SPLIT_ = false, int MT_ = 32, bool NIN_ = true, bool EPW_ = false>
struct Cfg {
    static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_, BK = BK_, NST = NST_;
    static constexpr int GROUP_M = GROUP_ROWS_ / BM;  // tile-rows per group of the raster
    // KS > 1 splits K inside the workgroup: KS groups of WM x WN waves each own
    // the whole tile, group g taking sub-steps g, g + KS, ... of every stage
    // (the stage's loads are shared by all waves); after the K loop the groups'
    // accumulators are added exactly through LDS, and group 0 holds the sums.
    static constexpr int KS = KS_;
    // SPLIT: split-K across workgroups; a work item is a (tile, K slice) pair
    // and its INT32 partial sums go to a slice of the workspace (see splitk_reduce)
    static constexpr bool SPLIT = SPLIT_;
    static constexpr int WG = WM * WN;                // waves per K group
    static constexpr int WAVES = WG * KS;
    static constexpr int THREADS = WAVES * 64;
    static constexpr int TM = BM / WM, TN = BN / WN;  // outputs per wave
    // MFMA tile: MT x MT outputs over KSUB bytes of K, ACC_N accumulator
    // registers per lane (32 x 32 x 32 bytes or 16 x 16 x 64 bytes)
    static constexpr int MT = MT_;
    static constexpr int KSUB = MT == 16 ? 64 : 32;
    static constexpr int ACC_N = MT * MT / 64;
    static constexpr int MI = TM / MT;                 // MFMA tiles per wave along M
    static constexpr int NI = TN / MT;                 // MFMA tiles per wave along N
    static constexpr int NQ = MI + NI;                 // fragments per sub-step
    static constexpr int NMFMA = MI * NI;              // MFMAs per sub-step
    // Fragment registers: with room to spare the next sub-step's fragments go
    // to fresh registers early in the sub-step; where the accumulators leave
    // no room (RECYCLE) each is read into the register of the fragment it
    // replaces, right after that fragment's last MFMA.
    static constexpr bool RECYCLE = NMFMA * ACC_N + 2 * NQ * 4 > 200;
    // MFMA order within a sub-step: with NIN the weight sub-tiles innermost where
    // they are the more numerous, so that a recycled activation fragment is read
    // while NI MFMAs still run, not MI (INT8 256 x 256: 0.9-1.5% faster on the FFN
    // and attention shapes; the BF16 variant then spills and ran 3% slower)
    static constexpr bool N_INNER = NIN_ && W8A8_ORDER_N_INNER && NI > MI;
    static constexpr int CPR = BK / 16;                // 16-byte chunks per LDS row
    static constexpr int RPI = 64 / CPR;               // rows one 1-KB wave instruction fills
    static constexpr int STAGE = (BM + BN) * BK;       // bytes per stage (A tile then B tile)
    static constexpr int SUB = BK / KSUB;              // MFMA sub-steps per stage
    static constexpr int SUBW = SUB / KS;              // ... of them for each wave
    static constexpr int LPW_A = BM / WAVES / RPI;     // A load instructions per wave per stage
    static constexpr int LPW_B = BN / WAVES / RPI;     // B load instructions per wave per stage
    static constexpr int NLOAD = LPW_A + LPW_B;
    static constexpr int WAVES_PER_SIMD = (WAVES + 3) / 4;
    // epilogue staging (see store_bf16)
    static constexpr int OUT_ROW = BN * 2 + 16;        // bytes per staged output row
    static constexpr int PM = 32 / MT;                 // MFMA row tiles per staging pass
    static constexpr int NPASS = MI / PM;              // staging passes
    static constexpr int SROWS = WM * 32;              // staged rows per pass
    static constexpr int RCH = BN / 8;                 // 16-byte chunks per output row
    static constexpr int RPINS = 64 / RCH;             // output rows per copy-out instruction
    static constexpr int RPW = SROWS / WAVES;          // staged rows each wave copies per pass
    static constexpr int EPI_BYTES = SROWS * OUT_ROW;
    // LDS: K ring (from byte STAGE on also the staging area), then the tile's
    // row scales, column scales and bias as binary32.  Where the ring fills the
    // 160 KB of LDS, the scales go in the ring above the staging area instead:
    // they are then written only once the K loop is done with the ring.
    // bytes the groups g > 0 pass their accumulators through (KS > 1)
    static constexpr int RED_WAVE = NI * MI * ACC_N * 64 * 4;
    static constexpr int RED_BYTES = (KS - 1) * WG * RED_WAVE;
    // EPW: the epilogue stages each wave's outputs in a 2 KB area of its own
    // past the ring (store_perwave), so the ring holds no staging area
    static constexpr bool EPW = EPW_;
    static constexpr int PW_BYTES = 16 * 128;  // 16 rows x 64 bf16 columns
    static constexpr int RING0 = EPW                              ? NST * STAGE
                                 : NST * STAGE > STAGE + EPI_BYTES ? NST * STAGE
                                                                   : STAGE + EPI_BYTES;
    static constexpr int RING = RING0 > RED_BYTES ? RING0 : RED_BYTES;
    static constexpr int PW_OFF = RING;
    static constexpr int RING_PW = EPW ? RING + WAVES * PW_BYTES : RING;
    static constexpr int SCALE_BYTES = (BM + 2 * BN) * 4;
    static constexpr bool SCALES_IN_RING = RING_PW + SCALE_BYTES > 160 * 1024;
    static constexpr int SCALE_OFF = SCALES_IN_RING ? STAGE + EPI_BYTES : RING_PW;
    // Epilogue straight from registers (store_direct): 16 x 16 MFMA tiles in
    // pairs, no K groups, and not the register-tight tiles (on the 256 x 256
    // tile it measured level on FFN up and 0.7-1.1% slower on FFN down, whose
    // 64-byte non-temporal row pieces drain slower than full 128-byte rows;
    // the INT8 192 x 256 tile gained 0.8-2.3% on the ~2300-row text projection,
    // in three runs).  With no
    // barrier at its end, the next tile's scales go to the other of two scale
    // buffers while slower waves still read these.
    static constexpr bool DIRECT_OK = MT == 16 && NI % 2 == 0 && KS == 1 && !RECYCLE && !EPW &&
                                      !SCALES_IN_RING && RING + 2 * SCALE_BYTES <= 160 * 1024;
    static constexpr int SCALE_BUFS = DIRECT_OK || EPW ? 2 : 1;
    static constexpr int SMEM = SCALES_IN_RING ? RING : RING_PW + SCALE_BUFS * SCALE_BYTES;
    static_assert(!EPW || (MT == 16 && NI % 4 == 0 && KS == 1 && !SCALES_IN_RING),
                  "per-wave epilogue: 16 x 16 tiles in groups of four, no K groups");
    static_assert(SMEM <= 160 * 1024 && SCALE_OFF + SCALE_BYTES <= SMEM, "LDS budget");
    static_assert(BM % (WAVES * RPI) == 0 && BN % (WAVES * RPI) == 0, "load split");
    static_assert(TM % 32 == 0 && TN % 32 == 0, "wave tile");
    static_assert((MT == 16 || MT == 32) && BK % KSUB == 0, "MFMA tile");
    static_assert(RPW % RPINS == 0 && 32 % RPW == 0, "copy-out rows per wave");
    static constexpr int SA_PT = (BM + THREADS - 1) / THREADS;  // row scales per thread
    static constexpr int SW_PT = (BN + THREADS - 1) / THREADS;  // column scales per thread
    static_assert(GROUP_M >= 1, "raster group");
    static_assert(KS >= 1 && SUB % KS == 0, "sub-steps per K group");
    static_assert(KS == 1 || !SCALES_IN_RING, "the K-group reduction uses the ring");
};

// Tile configurations: BM, BN, WM, WN, BK, NST, raster group rows, K groups,
// split-K; the MFMA tile edge (32 or 16) is set per tier and element type below.
#ifndef W8A8_LARGE_CFG
#define W8A8_LARGE_CFG 256, 256, 4, 2, 128, 2, GROUP_ROWS, 1, false
#endif
#ifndef W8A8_MID_CFG
#define W8A8_MID_CFG 192, 256, 2, 4, 128, 2, GROUP_ROWS, 1, false
#endif
// The small tiers split K between two groups of waves (two waves per SIMD, so
// each hides the other's fragment-read latency): INT8 2048^3 and 512 x 4096 x
// 4096 20.4 -> 18.0 us; BF16 2048^3 22.1 -> 20.7 us, 512 x 4096 x 4096
// 36.4 -> 30.2 us (the BF16 fp32 sums then add two partial chains).
#ifndef W8A8_SMALL_CFG
#define W8A8_SMALL_CFG 128, 128, 2, 2, 128, 2, GROUP_ROWS, 2, false
#endif
// small tiles with a 3-deep ring, for K loops of 32 stages or more (see launch_tiles)
#ifndef W8A8_SMALL_DEEP_CFG
#define W8A8_SMALL_DEEP_CFG 128, 128, 2, 2, 128, 3, GROUP_ROWS, 2, false
#endif
#ifndef W8A8_TINY_CFG
#define W8A8_TINY_CFG 64, 64, 2, 2, 128, 2, GROUP_ROWS, 1, false
#endif
// MFMA tile edge of each tier, INT8 and BF16.
#ifndef W8A8_I8_LARGE_MT
#define W8A8_I8_LARGE_MT 16
#endif
#ifndef W8A8_I8_MID_MT
#define W8A8_I8_MID_MT 16
#endif
#ifndef W8A8_I8_SMALL_MT
#define W8A8_I8_SMALL_MT 32
#endif
#ifndef W8A8_I8_TINY_MT
#define W8A8_I8_TINY_MT 32
#endif
// the INT8 256 x 256 tier stages its epilogue per wave (store_perwave)
#ifndef W8A8_I8_LARGE_EPW
#define W8A8_I8_LARGE_EPW 1
#endif
#ifndef W8A8_BF16_LARGE_MT
#define W8A8_BF16_LARGE_MT 16
#endif
#ifndef W8A8_BF16_MID_MT
#define W8A8_BF16_MID_MT 16
#endif
#ifndef W8A8_BF16_SMALL_MT
#define W8A8_BF16_SMALL_MT 32
#endif
#ifndef W8A8_BF16_TINY_MT
#define W8A8_BF16_TINY_MT 32
#endif
template <class E> struct Tiers {  // BF16
    typedef Cfg<W8A8_LARGE_CFG, W8A8_BF16_LARGE_MT, false> Large;
    typedef Cfg<W8A8_MID_CFG, W8A8_BF16_MID_MT> Mid;
    typedef Cfg<W8A8_SMALL_CFG, W8A8_BF16_SMALL_MT> Small;
    typedef Cfg<W8A8_SMALL_DEEP_CFG, W8A8_BF16_SMALL_MT> Deep;
    typedef Cfg<W8A8_TINY_CFG, W8A8_BF16_TINY_MT> Tiny;
};
template <> struct Tiers<ElemI8> {
    typedef Cfg<W8A8_LARGE_CFG, W8A8_I8_LARGE_MT, true, W8A8_I8_LARGE_EPW> Large;
    typedef Cfg<W8A8_MID_CFG, W8A8_I8_MID_MT> Mid;
    typedef Cfg<W8A8_SMALL_CFG, W8A8_I8_SMALL_MT> Small;
    typedef Cfg<W8A8_SMALL_DEEP_CFG, W8A8_I8_SMALL_MT> Deep;
    typedef Cfg<W8A8_TINY_CFG, W8A8_I8_TINY_MT> Tiny;
};

// Physical chunk of logical chunk c in LDS row r.  A ds_read_b128 takes four
// LDS cycles of 16 lanes when free of bank conflicts; a 32 x 32 MFMA fragment
// read has 32 lanes on 32 consecutive rows at one chunk, a 16 x 16 one 16
// consecutive rows at four chunks.  Each swizzle here was measured free of
// conflicts with SQ_LDS_BANK_CONFLICT, on the fragment reads of the kernel and
// on the same lane pattern alone: the 32 x 32 swizzle on 16 x 16 reads and
// c ^ ((r >> 2) & 3) on 64-byte rows conflicted two ways, 64-byte rows with no
// swizzle two ways and 128-byte rows with none four.  All are XOR-separable
// over blocks of 8 rows (the loads) and of MT rows (the fragment sub-tiles).
template <int BK, int MT>
__device__ __forceinline__ int swz(int r, int c) {
    if (BK == 128) return MT == 16 ? c ^ ((r ^ (r >> 2)) & 7) : c ^ ((r ^ (r >> 3)) & 7);
    return c ^ ((r >> 1) & 3);
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

// Element i of a bias vector of `count` elements that may be absent (NULL).
// A buffer load over an empty range returns 0, so there is no branch on the
// pointer: the load defines its register with no phi to resolve, and stays in
// flight until its value is used.
__device__ __forceinline__ uint32_t load_bias_bits(const uint16_t* bias, int count, int i) {
#if defined(__HIP_DEVICE_COMPILE__)
    const rsrc_t r = __builtin_amdgcn_make_buffer_rsrc((void*)bias, (short)0, bias ? 2 * count : 0,
                                                      kRawBufferWord3);
    return (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(r, 2 * i, 0, 0);
#else
    return 0u;
#endif
}

// Per-tile addressing.  Each operand is read through a buffer resource based
// at the tile's first row and sized to the rows that exist, so rows past M
// (or N) read as zero (the range check sees the lane offset, so the row part
// of the address stays in it); the K position of a stage goes in the scalar
// offset.  KB is the row length in bytes.
template <class C>
struct Ctx {
    rsrc_t rsrc[2];  // 0: activation panel, 1: weight panel
    // loads: lrow = (lane / CPR) * KB; lx = 16 x this lane's chunk before the
    // wave-uniform part of the swizzle (see stage_load_one)
    uint32_t lrow, lx, kb;
    int kofs;  // first K byte of the work item's slice (split-K), else 0
    // fragment reads: LDS byte offset of this lane's row in the wave's first
    // activation / weight sub-tile, and 16 x the physical chunk of its K-chunk
    // (lane / MT) in that row; every other read adds compile-time constants
    uint32_t fa, fw, ga, gw;
    int wave, lane, wm, wn, kg;  // kg: the wave's K group
};

// Points the context's buffer resources at the operand panels of the tile
// whose first output row is m0 and first output column n0.
template <class C>
__device__ __forceinline__ void set_tile(Ctx<C>& c, const char* a, const char* w, int64_t M,
                                         int64_t N, int64_t KB, int64_t m0, int64_t n0) {
#if defined(__HIP_DEVICE_COMPILE__)
    const int64_t rows_a = (M - m0) < C::BM ? (M - m0) : C::BM;
    const int64_t rows_w = (N - n0) < C::BN ? (N - n0) : C::BN;
    c.rsrc[0] = __builtin_amdgcn_make_buffer_rsrc((void*)(a + m0 * KB), (short)0,
                                                  (int)(rows_a * KB), kRawBufferWord3);
    c.rsrc[1] = __builtin_amdgcn_make_buffer_rsrc((void*)(w + n0 * KB), (short)0,
                                                  (int)(rows_w * KB), kRawBufferWord3);
#endif
}

// The per-lane values of the context: tile-local, so the same for every
// tile.  The persistent loop recomputes them (a few VALU operations) from an
// opaque copy of the lane index at the end of each tile rather than keeping
// them live through the epilogue, where the accumulators fill the registers.
template <class C>
__device__ __forceinline__ void lane_ctx(Ctx<C>& c, int lane) {
    const int rsub = (int)((unsigned)lane / C::CPR), pc = (int)((unsigned)lane % C::CPR);
    c.lrow = (uint32_t)rsub * c.kb;
    // 128-byte rows: swz(r0 + rsub, pc) = pc ^ rsub ^ ((r0 >> 3) & 7) for r0 % 8 == 0
    // (MT = 32), pc ^ rsub ^ (rsub >> 2) ^ ((r0 >> 2) & 7) (MT = 16);
    // 64-byte rows: swz(r0 + rsub, pc) = pc ^ ((rsub >> 1) & 3) for r0 % 8 == 0
    c.lx = C::BK != 128 ? 16u * (uint32_t)(pc ^ ((rsub >> 1) & 3))
           : C::MT == 16  ? 16u * (uint32_t)(pc ^ rsub ^ (rsub >> 2))
                          : 16u * (uint32_t)(pc ^ rsub);
    // lane l reads row l % MT of a sub-tile at K-chunk l / MT of the sub-step
    const int hi = (int)((unsigned)lane / C::MT);
    const int lr = (int)((unsigned)lane % C::MT);
    const int ra = c.wm * C::TM + lr, rw = c.wn * C::TN + lr;
    c.fa = (uint32_t)(ra * C::BK);
    c.fw = (uint32_t)(C::BM * C::BK + rw * C::BK);
    // a K group's sub-steps are kg, kg + KS, ...: KSUB * kg shares no bit with
    // KSUB * KS * (the wave's own sub-step) or with 16 * hi, so it joins the
    // per-lane XOR term
    c.ga = (16u * (uint32_t)swz<C::BK, C::MT>(ra, hi)) ^ ((uint32_t)C::KSUB * (uint32_t)c.kg);
    c.gw = (16u * (uint32_t)swz<C::BK, C::MT>(rw, hi)) ^ ((uint32_t)C::KSUB * (uint32_t)c.kg);
}

template <class C>
__device__ __forceinline__ void make_ctx(Ctx<C>& c, int64_t KB, int wave, int lane) {
    c.kb = (uint32_t)KB;
    c.kofs = 0;
    c.wave = wave;
    c.lane = lane;
    c.kg = C::KS > 1 ? wave / C::WG : 0;
    c.wm = (wave % C::WG) % C::WM;
    c.wn = (wave % C::WG) / C::WM;
    lane_ctx<C>(c, lane);
}

// Load j (0 .. NLOAD-1) of one wave's share of a K stage: j < LPW_A loads A
// rows, the rest B rows.  The load covers tile rows r0 .. r0 + RPI - 1 (r0
// wave-uniform, a multiple of RPI); lane l takes row r0 + l / CPR, logical
// chunk l % CPR, which lands at LDS byte 16*l of the load's 1 KB, the physical
// chunk of the swizzle.  Its lane offset is row * KB + 16 * swz(row, chunk) =
// lrow + r0 * KB + (lx ^ 16 * ((r0 >> 3) & 7)) for 128-byte rows (r0 >> 2 for
// the MT = 16 swizzle; the XOR term
// is 0 for 64-byte rows): two VALU operations per load instead of a register
// per load held across the K loop.  lrow and lx are passed by the caller
// through an empty asm statement so that the compiler forms each offset here.
template <class C>
__device__ __forceinline__ void stage_load_one(const Ctx<C>& c, uint32_t lrow, uint32_t lx, int k0,
                                               char* lds_stage, int j) {
    static_assert(C::BK == 128 || C::BK == 64, "swizzle");
    const bool is_a = j < C::LPW_A;
    const int i = is_a ? j : j - C::LPW_A;
    const uint32_t r0 = (uint32_t)(c.wave * ((is_a ? C::BM : C::BN) / C::WAVES) + i * C::RPI);
    const uint32_t xr = C::BK != 128 ? 0u : 16u * ((r0 >> (C::MT == 16 ? 2 : 3)) & 7u);
    const uint32_t voff = lrow + r0 * c.kb + (lx ^ xr);
    char* dst = lds_stage + (is_a ? 0 : C::BM * C::BK) + r0 * C::BK;
#if defined(__HIP_DEVICE_COMPILE__)
    const int kpos = C::SPLIT ? k0 + c.kofs : k0;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(c.rsrc[is_a ? 0 : 1], (lds_void*)dst, 16, voff, kpos,
                                             0, W8A8_LOAD_POLICY);
#else
    (void)dst;
    (void)voff;
#endif
}

template <class C>
__device__ __forceinline__ void stage_load(const Ctx<C>& c, int k0, char* lds_stage) {
    uint32_t lrow = c.lrow, lx = c.lx;
    asm volatile("" : "+v"(lrow), "+v"(lx));
#pragma unroll
    for (int j = 0; j < C::NLOAD; ++j) stage_load_one<C>(c, lrow, lx, k0, lds_stage, j);
}

template <class C>
struct Frags {
    v4i a[C::MI];  // activation rows (MFMA B-operand), m sub-tiles
    v4i w[C::NI];  // weight rows (MFMA A-operand), n sub-tiles
};

template <class C, class E>
using AccT = typename E::template Mfma<C::MT>::acc_t;
template <class C, class E>
using Acc = AccT<C, E>[C::NI][C::MI];

// Fragment q of sub-step ks: q < MI -> activation sub-tile q, else weight
// sub-tile q - MI.  Lane l reads row l % MT of the sub-tile at K-chunk
// ch = (KSUB/16)*ks + l/MT, stored at physical chunk ch ^ f(row).  Sub-tile i
// starts MT*i rows further on, where f changes by 4*(i & 1) for 128-byte rows
// (both swizzles) and not at all for 64-byte rows; so 16 * (ch ^ f(row)) =
// g ^ (KSUB*ks) ^ (64*(i & 1)) (128-byte rows) with g = 16 * ((l/MT) ^
// f(first row)) from the context: one XOR-add per read.  ga, gw are that g for
// the two operands.
// The four per-lane fragment-read values of the context.
struct FragBase {
    uint32_t fa, fw, ga, gw;
};

template <class C>
__device__ __forceinline__ FragBase frag_base(const Ctx<C>& c) {
    FragBase b{c.fa, c.fw, c.ga, c.gw};
    return b;
}

template <class C>
__device__ __forceinline__ void read_frag(const char* lds_stage, const FragBase& fb, int ks, int q,
                                          Frags<C>& f) {
    const bool is_a = q < C::MI;
    const int i = is_a ? q : q - C::MI;
    const uint32_t k = (uint32_t)(C::KSUB * ks) ^ (C::BK == 128 ? 64u * (uint32_t)(i & 1) : 0u);
    const uint32_t off = ((is_a ? fb.ga : fb.gw) ^ k) + (is_a ? fb.fa : fb.fw);
    const v4i v = *reinterpret_cast<const v4i*>(lds_stage + off + i * C::MT * C::BK);
    if (is_a) f.a[i] = v;
    else f.w[i] = v;
}

// Keeps the first `valid` bytes of a 16-byte fragment (0 <= valid, even), zero
// beyond: the K tail of the last stage, whose loads ran on into the next row.
__device__ __forceinline__ v4i keep_bytes(v4i v, int valid) {
#pragma unroll
    for (int d = 0; d < 4; ++d) {
        const int keep = valid - 4 * d;
        v[d] = keep >= 4 ? v[d] : keep >= 2 ? (v[d] & 0xffff) : 0;
    }
    return v;
}

// Masks the fragments of sub-step ks of the last stage to the row's `tail`
// valid bytes of that stage.
template <class C>
__device__ __forceinline__ void mask_tail(Frags<C>& f, const Ctx<C>& c, int ks, int tail) {
    const int valid = tail - (C::KSUB * (ks + c.kg) + 16 * (int)((unsigned)c.lane / C::MT));
#pragma unroll
    for (int q = 0; q < C::MI; ++q) f.a[q] = keep_bytes(f.a[q], valid);
#pragma unroll
    for (int q = 0; q < C::NI; ++q) f.w[q] = keep_bytes(f.w[q], valid);
}

template <class C, class E>
__device__ __forceinline__ void mfma_one(Acc<C, E>& acc, const Frags<C>& f, int j) {
    const int ni = C::N_INNER ? j % C::NI : j / C::MI, mi = C::N_INNER ? j / C::NI : j % C::MI;
    acc[ni][mi] = E::template Mfma<C::MT>::run(f.w[ni], f.a[mi], acc[ni][mi]);
}

// The MFMAs of one sub-step, with (READ) the fragment reads of sub-step rks
// of buffer rbuf and (LOAD) this wave's loads of stage kload into lbuf placed
// between them (spread evenly); sched_barrier pins that order.  Without
// RECYCLE the next fragments go to fresh registers, one read after each of the
// first NQ MFMAs (any left over after the last); with it each fragment is read
// into the register it replaces once its last MFMA has issued.  The fragment
// bases (and the load offsets' lane values) are passed through an empty asm
// statement so that their per-read combinations are formed next to each read,
// not hoisted out of the K loop into registers of their own.
template <class C, class E, bool READ, bool LOAD>
__device__ __forceinline__ void mfma_step(const Ctx<C>& c, Acc<C, E>& acc, Frags<C>& cur,
                                          const char* rbuf, int rks, char* lbuf, int kload) {
    FragBase fb = frag_base(c);
    uint32_t lrow = c.lrow, lx = c.lx;
    asm volatile("" : "+v"(fb.fa), "+v"(fb.fw), "+v"(fb.ga), "+v"(fb.gw));
    if (LOAD) asm volatile("" : "+v"(lrow), "+v"(lx));
    auto loads_after = [&](int j) {
        if (LOAD) {
            // loads (j * NLOAD / NMFMA) .. ((j+1) * NLOAD / NMFMA) - 1 go after MFMA j
#pragma unroll
            for (int l = (j * C::NLOAD) / C::NMFMA; l < ((j + 1) * C::NLOAD) / C::NMFMA; ++l)
                stage_load_one<C>(c, lrow, lx, kload, lbuf, l);
        }
    };
    if constexpr (C::RECYCLE && C::N_INNER) {
#pragma unroll
        for (int j = 0; j < C::NMFMA; ++j) {
            mfma_one<C, E>(acc, cur, j);  // MFMA j uses a[j / NI] and w[j % NI]
            if (READ && j % C::NI == C::NI - 1) read_frag<C>(rbuf, fb, rks, j / C::NI, cur);
            if (READ && j >= (C::MI - 1) * C::NI)
                read_frag<C>(rbuf, fb, rks, C::MI + j - (C::MI - 1) * C::NI, cur);
            loads_after(j);
            __builtin_amdgcn_sched_barrier(0);
        }
    } else if constexpr (C::RECYCLE) {
#pragma unroll
        for (int j = 0; j < C::NMFMA; ++j) {
            mfma_one<C, E>(acc, cur, j);  // MFMA j uses w[j / MI] and a[j % MI]
            if (READ && j % C::MI == C::MI - 1)
                read_frag<C>(rbuf, fb, rks, C::MI + j / C::MI, cur);
            if (READ && j >= (C::NI - 1) * C::MI)
                read_frag<C>(rbuf, fb, rks, j - (C::NI - 1) * C::MI, cur);
            loads_after(j);
            __builtin_amdgcn_sched_barrier(0);
        }
    } else {
        Frags<C> nxt;
#pragma unroll
        for (int j = 0; j < C::NMFMA; ++j) {
            mfma_one<C, E>(acc, cur, j);
            if (READ && j < C::NQ) read_frag<C>(rbuf, fb, rks, j, nxt);
            loads_after(j);
            __builtin_amdgcn_sched_barrier(0);
        }
        if (READ) {
#pragma unroll
            for (int j = C::NMFMA; j < C::NQ; ++j) read_frag<C>(rbuf, fb, rks, j, nxt);
            cur = nxt;
        }
    }
}

// One K stage, held in ring buffer kt % NST.
// LOAD: stage kt+NST exists and is loaded into this buffer after the barrier.
// NEXT: stage kt+1 exists.  STEADY: exactly NST-2 newer stages are in flight.
template <class C, class E, bool LOAD, bool NEXT, bool STEADY>
__device__ __forceinline__ void k_stage(const Ctx<C>& c, char* smem, int kt, Acc<C, E>& acc,
                                        Frags<C>& cur, int tail = C::BK) {
    // tail: valid bytes of each row in this stage, < BK only in a BF16 last
    // stage (the INT8 path has whole stages)
    constexpr bool MAYBE_TAIL = !NEXT && E::BYTES == 2;
    char* buf = smem + (kt % C::NST) * C::STAGE;
    // the wave's sub-steps of the stage: KS * j (+ its group's kg, folded into
    // the fragment offsets), j = 0 .. SUBW - 1
#pragma unroll
    for (int j = 0; j + 1 < C::SUBW; ++j) {
        if (MAYBE_TAIL && tail < C::BK) mask_tail<C>(cur, c, C::KS * j, tail);
        mfma_step<C, E, true, false>(c, acc, cur, buf, C::KS * (j + 1), nullptr, 0);
    }
    char* next_buf = smem + ((kt + 1) % C::NST) * C::STAGE;
    if (MAYBE_TAIL && tail < C::BK) mask_tail<C>(cur, c, C::KS * (C::SUBW - 1), tail);
    if (NEXT) {
        // my loads of stage kt+1 have landed and my reads of stage kt are done ...
        if (STEADY) wait_vm_lgkm0<C::NLOAD * (C::NST - 2)>();
        else wait_vm_lgkm0<0>();
        __syncthreads();  // ... and everyone's: stage kt+1 visible, buffer kt % NST free
        __builtin_amdgcn_sched_barrier(0);
    }
    mfma_step<C, E, NEXT, LOAD>(c, acc, cur, next_buf, 0, buf, (kt + C::NST) * C::BK);
}

// Workgroup id -> (tile row, tile col), XCD-aware.  Tile indices fit in 32
// bits (the launcher checks), and 32-bit division is a short sequence where
// the 64-bit one is a long scalar routine on every tile of a persistent loop.
template <class C>
__device__ __forceinline__ void tile_of(int64_t bid, int64_t tm, int64_t tn, int64_t& tile_m,
                                        int64_t& tile_n) {
    constexpr uint32_t GROUP_M = C::GROUP_M;
    const uint32_t tm32 = (uint32_t)tm, tn32 = (uint32_t)tn, total = tm32 * tn32;
    uint32_t t = (uint32_t)bid;
    if (total % NUM_XCD == 0) {
        // XCD x (= bid % 8) takes tiles [x * total/8, (x+1) * total/8) in dispatch order
        t = (t % NUM_XCD) * (total / NUM_XCD) + t / NUM_XCD;
    }
    // grouped raster: walk GROUP_M tile-rows at a time, column by column
    const uint32_t per_group = GROUP_M * tn32;
    const uint32_t g = t / per_group;
    const uint32_t first_m = g * GROUP_M;
    const uint32_t gm = (tm32 - first_m) < GROUP_M ? (tm32 - first_m) : GROUP_M;
    const uint32_t r = t - g * per_group;
    const uint32_t rn = r / gm;
    tile_m = (int64_t)(first_m + (r - rn * gm));
    tile_n = (int64_t)rn;
}

// Calls f(integral_constant<int, P>) for P = 0, 1, ... in order.
template <class F, int... P>
__device__ __forceinline__ void for_each_pass(F& f, std::integer_sequence<int, P...>) {
    (f(std::integral_constant<int, P>{}), ...);
}

// Epilogue.  acc[ni][mi][i] holds D[n][m] for m = m0 + wm*TM + mi*MT +
// (lane % MT) and n = n0 + wn*TN + ni*MT + (MT/4)*(i/4) + 4*(lane / MT) +
// (i & 3): four consecutive columns per group of four registers (four groups
// for MT = 32, one for MT = 16).
//
// Stored straight from the accumulator layout, one wave instruction would
// touch 32 rows with 16 bytes each.  Instead the bf16 tile goes through LDS,
// in NPASS passes of WM*32 rows (pass p holds the rows of MFMA sub-tiles
// mi = p*PM .. p*PM + PM - 1, the wave's rows 32p .. 32p + 31),
// and is copied out so that each wave instruction writes whole tile rows
// (64 lanes x 16 bytes).  Staged rows are padded by 16 bytes: every LDS address
// is a per-lane base plus a compile-time offset, and the 16-byte row reads are
// free of bank conflicts.  `stage` must not overlap the K buffer that the next
// tile's first stage is being loaded into.  VEC_OUT: y rows are 16-byte
// aligned and N % 8 == 0, so every 16-byte chunk is stored whole; otherwise
// chunks are stored in 8-, 4- or 2-byte parts, as N and y's alignment allow.
// b_l holds the bias, -0.0 where there is none.
template <class C, class E, int ACT, bool VEC_OUT>
__device__ __forceinline__ void store_bf16(const Acc<C, E>& acc, uint16_t* __restrict__ y, int64_t M,
                                           int64_t N, int64_t m0, int64_t n0, int wave, int wm,
                                           int wn, int lane, const float* sa_l, const float* sw_l,
                                           const float* b_l, char* stage, int kg) {
    constexpr int G = C::ACC_N / 4;  // groups of 4 consecutive columns per MFMA tile
    constexpr int GS = C::MT / 4;    // column step between them
    // the column tiles this wave finalises: all, or with two K groups the
    // group's half, whose sums reduce_k_groups left in acc[0 .. NI/2)
    constexpr int NIS = C::KS == 2 ? C::NI / 2 : C::NI;
    const int cofs = C::KS == 2 ? kg * NIS * C::MT : 0;
    const int lr = (int)((unsigned)lane % C::MT);
    const int ncol = wn * C::TN + 4 * (int)((unsigned)lane / C::MT);  // this lane's first column
    char* wbase = stage + (wm * 32 + lr) * C::OUT_ROW + ncol * 2;
    const bool interior = (m0 + C::BM <= M) && (n0 + C::BN <= N);
    const int cc = (int)((unsigned)lane % C::RCH);  // this lane's 16-byte chunk of a row
    // copy-out: staged row s = wave*RPW + i*RPINS + lane/RCH is tile row
    // (s/32)*TM + p*32 + s%32 (RPW divides 32, so s/32 is fixed per wave)
    const int s0 = wave * C::RPW + (int)((unsigned)lane / C::RCH);
    const char* rbase = stage + s0 * C::OUT_ROW + cc * 16;
    const int trow0 = (s0 / 32) * C::TM + (s0 % 32);
    // one staging pass per MFMA row sub-tile, p a compile-time constant (a
    // runtime pass loop left the accumulators dynamically indexed, in scratch,
    // where the GELU body made the loop too large to unroll)
    auto pass = [&](auto pc) {
        constexpr int p = decltype(pc)::value;
        // row scales of the pass's PM sub-tile rows
        float sam[C::PM];
#pragma unroll
        for (int q = 0; q < C::PM; ++q)
            sam[q] = E::BYTES == 1 ? sa_l[wm * C::TM + (p * C::PM + q) * C::MT + lr] : 0.f;
        // column groups outermost: a group's column scales and bias are read
        // once for all PM rows, and the next group's are read while this one
        // is computed (read and used back to back, each group waited out the
        // LDS latency: 16 times per pass on the 256 x 256 tile)
        // (register-tight tiles: no prefetch, the reads go just before their use)
        constexpr bool PREF = !C::RECYCLE;
        v4f swv[2][G], bv[2][G];
        auto read_cols = [&](int ni, int buf) {
#pragma unroll
            for (int g = 0; g < G; ++g) {
                const int cl = ncol + cofs + ni * C::MT + GS * g;
                if constexpr (E::BYTES == 1) swv[buf][g] = *reinterpret_cast<const v4f*>(sw_l + cl);
                bv[buf][g] = *reinterpret_cast<const v4f*>(b_l + cl);
            }
        };
        // with more than two K groups only group 0 holds the sums; every wave
        // copies out
        if (C::KS <= 2 || kg == 0) {
            if (PREF) read_cols(0, 0);
#pragma unroll
            for (int ni = 0; ni < NIS; ++ni) {
                const int cb = PREF ? ni & 1 : 0;
                if (!PREF) read_cols(ni, 0);
                else if (ni + 1 < NIS) read_cols(ni + 1, cb ^ 1);
#pragma unroll
                for (int q = 0; q < C::PM; ++q) {
                    const int mi = p * C::PM + q;
#pragma unroll
                    for (int g = 0; g < G; ++g) {
                        float v[4];
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            if constexpr (E::BYTES == 1) {
                                const float t = (float)acc[ni][mi][4 * g + e];  // nearest even
                                const float u = __fmul_rn(sam[q], swv[cb][g][e]);
                                v[e] = __builtin_fmaf(t, u, bv[cb][g][e]);
                            } else {
                                const float t = acc[ni][mi][4 * g + e];
                                v[e] = __fadd_rn(t, bv[cb][g][e]);
                            }
                        }
                        uint2 o = make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
                        if (ACT == 1) {
                            // GELU-tanh of the bf16-rounded value, rounded to bf16 (gelu_bf16_rn)
                            o = make_uint2(gelu_bf16_rn(o.x & 0xffffu) | (gelu_bf16_rn(o.x >> 16) << 16),
                                           gelu_bf16_rn(o.y & 0xffffu) | (gelu_bf16_rn(o.y >> 16) << 16));
                        }
                        *reinterpret_cast<uint2*>(wbase + q * C::MT * C::OUT_ROW +
                                                  (cofs + ni * C::MT + GS * g) * 2) = o;
                    }
                }
                // register-tight tiles: keep the reads of later column groups
                // from being hoisted next to these (they would spill)
                if constexpr (C::RECYCLE) __builtin_amdgcn_sched_barrier(0);
            }
        }
        lds_barrier();
        constexpr int NI_OUT = C::RPW / C::RPINS;  // copy-out instructions per wave per pass
        v4i d[NI_OUT];
#pragma unroll
        for (int i = 0; i < NI_OUT; ++i)
            d[i] = *reinterpret_cast<const v4i*>(rbase + i * C::RPINS * C::OUT_ROW);
        const int64_t row = m0 + trow0 + p * 32;
        uint16_t* gbase = y + row * N + n0 + 8 * cc;
        if (VEC_OUT && interior) {
#pragma unroll
            for (int i = 0; i < NI_OUT; ++i) {
#if W8A8_STORE_NT
                __builtin_nontemporal_store(d[i], reinterpret_cast<v4i*>(gbase + i * C::RPINS * N));
#else
                *reinterpret_cast<v4i*>(gbase + i * C::RPINS * N) = d[i];
#endif
            }
        } else if (VEC_OUT) {
#pragma unroll
            for (int i = 0; i < NI_OUT; ++i)
                if (row + i * C::RPINS < M && n0 + 8 * cc < N)
                    *reinterpret_cast<v4i*>(gbase + i * C::RPINS * N) = d[i];
        } else {
            // rows not 16-byte aligned: the widest stores that N and y allow.
            // n0 and 8 * cc are multiples of 8, so with N % 4 == 0 (N % 2 == 0)
            // each 4-column (2-column) part of a chunk lies wholly inside or
            // wholly past column N, and its address is 8- (4-) byte aligned.
            const uintptr_t ya = reinterpret_cast<uintptr_t>(y);
            const bool w8 = N % 4 == 0 && ya % 8 == 0, w4 = N % 2 == 0 && ya % 4 == 0;
            const int64_t c0 = n0 + 8 * cc;
#pragma unroll
            for (int i = 0; i < NI_OUT; ++i) {
                if (row + i * C::RPINS >= M) continue;
                uint16_t* pr = gbase + i * C::RPINS * N;
                if (w8) {
#pragma unroll
                    for (int h = 0; h < 2; ++h)
                        if (c0 + 4 * h < N)
                            *reinterpret_cast<uint2*>(pr + 4 * h) =
                                make_uint2((uint32_t)d[i][2 * h], (uint32_t)d[i][2 * h + 1]);
                } else if (w4) {
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        if (c0 + 2 * j < N) *reinterpret_cast<uint32_t*>(pr + 2 * j) = (uint32_t)d[i][j];
                } else {
#pragma unroll
                    for (int e = 0; e < 8; ++e)
                        if (c0 + e < N)
                            pr[e] = (uint16_t)(((uint32_t)d[i][e >> 1] >> (16 * (e & 1))) & 0xffffu);
                }
            }
        }
        lds_barrier();  // the staging area is free again
    };
    for_each_pass(pass, std::make_integer_sequence<int, C::NPASS>{});
}

// Epilogue without LDS staging, for 16 x 16 MFMA tiles and 16-byte aligned
// output rows.  After the scale and bias arithmetic a lane holds, for each
// pair of adjacent MFMA tiles (ni, ni + 1) of one row tile mi, 4 columns of
// row lane % 16 in each: columns 4 * (lane / 16) .. + 3.  One
// v_permlane16_swap exchanges lanes 16-31 of the first tile's values with
// lanes 0-15 of the second's (and 48-63 with 32-47), after which lane l holds
// 8 consecutive columns (16 bytes) of row l % 16: tile ni + ((l / 16) & 1),
// columns 8 * (l / 32) .. + 7.  A store instruction then writes 64 contiguous
// bytes of each of 16 rows; there is no staging area, so no barrier.
template <class C, class E, int ACT>
__device__ __forceinline__ void store_direct(const Acc<C, E>& acc, uint16_t* __restrict__ y, int64_t M,
                                             int64_t N, int64_t m0, int64_t n0, int wm, int wn,
                                             int lane, const float* sa_l, const float* sw_l,
                                             const float* b_l) {
    static_assert(C::DIRECT_OK, "direct epilogue: 16 x 16 tiles in pairs");
    const int lr = (int)((unsigned)lane % 16), hi = (int)((unsigned)lane / 16);
    const bool interior = (m0 + C::BM <= M) && (n0 + C::BN <= N);
    float sam[C::MI];
#pragma unroll
    for (int mi = 0; mi < C::MI; ++mi)
        sam[mi] = E::BYTES == 1 ? sa_l[wm * C::TM + mi * 16 + lr] : 0.f;
    // this lane's store: tile 2 * pp + (hi & 1), columns 8 * (hi >> 1) .. + 7,
    // at base + mi * 16 rows + 32 * pp columns
    const int64_t col0 = n0 + wn * C::TN + 16 * (hi & 1) + 8 * (hi >> 1);
    const int64_t row0 = m0 + wm * C::TM + lr;
    uint16_t* base = y + row0 * N + col0;
    const int64_t rows_left = M - row0, cols_left = N - col0;
#pragma unroll
    for (int pp = 0; pp < C::NI / 2; ++pp) {
        // the pair's column scales and bias, shared by every row tile
        v4f swv[2], bv[2];
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int cl = wn * C::TN + (2 * pp + j) * 16 + 4 * hi;
            if constexpr (E::BYTES == 1) swv[j] = *reinterpret_cast<const v4f*>(sw_l + cl);
            bv[j] = *reinterpret_cast<const v4f*>(b_l + cl);
        }
#pragma unroll
        for (int mi = 0; mi < C::MI; ++mi) {
            uint32_t d[2][2];
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                float v[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    if constexpr (E::BYTES == 1) {
                        const float t = (float)acc[2 * pp + j][mi][e];  // nearest even
                        const float u = __fmul_rn(sam[mi], swv[j][e]);
                        v[e] = __builtin_fmaf(t, u, bv[j][e]);
                    } else {
                        v[e] = __fadd_rn(acc[2 * pp + j][mi][e], bv[j][e]);
                    }
                }
                uint32_t lo = pack_bf16x2(v[0], v[1]), hi2 = pack_bf16x2(v[2], v[3]);
                if (ACT == 1) {
                    // GELU-tanh of the bf16-rounded value, rounded to bf16 (gelu_bf16_rn)
                    lo = gelu_bf16_rn(lo & 0xffffu) | (gelu_bf16_rn(lo >> 16) << 16);
                    hi2 = gelu_bf16_rn(hi2 & 0xffffu) | (gelu_bf16_rn(hi2 >> 16) << 16);
                }
                d[j][0] = lo;
                d[j][1] = hi2;
            }
#pragma unroll
            for (int k = 0; k < 2; ++k) {
                const auto r = __builtin_amdgcn_permlane16_swap(d[0][k], d[1][k], false, false);
                d[0][k] = r[0];
                d[1][k] = r[1];
            }
            v4i o;
            o[0] = (int)d[0][0];
            o[1] = (int)d[0][1];
            o[2] = (int)d[1][0];
            o[3] = (int)d[1][1];
            v4i* dst = reinterpret_cast<v4i*>(base + (int64_t)(mi * 16) * N + 32 * pp);
            if (interior || (mi * 16 < rows_left && 32 * pp < cols_left)) {
#if W8A8_STORE_NT
                __builtin_nontemporal_store(o, dst);
#else
                *dst = o;
#endif
            }
        }
        // register-tight tiles: keep the next pair's reads from being hoisted
        if constexpr (C::RECYCLE) __builtin_amdgcn_sched_barrier(0);
    }
}

// Epilogue with a staging area per wave (C::EPW), 2 KB past the ring: a wave
// stages a piece of 16 rows x 64 columns of its own outputs (MFMA row tile mi,
// four column tiles), reads it back as 2 x 8 rows of 128 bytes and stores
// whole 128-byte row segments.  A wave reads only what it wrote itself and
// LDS executes a wave's instructions in order, so there is no barrier.  Row r
// of a piece (128 bytes) keeps its 8-byte slot s at s ^ f(r), f(r) =
// 2 * (r & 7) + (r >> 3), a permutation of 0 .. 15.  An 8-byte write
// instruction takes 16 lanes per LDS cycle, here 16 rows at the same logical
// slot, which the XOR spreads over all 16 slots of a row: free of bank
// conflicts (SQ_LDS_BANK_CONFLICT; with any swizzle of 16-byte chunks instead,
// each such group hits only the low halves of the chunks and takes two cycles).
// A 16-byte read of logical bytes 16c .. 16c + 15 of row r then finds them in
// chunk c ^ (r & 7), with the two halves exchanged in rows 8 .. 15 (f odd):
// the second read of each piece, so the exchange is a fixed register order.
template <class C, class E, int ACT>
__device__ __forceinline__ void store_perwave(const Acc<C, E>& acc, uint16_t* __restrict__ y,
                                              int64_t M, int64_t N, int64_t m0, int64_t n0, int wm,
                                              int wn, int lane, const float* sa_l, const float* sw_l,
                                              const float* b_l, char* pw) {
    static_assert(C::EPW, "per-wave epilogue");
    const int lr = (int)((unsigned)lane % 16), hi = (int)((unsigned)lane / 16);
    // writes: row lr, logical slot 4 * nl + hi, at wofs + ((32 * nl) ^ g)
    const uint32_t wofs = (uint32_t)(lr * 128);
    const uint32_t g = 8u * (uint32_t)(hi ^ (2 * (lr & 7) + (lr >> 3)));
    // reads: rows rr and rr + 8, logical chunk rc, at physical chunk rc ^ rr
    const int rr = (int)((unsigned)lane / 8), rc = (int)((unsigned)lane % 8);
    const uint32_t rofs0 = (uint32_t)(rr * 128 + 16 * (rc ^ rr));
    const uint32_t rofs1 = rofs0 + 8u * 128u;
    const bool interior = (m0 + C::BM <= M) && (n0 + C::BN <= N);
    const int64_t row0 = m0 + wm * C::TM + rr, col0 = n0 + wn * C::TN + 8 * rc;
    uint16_t* base = y + row0 * N + col0;
    const int64_t rows_left = M - row0, cols_left = N - col0;
    // the bf16 values of piece (mi, h) for column groups nl = 0 .. 3, packed
    auto piece = [&](auto mic, auto hc, uint2 (&o)[4]) __attribute__((always_inline)) {
        constexpr int mi = decltype(mic)::value, h = decltype(hc)::value;
        const float sam = E::BYTES == 1 ? sa_l[wm * C::TM + mi * 16 + lr] : 0.f;
#pragma unroll
        for (int nl = 0; nl < 4; ++nl) {
            const int ni = 4 * h + nl;
            const int cl = wn * C::TN + ni * 16 + 4 * hi;
            v4f swv = {}, bv;
            if constexpr (E::BYTES == 1) swv = *reinterpret_cast<const v4f*>(sw_l + cl);
            bv = *reinterpret_cast<const v4f*>(b_l + cl);
            float v[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                if constexpr (E::BYTES == 1) {
                    const float t = (float)acc[ni][mi][e];  // nearest even
                    const float u = __fmul_rn(sam, swv[e]);
                    v[e] = __builtin_fmaf(t, u, bv[e]);
                } else {
                    v[e] = __fadd_rn(acc[ni][mi][e], bv[e]);
                }
            }
            o[nl] = make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
            if (ACT == 1) {
                // GELU-tanh of the bf16-rounded value, rounded to bf16 (gelu_bf16_rn)
                o[nl] = make_uint2(gelu_bf16_rn(o[nl].x & 0xffffu) | (gelu_bf16_rn(o[nl].x >> 16) << 16),
                                   gelu_bf16_rn(o[nl].y & 0xffffu) | (gelu_bf16_rn(o[nl].y >> 16) << 16));
            }
        }
    };
    // Pieces in order mi, h, software-pipelined: a piece is staged and its
    // reads issued, then the next piece's values are computed while those
    // reads are in flight, and only then are they waited for and stored (the
    // next piece's writes come after this piece's reads, which LDS executes
    // first).
    constexpr int H = C::NI / 4, P = C::MI * H;
    uint2 o[4];
    piece(std::integral_constant<int, 0>{}, std::integral_constant<int, 0>{}, o);
    auto step = [&](auto pc) __attribute__((always_inline)) {
        constexpr int p = decltype(pc)::value, mi = p / H, h = p % H;
#pragma unroll
        for (int nl = 0; nl < 4; ++nl)
            *reinterpret_cast<uint2*>(pw + (wofs + ((32u * (uint32_t)nl) ^ g))) = o[nl];
        const v4i d0 = *reinterpret_cast<const v4i*>(pw + rofs0);
        const v4i e1 = *reinterpret_cast<const v4i*>(pw + rofs1);
        if constexpr (p + 1 < P)
            piece(std::integral_constant<int, (p + 1) / H>{}, std::integral_constant<int, (p + 1) % H>{}, o);
        const v4i d1 = {e1[2], e1[3], e1[0], e1[1]};  // rows 8 .. 15: halves exchanged
        uint16_t* dst = base + (int64_t)(mi * 16) * N + 64 * h;
        const bool cols_in = interior || 64 * h < cols_left;
        if (cols_in && (interior || mi * 16 < rows_left)) {
#if W8A8_STORE_NT
            __builtin_nontemporal_store(d0, reinterpret_cast<v4i*>(dst));
#else
            *reinterpret_cast<v4i*>(dst) = d0;
#endif
        }
        if (cols_in && (interior || mi * 16 + 8 < rows_left)) {
#if W8A8_STORE_NT
            __builtin_nontemporal_store(d1, reinterpret_cast<v4i*>(dst + 8 * N));
#else
            *reinterpret_cast<v4i*>(dst + 8 * N) = d1;
#endif
        }
        // register-tight tiles: keep the piece after next from being hoisted here
        if constexpr (C::RECYCLE) __builtin_amdgcn_sched_barrier(0);
    };
    for_each_pass(step, std::make_integer_sequence<int, P>{});
}

// The K groups' partial sums are added through LDS (the ring, which the K loop
// is done with).  With two groups each finalises half of the wave's column
// tiles, group g the tiles [g*NI/2, (g+1)*NI/2): it hands the other half to its
// partner wave (same slot in the other group), adds the partner's half of its
// own, and leaves the sums in acc[0 .. NI/2) (so that no accumulator index
// depends on the group, which would put the accumulators in scratch memory).
// Both groups then share the adds and the epilogue.  The sums are the same
// either way: exact for INT32, and for fp32 a + b, which is b + a.  With more
// groups, groups g > 0 hand everything to group 0, which adds them in order
// g = 1, 2, ....  Lane l's values of accumulator register group q of MFMA tile
// j of the handed range sit at ((j*MI + mi)*G + q)*1 KB + 16*l of the wave's
// area, so each 16-byte access of a wave is contiguous.  Every wave calls it
// (it holds two barriers).
template <class C, class E>
__device__ __forceinline__ void reduce_k_groups(Acc<C, E>& acc, char* smem, int kg, int slot,
                                                int lane) {
    if constexpr (C::KS == 2) {
        typedef std::conditional_t<E::BYTES == 1, v4i, v4f> V4;
        constexpr int G = C::ACC_N / 4, H = C::NI / 2;
        constexpr int HALF = H * C::MI * G * 1024;  // bytes one wave hands over
        static_assert(C::NI % 2 == 0 && 2 * C::WG * HALF <= C::RING, "K-group halves");
        const bool g1 = kg != 0;
        char* dst = smem + (kg * C::WG + slot) * HALF + 16 * lane;
#pragma unroll
        for (int j = 0; j < H; ++j)
#pragma unroll
            for (int mi = 0; mi < C::MI; ++mi)
#pragma unroll
                for (int q = 0; q < G; ++q) {
                    V4 v;
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        v[e] = g1 ? acc[j][mi][4 * q + e] : acc[H + j][mi][4 * q + e];
                    *reinterpret_cast<V4*>(dst + ((j * C::MI + mi) * G + q) * 1024) = v;
                }
        lds_barrier();
        const char* src = smem + ((1 - kg) * C::WG + slot) * HALF + 16 * lane;
#pragma unroll
        for (int j = 0; j < H; ++j)
#pragma unroll
            for (int mi = 0; mi < C::MI; ++mi)
#pragma unroll
                for (int q = 0; q < G; ++q) {
                    const V4 v = *reinterpret_cast<const V4*>(src + ((j * C::MI + mi) * G + q) * 1024);
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const auto own = g1 ? acc[H + j][mi][4 * q + e] : acc[j][mi][4 * q + e];
                        acc[j][mi][4 * q + e] = own + v[e];
                    }
                }
        lds_barrier();  // the ring is free again
    } else if constexpr (C::KS > 2) {
        typedef AccT<C, E> A;
        typedef std::conditional_t<E::BYTES == 1, v4i, v4f> V4;
        constexpr int G = C::ACC_N / 4;
        if (kg > 0) {
            char* dst = smem + ((kg - 1) * C::WG + slot) * C::RED_WAVE + 16 * lane;
#pragma unroll
            for (int ni = 0; ni < C::NI; ++ni)
#pragma unroll
                for (int mi = 0; mi < C::MI; ++mi)
#pragma unroll
                    for (int q = 0; q < G; ++q) {
                        const A& a = acc[ni][mi];
                        const V4 v = {a[4 * q], a[4 * q + 1], a[4 * q + 2], a[4 * q + 3]};
                        *reinterpret_cast<V4*>(dst + ((ni * C::MI + mi) * G + q) * 1024) = v;
                    }
        }
        lds_barrier();
        if (kg == 0) {
#pragma unroll
            for (int g = 1; g < C::KS; ++g) {
                const char* src = smem + ((g - 1) * C::WG + slot) * C::RED_WAVE + 16 * lane;
#pragma unroll
                for (int ni = 0; ni < C::NI; ++ni)
#pragma unroll
                    for (int mi = 0; mi < C::MI; ++mi)
#pragma unroll
                        for (int q = 0; q < G; ++q) {
                            const V4 v = *reinterpret_cast<const V4*>(
                                src + ((ni * C::MI + mi) * G + q) * 1024);
#pragma unroll
                            for (int e = 0; e < 4; ++e) acc[ni][mi][4 * q + e] += v[e];
                        }
            }
        }
        lds_barrier();  // the ring is free again
    }
}

// (with two K groups a wave stores its group's half of its column tiles, kg
// the group: their sums are in acc[0 .. NI/2), see reduce_k_groups)
template <class C>
__device__ __forceinline__ void store_i32(const Acc<C, ElemI8>& acc, int32_t* __restrict__ out,
                                          int64_t M, int64_t N, int64_t m0, int64_t n0, int wm,
                                          int wn, int lane, int kg) {
    constexpr int G = C::ACC_N / 4, GS = C::MT / 4;
    constexpr int NIS = C::KS == 2 ? C::NI / 2 : C::NI;
    const int ncol = wn * C::TN + (C::KS == 2 ? kg * NIS * C::MT : 0) +
                     4 * (int)((unsigned)lane / C::MT);
#pragma unroll
    for (int mi = 0; mi < C::MI; ++mi) {
        const int ml = wm * C::TM + mi * C::MT + (int)((unsigned)lane % C::MT);
        if (m0 + ml >= M) continue;
        int32_t* rowp = out + (m0 + ml) * N + n0 + ncol;
#pragma unroll
        for (int ni = 0; ni < NIS; ++ni)
#pragma unroll
            for (int g = 0; g < G; ++g) {
                if (n0 + ncol + ni * C::MT + GS * g >= N) continue;
                v4i v = {acc[ni][mi][4 * g], acc[ni][mi][4 * g + 1], acc[ni][mi][4 * g + 2],
                         acc[ni][mi][4 * g + 3]};
                *reinterpret_cast<v4i*>(rowp + ni * C::MT + GS * g) = v;
            }
    }
}

// Persistent kernel (PERSIST): the grid holds as many workgroups as fit on the
// GPU at once (or one per tile if there are fewer tiles), and workgroup b
// walks tiles b, b + grid, ...  While a tile's epilogue runs, the next tile's
// first K stage is already loading into ring buffer 0 and its scales into
// registers; the output is staged in the LDS above buffer 0.  Without PERSIST
// each workgroup does one tile (the GELU epilogue's binary64 slow path needs
// the registers that the tile loop's live state would take).
// a, w: [M x K] and [N x K] operands of E; sa, sw: INT8 row and column scales
// (unused for BF16); K in elements.
template <class C, class E, int OUT_I32, int ACT, bool PERSIST, bool VEC_OUT>
__global__ __launch_bounds__(C::THREADS)
__attribute__((amdgpu_waves_per_eu(C::WAVES_PER_SIMD, C::WAVES_PER_SIMD)))
void gemm_tiled(const void* __restrict__ a, const float* __restrict__ sa, int64_t M,
                const void* __restrict__ w, const float* __restrict__ sw, int64_t N, int64_t K,
                const uint16_t* __restrict__ bias, void* __restrict__ out, int kt_split) {
    constexpr int BM = C::BM, BN = C::BN, BK = C::BK, NST = C::NST, MI = C::MI;
    constexpr bool SCALES = !OUT_I32 && E::BYTES == 1;
    // K ring (from byte STAGE on, also the output staging area) and the
    // tile's row scales, column scales and bias (as binary32).  All of it is
    // one LDS object: with several, the compiler can no longer tell the
    // fragment reads from the in-flight direct-to-LDS loads and waits for
    // every load.
    __shared__ __attribute__((aligned(1024))) char smem[C::SMEM];
    // the epilogue straight from registers (INT8, 16-byte aligned output rows;
    // the BF16 192 x 256 kernel measured 1.5% slower with it), or staged per wave
    constexpr bool DIRECT = C::DIRECT_OK && VEC_OUT && !OUT_I32 && E::BYTES == 1;
    constexpr bool PERWAVE = C::EPW && !OUT_I32;
    static_assert(!PERWAVE || VEC_OUT, "the per-wave epilogue stores whole 16-byte chunks");
    constexpr bool NO_STAGE = DIRECT || PERWAVE;  // the ring holds no staging area
    float* sa_l = reinterpret_cast<float*>(smem + C::SCALE_OFF);
    float* sw_l = sa_l + BM;
    float* b_l = sw_l + BN;
    const char* ab = static_cast<const char*>(a);
    const char* wb = static_cast<const char*>(w);
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int kg = C::KS > 1 ? wave / C::WG : 0;       // K group (KS > 1)
    const int wm = (wave % C::WG) % C::WM, wn = (wave % C::WG) / C::WM;
    const int64_t tm = (M + BM - 1) / BM, tn = (N + BN - 1) / BN, tiles = tm * tn;
    const int64_t KB = K * E::BYTES;
    // split-K: K / BK stages in slices of kt_split, work item t = slice * tiles + tile
    const int64_t nslice = C::SPLIT ? (KB / BK) / kt_split : 1;
    const int64_t total = tiles * nslice;
    // INT8 rows are whole stages; a BF16 row may end inside its last stage
    const int KT = C::SPLIT ? kt_split : E::BYTES == 1 ? (int)(KB / BK) : (int)((KB + BK - 1) / BK);
    const int tail = (int)(KB - (int64_t)(KT - 1) * BK);  // valid bytes in the last stage
    int64_t t = blockIdx.x, tile_m, tile_n;
    int slice = 0;
    auto item = [&](int64_t ti) {
        if constexpr (C::SPLIT) {
            slice = (int)(ti / tiles);
            ti -= (int64_t)slice * tiles;
        }
        tile_of<C>(ti, tm, tn, tile_m, tile_n);
    };
    item(t);
    int64_t m0 = tile_m * BM, n0 = tile_n * BN;
    Ctx<C> c;
    make_ctx<C>(c, KB, wave, lane);
    if constexpr (C::SPLIT) c.kofs = slice * kt_split * BK;
    set_tile<C>(c, ab, wb, M, N, KB, m0, n0);

    // Epilogue operands of a tile: row scales, column scales and bias (the
    // bias stays in bf16 bits until it is written: converting it at once
    // would make the wave wait for the load).  They are loaded with the tile's
    // first stages (or during the previous tile's epilogue) and written to LDS
    // before its K loop; with the scales in the ring they are loaded during
    // the tile's last K stage instead and written once the K loop is done
    // with the ring, so no register holds them across the K loop.
    // Every thread loads (clamped indices; only threads below BM / BN store),
    // so that each load defines its register anew and nothing carries over
    // from the previous tile.
    float nsa[C::SA_PT] = {}, nsw[C::SW_PT] = {};
    uint32_t nb[C::SW_PT] = {};
    auto load_scales = [&](int64_t m0_, int64_t n0_) {
#pragma unroll
        for (int i = 0; i < C::SA_PT; ++i) {
            const int64_t m = m0_ + tid + i * C::THREADS;
            if (SCALES) nsa[i] = sa[m < M ? m : M - 1];
        }
        if (!OUT_I32) {
#pragma unroll
            for (int i = 0; i < C::SW_PT; ++i) {
                const int64_t n = n0_ + tid + i * C::THREADS < N ? n0_ + tid + i * C::THREADS : N - 1;
                if (SCALES) nsw[i] = sw[n];
                if constexpr (C::SCALES_IN_RING) {
                    // loaded during the last K stage: a branch on the pointer
                    // would make the wave wait for it there
                    const int64_t cnt = N - n0_ < BN ? N - n0_ : BN;
                    nb[i] = load_bias_bits(bias ? bias + n0_ : nullptr, (int)cnt, (int)(n - n0_));
                } else {
                    nb[i] = bias ? (uint32_t)bias[n] : 0u;
                }
            }
        }
    };
    if constexpr (!C::SCALES_IN_RING) load_scales(m0, n0);
    auto put_scales = [&]() {
        // an opaque copy of the thread index: the LDS addresses are formed
        // here, not kept in registers across the K loop
        int et = tid;
        asm volatile("" : "+v"(et));
        if constexpr (C::SCALES_IN_RING) {
            // every wave waits for its loads here, before the stores below
            // branch: a wait left inside the branch would leave the loads
            // pending, for the compiler, on the other path, and it would then
            // wait for them at the next reuse of their registers, behind the
            // next tile's first stage
#pragma unroll
            for (int i = 0; i < C::SA_PT; ++i)
                if (SCALES) asm volatile("" ::"v"(nsa[i]));
#pragma unroll
            for (int i = 0; i < C::SW_PT; ++i) {
                if (SCALES) asm volatile("" ::"v"(nsw[i]));
                if (!OUT_I32) asm volatile("" ::"v"(nb[i]));
            }
        }
#pragma unroll
        for (int i = 0; i < C::SA_PT; ++i)
            if (SCALES && et + i * C::THREADS < BM) sa_l[et + i * C::THREADS] = nsa[i];
#pragma unroll
        for (int i = 0; i < C::SW_PT; ++i) {
            const int e = et + i * C::THREADS;
            if (!OUT_I32 && e < BN) {
                if (SCALES) sw_l[e] = nsw[i];
                b_l[e] = bf16_bits_to_float(bias ? nb[i] : 0x8000u);  // -0.0 without a bias
            }
        }
    };
    for (int s = 0; s < NST; ++s)
        if (s < KT) stage_load<C>(c, s * BK, smem + s * C::STAGE);
    if constexpr (!C::SCALES_IN_RING) put_scales();
    if (KT >= NST) wait_vm_lgkm0<C::NLOAD * (NST - 1)>();
    else wait_vm_lgkm0<0>();
    __syncthreads();

    for (;;) {
        Acc<C, E> acc;
#pragma unroll
        for (int i = 0; i < C::NI; ++i)
#pragma unroll
            for (int j = 0; j < MI; ++j) acc[i][j] = (AccT<C, E>){};
        Frags<C> cur;
        const FragBase fb0 = frag_base(c);
#pragma unroll
        for (int q = 0; q < C::NQ; ++q) read_frag<C>(smem, fb0, 0, q, cur);

        int kt = 0;
        for (; kt + NST < KT; ++kt) k_stage<C, E, true, true, true>(c, smem, kt, acc, cur);
        if (kt == KT - NST && kt + 1 < KT) {
            k_stage<C, E, false, true, true>(c, smem, kt, acc, cur);
            ++kt;
        }
        for (; kt + 1 < KT; ++kt) k_stage<C, E, false, true, false>(c, smem, kt, acc, cur);
        if constexpr (C::SCALES_IN_RING) load_scales(m0, n0);
        k_stage<C, E, false, false, false>(c, smem, kt, acc, cur, tail);

        const int64_t t_next = t + gridDim.x;
        const bool has_next = PERSIST && t_next < total;
        int64_t m0n = 0, n0n = 0;
        lds_barrier();  // every wave is done reading the K ring
        reduce_k_groups<C, E>(acc, smem, kg, wave % C::WG, lane);
        if constexpr (C::SCALES_IN_RING) {
            put_scales();
            lds_barrier();
        }
        const int slice_now = slice;
        if (has_next) {
            item(t_next);
            m0n = tile_m * BM;
            n0n = tile_n * BN;
            // (the per-wave epilogue leaves no register for them: they are
            // loaded after it, from L2)
            if constexpr (!C::SCALES_IN_RING && !PERWAVE) load_scales(m0n, n0n);
            set_tile<C>(c, ab, wb, M, N, KB, m0n, n0n);
            if constexpr (C::SPLIT) c.kofs = slice * kt_split * BK;
            stage_load<C>(c, 0, smem);  // next tile's stage 0 -> buffer 0
            // without a staging area in the ring the later stages can go now too
            if constexpr (NO_STAGE) {
                for (int s = 1; s < NST; ++s)
                    if (s < KT) stage_load<C>(c, s * BK, smem + s * C::STAGE);
            }
        }
        // The epilogue's lane addresses depend only on the lane, and hoisted out
        // of the tile loop they would stay live across the K loop; an opaque
        // copy of the lane index keeps them local to the epilogue.
        int elane = lane;
        asm volatile("" : "+v"(elane));
        if constexpr (OUT_I32 != 0) {
            if (C::KS <= 2 || kg == 0)
                store_i32<C>(acc, reinterpret_cast<int32_t*>(out) + (int64_t)slice_now * M * N, M, N,
                             m0, n0, wm, wn, elane, kg);
        } else if constexpr (DIRECT) {
            store_direct<C, E, ACT>(acc, reinterpret_cast<uint16_t*>(out), M, N, m0, n0, wm, wn,
                                    elane, sa_l, sw_l, b_l);
        } else if constexpr (PERWAVE) {
            store_perwave<C, E, ACT>(acc, reinterpret_cast<uint16_t*>(out), M, N, m0, n0, wm, wn,
                                     elane, sa_l, sw_l, b_l, smem + C::PW_OFF + wave * C::PW_BYTES);
        } else {
            store_bf16<C, E, ACT, VEC_OUT>(acc, reinterpret_cast<uint16_t*>(out), M, N, m0, n0,
                                           wave, wm, wn, elane, sa_l, sw_l, b_l, smem + C::STAGE,
                                           kg);
        }
        if (!has_next) break;
        if constexpr (PERWAVE) load_scales(m0n, n0n);
        if constexpr (C::SCALE_BUFS == 2) {
            // the next tile's scales go to the other buffer: slower waves may
            // still be reading these
            const int flip = sa_l == reinterpret_cast<float*>(smem + C::SCALE_OFF) ? 1 : 0;
            sa_l = reinterpret_cast<float*>(smem + C::SCALE_OFF + flip * C::SCALE_BYTES);
            sw_l = sa_l + BM;
            b_l = sw_l + BN;
        }
        // this tile's epilogue is done with the old values (store_bf16 ends
        // with a barrier; store_direct's and store_perwave's reads are in the
        // other buffer)
        if constexpr (!C::SCALES_IN_RING) put_scales();
        wait_vm_lgkm0<0>();  // the next tile's stage 0 (and this tile's stores) are done ...
        __syncthreads();     // ... for every wave, and the staging area is free
        lane_ctx<C>(c, elane);
        if constexpr (!NO_STAGE) {
            for (int s = 1; s < NST; ++s)
                if (s < KT) stage_load<C>(c, s * BK, smem + s * C::STAGE);
        }
        t = t_next;
        m0 = m0n;
        n0 = n0n;
    }
}

template <class C>
int64_t tile_count(int64_t M, int64_t N) {
    return ((N + C::BN - 1) / C::BN) * ((M + C::BM - 1) / C::BM);
}

template <class C, class E, int OUT_I32, int ACT, bool VEC_OUT>
hipError_t launch_cfg(const void* a, const float* sa, int64_t M, const void* w, const float* sw,
                      int64_t N, int64_t K, const uint16_t* bias, void* out, int cus,
                      hipStream_t stream, int nslice = 1) {
    const int64_t tiles = tile_count<C>(M, N) * nslice;
    const int kt_split = C::SPLIT ? (int)(K * E::BYTES / C::BK / nslice) : 0;
    if (tiles >= (int64_t(1) << 31)) return hipErrorInvalidValue;  // tile indices are 32-bit
    constexpr bool persist = ACT == 0;
    // workgroups that fit on one CU at once (160 KB of LDS is the limit)
    constexpr int per_cu = (160 * 1024) / C::SMEM < 1 ? 1 : (160 * 1024) / C::SMEM;
    int64_t grid = tiles;
    if (persist) {
        const int64_t slots = (int64_t)cus * per_cu;
        grid = tiles < slots ? tiles : slots;
    }
    hipLaunchKernelGGL((gemm_tiled<C, E, OUT_I32, ACT, persist, VEC_OUT>), dim3((unsigned)grid),
                       dim3(C::THREADS), 0, stream, a, sa, M, w, sw, N, K, bias, out, kt_split);
    return hipGetLastError();
}

// Tile choice.  Larger tiles move less data per MFMA, which is what sets the
// clock under the power cap; smaller ones only pay off when the large ones
// leave most CUs idle.
template <class E, int OUT_I32, int ACT, bool VEC_OUT>
hipError_t launch_tiles(const void* a, const float* sa, int64_t M, const void* w, const float* sw,
                        int64_t N, int64_t K, const uint16_t* bias, void* out,
                        hipStream_t stream) {
    const int cus = cu_count();
    if (cus <= 0) return hipErrorInvalidDevice;
    typedef typename Tiers<E>::Large CfgLarge;
    typedef typename Tiers<E>::Mid CfgMid;
    if (2 * tile_count<CfgLarge>(M, N) >= cus) {
        // mid when its rounds x 3/4 of a large tile's work, with 7% for its
        // lower efficiency per MFMA, come to less than large's rounds
        const int64_t tl = tile_count<CfgLarge>(M, N), tmid = tile_count<CfgMid>(M, N);
        const int64_t rounds_l = (tl + cus - 1) / cus, rounds_mid = (tmid + cus - 1) / cus;
        if (8025 * rounds_mid < 10000 * rounds_l)
            return launch_cfg<CfgMid, E, OUT_I32, ACT, VEC_OUT>(a, sa, M, w, sw, N, K, bias, out,
                                                               cus, stream);
        return launch_cfg<CfgLarge, E, OUT_I32, ACT, VEC_OUT>(a, sa, M, w, sw, N, K, bias, out, cus,
                                                             stream);
    }
    typedef typename Tiers<E>::Small CSmall;
    typedef typename Tiers<E>::Deep CDeep;
    typedef typename Tiers<E>::Tiny CTiny;
    if (2 * tile_count<CSmall>(M, N) >= cus) {
        // A 3-deep ring keeps two stages of loads in flight: with one wave per
        // SIMD and 512 cycles of MFMAs per stage, the 2-deep ring's per-stage
        // load latency shows.  It pays on K loops of 32 stages or more
        // (2048 x 2048 x 2050 BF16: 33.7 -> 27.1 us; 512 x 4096 x 4096 INT8:
        // 22.4 -> 20.3 us) and costs 2-5% on 16 stages (2048^3 INT8); its
        // 96 KB of LDS leaves one workgroup per CU, so only where the tiles
        // take one round.
        if (K * E::BYTES >= 32 * CDeep::BK && tile_count<CDeep>(M, N) <= cus)
            return launch_cfg<CDeep, E, OUT_I32, ACT, VEC_OUT>(a, sa, M, w, sw, N, K, bias, out, cus,
                                                              stream);
        return launch_cfg<CSmall, E, OUT_I32, ACT, VEC_OUT>(a, sa, M, w, sw, N, K, bias, out, cus,
                                                           stream);
    }
    return launch_cfg<CTiny, E, OUT_I32, ACT, VEC_OUT>(a, sa, M, w, sw, N, K, bias, out, cus,
                                                      stream);
}

// ---- split-K across workgroups ----
// Shapes whose tiles leave most CUs idle (few rows or columns) and have a long
// K loop: the K stages are cut into S slices, the 128 x 128 tiles of all slices
// run at once (writing INT32 partial sums to S slices of the workspace), then
// splitk_reduce adds the slices in order s = 0 .. S-1 (exact in INT32: the
// scales come only after the whole accumulation) and applies the same
// epilogue as the tiled kernel, so the result is w8a8_gemm's bit for bit.
#ifndef W8A8_I8_SPLIT_MT
#define W8A8_I8_SPLIT_MT 32
#endif
typedef Cfg<128, 128, 2, 2, 128, 2, GROUP_ROWS, 2, true, W8A8_I8_SPLIT_MT> CfgSplit;

// Four consecutive outputs of one row per thread (N is a multiple of 64), in a
// grid-stride loop: acc = sum of the S partials, then exactly store_bf16's
// arithmetic (or the raw INT32 sum).
template <int OUT_I32, int ACT>
__global__ __launch_bounds__(256) void splitk_reduce(const int32_t* __restrict__ part, int nslice,
                                                     int64_t M, int64_t N,
                                                     const float* __restrict__ sa,
                                                     const float* __restrict__ sw,
                                                     const uint16_t* __restrict__ bias,
                                                     void* __restrict__ out) {
    const int64_t MN = M * N, quads = MN / 4;
    for (int64_t qd = (int64_t)blockIdx.x * 256 + threadIdx.x; qd < quads;
         qd += (int64_t)gridDim.x * 256) {
        const int64_t e0 = 4 * qd;
        v4i acc = __builtin_nontemporal_load(reinterpret_cast<const v4i*>(part + e0));
        for (int sl = 1; sl < nslice; ++sl)
            acc += __builtin_nontemporal_load(reinterpret_cast<const v4i*>(part + sl * MN + e0));
        if constexpr (OUT_I32 != 0) {
            __builtin_nontemporal_store(acc, reinterpret_cast<v4i*>(static_cast<int32_t*>(out) + e0));
        } else {
            const int64_t row = e0 / N, col = e0 - row * N;
            const float sam = sa[row];
            float v[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float b = bf16_bits_to_float(bias ? (uint32_t)bias[col + e] : 0x8000u);
                const float t = (float)acc[e];  // nearest even
                const float u = __fmul_rn(sam, sw[col + e]);
                v[e] = __builtin_fmaf(t, u, b);
            }
            uint2 o = make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
            if (ACT == 1)
                o = make_uint2(gelu_bf16_rn(o.x & 0xffffu) | (gelu_bf16_rn(o.x >> 16) << 16),
                               gelu_bf16_rn(o.y & 0xffffu) | (gelu_bf16_rn(o.y >> 16) << 16));
            typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
            const u32x2 ov = {o.x, o.y};
            __builtin_nontemporal_store(ov, reinterpret_cast<u32x2*>(static_cast<uint16_t*>(out) + e0));
        }
    }
}

}  // namespace

int splitk_slices(int64_t M, int64_t N, int64_t K) {
    // The slice count is a property of the shape alone (the library targets the
    // 256 CUs of an MI355X), so the workspace size needs no device query.
    constexpr int64_t kCUs = 256;
    if (M <= 0 || N <= 0) return 1;
    // only shapes the large tiles and the 128 x 128 tiles leave mostly idle
    if (2 * tile_count<Tiers<ElemI8>::Large>(M, N) >= kCUs || 2 * tile_count<CfgSplit>(M, N) >= kCUs)
        return 1;
    const int64_t tiles = tile_count<CfgSplit>(M, N), stages = K / CfgSplit::BK;
    int64_t S = kCUs / tiles;
    if (S > 8) S = 8;
    // whole stages per slice, at least 8 of them
    while (S > 1 && (stages % S != 0 || stages / S < 8)) --S;
    return (int)S;
}

size_t splitk_workspace_bytes(int64_t M, int64_t N, int64_t K) {
    const int S = splitk_slices(M, N, K);
    return S > 1 ? (size_t)S * (size_t)M * (size_t)N * sizeof(int32_t) : 0;
}

int launch_gemm_i8_splitk(const int8_t* qa, const float* sa, int64_t M, const int8_t* qw,
                          const float* sw, int64_t N, int64_t K, const uint16_t* bias, int act,
                          int out_kind, void* out, void* workspace, hipStream_t stream) {
    const int S = splitk_slices(M, N, K);
    if (S <= 1) return launch_gemm_i8(qa, sa, M, qw, sw, N, K, bias, act, out_kind, out, stream);
    const int cus = cu_count();
    if (cus <= 0) return -1;
    hipError_t e = launch_cfg<CfgSplit, ElemI8, 1, 0, true>(qa, sa, M, qw, sw, N, K, nullptr,
                                                          workspace, cus, stream, S);
    if (e != hipSuccess) return -1;
    const int64_t quads = M * N / 4;
    int64_t blocks = (quads + 255) / 256;
    if (blocks > (int64_t)cus * 8) blocks = (int64_t)cus * 8;
    const int32_t* part = static_cast<const int32_t*>(workspace);
    if (out_kind == 1)
        hipLaunchKernelGGL((splitk_reduce<1, 0>), dim3((unsigned)blocks), dim3(256), 0, stream, part,
                           S, M, N, sa, sw, bias, out);
    else if (act == 1)
        hipLaunchKernelGGL((splitk_reduce<0, 1>), dim3((unsigned)blocks), dim3(256), 0, stream, part,
                           S, M, N, sa, sw, bias, out);
    else
        hipLaunchKernelGGL((splitk_reduce<0, 0>), dim3((unsigned)blocks), dim3(256), 0, stream, part,
                           S, M, N, sa, sw, bias, out);
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

int launch_gemm_i8(const int8_t* qa, const float* sa, int64_t M, const int8_t* qw,
                   const float* sw, int64_t N, int64_t K, const uint16_t* bias, int act,
                   int out_kind, void* out, hipStream_t stream) {
    if (M == 0 || N == 0) return 0;
    hipError_t e;
    if (out_kind == 1)
        e = launch_tiles<ElemI8, 1, 0, true>(qa, sa, M, qw, sw, N, K, bias, out, stream);
    else if (act == 1)
        e = launch_tiles<ElemI8, 0, 1, true>(qa, sa, M, qw, sw, N, K, bias, out, stream);
    else
        e = launch_tiles<ElemI8, 0, 0, true>(qa, sa, M, qw, sw, N, K, bias, out, stream);
    return e == hipSuccess ? 0 : -1;
}

bool gemm_bf16_tiled_ok(const uint16_t* x, int64_t K, const uint16_t* w) {
    // rows of whole dwords (K even, 4-byte aligned operands: the 16-byte loads
    // are dword aligned; the last stage's tail is masked), and stage offsets
    // and buffer sizes that fit the 32-bit buffer addressing
    return K >= 2 && K % 2 == 0 && K <= (1 << 20) &&
           reinterpret_cast<uintptr_t>(x) % 4 == 0 && reinterpret_cast<uintptr_t>(w) % 4 == 0;
}

int launch_gemm_bf16_tiled(const uint16_t* x, int64_t M, int64_t K, const uint16_t* w, int64_t N,
                           const uint16_t* bias, int act, uint16_t* y, hipStream_t stream) {
    if (M == 0 || N == 0) return 0;
    const bool vec = N % 8 == 0 && reinterpret_cast<uintptr_t>(y) % 16 == 0;
    hipError_t e;
    if (act == 1)
        e = vec ? launch_tiles<ElemBF16, 0, 1, true>(x, nullptr, M, w, nullptr, N, K, bias, y, stream)
                : launch_tiles<ElemBF16, 0, 1, false>(x, nullptr, M, w, nullptr, N, K, bias, y, stream);
    else
        e = vec ? launch_tiles<ElemBF16, 0, 0, true>(x, nullptr, M, w, nullptr, N, K, bias, y, stream)
                : launch_tiles<ElemBF16, 0, 0, false>(x, nullptr, M, w, nullptr, N, K, bias, y, stream);
    return e == hipSuccess ? 0 : -1;
}

}  // namespace w8a8
