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

namespace w8a8 {

namespace {

// ---------------------------------------------------------------------------
// A workgroup of WM x WN waves owns a BM x BN output tile; wave (wm, wn) owns
// (BM/WM) x (BN/WN) outputs, i.e. MI x NI tiles of 32 x 32 MFMA accumulators.
// K is staged BK bytes at a time through an NST-deep ring of LDS buffers.
// Five configurations:
//   xl:    384 x 256 tile (INT8 without GELU only), 4 x 2 waves of 96 x 128:
//          7 fragment reads per 12 MFMAs instead of 6 per 8, and 17% fewer
//          operand bytes per MFMA.  Its two 80 KB K stages fill the LDS, so
//          the tile's scales live in the ring once the K loop is done, and its
//          192 accumulators leave no room for a second set of fragments.
//   large: 256 x 256 tile, 4 x 2 waves (two per SIMD, so one wave's load issue,
//          LDS waits and barrier arrival overlap the other's MFMAs), each wave
//          64 x 128.
//   mid:   192 x 256 tile, 2 x 4 waves of 96 x 64: three quarters of a large
//          tile's work, for row counts where large tiles leave many CUs idle
//          in their last round (the ~2300-row text projection: 160 large
//          tiles or 208 mid ones on 256 CUs).
//   small: 128 x 128 tile, 2 x 2 waves of 64 x 64 (a 3-deep K ring for long
//          K loops).
//   tiny:  64 x 64 tile, 2 x 2 waves of 32 x 32.
// The launcher takes the largest of large/small/tiny whose tile count covers
// at least half of the CUs (a large tile on a CU still outruns four small
// ones; measured on the 2378-row text projection, the 2048^3 audio GEMM and
// 1024 x 1024 x 4096), then xl or mid instead of large where their rounds of
// tiles per CU cost less (see launch_tiles).
//
// * Operands go global -> LDS directly (buffer_load_dwordx4 ... lds): a wave
//   instruction moves 1 KB (64 lanes x 16 bytes); lane l lands at LDS offset
//   16*l of that KB and is given the global chunk that belongs there under the
//   swizzle below.  A lane's offsets are fixed per tile and the stage's K
//   position is a scalar offset; each load's lane offset is formed from two
//   per-lane values and wave-uniform terms as it is issued (stage_load_one).
// * An LDS row r (BK bytes = BK/16 chunks) stores logical K-chunk c at physical
//   chunk c ^ f(r).  A fragment read has lane l on row l % 32 at logical chunk
//   l / 32; with f(r) = (r ^ (r >> 3)) & 7 for 128-byte rows and (r >> 2) & 3
//   for 64-byte rows these reads are free of LDS bank conflicts on gfx950
//   (measured with the SQ_LDS_BANK_CONFLICT counter; LDS serves 256 bytes per
//   clock, so a conflict-free ds_read_b128 takes 4 clocks).
// * MFMA roles are transposed (A-operand = weight rows, B-operand = activation
//   rows) so the accumulator holds D[n][m]: each lane ends with 4 consecutive
//   output columns of one row.
// * One barrier per K stage; the MFMAs of the stage's last K sub-step are
//   issued after it, interleaved with the next stage's first fragment reads and
//   the loads that refill the buffer just released.  The order of MFMAs, LDS
//   reads and loads within a sub-step is fixed with sched_barrier.
// * Tile order is XCD-aware: workgroup b runs on XCD b % 8, so each XCD is
//   given a contiguous range of tiles, walked in groups of GROUP_M tile-rows
//   (1024 rows; 1536 for the 384-row tiles: the 32 tiles an XCD runs at once
//   then form a 4 x 8 block, which halved the 384 x 256 kernel's operand
//   fetches beyond L2 and made it 1.0-1.4% faster than 768-row groups).
// ---------------------------------------------------------------------------
constexpr int NUM_XCD = 8;
// The W8A8_* macros below are the tuned defaults; each can be overridden on
// the compiler command line to measure an alternative.
#ifndef W8A8_GROUP_ROWS
#define W8A8_GROUP_ROWS 1024
#endif
#ifndef W8A8_XL_GROUP_ROWS
#define W8A8_XL_GROUP_ROWS 1536
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

// Operand element types.  mfma() takes 16 bytes of weight row (A operand) and
// activation row (B operand) per lane and accumulates a 32 x 32 tile.
struct ElemI8 {
    static constexpr int BYTES = 1;
    typedef v16i acc_t;
    static __device__ __forceinline__ acc_t mfma(v4i w, v4i a, acc_t c) {
        return __builtin_amdgcn_mfma_i32_32x32x32_i8(w, a, c, 0, 0, 0);
    }
};

struct ElemBF16 {
    static constexpr int BYTES = 2;
    typedef v16f acc_t;
    static __device__ __forceinline__ acc_t mfma(v4i w, v4i a, acc_t c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(v8bf, w),
                                                       __builtin_bit_cast(v8bf, a), c, 0, 0, 0);
    }
};

template <int BM_, int BN_, int WM_, int WN_, int BK_, int NST_, int GROUP_ROWS_ = GROUP_ROWS>
struct Cfg {
    static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_, BK = BK_, NST = NST_;
    static constexpr int GROUP_M = GROUP_ROWS_ / BM;  // tile-rows per group of the raster
    static constexpr int WAVES = WM * WN;
    static constexpr int THREADS = WAVES * 64;
    static constexpr int TM = BM / WM, TN = BN / WN;  // outputs per wave
    static constexpr int MI = TM / 32;                 // 32-row MFMA tiles per wave along M
    static constexpr int NI = TN / 32;                 // 32-col MFMA tiles per wave along N
    static constexpr int NQ = MI + NI;                 // fragments per sub-step
    static constexpr int NMFMA = MI * NI;              // MFMAs per sub-step
    // Fragment registers: with room to spare the next sub-step's fragments go
    // to fresh registers early in the sub-step; where the accumulators leave
    // no room (RECYCLE) each is read into the register of the fragment it
    // replaces, right after that fragment's last MFMA.
    static constexpr bool RECYCLE = NMFMA * 16 + 2 * NQ * 4 > 200;
    static constexpr int CPR = BK / 16;                // 16-byte chunks per LDS row
    static constexpr int RPI = 64 / CPR;               // rows one 1-KB wave instruction fills
    static constexpr int STAGE = (BM + BN) * BK;       // bytes per stage (A tile then B tile)
    static constexpr int SUB = BK / 32;                // 32-byte MFMA sub-steps per stage
    static constexpr int LPW_A = BM / WAVES / RPI;     // A load instructions per wave per stage
    static constexpr int LPW_B = BN / WAVES / RPI;     // B load instructions per wave per stage
    static constexpr int NLOAD = LPW_A + LPW_B;
    static constexpr int WAVES_PER_SIMD = (WAVES + 3) / 4;
    // epilogue staging (see store_bf16)
    static constexpr int OUT_ROW = BN * 2 + 16;        // bytes per staged output row
    static constexpr int SROWS = BM / MI;              // staged rows per pass (= WM * 32)
    static constexpr int RCH = BN / 8;                 // 16-byte chunks per output row
    static constexpr int RPINS = 64 / RCH;             // output rows per copy-out instruction
    static constexpr int RPW = SROWS / WAVES;          // staged rows each wave copies per pass
    static constexpr int EPI_BYTES = SROWS * OUT_ROW;
    // LDS: K ring (from byte STAGE on also the staging area), then the tile's
    // row scales, column scales and bias as binary32.  Where the ring fills the
    // 160 KB of LDS, the scales go in the ring above the staging area instead:
    // they are then written only once the K loop is done with the ring.
    static constexpr int RING = NST * STAGE > STAGE + EPI_BYTES ? NST * STAGE : STAGE + EPI_BYTES;
    static constexpr int SCALE_BYTES = (BM + 2 * BN) * 4;
    static constexpr bool SCALES_IN_RING = RING + SCALE_BYTES > 160 * 1024;
    static constexpr int SCALE_OFF = SCALES_IN_RING ? STAGE + EPI_BYTES : RING;
    static constexpr int SMEM = SCALES_IN_RING ? RING : RING + SCALE_BYTES;
    static_assert(SMEM <= 160 * 1024 && SCALE_OFF + SCALE_BYTES <= SMEM, "LDS budget");
    static_assert(BM % (WAVES * RPI) == 0 && BN % (WAVES * RPI) == 0, "load split");
    static_assert(TM % 32 == 0 && TN % 32 == 0, "wave tile");
    static_assert(RPW % RPINS == 0 && 32 % RPW == 0, "copy-out rows per wave");
    static_assert(THREADS >= BM && THREADS >= BN, "scale staging");
    static_assert(GROUP_M >= 1, "raster group");
};

// Tile configurations: BM, BN, WM, WN, BK, NST[, raster group rows].
#ifndef W8A8_XL_CFG
#define W8A8_XL_CFG 384, 256, 4, 2, 128, 2, W8A8_XL_GROUP_ROWS
#endif
#ifndef W8A8_LARGE_CFG
#define W8A8_LARGE_CFG 256, 256, 4, 2, 128, 2
#endif
#ifndef W8A8_MID_CFG
#define W8A8_MID_CFG 192, 256, 2, 4, 128, 2
#endif
typedef Cfg<W8A8_XL_CFG> CfgXL;
typedef Cfg<W8A8_LARGE_CFG> CfgLarge;
#ifndef W8A8_SMALL_CFG
#define W8A8_SMALL_CFG 128, 128, 2, 2, 128, 2
#endif
typedef Cfg<W8A8_MID_CFG> CfgMid;
typedef Cfg<W8A8_SMALL_CFG> CfgSmall;
// small tiles with a 3-deep ring, for K loops of 32 stages or more (see launch_tiles)
typedef Cfg<128, 128, 2, 2, 128, 3> CfgSmallDeep;
typedef Cfg<64, 64, 2, 2, 128, 2> CfgTiny;

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
    // fragment reads: LDS byte offset of this lane's row in the wave's first
    // activation / weight sub-tile, and 16 x the physical chunk of its K-chunk
    // (lane >> 5) in that row; every other read adds compile-time constants
    uint32_t fa, fw, ga, gw;
    int wave, lane, wm, wn;
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
    // 128-byte rows: swz(r0 + rsub, pc) = pc ^ rsub ^ ((r0 >> 3) & 7) for r0 % 8 == 0;
    // 64-byte rows: swz(r0 + rsub, pc) = pc ^ ((rsub >> 2) & 3) for r0 % 16 == 0
    c.lx = C::BK == 128 ? 16u * (uint32_t)(pc ^ rsub) : 16u * (uint32_t)(pc ^ ((rsub >> 2) & 3));
    const int hi = (int)((unsigned)lane >> 5);
    const int ra = c.wm * C::TM + (lane & 31), rw = c.wn * C::TN + (lane & 31);
    c.fa = (uint32_t)(ra * C::BK);
    c.fw = (uint32_t)(C::BM * C::BK + rw * C::BK);
    c.ga = 16u * (uint32_t)swz<C::BK>(ra, hi);
    c.gw = 16u * (uint32_t)swz<C::BK>(rw, hi);
}

template <class C>
__device__ __forceinline__ void make_ctx(Ctx<C>& c, int64_t KB, int wave, int lane) {
    c.kb = (uint32_t)KB;
    c.wave = wave;
    c.lane = lane;
    c.wm = wave % C::WM;
    c.wn = wave / C::WM;
    lane_ctx<C>(c, lane);
}

// Load j (0 .. NLOAD-1) of one wave's share of a K stage: j < LPW_A loads A
// rows, the rest B rows.  The load covers tile rows r0 .. r0 + RPI - 1 (r0
// wave-uniform, a multiple of RPI); lane l takes row r0 + l / CPR, logical
// chunk l % CPR, which lands at LDS byte 16*l of the load's 1 KB, the physical
// chunk of the swizzle.  Its lane offset is row * KB + 16 * swz(row, chunk) =
// lrow + r0 * KB + (lx ^ 16 * ((r0 >> 3) & 7)) for 128-byte rows (the XOR term
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
    const uint32_t xr = C::BK == 128 ? 16u * ((r0 >> 3) & 7u) : 0u;
    const uint32_t voff = lrow + r0 * c.kb + (lx ^ xr);
    char* dst = lds_stage + (is_a ? 0 : C::BM * C::BK) + r0 * C::BK;
#if defined(__HIP_DEVICE_COMPILE__)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(c.rsrc[is_a ? 0 : 1], (lds_void*)dst, 16, voff, k0,
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
using Acc = typename E::acc_t[C::NI][C::MI];

// Fragment q of sub-step ks: q < MI -> activation sub-tile q, else weight
// sub-tile q - MI.  Lane l reads row l % 32 of the sub-tile at K-chunk
// ch = 2*ks + l/32, stored at physical chunk ch ^ f(row).  Sub-tile i starts
// 32*i rows further on, where f changes by 4*(i & 1) for 128-byte rows and not
// at all for 64-byte rows; so 16 * (ch ^ f(row)) = g ^ (32*ks) ^ (64*(i & 1))
// (128-byte rows) with g = 16 * ((l/32) ^ f(first row)) from the context:
// one XOR-add per read.  ga, gw are that g for the two operands.
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
    const uint32_t k = (uint32_t)(32 * ks) ^ (C::BK == 128 ? 64u * (uint32_t)(i & 1) : 0u);
    const uint32_t off = ((is_a ? fb.ga : fb.gw) ^ k) + (is_a ? fb.fa : fb.fw);
    const v4i v = *reinterpret_cast<const v4i*>(lds_stage + off + i * 32 * C::BK);
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
    const int valid = tail - (32 * ks + 16 * (c.lane >> 5));
#pragma unroll
    for (int q = 0; q < C::MI; ++q) f.a[q] = keep_bytes(f.a[q], valid);
#pragma unroll
    for (int q = 0; q < C::NI; ++q) f.w[q] = keep_bytes(f.w[q], valid);
}

template <class C, class E>
__device__ __forceinline__ void mfma_one(Acc<C, E>& acc, const Frags<C>& f, int j) {
    const int ni = j / C::MI, mi = j % C::MI;
    acc[ni][mi] = E::mfma(f.w[ni], f.a[mi], acc[ni][mi]);
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
    if constexpr (C::RECYCLE) {
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
#pragma unroll
    for (int ks = 0; ks + 1 < C::SUB; ++ks) {
        if (MAYBE_TAIL && tail < C::BK) mask_tail<C>(cur, c, ks, tail);
        mfma_step<C, E, true, false>(c, acc, cur, buf, ks + 1, nullptr, 0);
    }
    char* next_buf = smem + ((kt + 1) % C::NST) * C::STAGE;
    if (MAYBE_TAIL && tail < C::BK) mask_tail<C>(cur, c, C::SUB - 1, tail);
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

// Epilogue.  acc[ni][mi][i] holds D[n][m] for m = m0 + wm*TM + mi*32 +
// (lane & 31) and n = n0 + wn*TN + ni*32 + 8*(i/4) + 4*(lane >> 5) + (i & 3):
// four consecutive columns per group of four registers.
//
// Stored straight from the accumulator layout, one wave instruction would
// touch 32 rows with 16 bytes each.  Instead the bf16 tile goes through LDS,
// in MI passes of BM/MI rows (pass p holds the rows of MFMA sub-tile mi = p),
// and is copied out so that each wave instruction writes whole tile rows
// (64 lanes x 16 bytes).  Staged rows are padded by 16 bytes: every LDS address
// is a per-lane base plus a compile-time offset, and the 16-byte row reads are
// free of bank conflicts.  `stage` must not overlap the K buffer that the next
// tile's first stage is being loaded into.  VEC_OUT: y rows are 16-byte
// aligned and N % 8 == 0, so every 16-byte chunk is stored whole; otherwise
// chunks are stored element by element.  b_l holds the bias, -0.0 where
// there is none.
template <class C, class E, int ACT, bool VEC_OUT>
__device__ __forceinline__ void store_bf16(const Acc<C, E>& acc, uint16_t* __restrict__ y, int64_t M,
                                           int64_t N, int64_t m0, int64_t n0, int wave, int wm,
                                           int wn, int lane, const float* sa_l, const float* sw_l,
                                           const float* b_l, char* stage) {
    const int half = lane >> 5;
    const int ncol = wn * C::TN + 4 * half;  // tile-local column of this lane's first group
    char* wbase = stage + (wm * 32 + (lane & 31)) * C::OUT_ROW + ncol * 2;
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
        float sam = 0.f;
        if constexpr (E::BYTES == 1) sam = sa_l[wm * C::TM + p * 32 + (lane & 31)];
#pragma unroll
        for (int ni = 0; ni < C::NI; ++ni) {
            v4f swv[4], bv[4];
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int cl = ncol + ni * 32 + 8 * g;
                if constexpr (E::BYTES == 1) swv[g] = *reinterpret_cast<const v4f*>(sw_l + cl);
                bv[g] = *reinterpret_cast<const v4f*>(b_l + cl);
            }
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                float v[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    if constexpr (E::BYTES == 1) {
                        const float t = (float)acc[ni][p][4 * g + e];  // nearest even
                        const float u = __fmul_rn(sam, swv[g][e]);
                        v[e] = __builtin_fmaf(t, u, bv[g][e]);
                    } else {
                        const float t = acc[ni][p][4 * g + e];
                        v[e] = __fadd_rn(t, bv[g][e]);
                    }
                }
                uint2 o = make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
                if (ACT == 1) {
                    // GELU-tanh of the bf16-rounded value, rounded to bf16 (gelu_bf16_rn)
                    o = make_uint2(gelu_bf16_rn(o.x & 0xffffu) | (gelu_bf16_rn(o.x >> 16) << 16),
                                   gelu_bf16_rn(o.y & 0xffffu) | (gelu_bf16_rn(o.y >> 16) << 16));
                }
                *reinterpret_cast<uint2*>(wbase + (ni * 32 + 8 * g) * 2) = o;
            }
            // register-tight tiles: keep the next column group's scale reads
            // from being hoisted next to this one's (they would spill)
            if constexpr (C::RECYCLE) __builtin_amdgcn_sched_barrier(0);
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
#pragma unroll
            for (int i = 0; i < NI_OUT; ++i) {
                if (row + i * C::RPINS >= M) continue;
                uint16_t* pr = gbase + i * C::RPINS * N;
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    if (n0 + 8 * cc + e < N)
                        pr[e] = (uint16_t)(((uint32_t)d[i][e >> 1] >> (16 * (e & 1))) & 0xffffu);
            }
        }
        lds_barrier();  // the staging area is free again
    };
    static_assert(C::MI >= 1 && C::MI <= 4, "epilogue passes");
    pass(std::integral_constant<int, 0>{});
    if constexpr (C::MI > 1) pass(std::integral_constant<int, 1>{});
    if constexpr (C::MI > 2) pass(std::integral_constant<int, 2>{});
    if constexpr (C::MI > 3) pass(std::integral_constant<int, 3>{});
}

template <class C>
__device__ __forceinline__ void store_i32(const Acc<C, ElemI8>& acc, int32_t* __restrict__ out,
                                          int64_t M, int64_t N, int64_t m0, int64_t n0, int wm,
                                          int wn, int lane) {
    const int ncol = wn * C::TN + 4 * (lane >> 5);
#pragma unroll
    for (int mi = 0; mi < C::MI; ++mi) {
        const int ml = wm * C::TM + mi * 32 + (lane & 31);
        if (m0 + ml >= M) continue;
        int32_t* rowp = out + (m0 + ml) * N + n0 + ncol;
#pragma unroll
        for (int ni = 0; ni < C::NI; ++ni)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                if (n0 + ncol + ni * 32 + 8 * g >= N) continue;
                v4i v = {acc[ni][mi][4 * g], acc[ni][mi][4 * g + 1], acc[ni][mi][4 * g + 2],
                         acc[ni][mi][4 * g + 3]};
                *reinterpret_cast<v4i*>(rowp + ni * 32 + 8 * g) = v;
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
                const uint16_t* __restrict__ bias, void* __restrict__ out) {
    constexpr int BM = C::BM, BN = C::BN, BK = C::BK, NST = C::NST, MI = C::MI;
    constexpr bool SCALES = !OUT_I32 && E::BYTES == 1;
    // K ring (from byte STAGE on, also the output staging area) and the
    // tile's row scales, column scales and bias (as binary32).  All of it is
    // one LDS object: with several, the compiler can no longer tell the
    // fragment reads from the in-flight direct-to-LDS loads and waits for
    // every load.
    __shared__ __attribute__((aligned(1024))) char smem[C::SMEM];
    float* sa_l = reinterpret_cast<float*>(smem + C::SCALE_OFF);
    float* sw_l = sa_l + BM;
    float* b_l = sw_l + BN;
    const char* ab = static_cast<const char*>(a);
    const char* wb = static_cast<const char*>(w);
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave % C::WM, wn = wave / C::WM;
    const int64_t tm = (M + BM - 1) / BM, tn = (N + BN - 1) / BN, total = tm * tn;
    const int64_t KB = K * E::BYTES;
    // INT8 rows are whole stages; a BF16 row may end inside its last stage
    const int KT = E::BYTES == 1 ? (int)(KB / BK) : (int)((KB + BK - 1) / BK);
    const int tail = (int)(KB - (int64_t)(KT - 1) * BK);  // valid bytes in the last stage
    int64_t t = blockIdx.x, tile_m, tile_n;
    tile_of<C>(t, tm, tn, tile_m, tile_n);
    int64_t m0 = tile_m * BM, n0 = tile_n * BN;
    Ctx<C> c;
    make_ctx<C>(c, KB, wave, lane);
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
    float nsa = 0.f, nsw = 0.f;
    uint32_t nb = 0;
    auto load_scales = [&](int64_t m0_, int64_t n0_) {
        if (SCALES) nsa = sa[m0_ + tid < M ? m0_ + tid : M - 1];
        if (!OUT_I32) {
            const int64_t n = n0_ + tid < N ? n0_ + tid : N - 1;
            if (SCALES) nsw = sw[n];
            if constexpr (C::SCALES_IN_RING) {
                // loaded during the last K stage: a branch on the pointer
                // would make the wave wait for it there
                const int64_t cnt = N - n0_ < BN ? N - n0_ : BN;
                nb = load_bias_bits(bias ? bias + n0_ : nullptr, (int)cnt, (int)(n - n0_));
            } else {
                nb = bias ? (uint32_t)bias[n] : 0u;
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
            if (SCALES) asm volatile("" ::"v"(nsa), "v"(nsw));
            if (!OUT_I32) asm volatile("" ::"v"(nb));
        }
        if (SCALES && et < BM) sa_l[et] = nsa;
        if (!OUT_I32 && et < BN) {
            if (SCALES) sw_l[et] = nsw;
            b_l[et] = bf16_bits_to_float(bias ? nb : 0x8000u);  // -0.0 without a bias
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
            for (int j = 0; j < MI; ++j) acc[i][j] = (typename E::acc_t){};
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
        if constexpr (C::SCALES_IN_RING) {
            put_scales();
            lds_barrier();
        }
        if (has_next) {
            tile_of<C>(t_next, tm, tn, tile_m, tile_n);
            m0n = tile_m * BM;
            n0n = tile_n * BN;
            if constexpr (!C::SCALES_IN_RING) load_scales(m0n, n0n);
            set_tile<C>(c, ab, wb, M, N, KB, m0n, n0n);
            stage_load<C>(c, 0, smem);  // next tile's stage 0 -> buffer 0
        }
        // The epilogue's lane addresses depend only on the lane, and hoisted out
        // of the tile loop they would stay live across the K loop; an opaque
        // copy of the lane index keeps them local to the epilogue.
        int elane = lane;
        asm volatile("" : "+v"(elane));
        if constexpr (OUT_I32 != 0) {
            store_i32<C>(acc, reinterpret_cast<int32_t*>(out), M, N, m0, n0, wm, wn, elane);
        } else {
            store_bf16<C, E, ACT, VEC_OUT>(acc, reinterpret_cast<uint16_t*>(out), M, N, m0, n0,
                                           wave, wm, wn, elane, sa_l, sw_l, b_l, smem + C::STAGE);
        }
        if (!has_next) break;
        // this tile's epilogue is done with the old values
        if constexpr (!C::SCALES_IN_RING) put_scales();
        wait_vm_lgkm0<0>();  // the next tile's stage 0 (and this tile's stores) are done ...
        __syncthreads();     // ... for every wave, and the staging area is free
        lane_ctx<C>(c, elane);
        for (int s = 1; s < NST; ++s)
            if (s < KT) stage_load<C>(c, s * BK, smem + s * C::STAGE);
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
                      hipStream_t stream) {
    const int64_t tiles = tile_count<C>(M, N);
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
                       dim3(C::THREADS), 0, stream, a, sa, M, w, sw, N, K, bias, out);
    return hipGetLastError();
}

// Tile choice.  Larger tiles move less data per MFMA, which is what sets the
// clock under the power cap; smaller ones only pay off when the large ones
// leave most CUs idle.  xl (1.5x the work of a large tile) is taken when it
// needs no more rounds of persistent tiles than large does (rounds x 1.5 <=
// large's rounds) and either K >= 8192 or there are at least 4 xl tiles per
// CU: measured 2-3% faster on the FFN up (24576 x 16384 x 4096, 16 tiles per
// CU) and down (K = 16384) projections and 3.5% faster on 24576 x 4096 x 4096
// and 12288 x 8192 x 4096 (4 tiles per CU); with 1 tile per CU it is not taken.
template <class E, int OUT_I32, int ACT, bool VEC_OUT>
hipError_t launch_tiles(const void* a, const float* sa, int64_t M, const void* w, const float* sw,
                        int64_t N, int64_t K, const uint16_t* bias, void* out,
                        hipStream_t stream) {
    const int cus = cu_count();
    if (cus <= 0) return hipErrorInvalidDevice;
    if constexpr (E::BYTES == 1 && ACT == 0) {
        const int64_t txl = tile_count<CfgXL>(M, N), tl = tile_count<CfgLarge>(M, N);
        const int64_t rounds_xl = (txl + cus - 1) / cus, rounds_l = (tl + cus - 1) / cus;
        if (2 * txl >= cus && 3 * rounds_xl <= 2 * rounds_l && (K >= 8192 || txl >= 4 * (int64_t)cus))
            return launch_cfg<CfgXL, E, OUT_I32, ACT, VEC_OUT>(a, sa, M, w, sw, N, K, bias, out,
                                                              cus, stream);
    }
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
    if (2 * tile_count<CfgSmall>(M, N) >= cus) {
        // A 3-deep ring keeps two stages of loads in flight: with one wave per
        // SIMD and 512 cycles of MFMAs per stage, the 2-deep ring's per-stage
        // load latency shows.  It pays on K loops of 32 stages or more
        // (2048 x 2048 x 2050 BF16: 33.7 -> 27.1 us; 512 x 4096 x 4096 INT8:
        // 22.4 -> 20.3 us) and costs 2-5% on 16 stages (2048^3 INT8); its
        // 96 KB of LDS leaves one workgroup per CU, so only where the tiles
        // take one round.
        if (K * E::BYTES >= 32 * CfgSmallDeep::BK && tile_count<CfgSmallDeep>(M, N) <= cus)
            return launch_cfg<CfgSmallDeep, E, OUT_I32, ACT, VEC_OUT>(a, sa, M, w, sw, N, K, bias,
                                                                     out, cus, stream);
        return launch_cfg<CfgSmall, E, OUT_I32, ACT, VEC_OUT>(a, sa, M, w, sw, N, K, bias, out, cus,
                                                             stream);
    }
    return launch_cfg<CfgTiny, E, OUT_I32, ACT, VEC_OUT>(a, sa, M, w, sw, N, K, bias, out, cus,
                                                        stream);
}

}  // namespace

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
