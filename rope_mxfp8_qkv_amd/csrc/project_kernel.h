// The pass-1 projection kernel, shared by the launchers in project*.hip (internal header).
//
// Pass 1 ([QKV-CTE] "Upstream behavior": O[S, I] = A[S, H] @ W[H, I] + bias; "Applies to /
// Pattern": every output tile accumulates over the whole contraction, then is dequantised,
// bias-added and stored; "Design 1)" step a: per-token sums of squares of the Q and K
// segments of the un-normalised output).
//
// gfx950 design
//  * Block tile 256 output channels x 256 tokens, 4 wavefronts (2 x 2), each 128 x 128 =
//    4 x 4 fragments of V_MFMA_SCALE_F32_32X32X64_F8F6F4 (fp32 accumulators, 256 AGPRs/lane).
//  * Roles are swapped with respect to O = A W: the MFMA "A" operand is the weight (rows =
//    output channels, its E8M0 block exponents feed the MFMA's A-scale directly) and the "B"
//    operand is the ROW_MX activation (B-scale = 2^0; the fp32 row scale is applied in the
//    epilogue).  The accumulator then holds, per lane, 4-channel runs of one token.
//  * Operand lane layout of the 32x32x64 MFMA (K = 64 bytes per row): lane group g = lane / 32
//    holds bytes [16g, 16g + 16) and [32 + 16g, 32 + 16g + 16) of row lane % 32; the exponent
//    of K-block b (32 bytes) of row m comes from lane m + 32 b, byte op_sel.
//  * Operands reach LDS by direct global->LDS DMA (no staging registers), both as pre-swizzled
//    16 KiB stage images, 1 KiB contiguous per wave instruction: the weight from its one-time
//    prepack, the activation from a per-call repack of its rows (which are only 4-byte aligned
//    in the packed [T, H + 4] layout, too little for 16-byte DMA).  Four LDS stage
//    buffers (4 x 32 KiB) let each stage be requested four K-steps before it is consumed; the
//    fragments of step s + 1 are read from LDS while the 16 MFMAs of step s run.  The DMAs are
//    issued from inline assembly with explicit vmcnt waits, because the compiler would
//    otherwise wait for every outstanding DMA before each LDS read.
//  * LDS image of a stage: 256 rows x 64 K-bytes, 16-byte chunk c of row r at chunk position
//    c ^ stage_swizzle(r): the 16 consecutive rows one ds_read_b128 serves at a logical chunk
//    land on 16 distinct 16-byte bank groups of a 256-byte window (and any 8 aligned rows on
//    8 distinct groups of a 128-byte window).
//  * Epilogue: x = acc * a_scale[token] * c[channel] + bias[channel] in fp32, sums of x^2 per
//    token over the Q and K columns (V excluded) written as one partial per 128 channels
//    (groups holding only V write none), bf16 round-to-nearest-even (V_CVT_PK_BF16_F32),
//    transposed through LDS so every global store is a coalesced 16-byte vector along a token
//    row.  A small second kernel adds the partials in a fixed order (deterministic, no atomics).
//  * Tile order and scheduling: one persistent block per CU.  The tiles are split into 8
//    contiguous ranges, one per XCD, walked in groups of 4 token tiles x all channel tiles;
//    a block claims tiles one at a time from its own XCD's range (an atomic counter), so the
//    tiles resident on one XCD at any time share activation rows and weight columns in its
//    L2, and it prefetches the next tile's first stages while the current tile's epilogue
//    runs.
#pragma once

#include <algorithm>
#include <type_traits>

#include "device_common.h"
#include "internal.h"

namespace qkvmx {

namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef uint32_t u32x2_a8 __attribute__((ext_vector_type(2), aligned(8)));
typedef uint32_t u32x4_a4 __attribute__((ext_vector_type(4), aligned(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kGroupM = 4;                         // token tiles per raster group
constexpr int kXcds = 8;
constexpr int kHwRegXccId = 20 | (31 << 11);        // s_getreg operand: XCC_ID, bits [31:0]
constexpr int kBufs = 4;                           // LDS stage buffers
constexpr int kBufferRsrcWord3 = 0x00020000;        // buffer descriptor word 3 (gfx9 family)
constexpr int kNonTemporal = 2;                    // buffer store cache policy: streaming
constexpr uint32_t kDropOffset = 0x80000000u;      // outside any descriptor range (<= 2^31 - 1)
// Unconditional stores ending an epilogue.  The next tile waits with vmcnt(kTailStores), i.e.
// for everything but those stores, which is its DMAs only if vector memory operations complete
// in issue order.  LLVM's AMDGPU memory-model documentation (AMDGPUUsage, memory model of the
// GFX9 family including GFX90A/GFX942) states that vector memory operations report completion
// to the wavefront in execution order, the exception being FLAT instructions that access LDS
// memory; the DMAs here are global (not FLAT) loads and the stores buffer stores.  The
// backend's own wait insertion relies on the same order (a load followed by two stores is
// waited for with vmcnt(2) before the load's value is used, as compiled for gfx950).
constexpr int kTailStores = 8;
constexpr int kDmaPerStage = 8;                    // per wave: 4 (weight) + 4 (activation)
                                                   // (+ 2 exponent DMAs every 4th stage)

struct ProjectArgs {
  const uint8_t* a_codes;
  int64_t a_stride;
  const uint8_t* a_scales;
  int64_t s_stride;
  const uint8_t* w_img;        // [NT][KS][16 KiB]
  const uint8_t* w_scales;     // [KS / 4][NT * 256][2] dwords
  const uint8_t* x_img;        // activation stage images [MT][KS][16 KiB] (workspace; ROW_MX)
  const uint8_t* x_scales;     // MX block-32 activations: exponent images [MT][KS / 4][256][2]
                               // dwords (workspace), the weight exponents' format
  const float* chan_scale;     // [I] or null
  const uint16_t* bias;        // [I] or null
  int64_t T, H, I, Iq, Ik;
  int64_t d;                   // head_dim (NBSd addressing)
  int KS;                      // K-stages of 64 bytes (multiple of 4)
  int tiles_m, tiles_n;
  uint16_t* out;
  float* ws;                   // [P][T][2] or null
  unsigned* ctr;               // [8] tile counters, one per XCD (zeroed by the repack kernel)
  // per-head qk-norm fused into the epilogue: gamma (and LayerNorm beta, may be null) of the Q
  // and K segments, bf16 [d] each; rotate-half tables fp32 [T, d] (null: no RoPE)
  const uint16_t* hq_gamma;
  const uint16_t* hk_gamma;
  const uint16_t* hq_beta;
  const uint16_t* hk_beta;
  float h_eps;
  const float* cos_tab;
  const float* sin_tab;
  // split contraction: work unit v is tile v / ksplit over K-stages [kz * ks_chunk,
  // min(KS, (kz + 1) * ks_chunk)), kz = v % ksplit; its fp32 accumulators go to plane kz of
  // part ([ksplit][T][I]), summed by split_reduce_kernel
  int ksplit;
  int ks_chunk;
  float* part;
};

__device__ __forceinline__ int lds_off(int row, int chunk) {
  return row * kStage + ((chunk ^ stage_swizzle(row)) << 4);
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const uint8_t*)(p);
}

// Global -> LDS DMA in the scalar-base form: lane L reads sbase + voff_L (+ the immediate
// offset) and writes LDS at M0 (+ the immediate offset) + 16 L (dwordx4) or + 4 L (dword).
// The wave-uniform part of every source address stays in SGPRs; the only vector operand is
// the lane's byte offset.
//
// 1 KiB block i (0..3) of a stage image: the immediate offset 1024 i is added to both the
// global and the LDS address, so M0 only carries the stage buffer (base + Q * kStageImage);
// the switch folds away once i is a constant.
template <int Q>
__device__ __forceinline__ void dma16_blk(uint32_t base, const uint8_t* sbase, uint32_t voff,
                                          int i) {
#define QKVMX_DMA_BLK(OFF)                                                                  \
  asm volatile("s_add_u32 m0, %0, %3\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2 offset:" #OFF \
               :: "s"(base), "v"(voff), "s"(sbase), "n"(Q * kStageImage) : "memory", "m0", "scc")
  switch (i) {
    case 0: QKVMX_DMA_BLK(0); break;
    case 1: QKVMX_DMA_BLK(1024); break;
    case 2: QKVMX_DMA_BLK(2048); break;
    default: QKVMX_DMA_BLK(3072); break;
  }
#undef QKVMX_DMA_BLK
}
// Dword DMA from a per-lane 64-bit address (lane L: 4 bytes from g_L to LDS lds + 4 L).
__device__ __forceinline__ void dma4g(uint32_t lds, const void* g) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dword %1, off"
               :: "s"(lds), "v"(g) : "memory", "m0");
}
// 16-byte DMA, scalar base + per-lane offset (lane L: 16 bytes from sbase + voff_L to LDS
// lds + 16 L).
__device__ __forceinline__ void dma16(uint32_t lds, const void* sbase, uint32_t voff) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2"
               :: "s"(lds), "v"(voff), "s"(sbase) : "memory", "m0");
}
__device__ __forceinline__ void dma4(uint32_t lds, const uint8_t* sbase, uint32_t voff) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dword %1, %2"
               :: "s"(lds), "v"(voff), "s"(sbase) : "memory", "m0");
}
// The lane index, computed afresh (V_MBCNT) where it is needed: as volatile asm it is neither
// merged with an earlier copy nor hoisted, so lane-derived values need no register (or spill
// slot) across the K-steps.
__device__ __forceinline__ int fresh_lane() {
  int r;
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(r));
  return r;
}

// v + (v of lane ^ 32): the two lane halves' partial sums combined.  V_PERMLANE32_SWAP with
// both operands v leaves, in every lane l, the pair (v[l % 32], v[l % 32 + 32]), so lane l and
// lane l ^ 32 add the same two values in the same order (identical results) with one VALU
// instruction instead of an LDS permute.
__device__ __forceinline__ float add_xor32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                  false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

template <int N>
__device__ __forceinline__ void wait_vm() {
  asm volatile("s_waitcnt vmcnt(%0)" :: "n"(N) : "memory");
}

// Instruction-group masks of __builtin_amdgcn_sched_group_barrier.
constexpr int kSchedMfma = 0x008, kSchedDsRead = 0x100;

// Token tile and channel tile of tile index `tile` in the grouped raster order: groups of
// kGroupM token tiles, walked channel tile by channel tile.
struct Tile {
  int tm, tn;
  int kz;          // K chunk (split contraction; 0 otherwise)
};
__device__ __forceinline__ Tile decode_tile(int tile, int tiles_m, int tiles_n) {
  const int group = tile / (kGroupM * tiles_n);
  const int first_m = group * kGroupM;
  const int gm = min(tiles_m - first_m, kGroupM);
  const int in_group = tile % (kGroupM * tiles_n);
  return Tile{first_m + in_group % gm, in_group / gm, 0};
}

// kMx: MX block-32 activations (E4M3 rows with one E8M0 exponent per 32 elements).  Their
// exponents, re-laid per call in the weight exponents' format, feed the MFMA's B-scale as the
// weight's feed the A-scale, and the epilogue has no row scale.
// kHead: 0 = plain epilogue with the segment sums of squares; 1 / 2 = per-head RMS_NORM /
// LAYER_NORM of the Q and K heads fused into the epilogue (head_dim 64 or 128, segments
// multiples of 128 channels, no channel scale, no sums), with rotate-half RoPE when kRope.
// kSplit: split contraction (work units = tile x K chunk); the epilogue only stores the raw
// fp32 accumulators of its chunk (scales, bias, rounding and sums are split_reduce_kernel's).
template <bool kChanScale, bool kBias, bool kNbsd, bool kMx, int kHead = 0, bool kRope = false,
          bool kSplit = false>
__global__ void __launch_bounds__(kThreads, 1) project_kernel(const ProjectArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t lds_w[kBufs][kStageImage];
  __shared__ __attribute__((aligned(16))) uint8_t lds_x[kBufs][kStageImage];
  __shared__ __attribute__((aligned(16))) uint8_t lds_sc[2][kTileN * 8];
  // MX: activation exponents of a superstep (2 ring slots, the layout of lds_sc)
  __shared__ __attribute__((aligned(16))) uint8_t lds_xsc[kMx ? 2 : 1][kMx ? kTileM * 8 : 16];
  // epilogue operands, double-buffered (the next tile's arrive while the current tile's are
  // in use): channel scale and row scale (fp32) and the bias, DMA-copied as raw bf16 pairs and
  // widened to fp32 at the start of the tile
  __shared__ __attribute__((aligned(16))) float lds_cs[2][kTileN];
  __shared__ __attribute__((aligned(16))) float lds_sa[2][kTileM];
  __shared__ __attribute__((aligned(16))) uint32_t lds_braw[2][kTileN / 2];
  __shared__ __attribute__((aligned(16))) float lds_bias[2][kTileN];
  // per-head qk-norm: gamma of the Q and the K segment, then their LayerNorm beta (0 when
  // absent), widened to fp32 once per kernel (head_dim <= 128; every head of a segment shares
  // them, so each epilogue pass reads them from LDS instead of global memory)
  __shared__ __attribute__((aligned(16))) float lds_hgb[kHead ? 4 : 1][kHead ? 128 : 4];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform, kept in SGPRs
  const int wn = wave & 1;        // channel half of the block tile
  const int wm = wave >> 1;       // token half

  // ---- tile scheduler ----
  // The tiles are split into 8 contiguous ranges, one per XCD (grouped raster order inside
  // each).  A block claims its tiles one at a time from the counter of the XCD it runs on
  // (read from the XCC_ID register), so the tiles in flight on an XCD always form a compact
  // window that shares operand stage images in that XCD's L2; once that range is used up it
  // takes tiles from the other XCDs' ranges.  Thread 0 claims; the tile id reaches the block
  // through LDS.
  __shared__ int lds_tile[2];
  const int ntiles = a.tiles_m * a.tiles_n * (kSplit ? a.ksplit : 1);
  auto decode = [&](int v) -> Tile {
    if (!kSplit) return decode_tile(v, a.tiles_m, a.tiles_n);
    Tile u = decode_tile(v / a.ksplit, a.tiles_m, a.tiles_n);
    u.kz = v % a.ksplit;
    return u;
  };
  const int per = ntiles / kXcds, rem = ntiles % kXcds;
  const int my_xcd = __builtin_amdgcn_s_getreg(kHwRegXccId) & (kXcds - 1);
  auto range_first = [&](int x) { return x < rem ? x * (per + 1) : rem * (per + 1) + (x - rem) * per; };
  auto range_count = [&](int x) { return per + (x < rem ? 1 : 0); };
  // tile for ticket k of this XCD's counter, else the first one left in another range (-1:
  // none left anywhere); thread 0 only
  auto claim = [&](int k) -> int {
    if (k < range_count(my_xcd)) return range_first(my_xcd) + k;
    for (int d = 1; d < kXcds; ++d) {
      const int x = (my_xcd + d) & (kXcds - 1);
      const int kx = (int)atomicAdd(&a.ctr[x], 1u);
      if (kx < range_count(x)) return range_first(x) + kx;
    }
    return -1;
  };
  if (tid == 0) lds_tile[0] = claim((int)atomicAdd(&a.ctr[my_xcd], 1u));
  if (kHead != 0) {
    for (int i = tid; i < 4 * 128; i += kThreads) {
      const int which = i >> 7, j = i & 127;
      const uint16_t* src = which == 0 ? a.hq_gamma : which == 1 ? a.hk_gamma
                          : which == 2 ? a.hq_beta : a.hk_beta;
      lds_hgb[which][j] = (src && j < a.d) ? bf16_to_f32(src[j]) : 0.0f;
    }
  }
  __syncthreads();
  const int first_tile = __builtin_amdgcn_readfirstlane(lds_tile[0]);
  if (first_tile < 0) return;             // the whole block, nothing left
  Tile t = decode(first_tile);

  // ---- DMA sources of the current tile (wave-uniform bases, in SGPRs) ----
  // weight: wave w copies 1 KiB blocks 4 w .. 4 w + 3 of each 16 KiB stage image;
  // exponents: each wave copies 512 bytes (two dword DMAs) of the 2 KiB per superstep;
  // activation: same scheme as the weight, from the per-call stage images; MX exponents: as
  // the weight's, from their per-call images
  const uint32_t wdst = lds_addr(&lds_w[0][0]) + wave * 4096;
  const uint32_t xdst = lds_addr(&lds_x[0][0]) + wave * 4096;
  const uint32_t sdst = lds_addr(&lds_sc[0][0]) + wave * 512;
  const uint32_t xsdst = lds_addr(&lds_xsc[0][0]) + wave * 512;
  const int64_t s_step = (int64_t)a.tiles_n * kTileN * 2 * 4;       // bytes per superstep
  const int64_t xs_step = (int64_t)kTileM * 2 * 4;                  // MX: per superstep
  const uint8_t* wbase;
  const uint8_t* xbase;
  const uint8_t* sbase;
  const uint8_t* xsbase;
  auto set_sources = [&](Tile u) {
    wbase = a.w_img + ((int64_t)u.tn * a.KS) * kStageImage + wave * 4096;
    sbase = a.w_scales + ((int64_t)u.tn * kTileN * 2) * 4 + wave * 512;
    xbase = a.x_img + ((int64_t)u.tm * a.KS) * kStageImage + wave * 4096;
    if (kMx) xsbase = a.x_scales + (int64_t)u.tm * (a.KS / 4) * xs_step + wave * 512;
    if (kSplit) {                 // the unit's K chunk starts ks0 stages (ks0 / 4 supersteps) on
      const int64_t ks0 = (int64_t)u.kz * a.ks_chunk;
      wbase += ks0 * kStageImage;
      xbase += ks0 * kStageImage;
      sbase += (ks0 / 4) * s_step;
      if (kMx) xsbase += (ks0 / 4) * xs_step;
    }
  };
  set_sources(t);

  // DMA of stage t (t % 4 == Q) into buffer Q; a stage opening a superstep also brings that
  // superstep's exponents into ring slot (t / 4) % 2.
  auto issue = [&](auto q_c, int t) __attribute__((always_inline)) {
    constexpr int Q = decltype(q_c)::value;
    const uint32_t lv = fresh_lane();
    const uint32_t voff16 = lv * 16, voff4 = lv * 4;
    if (Q == 0) {
      const int64_t sup = t >> 2;
      const uint32_t slot = sdst + (uint32_t)(sup & 1) * 2048;
      dma4(slot, sbase + sup * s_step, voff4);
      dma4(slot + 256, sbase + sup * s_step + 256, voff4);
      if (kMx) {
        const uint32_t xslot = xsdst + (uint32_t)(sup & 1) * 2048;
        dma4(xslot, xsbase + sup * xs_step, voff4);
        dma4(xslot + 256, xsbase + sup * xs_step + 256, voff4);
      }
    }
    const uint8_t* const wsrc_t = wbase + (int64_t)t * kStageImage;
    const uint8_t* const xsrc_t = xbase + (int64_t)t * kStageImage;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      dma16_blk<Q>(wdst, wsrc_t, voff16, i);
      dma16_blk<Q>(xdst, xsrc_t, voff16, i);
    }
  };

  // DMA of tile u's epilogue operands into operand buffer e (one dword per lane, indices
  // clamped to the last row / channel): wave w brings the row scales of tokens 64 w ..
  // 64 w + 63 and the channel scales of channels 64 w .. 64 w + 63; waves 0 and 1 bring the
  // 128 bf16 pairs of the tile's bias.
  auto issue_ops = [&](Tile u, int e) {
    const int lv = fresh_lane();
    if (!kMx) {
      const int64_t m = min((int64_t)u.tm * kTileM + wave * 64 + lv, a.T - 1);
      dma4g(lds_addr(&lds_sa[e][wave * 64]), a.a_scales + m * a.s_stride);
    }
    if (kChanScale) {
      const int64_t n = min((int64_t)u.tn * kTileN + wave * 64 + lv, a.I - 1);
      dma4g(lds_addr(&lds_cs[e][wave * 64]), a.chan_scale + n);
    }
    if (kBias && wave < 2) {
      const int64_t n2 = min((int64_t)u.tn * kTileN + 2 * (wave * 64 + lv), a.I - 2);
      dma4g(lds_addr(&lds_braw[e][wave * 64]), a.bias + n2);
    }
  };

  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  using I3 = std::integral_constant<int, 3>;
  using Yes = std::true_type;
  using No = std::false_type;
  using W40 = std::integral_constant<int, 2 * kDmaPerStage>;
  using W20 = std::integral_constant<int, kDmaPerStage>;
  using W0 = std::integral_constant<int, 0>;
  using WN = std::integral_constant<int, -1>;
  using Z = std::true_type;                       // step starts the accumulators from zero
  using NZ = std::false_type;

  // lane-derived LDS offsets of the K-steps, recomputed at the start of every tile (from a
  // fresh lane index) so that none of them is live across the epilogue
  int rw0, rw1, rx0, rx1, rsc, rxs;
  uint32_t kvoff16;
  auto set_lane_offsets = [&]() {
    const int lv = fresh_lane();
    const int g = lv >> 5;
    const int fr = lv & 31;             // fragment row of this lane
    const int w_row0 = wn * 128 + fr;   // + 32 cf
    const int x_row0 = wm * 128 + fr;   // + 32 tf
    // the two 16-byte halves a lane feeds to the MFMA: chunks g and 2 + g of its row; rows
    // 32 f apart share the swizzle, so fragment f sits 32 * 64 * f bytes further on
    rw0 = lds_off(w_row0, g); rw1 = lds_off(w_row0, 2 + g);
    rx0 = lds_off(x_row0, g); rx1 = lds_off(x_row0, 2 + g);
    rsc = (w_row0 * 2 + g) * 4;         // + 32 * 8 cf: this lane's exponent dword
    rxs = (x_row0 * 2 + g) * 4;         // + 32 * 8 tf: MX, this lane's activation exponents
    kvoff16 = lv * 16;
  };

  v16f acc[4][4];
  v8i wf[2][4], xf[2][4];
  uint32_t sc[2][4], xs[2][4];
  auto fload = [&](int buf, v8i (&wd)[4], v8i (&xd)[4]) {
#pragma unroll
    for (int f = 0; f < 4; ++f) {
      const uint4 p0 = *reinterpret_cast<const uint4*>(&lds_w[buf][rw0 + 2048 * f]);
      const uint4 p1 = *reinterpret_cast<const uint4*>(&lds_w[buf][rw1 + 2048 * f]);
      wd[f] = v8i{(int)p0.x, (int)p0.y, (int)p0.z, (int)p0.w,
                  (int)p1.x, (int)p1.y, (int)p1.z, (int)p1.w};
      const uint4 q0 = *reinterpret_cast<const uint4*>(&lds_x[buf][rx0 + 2048 * f]);
      const uint4 q1 = *reinterpret_cast<const uint4*>(&lds_x[buf][rx1 + 2048 * f]);
      xd[f] = v8i{(int)q0.x, (int)q0.y, (int)q0.z, (int)q0.w,
                  (int)q1.x, (int)q1.y, (int)q1.z, (int)q1.w};
    }
  };
  auto sload = [&](int slot, uint32_t (&sd)[4]) {
#pragma unroll
    for (int cf = 0; cf < 4; ++cf)
      sd[cf] = *reinterpret_cast<const uint32_t*>(&lds_sc[slot][rsc + 256 * cf]);
  };
  auto xsload = [&](int slot, uint32_t (&xd)[4]) {
    if (kMx) {
#pragma unroll
      for (int tf = 0; tf < 4; ++tf)
        xd[tf] = *reinterpret_cast<const uint32_t*>(&lds_xsc[slot][rxs + 256 * tf]);
    }
  };

  // ---- software pipeline over K-steps of 64 bytes ----
  // Step s: fragments of stage s are in registers [s & 1].  The step requests stage s + 4
  // into the buffer stage s occupied (every wave read stage s's fragments during step s - 1,
  // before the barrier that ended it) while it issues its 16 MFMAs and reads stage s + 1's
  // fragments (and, on the last step of a superstep, the next superstep's exponents).  It
  // ends by waiting for its own DMA of stage s + 2 (the two most recent DMA groups, of stages
  // s + 3 and s + 4, may stay in flight) and a barrier, after which stage s + 2 is complete in
  // LDS for all waves.  Each stage thus has three steps to arrive.
  //
  // One K-step is 16 issue slots, each one MFMA followed by one fragment read for the next
  // step and (in the first slots) one DMA request, separated by hard scheduling barriers: the
  // DMAs of the four wavefronts then trickle out one per MFMA instead of arriving at the
  // address unit as one burst after the barrier, and every MFMA has independent work behind it.
  const int KS = a.KS;
  auto step = [&](auto q_c, int s, auto issue_c, auto wait_c, auto zero_c)
                  __attribute__((always_inline)) {
    constexpr int q = decltype(q_c)::value;        // step within the 256-K superstep
    constexpr bool from_zero = decltype(zero_c)::value;   // first K-step: accumulators start at 0
    constexpr int p = q & 1;
    constexpr bool do_issue = decltype(issue_c)::value;
    constexpr int nwait = decltype(wait_c)::value;
    constexpr int nb = (q + 1) & (kBufs - 1);      // buffer of stage s + 1 (s % 4 == q)
    const int t = s + 4;                           // stage requested by this step
    const uint8_t* const wsrc_t = wbase + (int64_t)t * kStageImage;
    const uint8_t* const xsrc_t = xbase + (int64_t)t * kStageImage;
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const int cf = k >> 2, tf = k & 3;
      acc[cf][tf] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
          wf[p][cf], xf[p][tf], from_zero ? v16f{} : acc[cf][tf], 0, 0, q, (int)sc[0][cf],
          kMx ? q : 0, kMx ? (int)xs[0][tf] : 0x7F7F7F7F);
      // fragment k / 2 of stage s + 1: even k -> weight fragment, odd k -> activation fragment
      const int f = k >> 2, half = (k >> 1) & 1;
      if ((k & 1) == 0) {
        const uint4 v = *reinterpret_cast<const uint4*>(&lds_w[nb][(half ? rw1 : rw0) + 2048 * f]);
        if (half == 0) { wf[p ^ 1][f][0] = (int)v.x; wf[p ^ 1][f][1] = (int)v.y; wf[p ^ 1][f][2] = (int)v.z; wf[p ^ 1][f][3] = (int)v.w; }
        else { wf[p ^ 1][f][4] = (int)v.x; wf[p ^ 1][f][5] = (int)v.y; wf[p ^ 1][f][6] = (int)v.z; wf[p ^ 1][f][7] = (int)v.w; }
      } else {
        const uint4 v = *reinterpret_cast<const uint4*>(&lds_x[nb][(half ? rx1 : rx0) + 2048 * f]);
        if (half == 0) { xf[p ^ 1][f][0] = (int)v.x; xf[p ^ 1][f][1] = (int)v.y; xf[p ^ 1][f][2] = (int)v.z; xf[p ^ 1][f][3] = (int)v.w; }
        else { xf[p ^ 1][f][4] = (int)v.x; xf[p ^ 1][f][5] = (int)v.y; xf[p ^ 1][f][6] = (int)v.z; xf[p ^ 1][f][7] = (int)v.w; }
      }
      if (do_issue) {
        if (k < 8) {
          const int i = k >> 1;
          if ((k & 1) == 0)
            dma16_blk<q>(wdst, wsrc_t, kvoff16, i);
          else
            dma16_blk<q>(xdst, xsrc_t, kvoff16, i);
        } else if (q == 0 && (k == 8 || k == 9)) {
          const int64_t sup = t >> 2;
          const uint32_t slot = sdst + (uint32_t)(sup & 1) * 2048;
          dma4(slot + (k - 8) * 256, sbase + sup * s_step + (k - 8) * 256, kvoff16 >> 2);
        } else if (kMx && q == 0 && (k == 10 || k == 11)) {
          const int64_t sup = t >> 2;
          const uint32_t xslot = xsdst + (uint32_t)(sup & 1) * 2048;
          dma4(xslot + (k - 10) * 256, xsbase + sup * xs_step + (k - 10) * 256, kvoff16 >> 2);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    if (q == 3) {
      sload(((s >> 2) + 1) & 1, sc[1]);
      xsload(((s >> 2) + 1) & 1, xs[1]);
#pragma unroll
      for (int cf = 0; cf < 4; ++cf) sc[0][cf] = sc[1][cf];
      if (kMx) {
#pragma unroll
        for (int tf = 0; tf < 4; ++tf) xs[0][tf] = xs[1][tf];
      }
    }
    if (nwait >= 0) wait_vm<(nwait < 0 ? 0 : nwait)>();
    __syncthreads();
  };

  // ---- epilogue of tile u (operands in buffer e), through stage buffer 3 ----
  // x = acc * a_scale * c + bias (fp32) -> sums of squares from the fp32 values, bf16.  Four
  // passes of 32 tokens: each wave packs its 32 x 128 bf16 block into an 8 KiB LDS area
  // (token rows of 256 bytes, 16-byte chunk j of row r at chunk position j ^ (r & 15), its two
  // 8-byte halves swapped when bit 4 of r is set, so the 32 rows of one 8-byte store phase hit
  // distinct banks), reads it back row-contiguous (16 lanes per row, 4 rows per instruction,
  // all eight reads in flight before their stores) and stores 16-byte vectors.  Streaming
  // (non-temporal) stores: the output is not re-read by this kernel, and keeping it out of L2
  // leaves L2 to the operand stage images that neighbouring tiles share.
  // With `more`, pass p (p < 3) also requests the next tile's stage p and pass 3 its epilogue
  // operands, so the address unit works through them while the passes compute instead of
  // receiving them as one burst.  Pass 3 ends with exactly kTailStores unconditional stores
  // per wave after its last DMA (vector memory operations complete in issue order), so the
  // next tile only waits for the DMAs, not for those stores.
  auto epilogue = [&](Tile u, int e, bool more, Tile nxt) __attribute__((always_inline)) {
    // lane-derived addresses are recomputed here from a fresh lane index, so the compiler
    // cannot hoist them out of the tile loop and keep them live through the K-steps
    const int el = fresh_lane();
    const int g = el >> 5, fr = el & 31;
    uint8_t* const otile = (wm == 0 ? &lds_w[3][0] : &lds_x[3][0]) + wn * 8192;
    const int64_t m0 = (int64_t)u.tm * kTileM, n0 = (int64_t)u.tn * kTileN;
    const int jc = el & 15;
    const int64_t ch = n0 + wn * 128 + jc * 8;
    const bool ch_ok = ch < a.I;
    // The tile's output through a buffer descriptor (raw, stride 0); the per-store step is one
    // token row.  BSD [T, I]: the descriptor's range ends where the output array ends, so
    // stores to token rows >= T fall outside it and the hardware's range check drops them (no
    // per-store predicate); in-tile offsets are < 256 * I * 2, which the host keeps below 2^31.
    // NBSd [I / d, T, d]: a row >= T of one head would alias the next head's first rows, so
    // invalid stores get an offset of 2^31, beyond every range the descriptor can hold.
    __amdgpu_buffer_rsrc_t orsrc;
    uint32_t row_bytes, lane_off;
    int rows_left = 0;             // NBSd: this lane's valid token rows (0 for channels >= I)
    if (!kNbsd) {
      const int64_t out_left = ((a.T - m0) * a.I - n0) * 2;
      orsrc = __builtin_amdgcn_make_buffer_rsrc(
          a.out + m0 * a.I + n0, (short)0, (int)(uint32_t)min(out_left, (int64_t)0x7FFFFFFF),
          kBufferRsrcWord3);
      row_bytes = (uint32_t)a.I * 2;
      lane_off = (uint32_t)(wm * 128 + (el >> 4)) * row_bytes + (uint32_t)(wn * 128 + jc * 8) * 2;
    } else {
      // element (token t, channel c) at ((c / d) * T + t) * d + c % d; base = the tile's first
      // head hb at token m0
      // channels < I < 2^22 and d < 2^11: 32-bit unsigned division (a 64-bit one expands into
      // a long branchy sequence)
      const uint32_t dd = (uint32_t)a.d;
      const int64_t hb = (uint32_t)n0 / dd;
      const int64_t base_el = hb * a.T * a.d + m0 * a.d;
      const int64_t hh = (uint32_t)ch / dd, jj = ch - hh * a.d;
      const int64_t out_left = (a.T * a.I - base_el) * 2;
      orsrc = __builtin_amdgcn_make_buffer_rsrc(
          a.out + base_el, (short)0, (int)(uint32_t)min(out_left, (int64_t)0x7FFFFFFF),
          kBufferRsrcWord3);
      row_bytes = (uint32_t)a.d * 2;
      lane_off = (uint32_t)((((hh - hb) * a.T + wm * 128 + (el >> 4)) * a.d + jj) * 2);
      rows_left = ch_ok ? (int)min(max(a.T - (m0 + wm * 128 + (el >> 4)), (int64_t)0), (int64_t)256)
                        : 0;
    }
    float sq_q[4] = {0.f, 0.f, 0.f, 0.f}, sq_k[4] = {0.f, 0.f, 0.f, 0.f};
    // number of this wave's 8-channel groups (of 16) inside Q, and inside Q or K (uniform)
    const int64_t c0 = n0 + wn * 128;
    const int gq = __builtin_amdgcn_readfirstlane((int)min(max((a.Iq - c0) / 8, (int64_t)0), (int64_t)16));
    const int gqk = __builtin_amdgcn_readfirstlane((int)min(max((a.Iq + a.Ik - c0) / 8, (int64_t)0), (int64_t)16));
    // Per-head qk-norm pass (kHead != 0).  Lane (fr, g) holds, for its token, the 64 values
    // cf * 32 + rq * 8 + 4 g + i of the wave's 128 channels and its partner lane (fr, g ^ 1) the
    // other 64: with head_dim 128 the wave's channels are one head, with 64 they are two (cf 0-1
    // and 2-3), and in both cases the rotate-half partner j + d/2 of a value sits in the same
    // lane (cf + 2, resp. cf + 1).  A head's statistics are the lane's partial sums plus the
    // partner's; the segment of the wave (Q, K or neither) is wave-uniform because the segment
    // boundaries are multiples of 128 channels.
    const int hseg = kHead == 0 ? 0 : __builtin_amdgcn_readfirstlane(
        c0 < a.Iq ? 1 : (c0 < a.Iq + a.Ik ? 2 : 0));
    // The rotate-half table values of a pass (first half of each token row: its two halves
    // hold the same angle).  Loaded straight into the MFMA layout, every 16-byte load
    // instruction would touch 32 token rows (32 cache lines for 1 KiB); instead the two waves
    // that share a token half (wn = 0, 1) split the tables: wave wn DMA-copies the first 256
    // bytes of its 32 token rows of cos (wn = 0) or sin (wn = 1) into its own LDS output area,
    // 4 consecutive rows (8 cache lines) per instruction, token row r at r * 256 bytes with
    // 16-byte chunk c at position c ^ (r % 16); after a block barrier each wave reads both
    // tables from the pair's two areas in the MFMA layout (16 lanes: 16 rows, one chunk, every
    // bank once), and a second barrier frees the areas for the pass's packed x.  Pass 0's copy
    // goes out before the epilogue's first DMAs, pass tf + 1's after pass tf's read-back, ahead
    // of its 8 stores.  Only tiles with Q or K channels copy (a block-uniform test, so every
    // wavefront meets the same barriers).
    const bool tabs = kRope && kHead != 0 && n0 < a.Iq + a.Ik;
    float4 ct[2][4], st[2][4];       // entry [cf][rq]: positions cf * 32 + rq * 8 + 4 g .. + 3
    auto dma_tabs = [&](int tf) __attribute__((always_inline)) {
      // rows tok0 + r, r < 32, clamped to the last token; the scalar base is the pass's first
      // row (clamped), so the per-lane offsets stay below 32 rows
      const int64_t tok0 = m0 + wm * 128 + tf * 32;
      const int64_t base_tok = min(tok0, a.T - 1);
      const int last = (int)(a.T - 1 - base_tok);           // rows past it repeat it
      const float* const tab = (wn == 0 ? a.cos_tab : a.sin_tab) + base_tok * a.d;
      const uint32_t row_bytes_t = (uint32_t)a.d * 4;
      const int lv = fresh_lane();
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // this wave's reads of its area
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int r = 4 * k + (lv >> 4);
        const uint32_t voff = (uint32_t)min(r + (int)(tok0 - base_tok), last) * row_bytes_t +
                              ((uint32_t)((lv & 15) ^ (r & 15)) << 4);
        dma16(lds_addr(otile) + 1024 * k, tab, voff);
      }
    };
    auto tabs_from_lds = [&]() __attribute__((always_inline)) {
      const uint8_t* const pc = otile - wn * 8192;          // the pair's cos area (wn = 0)
      const uint8_t* const ps = pc + 8192;                  // its sin area (wn = 1)
#pragma unroll
      for (int cf = 0; cf < 2; ++cf)
#pragma unroll
        for (int rq = 0; rq < 4; ++rq) {
          if (cf == 0 || a.d == 128) {
            const int off = fr * 256 + (((cf * 8 + rq * 2 + g) ^ (fr & 15)) << 4);
            ct[cf][rq] = *reinterpret_cast<const float4*>(pc + off);
            st[cf][rq] = *reinterpret_cast<const float4*>(ps + off);
          }
        }
    };
    auto head_pass = [&](int tf, float sa) __attribute__((always_inline)) {
      float xv[4][4][4];
#pragma unroll
      for (int cf = 0; cf < 4; ++cf)
#pragma unroll
        for (int rq = 0; rq < 4; ++rq) {
          const float4 b4 = *reinterpret_cast<const float4*>(
              &lds_bias[e][wn * 128 + cf * 32 + rq * 8 + g * 4]);
          const float bs[4] = {b4.x, b4.y, b4.z, b4.w};
#pragma unroll
          for (int i = 0; i < 4; ++i) xv[cf][rq][i] = fmaf(acc[cf][tf][rq * 4 + i], sa, bs[i]);
        }
      if (hseg != 0) {
        const bool d64 = a.d == 64;
        const float inv_d = 1.0f / (float)a.d;
        // head sums of a per-cf quantity: entry h of the result belongs to head h (cf 2h, 2h+1)
        // when d = 64; with d = 128 both entries are the whole wave's sum
        auto head_sums = [&](const float (&pc)[4], float (&hs)[2]) __attribute__((always_inline)) {
          float h0 = pc[0] + pc[1], h1 = pc[2] + pc[3];
          if (!d64) { h0 = h0 + h1; h1 = h0; }
          hs[0] = add_xor32(h0);
          hs[1] = add_xor32(h1);
        };
        float mean[2] = {0.f, 0.f}, r[2];
        if (kHead == 2) {                                  // LayerNorm: centre first
          float p1[4];
#pragma unroll
          for (int cf = 0; cf < 4; ++cf) {
            float t = 0.f;
#pragma unroll
            for (int rq = 0; rq < 4; ++rq)
#pragma unroll
              for (int i = 0; i < 4; ++i) t += xv[cf][rq][i];
            p1[cf] = t;
          }
          float h1[2];
          head_sums(p1, h1);
          mean[0] = h1[0] * inv_d;
          mean[1] = h1[1] * inv_d;
        }
        float p2[4];
#pragma unroll
        for (int cf = 0; cf < 4; ++cf) {
          float t = 0.f;
#pragma unroll
          for (int rq = 0; rq < 4; ++rq)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const float c = xv[cf][rq][i] - mean[cf >> 1];
              t = fmaf(c, c, t);
            }
          p2[cf] = t;
        }
        float h2[2];
        head_sums(p2, h2);
        r[0] = 1.0f / sqrtf(h2[0] * inv_d + a.h_eps);
        r[1] = 1.0f / sqrtf(h2[1] * inv_d + a.h_eps);
        const float* gam = &lds_hgb[hseg - 1][0];
        const float* bet = &lds_hgb[hseg + 1][0];
#pragma unroll
        for (int cf = 0; cf < 4; ++cf)
#pragma unroll
          for (int rq = 0; rq < 4; ++rq) {
            // in-head position of the lane's 4 values
            const int p0 = (d64 ? (cf & 1) : cf) * 32 + rq * 8 + g * 4;
            const float4 g4 = *reinterpret_cast<const float4*>(gam + p0);
            const float gv[4] = {g4.x, g4.y, g4.z, g4.w};
            float bv[4] = {0.f, 0.f, 0.f, 0.f};
            if (kHead == 2) {
              const float4 b4 = *reinterpret_cast<const float4*>(bet + p0);
              bv[0] = b4.x; bv[1] = b4.y; bv[2] = b4.z; bv[3] = b4.w;
            }
#pragma unroll
            for (int i = 0; i < 4; ++i)
              xv[cf][rq][i] = fmaf((xv[cf][rq][i] - mean[cf >> 1]) * r[cf >> 1], gv[i], bv[i]);
          }
        if (kRope) {
          // rotate-half pairs (j, j + d/2) with the angle of position j of the token's row
          auto rot = [&](int lo, int hi, int rq, float4 c4, float4 s4) __attribute__((always_inline)) {
            const float c[4] = {c4.x, c4.y, c4.z, c4.w}, sn[4] = {s4.x, s4.y, s4.z, s4.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const float yl = xv[lo][rq][i], yh = xv[hi][rq][i];
              xv[lo][rq][i] = yl * c[i] - yh * sn[i];
              xv[hi][rq][i] = yh * c[i] + yl * sn[i];
            }
          };
          if (!d64) {
#pragma unroll
            for (int cf = 0; cf < 2; ++cf)
#pragma unroll
              for (int rq = 0; rq < 4; ++rq) rot(cf, cf + 2, rq, ct[cf][rq], st[cf][rq]);
          } else {
#pragma unroll
            for (int rq = 0; rq < 4; ++rq) {
              rot(0, 1, rq, ct[0][rq], st[0][rq]);
              rot(2, 3, rq, ct[0][rq], st[0][rq]);
            }
          }
        }
      }
#pragma unroll
      for (int cf = 0; cf < 4; ++cf)
#pragma unroll
        for (int rq = 0; rq < 4; ++rq) {
          const int chunk = cf * 4 + rq;
          u32x2_a8 o = {pack_bf16x2(xv[cf][rq][0], xv[cf][rq][1]),
                        pack_bf16x2(xv[cf][rq][2], xv[cf][rq][3])};
          *reinterpret_cast<u32x2_a8*>(otile + fr * 256 + ((chunk ^ (fr & 15)) << 4) +
                                       ((g ^ (fr >> 4)) & 1) * 8) = o;
        }
    };
    if (tabs) dma_tabs(0);
#pragma unroll
    for (int tf = 0; tf < 4; ++tf) {
      if (more) {
        if (tf == 0) issue(I0{}, 0);
        if (tf == 1) issue(I1{}, 1);
        if (tf == 2) issue(I2{}, 2);
      }
      if (tabs) {
        // this wave's copy has landed once at most the memory operations issued after it are
        // outstanding: pass 0: the next tile's stage 0 (2 dword + 8 16-byte DMAs); later passes:
        // the previous pass's 8 stores and this pass's stage (8 DMAs; none in pass 3)
        if (tf == 0) {
          if (more) asm volatile("s_waitcnt vmcnt(10)\n\ts_barrier" ::: "memory");
          else asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
        } else if (tf < 3) {
          if (more) asm volatile("s_waitcnt vmcnt(16)\n\ts_barrier" ::: "memory");
          else asm volatile("s_waitcnt vmcnt(8)\n\ts_barrier" ::: "memory");
        } else {
          asm volatile("s_waitcnt vmcnt(8)\n\ts_barrier" ::: "memory");
        }
        tabs_from_lds();
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
      }
      // this pass's operands to registers first, under one LDS wait: the row scale of this
      // lane's token and the bias (and channel scale) of its 16 channel quads
      const float sa = kMx ? 1.0f : lds_sa[e][wm * 128 + tf * 32 + fr];
      if (kHead != 0) {
        head_pass(tf, sa);
      } else {
#pragma unroll
      for (int cf = 0; cf < 4; ++cf) {
        float4 bq[1][4], cq[1][4];
#pragma unroll
        for (int rq = 0; rq < 4; ++rq) {
          const int cl = cf * 32 + rq * 8 + g * 4;
          bq[0][rq] = *reinterpret_cast<const float4*>(&lds_bias[e][wn * 128 + cl]);
          if (kChanScale) cq[0][rq] = *reinterpret_cast<const float4*>(&lds_cs[e][wn * 128 + cl]);
        }
#pragma unroll
        for (int rq = 0; rq < 4; ++rq) {
          const int cl = cf * 32 + rq * 8 + g * 4;        // 4 consecutive channels (local)
          const float bs[4] = {bq[0][rq].x, bq[0][rq].y, bq[0][rq].z, bq[0][rq].w};
          float cs[4] = {1.f, 1.f, 1.f, 1.f};
          if (kChanScale) {
            cs[0] = cq[0][rq].x; cs[1] = cq[0][rq].y; cs[2] = cq[0][rq].z; cs[3] = cq[0][rq].w;
          }
          // 0/1 masks of the Q and K segments (multiplies rather than branches keep the
          // epilogue straight-line code); segment boundaries are multiples of 16 channels, so
          // the 8-channel group cf * 32 + rq * 8 lies in one segment and the masks are
          // wave-uniform
          const int gi = cf * 4 + rq;
          const float mq = gi < gq ? 1.f : 0.f;
          const float mk = gi >= gq && gi < gqk ? 1.f : 0.f;
          float x[4];
#pragma unroll
          for (int i = 0; i < 4; ++i)
            x[i] = kChanScale ? acc[cf][tf][rq * 4 + i] * sa * cs[i] + bs[i]
                              : fmaf(acc[cf][tf][rq * 4 + i], sa, bs[i]);
          const float s2 = x[0] * x[0] + x[1] * x[1] + x[2] * x[2] + x[3] * x[3];
          sq_q[tf] = fmaf(mq, s2, sq_q[tf]);
          sq_k[tf] = fmaf(mk, s2, sq_k[tf]);
          const int chunk = cf * 4 + rq;
          u32x2_a8 o = {pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3])};
          *reinterpret_cast<u32x2_a8*>(otile + fr * 256 + ((chunk ^ (fr & 15)) << 4) +
                                       ((g ^ (fr >> 4)) & 1) * 8) = o;
        }
      }
      }
      if (tf == 3) {
        // every pass's sums are complete: the per-token partials go out before the last
        // DMAs, then the next tile's epilogue operands
        if (kHead == 0 && a.ws && n0 + wn * 128 < a.Iq + a.Ik) {   // channels overlap Q or K
          const int64_t p = (int64_t)u.tn * 2 + wn;
#pragma unroll
          for (int tq = 0; tq < 4; ++tq) {
            const float q = add_xor32(sq_q[tq]);
            const float k = add_xor32(sq_k[tq]);
            const int64_t tok = m0 + wm * 128 + tq * 32 + fr;
            if (g == 0 && tok < a.T) {
              u32x2_a8 o = {__float_as_uint(q), __float_as_uint(k)};
              *reinterpret_cast<u32x2_a8*>(a.ws + (p * a.T + tok) * 2) = o;
            }
          }
        }
        if (more) issue_ops(nxt, e ^ 1);
        __builtin_amdgcn_sched_barrier(0);
      }
      const uint32_t obyte = lane_off + (uint32_t)(tf * 32) * row_bytes;
      uint4 v[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int row = j * 4 + (el >> 4);
        v[j] = *reinterpret_cast<const uint4*>(otile + row * 256 + ((jc ^ (row & 15)) << 4));
      }
      if (tabs && tf < 3) dma_tabs(tf + 1);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        // bit 4 of the row is bit 2 of j: those rows hold their 8-byte halves swapped
        const u32x4 o = ((j >> 2) & 1) ? u32x4{v[j].z, v[j].w, v[j].x, v[j].y}
                                       : u32x4{v[j].x, v[j].y, v[j].z, v[j].w};
        if (!kNbsd) {
          const uint32_t off = ch_ok ? obyte + (uint32_t)(j * 4) * row_bytes : kDropOffset;
          __builtin_amdgcn_raw_buffer_store_b128(o, orsrc, (int)off, 0, kNonTemporal);
        } else {
          const bool ok = tf * 32 + j * 4 < rows_left;
          const uint32_t off = ok ? obyte + (uint32_t)(j * 4) * row_bytes : kDropOffset;
          __builtin_amdgcn_raw_buffer_store_b128(o, orsrc, (int)off, 0, kNonTemporal);
        }
      }
      // the pass's sums are formed here, from registers (otherwise the compiler sinks every
      // pass's sum-of-squares arithmetic below the last pass, parking the fp32 values in
      // AGPRs meanwhile)
      asm volatile("" :: "v"(sq_q[tf]), "v"(sq_k[tf]));
      __builtin_amdgcn_sched_barrier(0);      // passes stay in order: bounded register use
    }
  };

  // ---- split contraction: the unit's raw fp32 accumulators to its plane ----
  // The next unit's stages 0-2 are requested first; then each lane stores its 64 accumulator
  // quads (4 consecutive channels of one token, 16 bytes) through a buffer descriptor over
  // the unit's [T, I] plane.  Quads outside [T, I] get an offset beyond the descriptor's range
  // and the hardware drops them, so all 64 stores are issued unconditionally and the next
  // unit's wait for all but the last kTailStores memory operations covers its DMAs.  Split
  // calls have at most 128 tiles of 256 x 256, so a plane holds at most 2^25 bytes and every
  // offset fits the descriptor's 32 bits.
  auto split_store = [&](Tile u, bool more) __attribute__((always_inline)) {
    if (more) {
      issue(I0{}, 0);
      issue(I1{}, 1);
      issue(I2{}, 2);
    }
    __builtin_amdgcn_sched_barrier(0);
    const int el = fresh_lane();
    const int g = el >> 5, fr = el & 31;
    const int64_t plane = a.T * a.I;
    const __amdgpu_buffer_rsrc_t prs = __builtin_amdgcn_make_buffer_rsrc(
        a.part + (int64_t)u.kz * plane, (short)0,
        (int)(uint32_t)min(plane * 4, (int64_t)0x7FFFFFFF), kBufferRsrcWord3);
    const int64_t tok0 = (int64_t)u.tm * kTileM + wm * 128 + fr;
    const int64_t ch0 = (int64_t)u.tn * kTileN + wn * 128 + g * 4;
#pragma unroll
    for (int tf = 0; tf < 4; ++tf) {
      const int64_t tok = tok0 + tf * 32;
#pragma unroll
      for (int cf = 0; cf < 4; ++cf)
#pragma unroll
        for (int rq = 0; rq < 4; ++rq) {
          const int64_t ch = ch0 + cf * 32 + rq * 8;
          const uint32_t off =
              (tok < a.T && ch < a.I) ? (uint32_t)((tok * a.I + ch) * 4) : kDropOffset;
          const u32x4 v = {__float_as_uint(acc[cf][tf][rq * 4]),
                           __float_as_uint(acc[cf][tf][rq * 4 + 1]),
                           __float_as_uint(acc[cf][tf][rq * 4 + 2]),
                           __float_as_uint(acc[cf][tf][rq * 4 + 3])};
          __builtin_amdgcn_raw_buffer_store_b128(v, prs, (int)off, 0, 0);
        }
    }
  };

  // ---- tile loop ----
  // Before the first tile: its stages 0-2 and epilogue operands requested and awaited.  Each
  // tile then: waits for everything in flight except the previous epilogue's last
  // kTailStores stores, barrier (stage buffer 3, the previous epilogue's staging area, is
  // free; stages 0-2 and the operands are visible), requests stage 3, widens the bias, reads
  // stage 0's fragments, barrier, runs the K-steps.  Once the last DMA has landed (two K-steps
  // before the end) thread 0 draws a ticket for the next tile; after the last K-step it turns
  // the ticket into a tile id, published through LDS, and the epilogue's passes request that
  // tile's stages 0-2 and epilogue operands one after another.
  issue(I0{}, 0);
  issue(I1{}, 1);
  issue(I2{}, 2);
  if (!kSplit) issue_ops(t, 0);
  wait_vm<0>();
  // the tile body, instantiated for operand buffer e = 0 and e = 1 (tiles alternate), so the
  // buffer index is a constant everywhere; returns whether another tile follows
  auto tile_iter = [&](auto e_c) __attribute__((always_inline)) -> bool {
    constexpr int e = decltype(e_c)::value;
    // the previous epilogue's DMAs have landed; its last kTailStores stores may be in flight
    wait_vm<kTailStores>();
    __syncthreads();
    issue(I3{}, 3);
    {
      const int lt = wave * 64 + fresh_lane();
      const uint32_t w = lds_braw[e][lt >> 1];
      lds_bias[e][lt] = kBias ? bf16_to_f32((lt & 1) ? w >> 16 : w & 0xFFFFu) : 0.0f;
    }
    set_lane_offsets();
    fload(0, wf[0], xf[0]);
    sload(0, sc[0]);
    xsload(0, xs[0]);
    __syncthreads();
    // the trip count is re-read through an opaque copy each tile: a loop-invariant test hoisted
    // out of the tile loop would be kept in a register (or spilled) across the whole tile
    int ks_opaque = kSplit ? min(a.ks_chunk, a.KS - t.kz * a.ks_chunk) : KS;
    asm volatile("" : "+s"(ks_opaque));
    const int kend = kSplit ? ks_opaque : KS;     // K-stages of this unit
    // K-step 0 feeds zero accumulators to its MFMAs (no separate clearing of the 256 AGPRs)
    if (ks_opaque > 4) {
      step(I0{}, 0, Yes{}, W40{}, Z{});
      step(I1{}, 1, Yes{}, W40{}, NZ{});
      step(I2{}, 2, Yes{}, W40{}, NZ{});
      step(I3{}, 3, Yes{}, W40{}, NZ{});
      for (int s = 4; s < ks_opaque - 4; s += 4) {
        step(I0{}, s, Yes{}, W40{}, NZ{});
        step(I1{}, s + 1, Yes{}, W40{}, NZ{});
        step(I2{}, s + 2, Yes{}, W40{}, NZ{});
        step(I3{}, s + 3, Yes{}, W40{}, NZ{});
      }
      // last superstep: nothing left to request; the waits shrink with the groups in flight
      step(I0{}, kend - 4, No{}, W20{}, NZ{});
    } else {
      step(I0{}, 0, No{}, W20{}, Z{});             // one superstep only
    }
    step(I1{}, kend - 3, No{}, W0{}, NZ{});
    // every DMA has landed: draw the ticket for the next tile now (its latency passes during
    // the last two K-steps); the claim is published after them
    unsigned ticket;
    if (tid == 0) ticket = atomicAdd(&a.ctr[my_xcd], 1u);
    step(I2{}, kend - 2, No{}, WN{}, NZ{});
    step(I3{}, kend - 1, No{}, WN{}, NZ{});
    // pin the accumulators here: without this the compiler sinks the last superstep's MFMAs
    // (their results are only read by the epilogue) below the next tile's DMA requests
#pragma unroll
    for (int cf = 0; cf < 4; ++cf)
#pragma unroll
      for (int tf = 0; tf < 4; ++tf) asm volatile("" : "+a"(acc[cf][tf]));
    __builtin_amdgcn_sched_barrier(0);

    const Tile cur = t;
    if (tid == 0) lds_tile[e] = claim((int)ticket);
    __syncthreads();
    const int next_tile = __builtin_amdgcn_readfirstlane(lds_tile[e]);
    const bool more = next_tile >= 0;
    if (more) {
      t = decode(next_tile);
      set_sources(t);
    }
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (kSplit)
      split_store(cur, more);
    else
      epilogue(cur, e, more, t);
    return more;
  };
  for (;;) {
    if (!tile_iter(std::integral_constant<int, 0>{})) break;
    if (!tile_iter(std::integral_constant<int, 1>{})) break;
  }
}

// Activation codes [T, stride] (rows only 4-byte aligned in the packed [T, H + 4] layout) ->
// the stage images the projection DMA-copies: per (token tile tm, K-stage t) 256 rows x 64
// bytes with 16-byte chunk c of row r at chunk position c ^ stage_swizzle(r); zero past T or H.
// One thread per 16-byte position.
__global__ void __launch_bounds__(256) act_repack_kernel(const uint8_t* __restrict__ a,
                                                         int64_t stride, int64_t T, int64_t H,
                                                         int KS, uint8_t* __restrict__ img,
                                                         unsigned* __restrict__ ctr) {
  // this kernel runs before every projection launch: it also resets the tile counters
  if (blockIdx.x == 0 && blockIdx.y == 0 && blockIdx.z == 0 && threadIdx.x < kXcds)
    ctr[threadIdx.x] = 0;
  const int p = blockIdx.x * blockDim.x + threadIdx.x;   // 0..1023
  const int64_t t = blockIdx.y;
  const int64_t tm = blockIdx.z;
  const int r = p >> 2;
  const int c = (p & 3) ^ stage_swizzle(r);
  const int64_t m = tm * kTileM + r;
  const int64_t k = t * kStage + 16 * c;
  uint4 o = make_uint4(0, 0, 0, 0);
  if (m < T && k < H) {
    const u32x4_a4 v = *reinterpret_cast<const u32x4_a4*>(a + m * stride + k);
    o = make_uint4(v.x, v.y, v.z, v.w);
  }
  reinterpret_cast<uint4*>(img)[(tm * KS + t) * (kStageImage / 16) + p] = o;
}

// Zeroes the per-XCD tile counters (for launches without an activation repack, which
// otherwise does it).
__global__ void __launch_bounds__(64) reset_counters_kernel(unsigned* __restrict__ ctr) {
  if (threadIdx.x < kXcds) ctr[threadIdx.x] = 0;
}

// MX activation exponents [T, stride] -> per (token tile tm, superstep s) [256 tokens][2]
// dwords: byte q of dword g of token r = exponent of K-block 8 s + 2 q + g of row 256 tm + r,
// 127 (2^0) past T or H (whose codes are zero).  One thread per (token, dword).
__global__ void __launch_bounds__(256) act_scale_repack_kernel(const uint8_t* __restrict__ e8,
                                                               int64_t stride, int64_t T,
                                                               int64_t H, uint32_t* __restrict__ img) {
  const int64_t s = blockIdx.y, tm = blockIdx.z;
  const int idx = blockIdx.x * blockDim.x + threadIdx.x;       // 0 .. 511
  const int r = idx >> 1, g = idx & 1;
  const int64_t m = tm * kTileM + r;
  const int64_t nblocks = H / 32;
  uint32_t w = 0;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int64_t b = 8 * s + 2 * q + g;
    const uint32_t e = (m < T && b < nblocks) ? e8[m * stride + b] : 127u;
    w |= e << (8 * q);
  }
  img[((tm * gridDim.y + s) * kTileM + r) * 2 + g] = w;
}

// ssq[t] = sum over partials p < P of ws[p][t]; P = 0 gives zeros.  A block covers 64 tokens
// with 8 wavefronts: wavefront w adds the partials p = w, w + 8, ... of its lane's token in
// increasing p (each load instruction reads 512 contiguous bytes), then wavefront 0 adds the
// eight results in w order.  The order is fixed, so the sums are reproducible run to run.
constexpr int kReduceWaves = 8;
__global__ void __launch_bounds__(64 * kReduceWaves) ssq_reduce_kernel(const float* __restrict__ ws,
                                                                       int64_t P, int64_t T,
                                                                       float* __restrict__ ssq) {
  __shared__ float2 part[kReduceWaves][64];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int64_t t = (int64_t)blockIdx.x * 64 + lane;
  float q = 0.f, k = 0.f;
  if (t < T) {
#pragma unroll 4
    for (int64_t p = w; p < P; p += kReduceWaves) {
      const float2 v = reinterpret_cast<const float2*>(ws)[p * T + t];
      q += v.x;
      k += v.y;
    }
  }
  part[w][lane] = make_float2(q, k);
  __syncthreads();
  if (w == 0 && t < T) {
    float2 r = part[0][lane];
#pragma unroll
    for (int i = 1; i < kReduceWaves; ++i) {
      r.x += part[i][lane].x;
      r.y += part[i][lane].y;
    }
    reinterpret_cast<float2*>(ssq)[t] = r;
  }
}

// Split contraction, second pass: token t's row of every plane summed in plane order, then the
// projection's epilogue on the sum: x = acc * a_scale * c + bias (fp32), bf16 out (BSD [T, I],
// or NBSd [I / d, T, d] with kNbsd), and the sums of squares of the fp32 x over the Q and the
// K segment.  One block per token, four channels per thread and step (I, d and the segment
// bounds are multiples of 16, so a quad never straddles a head or a segment boundary); the
// block's sums are combined in a fixed order.
template <bool kRowScale, bool kChanScale, bool kBias, bool kNbsd>
__global__ void __launch_bounds__(256) split_reduce_kernel(
    const float* __restrict__ part, int S, int64_t T, int64_t I, int64_t Iq, int64_t Ik,
    int64_t d, const uint8_t* __restrict__ a_scales, int64_t s_stride,
    const float* __restrict__ chan, const uint16_t* __restrict__ bias, uint16_t* __restrict__ out,
    float* __restrict__ ssq) {
  __shared__ float2 red[4];
  const int64_t t = blockIdx.x;
  const float sa = kRowScale ? *reinterpret_cast<const float*>(a_scales + t * s_stride) : 1.0f;
  const int64_t plane = T * I;
  const float* const row = part + t * I;
  float q = 0.f, k = 0.f;
  for (int64_t c = (int64_t)threadIdx.x * 4; c < I; c += 1024) {
    float4 acc = *reinterpret_cast<const float4*>(row + c);
    for (int z = 1; z < S; ++z) {
      const float4 p = *reinterpret_cast<const float4*>(row + z * plane + c);
      acc.x += p.x; acc.y += p.y; acc.z += p.z; acc.w += p.w;
    }
    const float av[4] = {acc.x, acc.y, acc.z, acc.w};
    float bs[4] = {0.f, 0.f, 0.f, 0.f}, cs[4] = {1.f, 1.f, 1.f, 1.f};
    if (kBias) {
      const uint2 bw = *reinterpret_cast<const uint2*>(bias + c);
      bs[0] = bf16_to_f32(bw.x & 0xFFFFu); bs[1] = bf16_to_f32(bw.x >> 16);
      bs[2] = bf16_to_f32(bw.y & 0xFFFFu); bs[3] = bf16_to_f32(bw.y >> 16);
    }
    if (kChanScale) {
      const float4 c4 = *reinterpret_cast<const float4*>(chan + c);
      cs[0] = c4.x; cs[1] = c4.y; cs[2] = c4.z; cs[3] = c4.w;
    }
    float x[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      x[i] = kChanScale ? av[i] * sa * cs[i] + bs[i] : fmaf(av[i], sa, bs[i]);
    const float s2 = x[0] * x[0] + x[1] * x[1] + x[2] * x[2] + x[3] * x[3];
    if (c < Iq) q += s2;
    else if (c < Iq + Ik) k += s2;
    const u32x2_a8 o = {pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3])};
    const int64_t at = kNbsd ? ((c / d) * T + t) * d + c % d : t * I + c;
    *reinterpret_cast<u32x2_a8*>(out + at) = o;
  }
  if (ssq) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
      q += __shfl_xor(q, off);
      k += __shfl_xor(k, off);
    }
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = make_float2(q, k);
    __syncthreads();
    if (threadIdx.x == 0) {
      float2 r = red[0];
#pragma unroll
      for (int w = 1; w < 4; ++w) {
        r.x += red[w].x;
        r.y += red[w].y;
      }
      reinterpret_cast<float2*>(ssq)[t] = r;
    }
  }
}

}  // namespace

namespace {

// Split contraction (few tiles): project_kernel over tile x K-chunk units into the planes at
// `planes`, then split_reduce_kernel.  Returns false (nothing launched) when the call has
// enough tiles or its K range is a single superstep.
template <bool kMx>
bool launch_split(const ProjectArgs& a, bool chan, bool bias, bool nbsd, float* ssq,
                  uint8_t* planes, int cus, hipStream_t s, hipError_t* err) {
  const SplitPlan sp = split_plan(a.T, a.H, a.I);
  if (sp.chunks < 2 || !planes) return false;
  const int used = sp.chunks;
  ProjectArgs b = a;
  b.ksplit = used;
  b.ks_chunk = sp.stages_per_chunk;
  b.part = reinterpret_cast<float*>(planes);
  const int64_t units = (int64_t)a.tiles_m * a.tiles_n * used;
  const unsigned nblocks = (unsigned)std::min<int64_t>(units, std::max(cus, 1));
  hipLaunchKernelGGL((project_kernel<false, false, false, kMx, 0, false, true>), dim3(nblocks),
                     dim3(kThreads), 0, s, b);
  hipError_t e = hipGetLastError();
  if (e == hipSuccess) {
    const dim3 rg((unsigned)a.T), rb(256);
    const int variant = (chan ? 4 : 0) | (bias ? 2 : 0) | (nbsd ? 1 : 0);
#define QKVMX_SPLIT_REDUCE(C, B, N)                                                          \
  hipLaunchKernelGGL((split_reduce_kernel<!kMx, C, B, N>), rg, rb, 0, s, b.part, used, a.T, a.I, \
                     a.Iq, a.Ik, a.d, a.a_scales, a.s_stride, a.chan_scale, a.bias, a.out, ssq)
    switch (variant) {
      case 0: QKVMX_SPLIT_REDUCE(false, false, false); break;
      case 1: QKVMX_SPLIT_REDUCE(false, false, true); break;
      case 2: QKVMX_SPLIT_REDUCE(false, true, false); break;
      case 3: QKVMX_SPLIT_REDUCE(false, true, true); break;
      case 4: QKVMX_SPLIT_REDUCE(true, false, false); break;
      case 5: QKVMX_SPLIT_REDUCE(true, false, true); break;
      case 6: QKVMX_SPLIT_REDUCE(true, true, false); break;
      default: QKVMX_SPLIT_REDUCE(true, true, true); break;
    }
#undef QKVMX_SPLIT_REDUCE
    e = hipGetLastError();
  }
  *err = e;
  return true;
}

// Persistent project_kernel launch (one block per compute unit, each walking its XCD's tile
// range), then the fixed-order sum of the partials when ssq is requested.  Calls with few
// tiles take the split contraction instead when `planes` is given.
template <bool kMx>
hipError_t launch_core(const ProjectArgs& a, bool chan, bool bias, bool nbsd, float* ssq,
                       hipStream_t s, uint8_t* planes) {
  int dev = 0, cus = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  if (launch_split<kMx>(a, chan, bias, nbsd, ssq, planes, cus, s, &e)) return e;
  const int64_t ntiles = (int64_t)a.tiles_m * a.tiles_n;
  const unsigned nblocks = (unsigned)std::min<int64_t>(ntiles, std::max(cus, 1));
  const dim3 grid(nblocks), block(kThreads);
  const int variant = (chan ? 4 : 0) | (bias ? 2 : 0) | (nbsd ? 1 : 0);
  switch (variant) {
    case 0: hipLaunchKernelGGL((project_kernel<false, false, false, kMx>), grid, block, 0, s, a); break;
    case 1: hipLaunchKernelGGL((project_kernel<false, false, true, kMx>), grid, block, 0, s, a); break;
    case 2: hipLaunchKernelGGL((project_kernel<false, true, false, kMx>), grid, block, 0, s, a); break;
    case 3: hipLaunchKernelGGL((project_kernel<false, true, true, kMx>), grid, block, 0, s, a); break;
    case 4: hipLaunchKernelGGL((project_kernel<true, false, false, kMx>), grid, block, 0, s, a); break;
    case 5: hipLaunchKernelGGL((project_kernel<true, false, true, kMx>), grid, block, 0, s, a); break;
    case 6: hipLaunchKernelGGL((project_kernel<true, true, false, kMx>), grid, block, 0, s, a); break;
    default: hipLaunchKernelGGL((project_kernel<true, true, true, kMx>), grid, block, 0, s, a); break;
  }
  e = hipGetLastError();
  if (e != hipSuccess || !ssq) return e;
  // only the partials of 128-channel groups that overlap Q or K are written and summed
  const int64_t P = ceil_div(a.Iq + a.Ik, (int64_t)kPartialN);
  hipLaunchKernelGGL(ssq_reduce_kernel, dim3((unsigned)ceil_div(a.T, 64)),
                     dim3(64 * kReduceWaves), 0, s, a.ws, P, a.T, ssq);
  return hipGetLastError();
}

ProjectArgs common_args(const uint8_t* w_packed, const float* chan_scale, const uint16_t* bias,
                        int64_t T, int64_t H, int64_t I, int64_t Iq, int64_t Ik, int64_t d,
                        uint16_t* out) {
  ProjectArgs a{};
  a.w_img = w_packed;
  a.w_scales = w_packed + packed_scales_offset(H, I);
  a.chan_scale = chan_scale; a.bias = bias;
  a.T = T; a.H = H; a.I = I; a.Iq = Iq; a.Ik = Ik; a.d = d;
  a.KS = (int)packed_stages(H);
  a.tiles_m = (int)ceil_div(T, kTileM);
  a.tiles_n = (int)packed_tiles_n(I);
  a.out = out;
  return a;
}

}  // namespace

}  // namespace qkvmx
