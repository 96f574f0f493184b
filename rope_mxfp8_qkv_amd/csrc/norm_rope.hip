// Pass 2 ([QKV-CTE] "Design 1)" steps b-c, "Design 2)", "Design 5)"): across-heads RMSNorm and
// rotate-half RoPE applied in place to the Q and K heads of the bf16 projection output, in the
// BSD [T, I] or the NBSd [I / d, T, d] layout; V is never read or written.  HBM-bound: per token
// 4 * (Iq + Ik) bytes of Q/K plus the token's cos/sin rows (8 * d bytes) and its two sums; gamma
// is shared by all tokens and stays cached.
//
// Every thread owns an 8-lane chunk j0 of its token's heads together with the chunk's
// rotate-half partners j0 + d/2 .. j0 + d/2 + 7.  The token's cos/sin values for those 16 lanes
// and its inv_rms are loaded once per thread and reused for every head, as the pages broadcast
// the position-only tables across heads; each head costs two independent 16-byte loads of x
// (plus gamma, an L1/L2 hit) and two 16-byte streaming stores.  inv_rms is folded into the gamma
// multiply.  The two layouts differ only in how threads map to (token, head): see the kernels.
// BSD: blocks of 4 tokens (256 threads), ten heads' loads in flight per thread before their
// stores, streaming loads and stores of x, and the blocks visit the tokens from the last one
// down: the projection writes its output token tile by token tile upwards, so the rows it
// wrote last are still in the 256 MB last-level cache when this pass starts, and reading them
// first finds them there instead of after the cache has turned over.  That order and block
// shape moved the most bytes per second right after the projection in interleaved A/B runs at
// the full video shape (blocks of 8, 16 and 2 tokens, batch depths 5 and 10, cached loads).
// NBSd has its own order (see its kernel).
#include "device_common.h"
#include "internal.h"

namespace qkvmx {

namespace {

constexpr int kThreadsPerToken = 64;
constexpr int kTokensPerBlock = 4;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

struct NormRopeArgs {
  uint16_t* qkv;
  const float* ssq;
  const uint16_t* gq;
  const uint16_t* gk;
  const float* cos_tab;
  const float* sin_tab;
  int64_t T;
  int64_t I;
  int nq, nkv, d;
  int heads_q;       // heads of the Q segment that are touched (0 if Q is untouched)
  int heads;         // touched heads in total (Q heads first, then K heads)
  float eps;
  bool norm_q, norm_k, rope;
};

__device__ __forceinline__ void unpack8(const uint4 v, float (&f)[8]) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    f[2 * e] = bf16_to_f32(w[e] & 0xFFFFu);
    f[2 * e + 1] = bf16_to_f32(w[e] >> 16);
  }
}

__device__ __forceinline__ u32x4 pack8(const float (&f)[8]) {
  return u32x4{pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3]), pack_bf16x2(f[4], f[5]),
               pack_bf16x2(f[6], f[7])};
}

__device__ __forceinline__ void load8f(const float* p, float (&f)[8]) {
  const float4 a = reinterpret_cast<const float4*>(p)[0];
  const float4 b = reinterpret_cast<const float4*>(p)[1];
  f[0] = a.x; f[1] = a.y; f[2] = a.z; f[3] = a.w;
  f[4] = b.x; f[5] = b.y; f[6] = b.z; f[7] = b.w;
}

// One token's work for one thread: the 8-lane chunk j0 (and its rotate-half partners
// j0 + d/2 ..) of the touched heads h = h0, h0 + hstep, ... below hend; base_of(h, is_k)
// addresses the head's d elements for this token.  The token's cos/sin values and inv_rms are loaded once and
// reused for every head.  Heads are taken kBatch at a time: the loads of a whole batch are
// issued before any of its stores, so each block keeps its tokens' Q/K bytes in flight at once,
// and both the loads and the stores of x are non-temporal (x is touched exactly once; with
// both streaming, the in-place read-modify-write of the strided Q/K columns sustains a higher
// DRAM rate than with cached accesses).  gamma and the tables are re-read by every token and
// stay cached.
constexpr int kBatch = 10;
template <typename BaseOf>
__device__ __forceinline__ void apply_token(const NormRopeArgs& a, int64_t token, int j0, int h0,
                                            int hstep, int hend, BaseOf base_of) {
  const int half = a.d / 2;
  float clo[8], chi[8], slo[8], shi[8];
  if (a.rope) {
    const float* cr = a.cos_tab + token * a.d;
    const float* sr = a.sin_tab + token * a.d;
    load8f(cr + j0, clo);
    load8f(cr + half + j0, chi);
    load8f(sr + j0, slo);
    load8f(sr + half + j0, shi);
  }
  float rq = 1.0f, rk = 1.0f;
  if (a.norm_q) rq = 1.0f / sqrtf(a.ssq[token * 2] / (float)(a.nq * a.d) + a.eps);
  if (a.norm_k) rk = 1.0f / sqrtf(a.ssq[token * 2 + 1] / (float)(a.nkv * a.d) + a.eps);
  for (int hb = h0; hb < hend; hb += kBatch * hstep) {
    u32x4 xlo[kBatch], xhi[kBatch];
#pragma unroll
    for (int b = 0; b < kBatch; ++b) {
      const int h = hb + b * hstep;
      if (h < hend) {
        const uint16_t* base = base_of(h, h >= a.heads_q);
        xlo[b] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(base + j0));
        xhi[b] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(base + half + j0));
      }
    }
#pragma unroll
    for (int b = 0; b < kBatch; ++b) {
      const int h = hb + b * hstep;
      if (h >= hend) break;
      const bool is_k = h >= a.heads_q;
      uint16_t* base = base_of(h, is_k);
      float lo[8], hi[8];
      unpack8(make_uint4(xlo[b].x, xlo[b].y, xlo[b].z, xlo[b].w), lo);
      unpack8(make_uint4(xhi[b].x, xhi[b].y, xhi[b].z, xhi[b].w), hi);
      const bool norm = is_k ? a.norm_k : a.norm_q;
      if (norm) {
        const float r = is_k ? rk : rq;
        const uint16_t* g = is_k ? a.gk + (int64_t)(h - a.heads_q) * a.d : a.gq + (int64_t)h * a.d;
        float glo[8], ghi[8];
        unpack8(*reinterpret_cast<const uint4*>(g + j0), glo);
        unpack8(*reinterpret_cast<const uint4*>(g + half + j0), ghi);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          lo[e] = lo[e] * (glo[e] * r);
          hi[e] = hi[e] * (ghi[e] * r);
        }
      }
      if (a.rope) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float ol = lo[e] * clo[e] - hi[e] * slo[e];
          const float oh = hi[e] * chi[e] + lo[e] * shi[e];
          lo[e] = ol;
          hi[e] = oh;
        }
      }
      __builtin_nontemporal_store(pack8(lo), reinterpret_cast<u32x4*>(base + j0));
      __builtin_nontemporal_store(pack8(hi), reinterpret_cast<u32x4*>(base + half + j0));
    }
  }
}

// BSD [T, I]: 64 threads per token; thread (j, hg) owns chunk j0 = 8 j of heads hg, hg + G, ...
// (G = 64 / (d / 16) head groups), so one wave instruction covers G heads of one token row.
__global__ void __launch_bounds__(kThreadsPerToken * kTokensPerBlock) norm_rope_kernel(
    const NormRopeArgs a) {
  // blocks from the last token down (see the file comment)
  const int64_t token = (int64_t)(gridDim.x - 1 - blockIdx.x) * kTokensPerBlock +
                        (threadIdx.x / kThreadsPerToken);
  if (token >= a.T) return;
  const int lane = threadIdx.x % kThreadsPerToken;
  const int cpd = a.d / 16;                 // chunks per head half-pair
  const int ngroups = kThreadsPerToken / cpd;
  const int hg = lane / cpd;
  if (hg >= ngroups) return;                // lanes past the last whole group (64 % cpd != 0)
  uint16_t* row = a.qkv + token * a.I;
  apply_token(a, token, (lane % cpd) * 8, hg, ngroups, a.heads, [&](int h, bool is_k) {
    // Q heads come first; the K segment starts at nq * d
    return row + (is_k ? (int64_t)a.nq * a.d + (int64_t)(h - a.heads_q) * a.d : (int64_t)h * a.d);
  });
}

// NBSd [I / d, T, d] ([QKV-CTE] "Interface": output_layout; "Design 2)": each head occupies its
// own block of rows, d contiguous): lane -> (token, chunk) with the chunk fastest, so for each
// head one wave instruction covers 64 / (d / 16) consecutive tokens of that head, contiguous in
// memory.  A block takes kTokensPerBlock wavefronts' tokens and one group of kBatch touched
// heads (one batch per thread).  The blocks walk the heads group by group, each group's tokens
// from the first up: the blocks in flight then cover one contiguous stretch of each of a few
// head blocks of rows, instead of short runs in all of them (measured at the full video shape
// right after the projection: 0.580 ms, against 0.590 with each group's tokens from the last
// down, 0.657 with every thread walking all heads of its token, 0.633 / 0.594 with groups of 5
// / 20 heads).
__global__ void __launch_bounds__(kThreadsPerToken * kTokensPerBlock) norm_rope_nbsd_kernel(
    const NormRopeArgs a) {
  const int cpd = a.d / 16;
  const int tpw = kThreadsPerToken / cpd;   // tokens per wavefront
  const int lane = threadIdx.x % kThreadsPerToken, wave = threadIdx.x / kThreadsPerToken;
  const int slot = lane / cpd;
  if (slot >= tpw) return;                  // lanes past the last whole token (64 % cpd != 0)
  const int ngroups = (a.heads + kBatch - 1) / kBatch;
  const unsigned ntb = gridDim.x / (unsigned)ngroups;   // token blocks per head group
  const int hgp = (int)(blockIdx.x / ntb);
  const int64_t tblk = (int64_t)(blockIdx.x % ntb);
  const int64_t token = (tblk * kTokensPerBlock + wave) * tpw + slot;
  if (token >= a.T) return;
  const int h0 = hgp * kBatch;
  apply_token(a, token, (lane % cpd) * 8, h0, 1, min(h0 + kBatch, a.heads), [&](int h, bool is_k) {
    // head index in the output: Q heads first, then K heads (which follow all nq Q heads)
    const int64_t hid = is_k ? (int64_t)a.nq + (h - a.heads_q) : (int64_t)h;
    return a.qkv + (hid * a.T + token) * a.d;
  });
}

}  // namespace

hipError_t launch_norm_rope(uint16_t* qkv, const float* ssq, const uint16_t* q_gamma,
                            const uint16_t* k_gamma, const float* cos_tab, const float* sin_tab,
                            int64_t T, int nq, int nkv, int d, float eps, uint32_t flags,
                            bool nbsd, hipStream_t s) {
  NormRopeArgs a;
  a.qkv = qkv; a.ssq = ssq; a.gq = q_gamma; a.gk = k_gamma; a.cos_tab = cos_tab;
  a.sin_tab = sin_tab; a.T = T; a.I = (int64_t)(nq + 2 * nkv) * d;
  a.nq = nq; a.nkv = nkv; a.d = d; a.eps = eps;
  a.norm_q = flags & 1u; a.norm_k = (flags & 2u) && nkv > 0; a.rope = flags & 4u;
  const bool q_on = a.norm_q || a.rope;
  const bool k_on = nkv > 0 && (a.norm_k || a.rope);
  a.heads_q = q_on ? nq : 0;
  a.heads = a.heads_q + (k_on ? nkv : 0);
  if (a.heads == 0 || T == 0) return hipSuccess;        // nothing to do
  if (d / 16 > kThreadsPerToken) return hipErrorInvalidValue;
  if (nbsd) {
    const int64_t per_block = (int64_t)kTokensPerBlock * (kThreadsPerToken / (d / 16));
    const int64_t ngroups = ceil_div((int64_t)a.heads, (int64_t)kBatch);
    const int64_t nblocks = ceil_div(T, per_block) * ngroups;
    if (nblocks > 0x7FFFFFFF) return hipErrorInvalidValue;
    hipLaunchKernelGGL(norm_rope_nbsd_kernel, dim3((unsigned)nblocks),
                       dim3(kThreadsPerToken * kTokensPerBlock), 0, s, a);
  } else {
    hipLaunchKernelGGL(norm_rope_kernel, dim3((unsigned)ceil_div(T, kTokensPerBlock)),
                       dim3(kThreadsPerToken * kTokensPerBlock), 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace qkvmx
