// Uniform asymmetric quantizers for the packed cache, and the fp16 window append.
//
// Keys are quantized per channel over blocks of 32 tokens, values per token over
// groups of 32 channels ("The KV cache has a geometry problem", sections on keys and
// values; KIVI post, "Method" and "Experiments").  Per group: the minimum is the zero
// point, the step is the range over 2^B - 1, each element is rounded to the nearest
// step ("Quantization error in practice").  Every operation below is one IEEE fp32
// operation (the library is built with contraction off), so the codes and the
// (scale, min) metadata are reproducible bit for bit.
//
// One workgroup of 256 threads handles one (batch, head, 32-token block): it stages
// the 32 x 128 fp16 tile in LDS with coalesced 16-byte loads, computes the group
// statistics with one thread per group, then writes the packed words with one thread
// per output word, so every global store is coalesced.
#include "kvq_common.h"

namespace kvq {
namespace {

constexpr int kThreads = 256;

struct GroupQ {
  float mn;
  float inv;
  uint32_t meta;
};

// Statistics of one group from its fp32 min and max (exact fp16 values).
__device__ __forceinline__ GroupQ group_params(float mn, float mx, float levels) {
  mn = mn + 0.0f;                              // -0 -> +0
  mx = mx + 0.0f;
  const uint16_t min_h = f32_to_f16_bits(mn);  // exact
  const uint16_t scale_h = f32_to_f16_bits((mx - mn) / levels);
  const float s = f16_bits_to_f32(scale_h);
  GroupQ g;
  g.mn = mn;
  g.inv = (s == 0.0f) ? 0.0f : 1.0f / s;
  g.meta = (uint32_t)scale_h | ((uint32_t)min_h << 16);
  return g;
}

__device__ __forceinline__ uint32_t code_of(float x, float mn, float inv, float levels) {
  float r = rintf((x - mn) * inv);
  r = fminf(fmaxf(r, 0.0f), levels);
  return (uint32_t)r;
}

// Stage a 32-token x 128-channel fp16 tile (rows of 256 bytes) in LDS.
__device__ __forceinline__ void load_tile(uint16_t (*tile)[kHeadDim], const uint16_t* src,
                                          int64_t stride_t) {
  const int t = threadIdx.x >> 3;            // token 0..31
  const int c = (threadIdx.x & 7) * 16;      // 16 channels = 32 bytes
  const uint4* p = reinterpret_cast<const uint4*>(src + t * stride_t + c);
  uint4 a = p[0];
  uint4 b = p[1];
  uint4* d = reinterpret_cast<uint4*>(&tile[t][c]);
  d[0] = a;
  d[1] = b;
}

template <int KB, int VB>
__global__ __launch_bounds__(kThreads) void quant_uniform_kernel(QuantArgs a) {
  __shared__ __align__(16) uint16_t tile[kGroup][kHeadDim];
  __shared__ __align__(16) float2 st[kHeadDim];   // K: [channel]; V: [group][token]

  const int64_t job = blockIdx.x;
  const int blk = (int)(job % a.n_blocks);
  const int64_t bh = job / a.n_blocks;
  const int b = (int)(bh / a.kv_heads);
  const int h = (int)(bh % a.kv_heads);
  const int64_t dst = bh * a.cap_blocks + a.blk0 + blk;   // [B][H][cap_blocks]
  const int tid = threadIdx.x;
  KVQ_CHECK(a.blk0 + blk < a.cap_blocks, kDbgWrite);

  if constexpr (KB != 0) {
   if (a.k != nullptr) {
    constexpr float L = (float)((1 << KB) - 1);
    constexpr int WK = kHeadDim * KB / 32;      // words per token row
    constexpr int CPW = 32 / KB;                // channels per word
    load_tile(tile, a.k + b * a.ks_b + h * a.ks_h + (int64_t)blk * kGroup * a.ks_t, a.ks_t);
    __syncthreads();
    if (tid < kHeadDim) {                       // one thread per channel
      float mn = f16_bits_to_f32(tile[0][tid]);
      float mx = mn;
#pragma unroll
      for (int t = 1; t < kGroup; ++t) {
        const float x = f16_bits_to_f32(tile[t][tid]);
        mn = fminf(mn, x);
        mx = fmaxf(mx, x);
      }
      const GroupQ g = group_params(mn, mx, L);
      a.k_meta[dst * kHeadDim + tid] = g.meta;
      st[tid] = make_float2(g.mn, g.inv);
    }
    __syncthreads();
    // Word wi = t * WK + col holds channels col*CPW .. col*CPW + CPW - 1 of token t.
    // 4-bit codes: a thread keeps one column for all its words, so it reads its
    // channels' (min, 1/scale) once, and reads each token's 8 fp16 values as one 16-byte
    // vector; the lanes of one token read a contiguous row (per-code 2-byte reads of the
    // same values conflicted heavily in the LDS banks and took twice as long).  2-bit
    // codes: one word per thread, per-code reads (measured faster for that layout).
   if constexpr (KB == 4) {
    const int col = tid % WK;
    const int c0 = col * CPW;
    float gmn[CPW], ginv[CPW];
#pragma unroll
    for (int j = 0; j < CPW; j += 2) {
      const float4 g = *reinterpret_cast<const float4*>(&st[c0 + j]);
      gmn[j] = g.x; ginv[j] = g.y; gmn[j + 1] = g.z; ginv[j + 1] = g.w;
    }
#pragma unroll
    for (int i = 0; i < (kGroup * WK) / kThreads; ++i) {
      const int t = tid / WK + i * (kThreads / WK);
      uint32_t x[CPW / 2];                      // CPW fp16 values, two per word
#pragma unroll
      for (int k = 0; k < CPW / 8; ++k) {
        const uint4 u = *reinterpret_cast<const uint4*>(&tile[t][c0 + 8 * k]);
        x[4 * k] = u.x; x[4 * k + 1] = u.y; x[4 * k + 2] = u.z; x[4 * k + 3] = u.w;
      }
      uint32_t word = 0;
#pragma unroll
      for (int j = 0; j < CPW; ++j) {
        const float v = (j & 1) ? hi_f16(x[j >> 1]) : lo_f16(x[j >> 1]);
        word |= code_of(v, gmn[j], ginv[j], L) << (KB * j);
      }
      a.k_codes[dst * (kGroup * WK) + t * WK + col] = word;
    }
   } else {
#pragma unroll
    for (int i = 0; i < (kGroup * WK) / kThreads; ++i) {
      const int wi = tid + i * kThreads;
      const int t = wi / WK;
      const int c0 = (wi % WK) * CPW;
      uint32_t word = 0;
#pragma unroll
      for (int j = 0; j < CPW; ++j) {
        const float2 g = st[c0 + j];
        const uint32_t q = code_of(f16_bits_to_f32(tile[t][c0 + j]), g.x, g.y, L);
        word |= q << (KB * j);
      }
      a.k_codes[dst * (kGroup * WK) + wi] = word;
    }
   }
    __syncthreads();
   }
  }

  if constexpr (VB != 0) {
   if (a.v != nullptr) {
    constexpr float L = (float)((1 << VB) - 1);
    load_tile(tile, a.v + b * a.vs_b + h * a.vs_h + (int64_t)blk * kGroup * a.vs_t, a.vs_t);
    __syncthreads();
    if (tid < kGroup * (kHeadDim / kGroup)) {   // one thread per (token, group)
      const int t = tid >> 2;
      const int g4 = tid & 3;
      const uint4* p = reinterpret_cast<const uint4*>(&tile[t][g4 * kGroup]);
      float mn = 0.f, mx = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint4 u = p[i];
        const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const float x0 = lo_f16(w[k]);
          const float x1 = hi_f16(w[k]);
          if (i == 0 && k == 0) {
            mn = fminf(x0, x1);
            mx = fmaxf(x0, x1);
          } else {
            mn = fminf(mn, fminf(x0, x1));
            mx = fmaxf(mx, fmaxf(x0, x1));
          }
        }
      }
      const GroupQ g = group_params(mn, mx, L);
      a.v_meta[(dst * kGroup + t) * (kHeadDim / kGroup) + g4] = g.meta;
      st[g4 * kGroup + t] = make_float2(g.mn, g.inv);
    }
    __syncthreads();
    // Tiled value layout: 8-token x 8-channel tiles in (token octet, channel octet)
    // order, 2*VB words each.  Word i (and i + 4 for 4-bit codes) of a tile holds token
    // pair i: the even token in bits 0..15, the odd one in bits 16..31, the tile's
    // channels VB bits apart from bit 0 of each half.
    constexpr int F = 16 / VB;                  // channels per half word
    constexpr int WT = 2 * VB;                  // words per tile
#pragma unroll
    for (int i = 0; i < (kHeadDim * VB) / kThreads; ++i) {
      const int wi = tid + i * kThreads;        // word index within the block
      const int tl = wi / WT, m = wi % WT;
      const int t0 = 8 * (tl / (kHeadDim / 8)) + 2 * (m & 3);
      const int c0 = 8 * (tl % (kHeadDim / 8)) + F * (m >> 2);
      const int g4 = c0 / kGroup;
      uint32_t word = 0;
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const float2 g = st[g4 * kGroup + t0 + hh];
#pragma unroll
        for (int j = 0; j < F; ++j) {
          const uint32_t q = code_of(f16_bits_to_f32(tile[t0 + hh][c0 + j]), g.x, g.y, L);
          word |= q << (16 * hh + VB * j);
        }
      }
      a.v_codes[dst * (kHeadDim * VB) + wi] = word;
    }
   }
  }
}

// Window append: one 16-byte chunk per thread, K rows then V rows.
__global__ __launch_bounds__(256) void append_kernel(AppendArgs a) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t per = (int64_t)a.rows * (kHeadDim / 8);   // 16-byte chunks per tensor
  if (i >= 2 * per) return;
  const bool is_v = i >= per;
  const int64_t j = is_v ? i - per : i;
  const int64_t row = j / (kHeadDim / 8);
  const int c = (int)(j % (kHeadDim / 8));
  const uint16_t* src = (is_v ? a.v_new : a.k_new) + row * kHeadDim + c * 8;
  KVQ_CHECK(a.slot >= 0 && a.slot < a.residual_len, kDbgWrite);
  uint16_t* dst = (is_v ? a.v_resid : a.k_resid) +
                  (row * a.residual_len + a.slot) * kHeadDim + c * 8;
  *reinterpret_cast<uint4*>(dst) = *reinterpret_cast<const uint4*>(src);
}

}  // namespace

hipError_t launch_quant_uniform(const QuantArgs& a, int batch, int k_bits, int v_bits,
                                hipStream_t s) {
  const int64_t jobs = (int64_t)batch * a.kv_heads * a.n_blocks;
  if (jobs == 0) return hipSuccess;
  dim3 grid((unsigned)jobs), block(kThreads);
  const int kb = a.k ? k_bits : 0;
  const int vb = a.v ? v_bits : 0;
#define KVQ_QL(KB_, VB_) \
  if (kb == KB_ && vb == VB_) { quant_uniform_kernel<KB_, VB_><<<grid, block, 0, s>>>(a); return hipGetLastError(); }
  KVQ_QL(2, 2) KVQ_QL(2, 4) KVQ_QL(4, 2) KVQ_QL(4, 4)
  KVQ_QL(2, 0) KVQ_QL(4, 0) KVQ_QL(0, 2) KVQ_QL(0, 4)
#undef KVQ_QL
  return hipErrorInvalidValue;
}

hipError_t launch_append(const AppendArgs& a, hipStream_t s) {
  const int64_t n = 2LL * a.rows * (kHeadDim / 8);
  append_kernel<<<dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s>>>(a);
  return hipGetLastError();
}

uint32_t debug_take_quant_uniform() { return debug_take_local(); }

}  // namespace kvq
