// Decode attention computed directly over the packed uniform cache.
//
// Every generated token reads the whole cache, so the step is bound by streaming
// the packed codes and metadata from HBM ("The KV cache has a geometry problem",
// section "Why the KV cache is a problem"; KIVI post, "Experiments": loading the
// cache dominates long-context generation).  Scores are q . k_hat over the packed
// tokens (dequantization fused) and over the fp16 window, then a softmax over all
// of them and the p-weighted sum of v_hat.
//
// Algebra used to keep the inner loops to one multiply-add per code:
//   q . k_hat_t = sum_d (q_d * scale_d) * code_td + sum_d q_d * min_d      (keys)
//   sum_t p_t v_hat_td = sum_t (p_t * scale_tg) * code_td + sum_t p_t * min_tg
// so a block needs one per-channel vector q*scale (keys) and one per-token
// vector p*scale (values), staged in LDS, and the min terms are one reduction.
//
// Unpacking: a 2-bit (or 4-bit) field moved into the low mantissa bits of an fp16
// half word is an fp16 subnormal of value code * 2^(pos - 24); one AND extracts two
// such codes (both fp16 halves of a register), and v_fma_mix_f32 multiplies an fp16
// half by an fp32 operand.  The power of two 2^(24 - pos) is folded into the staged
// q*scale / p*scale values.  Products are exact; sums are fp32.
//
// Work split: a workgroup of 4 waves handles one (batch, kv head) and a range of
// blocks (split-K over the context, as in flash-decoding); a wave streams one
// 32-token block at a time (lane = token x channel half for keys, lane = channel
// pair for values), with the next block's loads in flight.  The fp16 window is an
// extra split.  Waves merge in LDS.  With one split per (batch, kv head) the
// workgroup writes the output; otherwise it writes a (max, sum, output) partial and a
// second small launch merges the splits.
#include "kvq_common.h"

namespace kvq {
namespace {

constexpr float kNegInf = -__builtin_inff();
constexpr int kWindowUnits = 4;   // a 32-token fp16 window chunk weighs as 4 packed blocks

// Bit position of field j (within its 16-bit half, after the shift used to reach
// it) for a word holding 32/B fields of B bits.
__host__ __device__ constexpr int field_pos(int bits, int j) {
  return bits == 2 ? (j < 5 ? 2 * j : j < 8 ? 2 * (j - 5) : j < 13 ? 2 * (j - 8) : 2 * (j - 13))
                   : 4 * (j & 1);
}
// 2^(24 - pos): undoes the subnormal scaling of a field.
__device__ __forceinline__ float field_scale(int bits, int j) {
  return __builtin_bit_cast(float, (uint32_t)(127 + 24 - field_pos(bits, j)) << 23);
}

// acc += sum_j w_j * field_j(word), with w the 32/B weights of the word's fields.
template <int B>
__device__ __forceinline__ float dot_word(uint32_t w, const float* wt, float acc) {
  if constexpr (B == 2) {
    const uint32_t w10 = w >> 10;
    uint32_t x;
    x = w & 0x00030003u;   acc = fmaf(wt[0], lo_f16(x), acc);  acc = fmaf(wt[8], hi_f16(x), acc);
    x = w & 0x000C000Cu;   acc = fmaf(wt[1], lo_f16(x), acc);  acc = fmaf(wt[9], hi_f16(x), acc);
    x = w & 0x00300030u;   acc = fmaf(wt[2], lo_f16(x), acc);  acc = fmaf(wt[10], hi_f16(x), acc);
    x = w & 0x00C000C0u;   acc = fmaf(wt[3], lo_f16(x), acc);  acc = fmaf(wt[11], hi_f16(x), acc);
    x = w & 0x03000300u;   acc = fmaf(wt[4], lo_f16(x), acc);  acc = fmaf(wt[12], hi_f16(x), acc);
    x = w10 & 0x00030003u; acc = fmaf(wt[5], lo_f16(x), acc);  acc = fmaf(wt[13], hi_f16(x), acc);
    x = w10 & 0x000C000Cu; acc = fmaf(wt[6], lo_f16(x), acc);  acc = fmaf(wt[14], hi_f16(x), acc);
    x = w10 & 0x00300030u; acc = fmaf(wt[7], lo_f16(x), acc);  acc = fmaf(wt[15], hi_f16(x), acc);
  } else {
    const uint32_t w8 = w >> 8;
    uint32_t x;
    x = w & 0x000F000Fu;  acc = fmaf(wt[0], lo_f16(x), acc);  acc = fmaf(wt[4], hi_f16(x), acc);
    x = w & 0x00F000F0u;  acc = fmaf(wt[1], lo_f16(x), acc);  acc = fmaf(wt[5], hi_f16(x), acc);
    x = w8 & 0x000F000Fu; acc = fmaf(wt[2], lo_f16(x), acc);  acc = fmaf(wt[6], hi_f16(x), acc);
    x = w8 & 0x00F000F0u; acc = fmaf(wt[3], lo_f16(x), acc);  acc = fmaf(wt[7], hi_f16(x), acc);
  }
  return acc;
}

// DPP lane permutations (gfx9 encodings): quad_perm, row mirrors, row broadcasts.
template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ float dpp(float old, float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(__builtin_bit_cast(int, old),
                                                               __builtin_bit_cast(int, x), CTRL,
                                                               ROW_MASK, 0xF, false));
}
constexpr int kQuadSwap1 = 0xB1;      // quad_perm [1,0,3,2]
constexpr int kQuadSwap2 = 0x4E;      // quad_perm [2,3,0,1]
constexpr int kRowHalfMirror = 0x141;
constexpr int kRowMirror = 0x140;
constexpr int kRowBcast15 = 0x142;
constexpr int kRowBcast31 = 0x143;

__device__ __forceinline__ float readlane63(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 63));
}
// Sum over all 64 lanes, returned wave-uniform.
__device__ __forceinline__ float wave_sum(float x) {
  x += dpp<kQuadSwap1>(0.f, x);
  x += dpp<kQuadSwap2>(0.f, x);
  x += dpp<kRowHalfMirror>(0.f, x);
  x += dpp<kRowMirror>(0.f, x);
  x += dpp<kRowBcast15, 0xA>(0.f, x);
  x += dpp<kRowBcast31, 0xC>(0.f, x);
  return readlane63(x);
}
// Max over all 64 lanes, returned wave-uniform.
__device__ __forceinline__ float wave_max(float x) {
  x = fmaxf(x, dpp<kQuadSwap1>(kNegInf, x));
  x = fmaxf(x, dpp<kQuadSwap2>(kNegInf, x));
  x = fmaxf(x, dpp<kRowHalfMirror>(kNegInf, x));
  x = fmaxf(x, dpp<kRowMirror>(kNegInf, x));
  x = fmaxf(x, dpp<kRowBcast15, 0xA>(kNegInf, x));
  x = fmaxf(x, dpp<kRowBcast31, 0xC>(kNegInf, x));
  return readlane63(x);
}
__device__ __forceinline__ float sum32(float x) {   // over lane bits 0..4
#pragma unroll
  for (int o = 1; o < 32; o <<= 1) x += __shfl_xor(x, o);
  return x;
}

template <int KB, int VB>
struct BlockRegs {
  uint32_t kc[kHeadDim * KB / 64];   // this lane's half of a token row
  uint32_t km[2];                    // key meta of channels 2l, 2l+1
  uint32_t vc[2 * VB];               // value rows of channels 2l, 2l+1
  uint32_t vm[2];                    // value meta of token t, groups 2h, 2h+1
};

template <int KB, int VB>
__device__ __forceinline__ void load_block(BlockRegs<KB, VB>& r, const DecodeArgs& a,
                                           int64_t blk, int lane) {
  constexpr int WK = kHeadDim * KB / 32;
  const int t = lane & 31, half = lane >> 5;
  const uint4* kp = reinterpret_cast<const uint4*>(a.k_codes + blk * (kGroup * WK) +
                                                   t * WK + half * (WK / 2));
#pragma unroll
  for (int i = 0; i < WK / 8; ++i) {
    const uint4 u = kp[i];
    r.kc[4 * i] = u.x; r.kc[4 * i + 1] = u.y; r.kc[4 * i + 2] = u.z; r.kc[4 * i + 3] = u.w;
  }
  const uint2 km = *reinterpret_cast<const uint2*>(a.k_meta + blk * kHeadDim + 2 * lane);
  r.km[0] = km.x; r.km[1] = km.y;
  const uint4* vp = reinterpret_cast<const uint4*>(a.v_codes + blk * (kHeadDim * VB) +
                                                   2 * lane * VB);
#pragma unroll
  for (int i = 0; i < VB / 2; ++i) {
    const uint4 u = vp[i];
    r.vc[4 * i] = u.x; r.vc[4 * i + 1] = u.y; r.vc[4 * i + 2] = u.z; r.vc[4 * i + 3] = u.w;
  }
  const uint2 vm = *reinterpret_cast<const uint2*>(a.v_meta + (blk * kGroup + t) * 4 + 2 * half);
  r.vm[0] = vm.x; r.vm[1] = vm.y;
}

template <int GQ>
struct WaveState {
  float m[GQ];        // running max (log2 domain), wave-uniform
  float l[GQ];        // this lane's sum of p over its tokens
  float o[GQ][2];     // output accumulators of channels 2l, 2l+1
  float mv[GQ][2];    // sum_t p_t * min_tg for groups 2h, 2h+1 (token lanes)
};

// Online softmax update for one head; s is this lane's token score (log2 units; the
// two lane halves hold the same tokens).  The block maximum is only reduced when some
// score exceeds the running maximum, which after the first blocks is rare.
__device__ __forceinline__ float softmax_step(float s, float& m, float& l, float& alpha) {
  alpha = 1.0f;
  if (__any(s > m)) {
    const float mn = fmaxf(m, wave_max(s));
    alpha = exp2f(m - mn);
    m = mn;
    l *= alpha;
  }
  const float p = exp2f(s - m);
  l += p;
  return p;
}

template <int KB, int VB, int GQ>
__device__ __forceinline__ void process_block(const BlockRegs<KB, VB>& r, WaveState<GQ>& st,
                                              const uint32_t* qreg, float (*qsL)[kHeadDim],
                                              float (*psL)[4][kGroup], float scale_log2,
                                              int lane) {
  constexpr int WK = kHeadDim * KB / 32;
  constexpr int CPW = 32 / KB;
  constexpr int TPW = 32 / VB;
  const int t = lane & 31, half = lane >> 5;

  // ---- keys: q*scale per channel into LDS, q.min reduced over the wave
  const float ks0 = lo_f16(r.km[0]), kn0 = hi_f16(r.km[0]);
  const float ks1 = lo_f16(r.km[1]), kn1 = hi_f16(r.km[1]);
  const float f0 = field_scale(KB, (2 * lane) % CPW), f1 = field_scale(KB, (2 * lane + 1) % CPW);
  float cmin[GQ];
#pragma unroll
  for (int j = 0; j < GQ; ++j) {
    const float q0 = lo_f16(qreg[j]), q1 = hi_f16(qreg[j]);
    *reinterpret_cast<float2*>(&qsL[j][2 * lane]) = make_float2(q0 * ks0 * f0, q1 * ks1 * f1);
    cmin[j] = q0 * kn0 + q1 * kn1;
  }
#pragma unroll
  for (int j = 0; j < GQ; ++j) cmin[j] = wave_sum(cmin[j]);

  float s[GQ];
#pragma unroll
  for (int j = 0; j < GQ; ++j) {
    float acc = 0.f;
#pragma unroll
    for (int wi = 0; wi < WK / 2; ++wi) {
      float wt[CPW];
      const float4* qp = reinterpret_cast<const float4*>(&qsL[j][half * 64 + wi * CPW]);
#pragma unroll
      for (int k = 0; k < CPW / 4; ++k) {
        const float4 v = qp[k];
        wt[4 * k] = v.x; wt[4 * k + 1] = v.y; wt[4 * k + 2] = v.z; wt[4 * k + 3] = v.w;
      }
      acc = dot_word<KB>(r.kc[wi], wt, acc);
    }
    acc += __shfl_xor(acc, 32);
    s[j] = (acc + cmin[j]) * scale_log2;
  }

  // ---- softmax
  float p[GQ], alpha[GQ];
#pragma unroll
  for (int j = 0; j < GQ; ++j) p[j] = softmax_step(s[j], st.m[j], st.l[j], alpha[j]);

  // ---- values: p*scale per token into LDS, p*min accumulated per lane
  const float vs0 = lo_f16(r.vm[0]), vn0 = hi_f16(r.vm[0]);
  const float vs1 = lo_f16(r.vm[1]), vn1 = hi_f16(r.vm[1]);
  const float ft = field_scale(VB, t % TPW);
#pragma unroll
  for (int j = 0; j < GQ; ++j) {
    psL[j][2 * half][t] = p[j] * vs0 * ft;
    psL[j][2 * half + 1][t] = p[j] * vs1 * ft;
    st.mv[j][0] = st.mv[j][0] * alpha[j] + p[j] * vn0;
    st.mv[j][1] = st.mv[j][1] * alpha[j] + p[j] * vn1;
  }
  const int gi = lane >> 4;
#pragma unroll
  for (int j = 0; j < GQ; ++j) {
    float wt[kGroup];
    const float4* pp = reinterpret_cast<const float4*>(&psL[j][gi][0]);
#pragma unroll
    for (int k = 0; k < kGroup / 4; ++k) {
      const float4 v = pp[k];
      wt[4 * k] = v.x; wt[4 * k + 1] = v.y; wt[4 * k + 2] = v.z; wt[4 * k + 3] = v.w;
    }
    float o0 = st.o[j][0] * alpha[j], o1 = st.o[j][1] * alpha[j];
#pragma unroll
    for (int w = 0; w < VB; ++w) {
      o0 = dot_word<VB>(r.vc[w], wt + w * TPW, o0);
      o1 = dot_word<VB>(r.vc[VB + w], wt + w * TPW, o1);
    }
    st.o[j][0] = o0;
    st.o[j][1] = o1;
  }
}

// One chunk of up to 32 fp16 window tokens.
template <int GQ>
__device__ __forceinline__ void process_window(const DecodeArgs& a, int64_t bh, int c,
                                               WaveState<GQ>& st, const uint32_t (*qh)[64],
                                               float (*pL)[kGroup], int lane) {
  const int t = lane & 31, half = lane >> 5;
  const int tok0 = c * kGroup;
  const int nvalid = min(kGroup, a.n_resid - tok0);
  const bool valid = t < nvalid;
  const uint16_t* kr = a.k_resid + (bh * a.residual_len + tok0) * kHeadDim;
  uint32_t kw[32];
  if (valid) {
    const uint4* kp = reinterpret_cast<const uint4*>(kr + t * kHeadDim + half * 64);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint4 u = kp[i];
      kw[4 * i] = u.x; kw[4 * i + 1] = u.y; kw[4 * i + 2] = u.z; kw[4 * i + 3] = u.w;
    }
  } else {
#pragma unroll
    for (int i = 0; i < 32; ++i) kw[i] = 0;
  }
  float p[GQ], alpha[GQ];
#pragma unroll
  for (int j = 0; j < GQ; ++j) {
    float acc = 0.f;
    const uint4* qp = reinterpret_cast<const uint4*>(&qh[j][half * 32]);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint4 u = qp[i];
      acc = __builtin_amdgcn_fdot2(as_h2(kw[4 * i]), as_h2(u.x), acc, false);
      acc = __builtin_amdgcn_fdot2(as_h2(kw[4 * i + 1]), as_h2(u.y), acc, false);
      acc = __builtin_amdgcn_fdot2(as_h2(kw[4 * i + 2]), as_h2(u.z), acc, false);
      acc = __builtin_amdgcn_fdot2(as_h2(kw[4 * i + 3]), as_h2(u.w), acc, false);
    }
    acc += __shfl_xor(acc, 32);
    const float s = valid ? acc * a.scale_log2 : kNegInf;
    p[j] = softmax_step(s, st.m[j], st.l[j], alpha[j]);
    if (half == 0) pL[j][t] = p[j];
  }
  const uint16_t* vr = a.v_resid + (bh * a.residual_len + tok0) * kHeadDim + 2 * lane;
#pragma unroll
  for (int j = 0; j < GQ; ++j) {
    st.o[j][0] *= alpha[j];
    st.o[j][1] *= alpha[j];
    st.mv[j][0] *= alpha[j];
    st.mv[j][1] *= alpha[j];
  }
  uint32_t vw[kGroup];
#pragma unroll
  for (int k = 0; k < kGroup; ++k)
    vw[k] = *reinterpret_cast<const uint32_t*>(vr + min(k, nvalid - 1) * kHeadDim);
#pragma unroll
  for (int j = 0; j < GQ; ++j) {
    const float4* pp = reinterpret_cast<const float4*>(&pL[j][0]);
    float o0 = st.o[j][0], o1 = st.o[j][1];
#pragma unroll
    for (int k4 = 0; k4 < kGroup / 4; ++k4) {
      const float4 p4 = pp[k4];
      const float pk[4] = {p4.x, p4.y, p4.z, p4.w};
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        o0 = fmaf(pk[u], lo_f16(vw[4 * k4 + u]), o0);
        o1 = fmaf(pk[u], hi_f16(vw[4 * k4 + u]), o1);
      }
    }
    st.o[j][0] = o0;
    st.o[j][1] = o1;
  }
}

// Work units: packed block i is unit i (0 <= i < n_blocks); window chunk c (32 fp16
// tokens) is units [n_blocks + kWindowUnits*c, n_blocks + kWindowUnits*(c+1)), weighted
// by its larger byte count.  A split covers a contiguous unit range; each wave of the
// split covers a contiguous sub-range: the packed blocks in it, and every window
// chunk whose first unit falls in it.
template <int KB, int VB, int GQ, int NW>
__global__ __launch_bounds__(NW * kWave) void decode_uniform_kernel(DecodeArgs a) {
  constexpr int NT = NW * kWave;
  __shared__ __align__(16) uint32_t qh[GQ][64];
  __shared__ __align__(16) float qsL[NW][GQ][kHeadDim];
  __shared__ __align__(16) float psL[NW][GQ][4][kGroup];
  __shared__ float wm[NW][GQ], wl[NW][GQ];
  __shared__ __align__(16) float wo[NW][GQ][kHeadDim];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform
  const int split = blockIdx.x % a.splits;
  const int64_t bh = blockIdx.x / a.splits;
  const int b = (int)(bh / a.kv_heads);
  const int hkv = (int)(bh % a.kv_heads);
  const int hq0 = hkv * GQ;

  uint32_t qreg[GQ];
#pragma unroll
  for (int j = 0; j < GQ; ++j) {
    qreg[j] = *reinterpret_cast<const uint32_t*>(a.q + ((int64_t)b * a.q_heads + hq0 + j) *
                                                           kHeadDim + 2 * lane);
    if (wave == 0) qh[j][lane] = qreg[j];
  }
  __syncthreads();

  WaveState<GQ> st;
#pragma unroll
  for (int j = 0; j < GQ; ++j) {
    st.m[j] = kNegInf;
    st.l[j] = 0.f;
    st.o[j][0] = st.o[j][1] = 0.f;
    st.mv[j][0] = st.mv[j][1] = 0.f;
  }

  const int nchunks = (a.n_resid + kGroup - 1) / kGroup;
  const int units = a.n_blocks + kWindowUnits * nchunks;
  const int s0 = (int)((int64_t)units * split / a.splits);
  const int s1 = (int)((int64_t)units * (split + 1) / a.splits);
  const int w0 = s0 + (int)((int64_t)(s1 - s0) * wave / NW);
  const int w1 = s0 + (int)((int64_t)(s1 - s0) * (wave + 1) / NW);

  // ---- window chunks first (their loads are short), then the packed blocks
  for (int c = 0; c < nchunks; ++c) {
    const int u = a.n_blocks + kWindowUnits * c;
    if (u >= w0 && u < w1)
      process_window<GQ>(a, bh, c, st, qh, reinterpret_cast<float(*)[kGroup]>(psL[wave]), lane);
  }
  const int b0 = w0, b1 = min(w1, a.n_blocks);
  if (b0 < b1) {
    const int64_t base = bh * a.cap_blocks;
    // Two blocks in flight ahead of the one being processed.  The prefetch index is
    // clamped rather than guarded so every iteration issues the same loads, and the
    // loop is unrolled by three with rotating roles so no register copy has to wait
    // for the loads just issued.
    const int last = b1 - 1;
    BlockRegs<KB, VB> r0, r1, r2;
    load_block<KB, VB>(r0, a, base + b0, lane);
    load_block<KB, VB>(r1, a, base + min(b0 + 1, last), lane);
    for (int i = b0; i < b1; i += 3) {
      load_block<KB, VB>(r2, a, base + min(i + 2, last), lane);
      process_block<KB, VB, GQ>(r0, st, qreg, qsL[wave], psL[wave], a.scale_log2, lane);
      if (i + 1 >= b1) break;
      load_block<KB, VB>(r0, a, base + min(i + 3, last), lane);
      process_block<KB, VB, GQ>(r1, st, qreg, qsL[wave], psL[wave], a.scale_log2, lane);
      if (i + 2 >= b1) break;
      load_block<KB, VB>(r1, a, base + min(i + 4, last), lane);
      process_block<KB, VB, GQ>(r2, st, qreg, qsL[wave], psL[wave], a.scale_log2, lane);
    }
  }

  // ---- finish the wave: totals of l and of the min terms, then the WG merge
  const int k_sel = (lane >> 4) & 1;
#pragma unroll
  for (int j = 0; j < GQ; ++j) {
    const float lt = sum32(st.l[j]);
    const float mv0 = sum32(st.mv[j][0]);
    const float mv1 = sum32(st.mv[j][1]);
    const float mvg = k_sel ? mv1 : mv0;
    if (lane == 0) {
      wm[wave][j] = st.m[j];
      wl[wave][j] = lt;
    }
    *reinterpret_cast<float2*>(&wo[wave][j][2 * lane]) =
        make_float2(st.o[j][0] + mvg, st.o[j][1] + mvg);
  }
  __syncthreads();

  const bool single = a.splits == 1;
  for (int idx = threadIdx.x; idx < GQ * kHeadDim; idx += NT) {
    const int j = idx >> 7, d = idx & 127;
    float M = kNegInf;
#pragma unroll
    for (int w = 0; w < NW; ++w) M = fmaxf(M, wm[w][j]);
    float L = 0.f, O = 0.f;
    if (M != kNegInf) {
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        const float e = exp2f(wm[w][j] - M);
        L += wl[w][j] * e;
        O += wo[w][j][d] * e;
      }
    }
    const int64_t row = (int64_t)b * a.q_heads + hq0 + j;
    if (single) {
      a.out[row * kHeadDim + d] = L > 0.f ? O / L : 0.f;
    } else {
      float* P = a.partials + (row * a.splits + split) * kPartialStride;
      P[d] = O;
      if (d == 0) {
        P[kHeadDim] = M;
        P[kHeadDim + 1] = L;
      }
    }
  }
}

// Combines the per-split (max, sum, output) partials of one (batch, query head) row.
// A separate launch: the kernel boundary makes every split's stores visible, which
// costs far less than device-scope fences in each workgroup of the main kernel.  The
// split weights are computed in parallel into LDS; each output channel then sums its
// splits with independent loads.
constexpr int kMergeThreads = 256;

__device__ __forceinline__ float block_reduce(float x, float* red, bool is_max) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float y = __shfl_xor(x, o);
    x = is_max ? fmaxf(x, y) : x + y;
  }
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = x;
  __syncthreads();
  float r = red[0];
#pragma unroll
  for (int w = 1; w < kMergeThreads / kWave; ++w) r = is_max ? fmaxf(r, red[w]) : r + red[w];
  __syncthreads();
  return r;
}

__global__ __launch_bounds__(kMergeThreads) void merge_splits_kernel(const float* partials,
                                                                    float* out, int splits) {
  __shared__ float wgt[kMaxSplits];
  __shared__ float red[kMergeThreads / kWave];
  __shared__ float half_o[kHeadDim];
  const int64_t row = blockIdx.x;
  const int tid = threadIdx.x;
  const float* P = partials + row * splits * kPartialStride;
  float m = kNegInf;
  for (int s = tid; s < splits; s += kMergeThreads) m = fmaxf(m, P[s * kPartialStride + kHeadDim]);
  const float M = block_reduce(m, red, true);
  float l = 0.f;
  for (int s = tid; s < splits; s += kMergeThreads) {
    const float e = M == kNegInf ? 0.f : exp2f(P[s * kPartialStride + kHeadDim] - M);
    wgt[s] = e;
    l += P[s * kPartialStride + kHeadDim + 1] * e;
  }
  const float L = block_reduce(l, red, false);     // its barrier also publishes wgt[]
  const int d = tid & (kHeadDim - 1), part = tid >> 7;
  float o0 = 0.f, o1 = 0.f, o2 = 0.f, o3 = 0.f;
  int s = part;
  for (; s + 6 < splits; s += 8) {
    o0 += P[s * kPartialStride + d] * wgt[s];
    o1 += P[(s + 2) * kPartialStride + d] * wgt[s + 2];
    o2 += P[(s + 4) * kPartialStride + d] * wgt[s + 4];
    o3 += P[(s + 6) * kPartialStride + d] * wgt[s + 6];
  }
  for (; s < splits; s += 2) o0 += P[s * kPartialStride + d] * wgt[s];
  const float o = (o0 + o1) + (o2 + o3);
  if (part == 1) half_o[d] = o;
  __syncthreads();
  if (part == 0) out[row * kHeadDim + d] = L > 0.f ? (o + half_o[d]) / L : 0.f;
}

}  // namespace

hipError_t launch_decode_uniform(const DecodeArgs& a, int k_bits, int v_bits, int gq,
                                 hipStream_t s) {
  const int64_t wgs = (int64_t)a.batch * a.kv_heads * a.splits;
  const int nw = a.waves_per_group;
  dim3 grid((unsigned)wgs), block((unsigned)(nw * kWave));
#define KVQ_DL(KB_, VB_, G_, NW_)                                                   \
  if (k_bits == KB_ && v_bits == VB_ && gq == G_ && nw == NW_) {                    \
    decode_uniform_kernel<KB_, VB_, G_, NW_><<<grid, block, 0, s>>>(a);             \
    hipError_t e_ = hipGetLastError();                                              \
    if (e_ != hipSuccess || a.splits == 1) return e_;                               \
    return launch_merge_splits(a, s);                                               \
  }
#define KVQ_DLB(G_, NW_) KVQ_DL(2, 2, G_, NW_) KVQ_DL(2, 4, G_, NW_) KVQ_DL(4, 2, G_, NW_) \
  KVQ_DL(4, 4, G_, NW_)
  KVQ_DLB(1, 4) KVQ_DLB(2, 4) KVQ_DLB(4, 4) KVQ_DLB(8, 4)
  KVQ_DLB(1, 8) KVQ_DLB(2, 8) KVQ_DLB(4, 8) KVQ_DLB(8, 8)
  KVQ_DLB(1, 16)
#undef KVQ_DLB
#undef KVQ_DL
  return hipErrorInvalidValue;
}

hipError_t launch_merge_splits(const DecodeArgs& a, hipStream_t s) {
  const int64_t rows = (int64_t)a.batch * a.q_heads;
  merge_splits_kernel<<<dim3((unsigned)rows), dim3(kMergeThreads), 0, s>>>(a.partials, a.out,
                                                                           a.splits);
  return hipGetLastError();
}

}  // namespace kvq
