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

// acc[T] += w0 * code(even token, channel T) + w1 * code(odd token, channel T) over the
// channels of one word of the tiled value layout (8 channels for 2-bit codes, 4 for
// 4-bit codes).  Each accumulator keeps the 2^(pos - 24) factor of its field position,
// which is undone once at the end.
template <int B>
__device__ __forceinline__ void vdot_word(uint32_t w, float w0, float w1, float* acc) {
  if constexpr (B == 2) {
    const uint32_t w10 = w >> 10;
    uint32_t x;
    x = w & 0x00030003u;   acc[0] = fmaf(w0, lo_f16(x), acc[0]);  acc[0] = fmaf(w1, hi_f16(x), acc[0]);
    x = w & 0x000C000Cu;   acc[1] = fmaf(w0, lo_f16(x), acc[1]);  acc[1] = fmaf(w1, hi_f16(x), acc[1]);
    x = w & 0x00300030u;   acc[2] = fmaf(w0, lo_f16(x), acc[2]);  acc[2] = fmaf(w1, hi_f16(x), acc[2]);
    x = w & 0x00C000C0u;   acc[3] = fmaf(w0, lo_f16(x), acc[3]);  acc[3] = fmaf(w1, hi_f16(x), acc[3]);
    x = w & 0x03000300u;   acc[4] = fmaf(w0, lo_f16(x), acc[4]);  acc[4] = fmaf(w1, hi_f16(x), acc[4]);
    x = w10 & 0x00030003u; acc[5] = fmaf(w0, lo_f16(x), acc[5]);  acc[5] = fmaf(w1, hi_f16(x), acc[5]);
    x = w10 & 0x000C000Cu; acc[6] = fmaf(w0, lo_f16(x), acc[6]);  acc[6] = fmaf(w1, hi_f16(x), acc[6]);
    x = w10 & 0x00300030u; acc[7] = fmaf(w0, lo_f16(x), acc[7]);  acc[7] = fmaf(w1, hi_f16(x), acc[7]);
  } else {
    const uint32_t w8 = w >> 8;
    uint32_t x;
    x = w & 0x000F000Fu;  acc[0] = fmaf(w0, lo_f16(x), acc[0]);  acc[0] = fmaf(w1, hi_f16(x), acc[0]);
    x = w & 0x00F000F0u;  acc[1] = fmaf(w0, lo_f16(x), acc[1]);  acc[1] = fmaf(w1, hi_f16(x), acc[1]);
    x = w8 & 0x000F000Fu; acc[2] = fmaf(w0, lo_f16(x), acc[2]);  acc[2] = fmaf(w1, hi_f16(x), acc[2]);
    x = w8 & 0x00F000F0u; acc[3] = fmaf(w0, lo_f16(x), acc[3]);  acc[3] = fmaf(w1, hi_f16(x), acc[3]);
  }
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// LDS rows of the per-block weights: 32 floats padded to 40, so that rows read by the
// lanes of one 8-lane LDS cycle start on different banks.
constexpr int kRow = 40;

// Lane roles inside a wave for one 32-token block:
//   keys   : lane = 4 * tp + q: tokens tp and tp + 16, channels 32q .. 32q + 31 (the
//            four lanes of a quad share a token pair and sum their partial scores);
//   values : lane = 16 * o + n: tokens 8o .. 8o + 7, channels 8n .. 8n + 7 (one tile);
//   meta   : key scale/min of channels 2*lane, 2*lane + 1; value scale/min of tokens
//            tp and tp + 16 in group q.
template <int KB, int VB>
struct BlockRegs {
  uint32_t ka[KB];     // token tp, channel quarter q
  uint32_t kb[KB];     // token tp + 16
  uint32_t km[2];      // key meta of channels 2l, 2l+1
  uint32_t vc[2 * VB]; // value tile
  uint32_t vm[2];      // value meta (tp, q), (tp + 16, q)
};

// Base pointers of one (batch, kv head) cache segment.
struct HeadPtrs {
  const uint32_t* kc;
  const uint32_t* km;
  const uint32_t* vc;
  const uint32_t* vm;
};

// Loads of block `blk` (wave-uniform) of a segment: the block's base address is scalar
// arithmetic, each lane adds a fixed 32-bit offset.
template <int KB, int VB>
__device__ __forceinline__ void load_block(BlockRegs<KB, VB>& r, const HeadPtrs& hp, int blk,
                                           int lane) {
  constexpr int WK = kHeadDim * KB / 32;            // words per token row
  const int tp = lane >> 2, q = lane & 3;
  const uint32_t* kp = hp.kc + (uint32_t)blk * (kGroup * WK);
  const uint32_t ka_off = (uint32_t)(tp * WK + q * KB), kb_off = ka_off + 16 * WK;
  if constexpr (KB == 2) {
    const uint2 x = *reinterpret_cast<const uint2*>(kp + ka_off);
    const uint2 y = *reinterpret_cast<const uint2*>(kp + kb_off);
    r.ka[0] = x.x; r.ka[1] = x.y; r.kb[0] = y.x; r.kb[1] = y.y;
  } else {
    const uint4 x = *reinterpret_cast<const uint4*>(kp + ka_off);
    const uint4 y = *reinterpret_cast<const uint4*>(kp + kb_off);
    r.ka[0] = x.x; r.ka[1] = x.y; r.ka[2] = x.z; r.ka[3] = x.w;
    r.kb[0] = y.x; r.kb[1] = y.y; r.kb[2] = y.z; r.kb[3] = y.w;
  }
  const uint2 km = *reinterpret_cast<const uint2*>(hp.km + (uint32_t)blk * kHeadDim +
                                                   (uint32_t)(2 * lane));
  r.km[0] = km.x; r.km[1] = km.y;
  const uint4* vp = reinterpret_cast<const uint4*>(hp.vc + (uint32_t)blk * (kHeadDim * VB) +
                                                   (uint32_t)(lane * 2 * VB));
#pragma unroll
  for (int i = 0; i < VB / 2; ++i) {
    const uint4 u = vp[i];
    r.vc[4 * i] = u.x; r.vc[4 * i + 1] = u.y; r.vc[4 * i + 2] = u.z; r.vc[4 * i + 3] = u.w;
  }
  const uint32_t* vm = hp.vm + (uint32_t)blk * (kGroup * 4);
  r.vm[0] = vm[(uint32_t)lane];
  r.vm[1] = vm[(uint32_t)lane + 64];
}

template <int GQ>
struct WaveState {
  float m[GQ];          // running max (log2 domain), wave-uniform
  float l[GQ];          // this lane's sum of p (every token counted by 4 lanes)
  float mv[GQ];         // sum of p * min over this lane's two tokens, group q
  float acc[GQ][8];     // packed values, channels 8n + T (field-scaled)
  float ow[GQ][8];      // fp16 window values, channels 8n + T
};

// Online softmax for one head over this lane's two scores; the running maximum is only
// reduced over the wave when some score exceeds it (after the first blocks: rarely).
template <int GQ>
__device__ __forceinline__ void softmax_pair(WaveState<GQ>& st, int j, float sA, float sB,
                                             float& pA, float& pB) {
  const float smax = fmaxf(sA, sB);
  if (__any(smax > st.m[j])) {
    const float mn = fmaxf(st.m[j], wave_max(smax));
    const float alpha = fast_exp2(st.m[j] - mn);     // 0 while m = -inf
    st.m[j] = mn;
    st.l[j] *= alpha;
    st.mv[j] *= alpha;
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      st.acc[j][t] *= alpha;
      st.ow[j][t] *= alpha;
    }
  }
  pA = fast_exp2(sA - st.m[j]);
  pB = fast_exp2(sB - st.m[j]);
  st.l[j] += pA + pB;
}

__device__ __forceinline__ float quad_sum(float x) {
  x += dpp<kQuadSwap1>(0.f, x);
  x += dpp<kQuadSwap2>(0.f, x);
  return x;
}

template <int KB, int VB, int GQ>
__device__ __forceinline__ void process_block(const BlockRegs<KB, VB>& r, WaveState<GQ>& st,
                                              const uint32_t* qreg, const float (*qf)[2],
                                              float cscale, float (*qsL)[4][kRow],
                                              float (*psL)[4][kRow], int lane) {
  constexpr int CPW = 32 / KB;                       // key channels per word
  const int tp = lane >> 2, q = lane & 3;
  const int n = lane & 15, o = lane >> 4;

  // ---- keys: q * scale of channels 2l, 2l+1 into LDS; q . min reduced over the wave
  const uint32_t kmin2 = __builtin_amdgcn_perm(r.km[1], r.km[0], 0x07060302u);
  float cmin[GQ];
#pragma unroll
  for (int j = 0; j < GQ; ++j) {
    *reinterpret_cast<float2*>(&qsL[j][lane >> 4][(2 * lane) & 31]) =
        make_float2(qf[j][0] * lo_f16(r.km[0]), qf[j][1] * lo_f16(r.km[1]));
    cmin[j] = __builtin_amdgcn_fdot2(as_h2(qreg[j]), as_h2(kmin2), 0.0f, false);
  }
#pragma unroll
  for (int j = 0; j < GQ; ++j) cmin[j] = wave_sum(cmin[j]) * cscale;

  const float vsA = lo_f16(r.vm[0]), vnA = hi_f16(r.vm[0]);
  const float vsB = lo_f16(r.vm[1]), vnB = hi_f16(r.vm[1]);
#pragma unroll
  for (int j = 0; j < GQ; ++j) {
    float wt[32];
    const float4* qp = reinterpret_cast<const float4*>(&qsL[j][q][0]);
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const float4 v = qp[k];
      wt[4 * k] = v.x; wt[4 * k + 1] = v.y; wt[4 * k + 2] = v.z; wt[4 * k + 3] = v.w;
    }
    float a0 = 0.f, a1 = 0.f, b0 = 0.f, b1 = 0.f;
#pragma unroll
    for (int e = 0; e < KB; e += 2) {
      a0 = dot_word<KB>(r.ka[e], wt + e * CPW, a0);
      a1 = dot_word<KB>(r.ka[e + 1], wt + (e + 1) * CPW, a1);
      b0 = dot_word<KB>(r.kb[e], wt + e * CPW, b0);
      b1 = dot_word<KB>(r.kb[e + 1], wt + (e + 1) * CPW, b1);
    }
    const float sA = quad_sum(a0 + a1) + cmin[j];
    const float sB = quad_sum(b0 + b1) + cmin[j];

    float pA, pB;
    softmax_pair<GQ>(st, j, sA, sB, pA, pB);

    // ---- values: p * scale of tokens tp, tp + 16 (group q) into LDS, p * min per lane
    psL[j][q][tp] = pA * vsA;
    psL[j][q][tp + 16] = pB * vsB;
    st.mv[j] = fmaf(pA, vnA, fmaf(pB, vnB, st.mv[j]));

    float wv[8];
    const float4* pp = reinterpret_cast<const float4*>(&psL[j][n >> 2][8 * o]);
    const float4 u0 = pp[0], u1 = pp[1];
    wv[0] = u0.x; wv[1] = u0.y; wv[2] = u0.z; wv[3] = u0.w;
    wv[4] = u1.x; wv[5] = u1.y; wv[6] = u1.z; wv[7] = u1.w;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if constexpr (VB == 2) {
        vdot_word<2>(r.vc[i], wv[2 * i], wv[2 * i + 1], st.acc[j]);
      } else {
        vdot_word<4>(r.vc[i], wv[2 * i], wv[2 * i + 1], st.acc[j]);
        vdot_word<4>(r.vc[i + 4], wv[2 * i], wv[2 * i + 1], st.acc[j] + 4);
      }
    }
  }
}

// One chunk of up to 32 fp16 window tokens, with the same lane roles as a packed block.
template <int GQ>
__device__ __forceinline__ void process_window(const DecodeArgs& a, int64_t bh, int c,
                                               WaveState<GQ>& st, const uint32_t (*qh)[64],
                                               float (*pL)[kGroup], int lane) {
  const int tp = lane >> 2, q = lane & 3;
  const int n = lane & 15, o = lane >> 4;
  const int tok0 = c * kGroup;
  const int nvalid = min(kGroup, a.n_resid - tok0);
  const uint16_t* kr = a.k_resid + (bh * a.residual_len + tok0) * kHeadDim + 32 * q;
  const uint16_t* vr = a.v_resid + (bh * a.residual_len + tok0) * kHeadDim + 8 * n;
  uint32_t ka[16], kb[16];
  {
    const uint4* pa = reinterpret_cast<const uint4*>(kr + min(tp, nvalid - 1) * kHeadDim);
    const uint4* pb = reinterpret_cast<const uint4*>(kr + min(tp + 16, nvalid - 1) * kHeadDim);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint4 x = pa[i], y = pb[i];
      ka[4 * i] = x.x; ka[4 * i + 1] = x.y; ka[4 * i + 2] = x.z; ka[4 * i + 3] = x.w;
      kb[4 * i] = y.x; kb[4 * i + 1] = y.y; kb[4 * i + 2] = y.z; kb[4 * i + 3] = y.w;
    }
  }
#pragma unroll
  for (int j = 0; j < GQ; ++j) {
    float accA = 0.f, accB = 0.f;
    const uint4* qp = reinterpret_cast<const uint4*>(&qh[j][16 * q]);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint4 u = qp[i];
      const uint32_t qw[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        accA = __builtin_amdgcn_fdot2(as_h2(ka[4 * i + k]), as_h2(qw[k]), accA, false);
        accB = __builtin_amdgcn_fdot2(as_h2(kb[4 * i + k]), as_h2(qw[k]), accB, false);
      }
    }
    const float sA = tp < nvalid ? quad_sum(accA) * a.scale_log2 : kNegInf;
    const float sB = tp + 16 < nvalid ? quad_sum(accB) * a.scale_log2 : kNegInf;
    float pA, pB;
    softmax_pair<GQ>(st, j, sA, sB, pA, pB);
    pL[j][tp] = pA;
    pL[j][tp + 16] = pB;
  }
  // the value rows are requested once the keys are consumed (fewer live registers)
  uint32_t vw[8][4];
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    const uint4 u =
        *reinterpret_cast<const uint4*>(vr + min(8 * o + t, nvalid - 1) * kHeadDim);
    vw[t][0] = u.x; vw[t][1] = u.y; vw[t][2] = u.z; vw[t][3] = u.w;
  }
#pragma unroll
  for (int j = 0; j < GQ; ++j) {
    const float4* pp = reinterpret_cast<const float4*>(&pL[j][8 * o]);
    const float4 u0 = pp[0], u1 = pp[1];
    const float pw[8] = {u0.x, u0.y, u0.z, u0.w, u1.x, u1.y, u1.z, u1.w};
#pragma unroll
    for (int t = 0; t < 8; ++t) {
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        st.ow[j][2 * k] = fmaf(pw[t], lo_f16(vw[t][k]), st.ow[j][2 * k]);
        st.ow[j][2 * k + 1] = fmaf(pw[t], hi_f16(vw[t][k]), st.ow[j][2 * k + 1]);
      }
    }
  }
}

// Work units: packed block i is unit i (0 <= i < n_blocks); window chunk c (32 fp16
// tokens) is units [n_blocks + kWindowUnits*c, n_blocks + kWindowUnits*(c+1)), weighted
// by its larger byte count.  A split covers a contiguous unit range: the packed blocks
// in it and every window chunk whose first unit falls in it.
template <int KB, int VB, int GQ, int NW>
__global__ __launch_bounds__(NW * kWave) void decode_uniform_kernel(DecodeArgs a) {
  constexpr int NT = NW * kWave;
  constexpr int CPW = 32 / KB;
  __shared__ __align__(16) uint32_t qh[GQ][64];
  __shared__ __align__(16) float qsL[NW][GQ][4][kRow];
  __shared__ __align__(16) float psL[NW][GQ][4][kRow];
  __shared__ float wm[NW][GQ], wl[NW][GQ];
  __shared__ __align__(16) float wo[NW][GQ][kHeadDim];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform
  const int split = blockIdx.x % a.splits;
  const int64_t bh = blockIdx.x / a.splits;
  const int b = (int)(bh / a.kv_heads);
  const int hkv = (int)(bh % a.kv_heads);
  const int hq0 = hkv * GQ;

  // query pair (channels 2l, 2l+1) per head, and the same times the key field scale and
  // the softmax scale (scores are kept in log2 units)
  uint32_t qreg[GQ];
  float qf[GQ][2];
  const float f0 = field_scale(KB, (2 * lane) % CPW), f1 = field_scale(KB, (2 * lane + 1) % CPW);
#pragma unroll
  for (int j = 0; j < GQ; ++j) {
    qreg[j] = *reinterpret_cast<const uint32_t*>(a.q + ((int64_t)b * a.q_heads + hq0 + j) *
                                                           kHeadDim + 2 * lane);
    qf[j][0] = lo_f16(qreg[j]) * f0 * a.scale_log2;
    qf[j][1] = hi_f16(qreg[j]) * f1 * a.scale_log2;
    if (wave == 0) qh[j][lane] = qreg[j];
  }
  __syncthreads();

  const float cscale = a.scale_log2;
  WaveState<GQ> st;
#pragma unroll
  for (int j = 0; j < GQ; ++j) {
    st.m[j] = kNegInf;
    st.l[j] = 0.f;
    st.mv[j] = 0.f;
#pragma unroll
    for (int t = 0; t < 8; ++t) st.acc[j][t] = st.ow[j][t] = 0.f;
  }

  const int nchunks = (a.n_resid + kGroup - 1) / kGroup;
  const int units = a.n_blocks + kWindowUnits * nchunks;
  const int s0 = (int)((int64_t)units * split / a.splits);
  const int s1 = (int)((int64_t)units * (split + 1) / a.splits);
  // Packed blocks of the split are dealt round-robin to the waves, so that at any time
  // the workgroup streams one contiguous stretch of each cache array; window chunks go
  // to the last waves (which get no more packed blocks than the others).
  const int bend = min(s1, a.n_blocks);
  const int first = s0 + wave;
  const int cnt = first < bend ? (bend - first + NW - 1) / NW : 0;

  // ---- window chunks first (their loads are short), then the packed blocks
  for (int c = 0; c < nchunks; ++c) {
    const int u = a.n_blocks + kWindowUnits * c;
    if (u >= s0 && u < s1 && NW - 1 - (c % NW) == wave)
      process_window<GQ>(a, bh, c, st, qh, reinterpret_cast<float(*)[kGroup]>(psL[wave]), lane);
  }
  if (cnt > 0) {
    const int64_t seg = bh * a.cap_blocks;
    const HeadPtrs hp = {a.k_codes + seg * (kGroup * kHeadDim * KB / 32),
                         a.k_meta + seg * kHeadDim, a.v_codes + seg * (kHeadDim * VB),
                         a.v_meta + seg * (kGroup * 4)};
    // Two blocks in flight ahead of the one being processed.  The prefetch index is
    // clamped rather than guarded so every iteration issues the same loads, and the
    // loop is unrolled by three with rotating roles so no register copy has to wait
    // for the loads just issued.
    const int last = cnt - 1;
    BlockRegs<KB, VB> r0, r1, r2;
    load_block<KB, VB>(r0, hp, first, lane);
    load_block<KB, VB>(r1, hp, first + min(1, last) * NW, lane);
    for (int k = 0; k < cnt; k += 3) {
      load_block<KB, VB>(r2, hp, first + min(k + 2, last) * NW, lane);
      process_block<KB, VB, GQ>(r0, st, qreg, qf, cscale, qsL[wave], psL[wave], lane);
      if (k + 1 >= cnt) break;
      load_block<KB, VB>(r0, hp, first + min(k + 3, last) * NW, lane);
      process_block<KB, VB, GQ>(r1, st, qreg, qf, cscale, qsL[wave], psL[wave], lane);
      if (k + 2 >= cnt) break;
      load_block<KB, VB>(r1, hp, first + min(k + 4, last) * NW, lane);
      process_block<KB, VB, GQ>(r2, st, qreg, qf, cscale, qsL[wave], psL[wave], lane);
    }
  }

  // ---- finish the wave: totals of l and of the min terms, value accumulators reduced
  // over the four token octets, then the WG merge
  const int n = lane & 15;
  float fs[8];
#pragma unroll
  for (int t = 0; t < 8; ++t) fs[t] = field_scale(VB, VB == 2 ? t : (t & 3));
#pragma unroll
  for (int j = 0; j < GQ; ++j) {
    const float lt = wave_sum(st.l[j]) * 0.25f;      // each token counted by four lanes
    float mvq = st.mv[j];                             // over the 16 lanes sharing q
    mvq += __shfl_xor(mvq, 4);
    mvq += __shfl_xor(mvq, 8);
    mvq += __shfl_xor(mvq, 16);
    mvq += __shfl_xor(mvq, 32);
    const float mvg = __shfl(mvq, n >> 2);            // group of channels 8n .. 8n + 7
    float ov[8];
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      float x = fmaf(st.acc[j][t], fs[t], st.ow[j][t]);
      x += __shfl_xor(x, 16);
      x += __shfl_xor(x, 32);
      ov[t] = x + mvg;
    }
    if (lane == 0) {
      wm[wave][j] = st.m[j];
      wl[wave][j] = lt;
    }
    if (lane < 16) {
      *reinterpret_cast<float4*>(&wo[wave][j][8 * n]) = make_float4(ov[0], ov[1], ov[2], ov[3]);
      *reinterpret_cast<float4*>(&wo[wave][j][8 * n + 4]) = make_float4(ov[4], ov[5], ov[6], ov[7]);
    }
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
  KVQ_DLB(1, 8) KVQ_DLB(1, 16)
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
