// Device helpers shared by the decode kernels over the packed uniform cache: field
// unpacking, wave reductions, the online-softmax state of the VALU paths, the fp16
// window chunk, and the end-of-wave / workgroup merge of (max, sum, output) partials.
#pragma once

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
constexpr int kRowRor4 = 0x124;      // rotate within a row of 16 lanes by 4
constexpr int kRowRor8 = 0x128;

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

// The running softmax maximum is raised only when a score exceeds it by more than this
// (log2 units): p = 2^(s - m) stays below 2^8, the rescaling of the accumulators
// becomes rare, and the final normalization is unchanged.
constexpr float kMaxSlack = 8.0f;

template <int GQ>
struct WaveState {
  float m[GQ];          // running max (log2 domain), wave-uniform
  float l[GQ];          // this lane's sum of p (every token counted by 4 lanes)
  float mv[GQ];         // sum of p * min over this lane's two tokens, group q
  float acc[GQ][8];     // values, channels 8n + T, in units of the packed fields' scale
};

// Online softmax for one head over this lane's two scores; the running maximum is only
// reduced over the wave when some score exceeds it (after the first blocks: rarely).
template <int GQ>
__device__ __forceinline__ void softmax_pair(WaveState<GQ>& st, int j, float sA, float sB,
                                             float& pA, float& pB) {
  const float smax = fmaxf(sA, sB);
  if (__any(smax > st.m[j] + kMaxSlack)) {
    const float mn = fmaxf(st.m[j], wave_max(smax));
    const float alpha = fast_exp2(st.m[j] - mn);     // 0 while m = -inf
    st.m[j] = mn;
    st.l[j] *= alpha;
    st.mv[j] *= alpha;
#pragma unroll
    for (int t = 0; t < 8; ++t) st.acc[j][t] *= alpha;
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

// One chunk of up to 32 fp16 window tokens, with the same lane roles as a packed block.
// Its value sums are folded into the packed accumulators, which carry the factor
// 2^(pos - 24) of the packed fields (VB-bit codes): a power of two, so exactly.
// The chunk's rows are read with plain loads, never streaming ones: each load instruction
// covers a quarter of every 128-byte line it touches (lanes 64 bytes apart) and the next
// three instructions need the rest, so the lines must stay in L2 between them.  With the
// streaming hint llama2_7b took 24.7 us, with plain loads 23.5-23.8 us.
template <int GQ, int VB>
__device__ __forceinline__ void process_window(const DecodeArgs& a, int64_t bh, int c,
                                               WaveState<GQ>& st, const uint32_t (*qh)[64],
                                               float (*pL)[kGroup], int lane) {
  const int tp = lane >> 2, q = lane & 3;
  const int n = lane & 15, o = lane >> 4;
  const Fp16Chunk ch = fp16_chunk(a, bh, c);
  const int nvalid = ch.nvalid;
  const uint16_t* kr = ch.k + 32 * q;
  const uint16_t* vr = ch.v + 8 * n;
  uint32_t ka[16], kb[16];
  {
    const uint16_t* pa = kr + min(tp, nvalid - 1) * kHeadDim;
    const uint16_t* pb = kr + min(tp + 16, nvalid - 1) * kHeadDim;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint4 x = reinterpret_cast<const uint4*>(pa)[i];
      const uint4 y = reinterpret_cast<const uint4*>(pb)[i];
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
    const uint4 u = *reinterpret_cast<const uint4*>(vr + min(8 * o + t, nvalid - 1) * kHeadDim);
    vw[t][0] = u.x; vw[t][1] = u.y; vw[t][2] = u.z; vw[t][3] = u.w;
  }
#pragma unroll
  for (int j = 0; j < GQ; ++j) {
    const float4* pp = reinterpret_cast<const float4*>(&pL[j][8 * o]);
    const float4 u0 = pp[0], u1 = pp[1];
    const float pw[8] = {u0.x, u0.y, u0.z, u0.w, u1.x, u1.y, u1.z, u1.w};
    float ow[8];
#pragma unroll
    for (int t = 0; t < 8; ++t) ow[t] = 0.f;
#pragma unroll
    for (int t = 0; t < 8; ++t) {
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        ow[2 * k] = fmaf(pw[t], lo_f16(vw[t][k]), ow[2 * k]);
        ow[2 * k + 1] = fmaf(pw[t], hi_f16(vw[t][k]), ow[2 * k + 1]);
      }
    }
#pragma unroll
    for (int t = 0; t < 8; ++t)
      st.acc[j][t] = fmaf(ow[t], 1.0f / field_scale(VB, VB == 2 ? t : (t & 3)), st.acc[j][t]);
  }
}

// Wave totals of a VALU state: l, the value min terms, the value accumulators reduced
// over the four token octets; written as one (max, sum, output[128]) partial per head.
template <int GQ, int VB>
__device__ __forceinline__ void finish_wave_state(const WaveState<GQ>& st, float* wm, float* wl,
                                                  float (*wo)[kHeadDim], int lane) {
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
      float x = st.acc[j][t] * fs[t];
      x += __shfl_xor(x, 16);
      x += __shfl_xor(x, 32);
      ov[t] = x + mvg;
    }
    if (lane == 0) {
      wm[j] = st.m[j];
      wl[j] = lt;
    }
    if (lane < 16) {
      *reinterpret_cast<float4*>(&wo[j][8 * n]) = make_float4(ov[0], ov[1], ov[2], ov[3]);
      *reinterpret_cast<float4*>(&wo[j][8 * n + 4]) = make_float4(ov[4], ov[5], ov[6], ov[7]);
    }
  }
}

template <int GQ>
__device__ __forceinline__ void init_wave_state(WaveState<GQ>& st) {
#pragma unroll
  for (int j = 0; j < GQ; ++j) {
    st.m[j] = kNegInf;
    st.l[j] = 0.f;
    st.mv[j] = 0.f;
#pragma unroll
    for (int t = 0; t < 8; ++t) st.acc[j][t] = 0.f;
  }
}

// Merge of NS (max, sum, output) partials per head in LDS: the workgroup writes the
// normalized output (one split) or its own partial for the split-merge launch.
template <int GQ, int NS>
__device__ __forceinline__ void merge_partials(const DecodeArgs& a, const float (*wm)[GQ],
                                               const float (*wl)[GQ],
                                               const float (*wo)[GQ][kHeadDim], int b, int hq0,
                                               int split) {
  const bool single = a.splits == 1;
  for (int idx = threadIdx.x; idx < GQ * kHeadDim; idx += blockDim.x) {
    const int j = idx >> 7, d = idx & 127;
    float M = kNegInf;
#pragma unroll
    for (int w = 0; w < NS; ++w) M = fmaxf(M, wm[w][j]);
    float L = 0.f, O = 0.f;
    if (M != kNegInf) {
#pragma unroll
      for (int w = 0; w < NS; ++w) {
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

}  // namespace
// Packed blocks of a split dealt to the NW waves of a workgroup when `chunks` window
// chunks (kWindowUnits each) go to the waves from the last one down, cyclically: the
// waves with one chunk fewer get kWindowUnits more blocks, the remainder goes one
// each to the first waves.  Counts never increase with the wave index, so round k of
// the deal is taken by waves 0..P_k-1 and the k-th block of wave w is block
// sum_v min(count_v, k) + w.  The counts form four runs: n0 waves of count c0, then
// n1 of c1, n2 of c2, n3 of c3 (plain scalars: no array the compiler would place in
// memory).
struct Deal {
  int n0, n1, n2, n3, c0, c1, c2, c3;
  __device__ __forceinline__ int count(int w) const {
    return c3 + (w < n0 + n1 + n2 ? c2 - c3 : 0) + (w < n0 + n1 ? c1 - c2 : 0) +
           (w < n0 ? c0 - c1 : 0);
  }
  __device__ __forceinline__ int index(int k, int w) const {
    return w + n0 * min(c0, k) + n1 * min(c1, k) + n2 * min(c2, k) + n3 * min(c3, k);
  }
};

// Block of round k (clamped to the wave's last round) for wave w of a split that
// starts at unit s0; wave-uniform.
__device__ __forceinline__ int block_of(const Deal d, int s0, int k, int last, int w) {
  return __builtin_amdgcn_readfirstlane(s0 + d.index(min(k, last), w));
}

__device__ __forceinline__ Deal deal_blocks(int nb, int chunks, int nw) {
  const int rem = chunks % nw;                  // waves with one chunk more than the rest
  const int na = nw - rem;                      // ... and those without it
  int ca = nb / nw, cb = ca, r = nb % nw;
  if (rem > 0) {
    const int extra = kWindowUnits * na;        // blocks that even out the extra chunk
    if (nb >= extra) {
      cb = (nb - extra) / nw;
      ca = cb + kWindowUnits;
      r = nb - extra - cb * nw;
    } else {
      cb = 0;
      ca = nb / na;
      r = nb % na;
    }
  }
  // the first r waves get one block more: all of class a first, then class b
  const int ra = min(r, na), rb = r - ra;
  Deal d;
  d.n0 = ra;           d.c0 = ca + 1;
  d.n1 = na - ra;      d.c1 = ca;
  d.n2 = rb;           d.c2 = cb + 1;
  d.n3 = nw - na - rb; d.c3 = cb;
  return d;
}

}  // namespace kvq
