// Decode attention over the non-uniform cache with outliers and RoPE after
// dequantization (KVQuant review, abstract items (ii)-(iv); "The KV cache has a
// geometry problem", section on rotary embeddings: quantize keys before the rotation,
// rotate after dequantization).
//
// Key t (position t) after dequantization: k~_d = lut[c_td] * s_d + m_d, or the exact
// fp16 value at an outlier.  With RoPE on interleaved pairs, q . R(t) k~ is
//   sum_i Re(a_i(t)) k~_2i + Im(a_i(t)) k~_2i+1,   a_i(t) = (q_2i + i q_2i+1) e^(-i t th_i)
// so one lane owns a channel pair i, keeps a_i for the current token and advances it
// by e^(-i th_i) per token (a complex product); each block restarts it from an angle
// t0 * th_i reduced modulo 2 pi in fp64.  Per-pair partial scores of the block's 32
// tokens are then summed across lanes (lanes 2t and 2t+1 end with token t).
// Outliers: the dense pass uses the stored code everywhere; one lane per CSR entry
// then computes a_col(t) * (x - dequant(code)) and token t adds its row's
// corrections in row order.
//
// Values: one lane per channel pair as well; o_d += (p_t * s_t) * lut[c_td] plus the
// per-token minimum term sum_t p_t m_t, identical for every channel.
// Code-book lookups: four codes in the four bytes of a word select bytes of the
// eight-entry fp16 table with v_perm_b32.
#include "kvq_common.h"

namespace kvq {
namespace {

constexpr float kNegInf = -__builtin_inff();
constexpr int kWindowUnits = 4;
constexpr double kTwoPi = 6.283185307179586476925286766559;

struct Lut {
  uint32_t lo_a, lo_b, hi_a, hi_b;   // low / high bytes of entries 0-3 and 4-7
};

__device__ __forceinline__ Lut load_lut(const uint16_t* lut) {
  uint32_t e[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) e[i] = lut[i];
  Lut r;
  r.lo_a = (e[0] & 255) | (e[1] & 255) << 8 | (e[2] & 255) << 16 | (e[3] & 255) << 24;
  r.lo_b = (e[4] & 255) | (e[5] & 255) << 8 | (e[6] & 255) << 16 | (e[7] & 255) << 24;
  r.hi_a = (e[0] >> 8) | (e[1] >> 8) << 8 | (e[2] >> 8) << 16 | (e[3] >> 8) << 24;
  r.hi_b = (e[4] >> 8) | (e[5] >> 8) << 8 | (e[6] >> 8) << 16 | (e[7] >> 8) << 24;
  return r;
}

// Four codes (one per byte, 0..7) -> their fp16 entries as two packed pairs.
__device__ __forceinline__ void lut4(const Lut& L, uint32_t codes, uint32_t& p01, uint32_t& p23) {
  const uint32_t lo = __builtin_amdgcn_perm(L.lo_b, L.lo_a, codes);
  const uint32_t hi = __builtin_amdgcn_perm(L.hi_b, L.hi_a, codes);
  p01 = __builtin_amdgcn_perm(hi, lo, 0x05010400u);
  p23 = __builtin_amdgcn_perm(hi, lo, 0x07030602u);
}

// Codes of tokens 4m..4m+3 of one channel's three nuq3 words, one per byte.
__device__ __forceinline__ uint32_t codes4(const uint32_t* w, int m) {
  const uint32_t lo = (w[m >> 2] >> (2 * (m & 3))) & 0x03030303u;
  const uint32_t hi = (w[2] >> m) & 0x01010101u;
  return lo | (hi << 2);
}

__device__ __forceinline__ uint32_t code_at(const uint32_t* w, int j) {
  const int jj = j & 15;
  const uint32_t lo = (w[j >> 4] >> (8 * (jj & 3) + 2 * (jj >> 2))) & 3u;
  const uint32_t hi = (w[2] >> (8 * (j & 3) + (j >> 2))) & 1u;
  return lo | (hi << 2);
}

__device__ __forceinline__ float lut_value(const uint16_t* lut, uint32_t c) {
  return f16_bits_to_f32(lut[c]);
}

// e^(-i phi) for phi = t * theta reduced modulo 2 pi in fp64.
__device__ __forceinline__ float2 rot_at(int64_t t, double theta) {
  double ph = fmod((double)t * theta, kTwoPi);
  float s, c;
  sincosf((float)ph, &s, &c);
  return make_float2(c, -s);
}

__device__ __forceinline__ float2 cmul(float2 a, float2 b) {
  return make_float2(fmaf(a.x, b.x, -(a.y * b.y)), fmaf(a.x, b.y, a.y * b.x));
}

__device__ __forceinline__ float sum32(float x) {
#pragma unroll
  for (int o = 1; o < 32; o <<= 1) x += __shfl_xor(x, o);
  return x;
}

template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ float dpp(float old, float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(__builtin_bit_cast(int, old),
                                                               __builtin_bit_cast(int, x), CTRL,
                                                               ROW_MASK, 0xF, false));
}
__device__ __forceinline__ float wave_max(float x) {
  x = fmaxf(x, dpp<0xB1>(kNegInf, x));
  x = fmaxf(x, dpp<0x4E>(kNegInf, x));
  x = fmaxf(x, dpp<0x141>(kNegInf, x));
  x = fmaxf(x, dpp<0x140>(kNegInf, x));
  x = fmaxf(x, dpp<0x142, 0xA>(kNegInf, x));
  x = fmaxf(x, dpp<0x143, 0xC>(kNegInf, x));
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 63));
}

// One in-row stage of the transposed reduction: DPP partner lanes hold the same token
// subsets; the lane with `high` set keeps v[H..2H), the other v[0..H), each adding the
// half its partner gives away.
template <int H, int CTRL>
__device__ __forceinline__ void row_stage(float (&v)[32], bool high) {
#pragma unroll
  for (int i = 0; i < H; ++i) {
    const float keep = high ? v[i + H] : v[i];
    const float send = high ? v[i] : v[i + H];
    v[i] = keep + dpp<CTRL>(0.f, send);
  }
}

__device__ __forceinline__ float bits_f(uint32_t x) { return __builtin_bit_cast(float, x); }
__device__ __forceinline__ uint32_t f_bits(float x) { return __builtin_bit_cast(uint32_t, x); }

// Sum over the 64 lanes of v[t] for the 32 tokens t: lane l ends with token l >> 1.
// Halves of the wave swap with v_permlane32_swap, rows with v_permlane16_swap (one
// instruction per pair of values), then mirror / half-mirror / quad DPP stages.
__device__ __forceinline__ float transpose_sum32(float (&v)[32], int lane) {
#pragma unroll
  for (int i = 0; i < 16; ++i) {               // lanes < 32 keep tokens 0..15
    const auto r = __builtin_amdgcn_permlane32_swap(f_bits(v[i]), f_bits(v[i + 16]), false,
                                                    false);
    v[i] = bits_f(r[0]) + bits_f(r[1]);
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) {                // even rows keep 8 of them, odd rows the rest
    const auto r = __builtin_amdgcn_permlane16_swap(f_bits(v[i]), f_bits(v[i + 8]), false,
                                                    false);
    v[i] = bits_f(r[0]) + bits_f(r[1]);
  }
  row_stage<4, 0x140>(v, lane & 8);            // row mirror: partner 15 - i
  row_stage<2, 0x141>(v, lane & 4);            // half-row mirror: partner 7 - i
  row_stage<1, 0x4E>(v, lane & 2);             // quad_perm [2,3,0,1]
  return v[0] + dpp<0xB1>(0.f, v[0]);          // quad_perm [1,0,3,2]
}

template <int GQ>
struct NuqState {
  float m[GQ], l[GQ], o[GQ][2], mv[GQ];
};

__device__ __forceinline__ float softmax_step(float s, float& m, float& l, float& alpha) {
  alpha = 1.0f;
  if (__any(s > m + 8.0f)) {               // the max may lag by 8 (log2): p < 2^8
    const float mn = fmaxf(m, wave_max(s));
    alpha = exp2f(m - mn);
    m = mn;
    l *= alpha;
  }
  const float p = exp2f(s - m);
  l += p;
  return p;
}

struct PairConsts {
  float2 q[8];        // (q_2i, q_2i+1) per query head
  float2 step;        // e^(-i theta_i)
  double theta;       // theta_i
  float ks0, km0, ks1, km1;   // key scale / min of channels 2i, 2i+1
};

// Softmax over the block's scores and the value accumulation shared by packed blocks
// and window chunks: s[] holds this lane's token (lane >> 1) score per head (log2
// units, -inf for missing tokens).
template <int GQ>
__device__ __forceinline__ void softmax_block(NuqState<GQ>& st, const float* s, float* p,
                                              float* alpha) {
#pragma unroll
  for (int j = 0; j < GQ; ++j) p[j] = softmax_step(s[j], st.m[j], st.l[j], alpha[j]);
}

// Block-invariant values shared by the waves of a workgroup (LDS).
template <int GQ>
struct NuqShared {
  float2 rot[kGroup][64];    // e^(-i j theta_i) for token j of a block, pair i
  float ks[kHeadDim], km[kHeadDim];
  float lutk[8], lutv[8];
};

// Per-wave scratch (LDS).
template <int GQ>
struct NuqWaveScratch {
  float ps[GQ][kGroup];      // p_t * scale_t of the block's tokens
  float2 qb[GQ][64];         // q e^(-i t0 theta_i) per head and pair: the block's first token
  uint32_t kc[kHeadDim][3];  // the block's key code words, per channel
  float corr[GQ][64];        // per CSR entry of the window: its score correction
  uint8_t tok[64];           // per CSR entry of the window: its token in the block
  float pv[GQ][kGroup];      // p_t of the block's tokens (value outliers)
  uint32_t vmeta[kGroup];    // value scale / min of the block's tokens
  float vcorr[GQ][kHeadDim]; // value-outlier corrections of the block, per channel
};

struct NuqBlockRegs {
  uint32_t kw[6], vw[6];     // key / value code words of channels 2l, 2l+1
  uint32_t vmeta;            // value scale / min of token lane >> 1
  int32_t r0, r1;            // CSR row of token lane >> 1
};

__device__ __forceinline__ void load_nuq_block(NuqBlockRegs& r, const DecodeArgs& a, int64_t bh,
                                               int64_t blk, int lane) {
  const int t = lane >> 1;
  const int64_t gblk = bh * a.cap_blocks + blk;
  const int64_t t0 = blk * kGroup;
  const uint32_t* kp = a.k_codes + (gblk * kHeadDim + 2 * lane) * 3;
  const uint32_t* vp = a.v_codes + (gblk * kHeadDim + 2 * lane) * 3;
  const uint2 k01 = *reinterpret_cast<const uint2*>(kp);
  const uint4 k25 = *reinterpret_cast<const uint4*>(kp + 2);
  const uint2 v01 = *reinterpret_cast<const uint2*>(vp);
  const uint4 v25 = *reinterpret_cast<const uint4*>(vp + 2);
  r.kw[0] = k01.x; r.kw[1] = k01.y; r.kw[2] = k25.x; r.kw[3] = k25.y; r.kw[4] = k25.z; r.kw[5] = k25.w;
  r.vw[0] = v01.x; r.vw[1] = v01.y; r.vw[2] = v25.x; r.vw[3] = v25.y; r.vw[4] = v25.z; r.vw[5] = v25.w;
  r.vmeta = a.v_meta[bh * (a.cap_blocks * kGroup) + t0 + t];
  r.r0 = r.r1 = 0;
  if (a.csr_rowptr) {
    const int32_t* rp = a.csr_rowptr + bh * (a.cap_blocks * kGroup + 1);
    r.r0 = rp[t0 + t];
    r.r1 = rp[t0 + t + 1];
  }
}

template <int GQ>
__device__ void process_nuq_block(const DecodeArgs& a, int64_t bh, int64_t t0,
                                  const NuqBlockRegs& r, const PairConsts& pc, const Lut& lk,
                                  const Lut& lv, NuqState<GQ>& st, const NuqShared<GQ>& sh,
                                  NuqWaveScratch<GQ>& ws, int lane) {
  const int t = lane >> 1;                  // this lane's token after the reduction
  const uint32_t* kw0 = r.kw;
  const uint32_t* kw1 = r.kw + 3;
  const uint32_t* vw0 = r.vw;
  const uint32_t* vw1 = r.vw + 3;

  // The block's CSR entries [e_begin, e_end): the first 64 are loaded now, one per
  // lane, so that the dense work below covers the load.
  const int64_t e_begin = max((int64_t)__builtin_amdgcn_readlane(r.r0, 0), (int64_t)0);
  const int64_t e_end =
      min((int64_t)__builtin_amdgcn_readlane(r.r1, 63), a.csr_capacity);
  uint32_t ent_first = 0;
  if (e_begin + lane < e_end) ent_first = a.csr_ent[bh * a.csr_capacity + e_begin + lane];
  // The block's value outliers: v_kv per token, 32 * v_kv entries from vbase.
  const int v_ne = a.v_out != nullptr ? kGroup * a.v_kv : 0;
  const int64_t vbase = (bh * (a.cap_blocks * kGroup) + (t0 - a.n_sink)) * a.v_kv;
  uint32_t vent_first = 0;
  if (lane < v_ne) vent_first = a.v_out[vbase + lane];

  // ---- keys: dequantize this lane's pair for the 32 tokens, then per head the
  // rotated-query partial scores and their sum across lanes
  float kd0[32], kd1[32];
#pragma unroll
  for (int m4 = 0; m4 < 8; ++m4) {
    uint32_t a01, a23, b01, b23;
    lut4(lk, codes4(kw0, m4), a01, a23);
    lut4(lk, codes4(kw1, m4), b01, b23);
    kd0[4 * m4 + 0] = fmaf(lo_f16(a01), pc.ks0, pc.km0);
    kd0[4 * m4 + 1] = fmaf(hi_f16(a01), pc.ks0, pc.km0);
    kd0[4 * m4 + 2] = fmaf(lo_f16(a23), pc.ks0, pc.km0);
    kd0[4 * m4 + 3] = fmaf(hi_f16(a23), pc.ks0, pc.km0);
    kd1[4 * m4 + 0] = fmaf(lo_f16(b01), pc.ks1, pc.km1);
    kd1[4 * m4 + 1] = fmaf(hi_f16(b01), pc.ks1, pc.km1);
    kd1[4 * m4 + 2] = fmaf(lo_f16(b23), pc.ks1, pc.km1);
    kd1[4 * m4 + 3] = fmaf(hi_f16(b23), pc.ks1, pc.km1);
  }
  const float2 base = rot_at(t0, pc.theta);
  float s[GQ];
  float2 qb[GQ];
#pragma unroll
  for (int j = 0; j < GQ; ++j) {
    float part[32];
    qb[j] = cmul(pc.q[j], base);
    float2 ar = qb[j];
#pragma unroll
    for (int k = 0; k < 32; ++k) {
      part[k] = fmaf(ar.x, kd0[k], ar.y * kd1[k]);
      ar = cmul(ar, pc.step);
    }
    s[j] = transpose_sum32(part, lane);
  }

  // ---- outliers: token t's CSR entries replace the dequantized code by the exact value.
  // Entries are taken in windows of 64, one per lane: the lanes of each token mark its
  // row's slots with the token, every entry lane computes its correction
  // comp(q e^(-i (t0 + t) theta)) * (x - dequant(code)) (the real part for an even
  // channel, the imaginary part for an odd one), and the lanes of token t add their
  // row's corrections in row order.
  if (e_begin < e_end) {
#pragma unroll
    for (int j = 0; j < GQ; ++j) ws.qb[j][lane] = qb[j];
    ws.kc[2 * lane][0] = kw0[0]; ws.kc[2 * lane][1] = kw0[1]; ws.kc[2 * lane][2] = kw0[2];
    ws.kc[2 * lane + 1][0] = kw1[0]; ws.kc[2 * lane + 1][1] = kw1[1]; ws.kc[2 * lane + 1][2] = kw1[2];
    for (int64_t w0 = e_begin; w0 < e_end; w0 += 64) {
      const bool has = w0 + lane < e_end;
      uint32_t ent = ent_first;
      if (w0 != e_begin) ent = has ? a.csr_ent[bh * a.csr_capacity + w0 + lane] : 0u;
      const int64_t lo = max((int64_t)r.r0, w0), hi = min((int64_t)r.r1, min(e_end, w0 + 64));
      if (!(lane & 1))
        for (int64_t e = lo; e < hi; ++e) ws.tok[e - w0] = (uint8_t)t;
      __builtin_amdgcn_wave_barrier();
      if (has) {
        const int te = ws.tok[lane] & (kGroup - 1);
        const int col = (int)(ent & (kHeadDim - 1));
        const int pr = col >> 1;
        const float x = f16_bits_to_f32((uint16_t)(ent >> 16));
        const float khat = fmaf(sh.lutk[code_at(ws.kc[col], te)], sh.ks[col], sh.km[col]);
        const float d = x - khat;
        const float2 e = sh.rot[te][pr];
        const bool odd = col & 1;
        const float u = odd ? e.y : e.x, v = odd ? e.x : -e.y;
#pragma unroll
        for (int j = 0; j < GQ; ++j) {
          const float2 b = ws.qb[j][pr];
          ws.corr[j][lane] = fmaf(b.x, u, b.y * v) * d;
        }
      }
      __builtin_amdgcn_wave_barrier();
      for (int64_t e = lo; e < hi; ++e) {
#pragma unroll
        for (int j = 0; j < GQ; ++j) s[j] += ws.corr[j][e - w0];
      }
      __builtin_amdgcn_wave_barrier();
    }
  }

  // ---- softmax (lanes 2t and 2t+1 both carry the corrected score of token t)
  float p[GQ], alpha[GQ];
#pragma unroll
  for (int j = 0; j < GQ; ++j) s[j] *= a.scale_log2;
  softmax_block<GQ>(st, s, p, alpha);

  // ---- values: p * scale per token into LDS, p * min per lane
  const float vs = lo_f16(r.vmeta), vm = hi_f16(r.vmeta);
#pragma unroll
  for (int j = 0; j < GQ; ++j) {
    ws.ps[j][t] = p[j] * vs;
    st.mv[j] = fmaf(p[j], vm, st.mv[j] * alpha[j]);     // every token counted twice
  }
#pragma unroll
  for (int j = 0; j < GQ; ++j) {
    float o0 = st.o[j][0] * alpha[j], o1 = st.o[j][1] * alpha[j];
    const float4* pp = reinterpret_cast<const float4*>(&ws.ps[j][0]);
#pragma unroll
    for (int m4 = 0; m4 < 8; ++m4) {
      const float4 w4 = pp[m4];
      uint32_t a01, a23, b01, b23;
      lut4(lv, codes4(vw0, m4), a01, a23);
      lut4(lv, codes4(vw1, m4), b01, b23);
      o0 = fmaf(w4.x, lo_f16(a01), o0); o0 = fmaf(w4.y, hi_f16(a01), o0);
      o0 = fmaf(w4.z, lo_f16(a23), o0); o0 = fmaf(w4.w, hi_f16(a23), o0);
      o1 = fmaf(w4.x, lo_f16(b01), o1); o1 = fmaf(w4.y, hi_f16(b01), o1);
      o1 = fmaf(w4.z, lo_f16(b23), o1); o1 = fmaf(w4.w, hi_f16(b23), o1);
    }
    st.o[j][0] = o0;
    st.o[j][1] = o1;
  }

  // ---- value outliers: each token's entries replace the dequantized value by the exact
  // one.  One lane per entry adds p_t * (x - v_hat) for its channel into LDS (the key
  // code-word scratch now holds the value code words); each lane then takes its two
  // channels' sums.
  if (v_ne > 0) {
    ws.kc[2 * lane][0] = vw0[0]; ws.kc[2 * lane][1] = vw0[1]; ws.kc[2 * lane][2] = vw0[2];
    ws.kc[2 * lane + 1][0] = vw1[0]; ws.kc[2 * lane + 1][1] = vw1[1];
    ws.kc[2 * lane + 1][2] = vw1[2];
    if (!(lane & 1)) {
      ws.vmeta[t] = r.vmeta;
#pragma unroll
      for (int j = 0; j < GQ; ++j) ws.pv[j][t] = p[j];
    }
    __builtin_amdgcn_wave_barrier();
    for (int e0 = 0; e0 < v_ne; e0 += 64) {
      const int e = e0 + lane;
      if (e < v_ne) {
        const uint32_t ent = e0 == 0 ? vent_first : a.v_out[vbase + e];
        const int te = (e / a.v_kv) & (kGroup - 1);
        const int d = (int)(ent & (kHeadDim - 1));
        const float x = f16_bits_to_f32((uint16_t)(ent >> 16));
        const uint32_t vmw = ws.vmeta[te];
        const float vhat = sh.lutv[code_at(ws.kc[d], te)] * lo_f16(vmw) + hi_f16(vmw);
#pragma unroll
        for (int j = 0; j < GQ; ++j) atomicAdd(&ws.vcorr[j][d], ws.pv[j][te] * (x - vhat));
      }
    }
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int j = 0; j < GQ; ++j) {
      const float2 cv = *reinterpret_cast<const float2*>(&ws.vcorr[j][2 * lane]);
      st.o[j][0] += cv.x;
      st.o[j][1] += cv.y;
      *reinterpret_cast<float2*>(&ws.vcorr[j][2 * lane]) = make_float2(0.f, 0.f);
    }
    __builtin_amdgcn_wave_barrier();
  }
}

// Up to 32 fp16 window tokens (positions n_packed + 32 c + j), rotated like the keys.
template <int GQ>
__device__ void process_nuq_window(const DecodeArgs& a, int64_t bh, int c,
                                   const PairConsts& pc, NuqState<GQ>& st,
                                   float (*psL)[kGroup], int lane) {
  const int t = lane >> 1;                  // this lane's token after the reduction
  const Fp16Chunk ch = fp16_chunk(a, bh, c);
  const int nvalid = ch.nvalid;
  const int64_t pos0 = ch.pos0;
  const uint16_t* kr = ch.k + 2 * lane;
  const uint16_t* vr = ch.v + 2 * lane;
  uint32_t kv[32];
#pragma unroll
  for (int k = 0; k < 32; ++k)
    kv[k] = *reinterpret_cast<const uint32_t*>(kr + min(k, nvalid - 1) * kHeadDim);
  const float2 base = rot_at(pos0, pc.theta);
  float s[GQ], p[GQ], alpha[GQ];
#pragma unroll
  for (int j = 0; j < GQ; ++j) {
    float part[32];
    float2 ar = cmul(pc.q[j], base);
#pragma unroll
    for (int k = 0; k < 32; ++k) {
      part[k] = fmaf(ar.x, lo_f16(kv[k]), ar.y * hi_f16(kv[k]));
      ar = cmul(ar, pc.step);
    }
    s[j] = transpose_sum32(part, lane) * a.scale_log2;
    if (t >= nvalid) s[j] = kNegInf;
  }
  softmax_block<GQ>(st, s, p, alpha);
#pragma unroll
  for (int j = 0; j < GQ; ++j) {
    psL[j][t] = p[j];
    st.mv[j] *= alpha[j];
  }
  uint32_t vv[32];
#pragma unroll
  for (int k = 0; k < 32; ++k)
    vv[k] = *reinterpret_cast<const uint32_t*>(vr + min(k, nvalid - 1) * kHeadDim);
#pragma unroll
  for (int j = 0; j < GQ; ++j) {
    float o0 = st.o[j][0] * alpha[j], o1 = st.o[j][1] * alpha[j];
#pragma unroll
    for (int k = 0; k < 32; ++k) {
      const float pk = psL[j][k];
      o0 = fmaf(pk, lo_f16(vv[k]), o0);
      o1 = fmaf(pk, hi_f16(vv[k]), o1);
    }
    st.o[j][0] = o0;
    st.o[j][1] = o1;
  }
}

template <int GQ, int NW>
__global__ __launch_bounds__(NW * kWave) void decode_nuq_kernel(DecodeArgs a) {
  constexpr int NT = NW * kWave;
  __shared__ NuqShared<GQ> sh;
  __shared__ __align__(16) NuqWaveScratch<GQ> wsc[NW];
  __shared__ float wm[NW][GQ], wl[NW][GQ];
  __shared__ __align__(16) float wo[NW][GQ][kHeadDim];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int split = blockIdx.x % a.splits;
  const int64_t bh = blockIdx.x / a.splits;
  const int b = (int)(bh / a.kv_heads);
  const int hkv = (int)(bh % a.kv_heads);
  const int hq0 = hkv * GQ;

  PairConsts pc;
#pragma unroll
  for (int j = 0; j < GQ; ++j) {
    const uint32_t qq = *reinterpret_cast<const uint32_t*>(
        a.q + ((int64_t)b * a.q_heads + hq0 + j) * kHeadDim + 2 * lane);
    pc.q[j] = make_float2(lo_f16(qq), hi_f16(qq));
  }
  pc.theta = a.rope_theta > 0.f ? pow((double)a.rope_theta, -2.0 * lane / kHeadDim) : 0.0;
  {
    const float2 r1 = rot_at(1, pc.theta);
    pc.step = r1;
  }
  if (a.n_blocks > 0) {
    const uint2 km = *reinterpret_cast<const uint2*>(a.k_meta + bh * kHeadDim + 2 * lane);
    pc.ks0 = lo_f16(km.x); pc.km0 = hi_f16(km.x);
    pc.ks1 = lo_f16(km.y); pc.km1 = hi_f16(km.y);
  } else {
    pc.ks0 = pc.km0 = pc.ks1 = pc.km1 = 0.f;
  }
  const Lut lk = load_lut(a.lut_k);
  const Lut lv = load_lut(a.lut_v);
  for (int j = wave; j < kGroup; j += NW) sh.rot[j][lane] = rot_at(j, pc.theta);
  if (wave == 0) {
    sh.ks[2 * lane] = pc.ks0; sh.km[2 * lane] = pc.km0;
    sh.ks[2 * lane + 1] = pc.ks1; sh.km[2 * lane + 1] = pc.km1;
    if (lane < 8) sh.lutk[lane] = lut_value(a.lut_k, lane);
    if (lane < 8) sh.lutv[lane] = lut_value(a.lut_v, lane);
  }
  __syncthreads();

  NuqState<GQ> st;
#pragma unroll
  for (int j = 0; j < GQ; ++j) {
    st.m[j] = kNegInf;
    st.l[j] = 0.f;
    st.o[j][0] = st.o[j][1] = 0.f;
    st.mv[j] = 0.f;
    *reinterpret_cast<float2*>(&wsc[wave].vcorr[j][2 * lane]) = make_float2(0.f, 0.f);
  }

  const int nchunks = fp16_chunks(a);
  const int units = a.n_blocks + kWindowUnits * nchunks;
  const int s0 = (int)((int64_t)units * split / a.splits);
  const int s1 = (int)((int64_t)units * (split + 1) / a.splits);
  const int w0 = s0 + (int)((int64_t)(s1 - s0) * wave / NW);
  const int w1 = s0 + (int)((int64_t)(s1 - s0) * (wave + 1) / NW);
  for (int c = 0; c < nchunks; ++c) {
    const int u = a.n_blocks + kWindowUnits * c;
    if (u >= w0 && u < w1) process_nuq_window<GQ>(a, bh, c, pc, st, wsc[wave].ps, lane);
  }
  const int b0 = w0, b1 = min(w1, a.n_blocks);
  if (b0 < b1) {
    // One block in flight ahead of the one being processed (clamped index, unrolled by
    // two so no register copy waits on the loads just issued).
    const int last = b1 - 1;
    NuqBlockRegs r0, r1;
    load_nuq_block(r0, a, bh, b0, lane);
    for (int i = b0; i < b1; i += 2) {
      load_nuq_block(r1, a, bh, min(i + 1, last), lane);
      process_nuq_block<GQ>(a, bh, a.n_sink + (int64_t)i * kGroup, r0, pc, lk, lv, st, sh, wsc[wave],
                            lane);
      if (i + 1 >= b1) break;
      load_nuq_block(r0, a, bh, min(i + 2, last), lane);
      process_nuq_block<GQ>(a, bh, a.n_sink + (int64_t)(i + 1) * kGroup, r1, pc, lk, lv, st, sh,
                            wsc[wave], lane);
    }
  }

  // ---- wave totals and the workgroup merge
#pragma unroll
  for (int j = 0; j < GQ; ++j) {
    float ltall = sum32(st.l[j]), mvall = sum32(st.mv[j]);
    ltall = (ltall + __shfl_xor(ltall, 32)) * 0.5f;      // every token counted by two lanes
    mvall = (mvall + __shfl_xor(mvall, 32)) * 0.5f;
    if (lane == 0) {
      wm[wave][j] = st.m[j];
      wl[wave][j] = ltall;
    }
    *reinterpret_cast<float2*>(&wo[wave][j][2 * lane]) =
        make_float2(st.o[j][0] + mvall, st.o[j][1] + mvall);
  }
  __syncthreads();
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
    if (a.splits == 1) {
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

hipError_t launch_decode_nuq(const DecodeArgs& a, int gq, hipStream_t s) {
  const int64_t wgs = (int64_t)a.batch * a.kv_heads * a.splits;
  const int nw = a.waves_per_group;
  dim3 grid((unsigned)wgs), block((unsigned)(nw * kWave));
#define KVQ_DN(G_, NW_)                                                   \
  if (gq == G_ && nw == NW_) {                                            \
    decode_nuq_kernel<G_, NW_><<<grid, block, 0, s>>>(a);                 \
    hipError_t e_ = hipGetLastError();                                    \
    if (e_ != hipSuccess || a.splits == 1) return e_;                     \
    return launch_merge_splits(a, s);                                     \
  }
  KVQ_DN(1, 4) KVQ_DN(2, 4) KVQ_DN(4, 4) KVQ_DN(8, 4)
#undef KVQ_DN
  return hipErrorInvalidValue;
}

const void* decode_nuq_fn(int gq, int nw) {
  if (nw != 4) return nullptr;
  if (gq == 1) return reinterpret_cast<const void*>(&decode_nuq_kernel<1, 4>);
  if (gq == 2) return reinterpret_cast<const void*>(&decode_nuq_kernel<2, 4>);
  if (gq == 4) return reinterpret_cast<const void*>(&decode_nuq_kernel<4, 4>);
  if (gq == 8) return reinterpret_cast<const void*>(&decode_nuq_kernel<8, 4>);
  return nullptr;
}

}  // namespace kvq
