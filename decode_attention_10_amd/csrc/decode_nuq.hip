// Decode attention over the non-uniform cache with outliers and RoPE after
// dequantization (KVQuant review, abstract items (ii)-(iv); "The KV cache has a
// geometry problem", section on rotary embeddings: quantize keys before the rotation,
// rotate after dequantization).
//
// Key t (position t) after dequantization: k~_d = lut[c_td] * s_d + m_d, or the exact
// fp16 value at an outlier.  With RoPE on interleaved pairs, q . R(t) k~ is
//   sum_i Re(a_i(t)) k~_2i + Im(a_i(t)) k~_2i+1,   a_i(t) = (q_2i + i q_2i+1) e^(-i t th_i)
// so one lane owns a channel pair i.  Each block starts from a_i(t0) = q e^(-i t0 th_i),
// where e^(-i t0 th_i) is carried from block to block in fp64 (one complex product by
// e^(-i 32 th_i) per block, started from an angle reduced modulo 2 pi at the wave's
// first block).  Inside the block chains advance by the three-term recurrence
// x(t+1) = 2 cos(th_i) x(t) - x(t-1), which every real-linear function of a_i(t) obeys
// (one chain over the 32 tokens with one query head, two chains from tokens 0 and 16
// otherwise); with one query head the chains carry s_2i Re(a), s_2i+1 Im(a) and
// m_2i Re(a) + m_2i+1 Im(a) (key scales and minima folded in), so a token costs three
// fmas of recurrence and two of score.  Per-pair partial scores of the block's 32 tokens
// are then summed across lanes (lanes 2t and 2t+1 end with token t).
// Outliers: the dense pass uses the stored code everywhere; one lane per CSR entry
// (which carries its token's place in the block) then computes
// a_col(t) * (x - dequant(code)), and the two lanes of token t add their row's
// corrections, every other entry each, in row order.
//
// Values: one lane per channel pair as well; o_d += (p_t * s_t) * lut[c_td] plus the
// per-token minimum term sum_t p_t m_t, identical for every channel; each token's
// value outliers (if any) add p_t * (x - dequant(code)) to their channels.  The weights
// p_t * s_t enter as fp16 (scaled by a per-wave power of two that keeps them below 2^15)
// in fp16 dot products with fp32 accumulation, two tokens per instruction.
// Code-book lookups: tables in LDS of code-book pairs (entry a + 2^B b = (lut[a],
// lut[b]) as fp16 halves), indexed per token by the two channels of a lane's key pair
// and per channel by two tokens of the values; four indices per word, one per byte.
// With several query heads the keys are dequantized through v_perm_b32 selections from
// the code book in registers (four codes in the four bytes of a word).
// Code widths B = 2, 3, 4 (kernel template); sink and window tokens are fp16 chunks.
#include "kvq_common.h"

namespace kvq {
namespace {

constexpr float kNegInf = -__builtin_inff();
constexpr int kWindowUnits = 4;

// Code book in registers: the low and the high bytes of the fp16 entries, four entries
// per register (entries 4i..4i+3 in lo[i] / hi[i]).
template <int B>
struct Lut {
  uint32_t lo[B == 4 ? 4 : 2], hi[B == 4 ? 4 : 2];
};

template <int B>
__device__ __forceinline__ Lut<B> load_lut(const uint16_t* lut) {
  constexpr int NR = B == 4 ? 4 : 2;
  Lut<B> r;
#pragma unroll
  for (int i = 0; i < NR; ++i) {
    r.lo[i] = r.hi[i] = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const uint32_t e = 4 * i + k < (1 << B) ? lut[4 * i + k] : 0u;
      r.lo[i] |= (e & 255u) << (8 * k);
      r.hi[i] |= (e >> 8) << (8 * k);
    }
  }
  return r;
}

// Four codes (one per byte) -> their fp16 entries as two packed pairs.  Eight entries
// fit one v_perm_b32 source pair; with 16 (nuq4) both halves are looked up and the
// code's high bit picks the byte.
template <int B>
__device__ __forceinline__ void lut4(const Lut<B>& L, uint32_t codes, uint32_t& p01,
                                     uint32_t& p23) {
  uint32_t lo, hi;
  if constexpr (B == 4) {
    const uint32_t c7 = codes & 0x07070707u;
    const uint32_t t = (codes >> 3) & 0x01010101u;
    const uint32_t sel = (t << 8) - t;            // 0xFF in the bytes of codes 8..15
    const uint32_t lo0 = __builtin_amdgcn_perm(L.lo[1], L.lo[0], c7);
    const uint32_t lo1 = __builtin_amdgcn_perm(L.lo[3], L.lo[2], c7);
    const uint32_t hi0 = __builtin_amdgcn_perm(L.hi[1], L.hi[0], c7);
    const uint32_t hi1 = __builtin_amdgcn_perm(L.hi[3], L.hi[2], c7);
    lo = (lo1 & sel) | (lo0 & ~sel);
    hi = (hi1 & sel) | (hi0 & ~sel);
  } else {
    lo = __builtin_amdgcn_perm(L.lo[1], L.lo[0], codes);
    hi = __builtin_amdgcn_perm(L.hi[1], L.hi[0], codes);
  }
  p01 = __builtin_amdgcn_perm(hi, lo, 0x05010400u);
  p23 = __builtin_amdgcn_perm(hi, lo, 0x07030602u);
}

// Codes of tokens 4m..4m+3 of one channel's B code words, one per byte.
template <int B>
__device__ __forceinline__ uint32_t codes4(const uint32_t* w, int m) {
  if constexpr (B == 4) {
    return (w[m >> 1] >> (4 * (m & 1))) & 0x0F0F0F0Fu;
  } else {
    const uint32_t lo = (w[m >> 2] >> (2 * (m & 3))) & 0x03030303u;
    if constexpr (B == 2) return lo;
    const uint32_t hi = (w[2] >> m) & 0x01010101u;
    return lo | (hi << 2);
  }
}

// codes4 for nuq3 (m is a constant of the unrolled loops): for m < 6 one shift and one
// mask of word m / 2; for m = 6, 7 the low bits from bits 6..7 of each byte of word
// m - 6 and the high bit from bit m of each byte of word 2, merged by one AND-OR.
__device__ __forceinline__ uint32_t codes4_3(const uint32_t* w, int m) {
  if (m < 6) return (w[m >> 1] >> (3 * (m & 1))) & 0x07070707u;
  return ((w[m - 6] >> 6) & 0x03030303u) | ((w[2] >> (m - 2)) & 0x04040404u);
}

// codes of tokens 4m..4m+3 (one per byte) for any width
template <int B>
__device__ __forceinline__ uint32_t codes_of(const uint32_t* w, int m) {
  if constexpr (B == 3) return codes4_3(w, m);
  else return codes4<B>(w, m);
}

// nuq3 pair-table indices, one per byte: for tokens 4m..4m+3, the key code of channel
// 2i plus 8 times that of channel 2i+1 (w0, w1: the two channels' words).  For m < 6
// one mask and one masked merge, the second field taken in place (bits 3..5 of a byte).
__device__ __forceinline__ uint32_t key_pair_index4(const uint32_t* w0, const uint32_t* w1,
                                                    int m) {
  if (m < 6) {
    const uint32_t a = w0[m >> 1], b = w1[m >> 1];
    if (m & 1) return ((a >> 3) & 0x07070707u) | (b & 0x38383838u);
    return (a & 0x07070707u) | ((b << 3) & 0x38383838u);
  }
  return codes4_3(w0, m) | (codes4_3(w1, m) << 3);
}

// nuq3 value pair-table indices of one channel, one per byte: byte k pairs tokens
// 8q + k and 8q + 4 + k.  For q < 3 these are the two whole codes at bits 0..5 of byte k
// of word q; for q = 3 they are assembled from the split codes of tokens 24..31.
__device__ __forceinline__ uint32_t value_pair_index4(const uint32_t* w, int q) {
  if (q < 3) return w[q] & 0x3F3F3F3Fu;
  uint32_t x = ((w[0] >> 6) & 0x03030303u) | ((w[2] >> 4) & 0x04040404u);   // token 24 + k
  x |= (w[1] >> 3) & 0x18181818u;                                          // 28 + k, low
  return x | ((w[2] >> 2) & 0x20202020u);                                  // 28 + k, high
}

// nuq2 pair-table indices, one per byte (16-entry tables: code of the first element plus
// 4 times that of the second).  Keys: channel 2i and 2i+1 of tokens 4m..4m+3, both at
// bits 8k + 2(m % 4) of word m / 4.  Values: tokens 8q + k and 8q + 4 + k of one channel,
// the adjacent fields at bits 8k + 4(q % 2) of word q / 2, so one shift and one mask.
__device__ __forceinline__ uint32_t key_pair_index4_2(const uint32_t* w0, const uint32_t* w1,
                                                      int m) {
  const int s = 2 * (m & 3);
  return ((w0[m >> 2] >> s) & 0x03030303u) | (((w1[m >> 2] >> s) << 2) & 0x0C0C0C0Cu);
}
__device__ __forceinline__ uint32_t value_pair_index4_2(const uint32_t* w, int q) {
  return (w[q >> 1] >> (4 * (q & 1))) & 0x0F0F0F0Fu;
}

// nuq4 pair-table indices (256-entry tables: code of the first element plus 16 times
// that of the second).  Keys: tokens 4m..4m+3 at bits 8k + 4(m % 2) of word m / 2.
// Values: tokens 8q + k and 8q + 4 + k are the low and high nibble of byte k of word q,
// so the code word is the index word.
__device__ __forceinline__ uint32_t key_pair_index4_4(const uint32_t* w0, const uint32_t* w1,
                                                      int m) {
  const int s = 4 * (m & 1);
  return ((w0[m >> 1] >> s) & 0x0F0F0F0Fu) | (((w1[m >> 1] >> s) << 4) & 0xF0F0F0F0u);
}

// Pair-table indices of any width.
template <int B>
__device__ __forceinline__ uint32_t key_pair_idx(const uint32_t* w0, const uint32_t* w1, int m) {
  if constexpr (B == 2) return key_pair_index4_2(w0, w1, m);
  else if constexpr (B == 4) return key_pair_index4_4(w0, w1, m);
  else return key_pair_index4(w0, w1, m);
}
template <int B>
__device__ __forceinline__ uint32_t value_pair_idx(const uint32_t* w, int q) {
  if constexpr (B == 2) return value_pair_index4_2(w, q);
  else if constexpr (B == 4) return w[q];
  else return value_pair_index4(w, q);
}

// 4 * (byte k of x): one v_lshlrev_b32 with a byte-select operand (SDWA).  Written out
// because the compiler, knowing the top bits of each index byte are clear, otherwise
// prefers a shift and a mask.  Arithmetic only, no memory access.
template <int K>
__device__ __forceinline__ uint32_t byte_times4(uint32_t x) {
  uint32_t r;
  if constexpr (K == 0)
    asm("v_lshlrev_b32_sdwa %0, 2, %1 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD "
        "src1_sel:BYTE_0" : "=v"(r) : "v"(x));
  else if constexpr (K == 1)
    asm("v_lshlrev_b32_sdwa %0, 2, %1 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD "
        "src1_sel:BYTE_1" : "=v"(r) : "v"(x));
  else if constexpr (K == 2)
    asm("v_lshlrev_b32_sdwa %0, 2, %1 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD "
        "src1_sel:BYTE_2" : "=v"(r) : "v"(x));
  else
    asm("v_lshlrev_b32_sdwa %0, 2, %1 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD "
        "src1_sel:BYTE_3" : "=v"(r) : "v"(x));
  return r;
}

// The table entry selected by byte K of a word of table indices (< 256 each).
template <int K>
__device__ __forceinline__ uint32_t pair_entry(const uint32_t* table, uint32_t idx4) {
  return *reinterpret_cast<const uint32_t*>(reinterpret_cast<const char*>(table) +
                                            byte_times4<K>(idx4));
}

__device__ __forceinline__ float lut_value(const uint16_t* lut, uint32_t c) {
  return f16_bits_to_f32(lut[c]);
}

// e^(-i phi) in fp64 for phi = t * theta reduced modulo 2 pi in fp64 (Cody-Waite: 2 pi
// as a 24-bit head, so that k * head is exact for the k < 2^29 of any position below
// 2^31, plus a tail; the reduced angle lies in [-pi, pi]).
constexpr double kTwoPiHi = 0x1.921fb4p+2;
constexpr double kTwoPiLo = 0x1.4442d18469899p-22;
constexpr double kInvTwoPi = 0x1.45f306dc9c883p-3;

__device__ __forceinline__ float2 cmul(float2 a, float2 b) {
  return make_float2(fmaf(a.x, b.x, -(a.y * b.y)), fmaf(a.x, b.y, a.y * b.x));
}

__device__ __forceinline__ double2 rot_at64(int64_t t, double theta) {
  const double x = (double)t * theta;
  const double k = rint(x * kInvTwoPi);
  const double ph = fma(-k, kTwoPiLo, fma(-k, kTwoPiHi, x));
  double s, c;
  sincos(ph, &s, &c);
  return make_double2(c, -s);
}

__device__ __forceinline__ double2 cmul64(double2 a, double2 b) {
  return make_double2(fma(a.x, b.x, -(a.y * b.y)), fma(a.x, b.y, a.y * b.x));
}

__device__ __forceinline__ float2 to_f32(double2 a) { return make_float2((float)a.x, (float)a.y); }

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

// Running state of a wave.  The value sums o are kept scaled by 2^-e (per head): the
// packed blocks' weights p_t * scale_t enter the fp16 dot products as p_t * scale_t * 2^-e,
// with e raised (and o rescaled) whenever a weight would reach 2^15, so no weight
// overflows fp16 and the largest keep 11 significant bits.
template <int GQ>
struct NuqState {
  float m[GQ], l[GQ], o[GQ][2], mv[GQ];
  int e[GQ];
};

__device__ __forceinline__ float softmax_step(float s, float& m, float& l, float& alpha) {
  alpha = 1.0f;
  if (__any(s > m + 8.0f)) {               // the max may lag by 8 (log2): p < 2^8
    const float mn = fmaxf(m, wave_max(s));
    alpha = __builtin_amdgcn_exp2f(m - mn);   // v_exp_f32: 0 while m = -inf
    m = mn;
    l *= alpha;
  }
  // s - m <= 8; results below 2^-126 flush to 0, a weight no output can feel
  const float p = __builtin_amdgcn_exp2f(s - m);
  l += p;
  return p;
}

struct PairConsts {
  float2 q[8];        // (q_2i, q_2i+1) per query head
  float2 step;        // e^(-i theta_i)
  float2 r16;         // e^(-i 16 theta_i)
  float tc;           // 2 cos(theta_i)
  double2 step32;     // e^(-i 32 theta_i): from one block to the next
  double theta;       // theta_i
  float ks0, km0, ks1, km1;   // key scale / min of channels 2i, 2i+1
};

// Any real-linear function x(t) of q e^(-i t theta) (its real part, its imaginary part,
// a combination of both) satisfies x(t+1) = 2 cos(theta) x(t) - x(t-1): one fma per
// token instead of a complex product.  An error made at token s reaches token t scaled
// by sin((t-s) theta) / sin(theta), at most t - s, so over the (at most) 32 tokens of a
// chain the recurrence keeps a relative error of ~2e-5 even where theta is tiny.
__device__ __forceinline__ float cheb_next(float tc, float cur, float prev) {
  return fmaf(tc, cur, -prev);
}

// The block's partial scores of this lane's pair for one head, from dequantized keys:
// two chains (tokens 0..15 and 16..31) of the rotated query q e^(-i t theta).
__device__ __forceinline__ void pair_scores(float (&part)[32], float2 qb, const PairConsts& pc,
                                            const float (&k0)[32], const float (&k1)[32]) {
  float2 a[2], b[2];           // the chain's values at tokens k and k + 1
  a[0] = qb;
  a[1] = cmul(qb, pc.r16);
  b[0] = cmul(a[0], pc.step);
  b[1] = cmul(a[1], pc.step);
#pragma unroll
  for (int k = 0; k < 16; ++k) {
#pragma unroll
    for (int ch = 0; ch < 2; ++ch)
      part[16 * ch + k] = fmaf(a[ch].x, k0[16 * ch + k], a[ch].y * k1[16 * ch + k]);
    if (k < 15) {
#pragma unroll
      for (int ch = 0; ch < 2; ++ch) {
        float2 n = b[ch];
        if (k < 14)
          n = make_float2(cheb_next(pc.tc, b[ch].x, a[ch].x), cheb_next(pc.tc, b[ch].y, a[ch].y));
        a[ch] = b[ch];
        b[ch] = n;
      }
    }
  }
}

// (u, v, w) of a rotated query c for one head with the key metadata folded in:
// u = s_2i Re(c), v = s_2i+1 Im(c), w = m_2i Re(c) + m_2i+1 Im(c), so that the pair's
// score of codes (l0, l1) is u l0 + v l1 + w.  All three are real-linear in c.
struct Uvw {
  float u, v, w;
};
__device__ __forceinline__ Uvw uvw_of(float2 c, const PairConsts& pc) {
  return Uvw{pc.ks0 * c.x, pc.ks1 * c.y, fmaf(pc.km0, c.x, pc.km1 * c.y)};
}
__device__ __forceinline__ Uvw cheb_next(float tc, const Uvw& cur, const Uvw& prev) {
  return Uvw{cheb_next(tc, cur.u, prev.u), cheb_next(tc, cur.v, prev.v),
             cheb_next(tc, cur.w, prev.w)};
}

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
  float lutk[16], lutv[16];
  // Code-book pairs: entry a + 2^B b (the first 4^B entries) holds (lut[a], lut[b]) as
  // fp16 halves.  Keys look up the two channels of a lane's pair at one token, values two
  // tokens of one channel.
  uint32_t tk[256], tv[256];
};

// Per-wave scratch (LDS).
template <int GQ, int B>
struct NuqWaveScratch {
  float ps[GQ][kGroup];      // window chunks: p_t of the chunk's tokens (scaled by 2^-e)
  uint16_t psh[GQ][kGroup];  // packed blocks: fp16 p_t * scale_t * 2^-e of the block's tokens
  float2 qb[GQ][64];         // q e^(-i t0 theta_i) per head and pair: the block's first token
  float corr[GQ][64];        // per CSR entry of the window: its score correction
  float pv[GQ][kGroup];      // p_t of the block's tokens (value outliers)
  uint32_t vmeta[kGroup];    // value scale / min of the block's tokens
  float vcorr[GQ][kHeadDim]; // value-outlier corrections of the block, per channel
};

template <int B>
struct NuqBlockRegs {
  uint32_t kw[2 * B], vw[2 * B];   // key / value code words of channels 2l, 2l+1
  uint32_t vmeta;            // value scale / min of token lane >> 1
};

// The block's outlier entries: key CSR entries [e_begin, e_begin + n), the first 64 of
// them (one per lane), the first 64 value-outlier entries, and this lane's token row.
// The block loop requests them one block ahead of their use, from row pointers loaded
// two blocks ahead, so that neither dependent load makes a wave wait.
struct NuqBlockEntries {
  int32_t e_begin, n;        // n entries from e_begin (at most one per code of the block)
  uint32_t ent, vent;
  uint32_t rows;             // row of token lane >> 1 relative to e_begin: lo | hi << 16
};

// A wave's (batch, kv head) streams, uniform: resolved once so that the block loop
// keeps a few base pointers in scalar registers instead of the whole argument block.
struct NuqStreams {
  const uint32_t* kc;        // key code words of packed block 0
  const uint32_t* vc;        // value code words of packed block 0
  const uint32_t* vm;        // value scale / min of packed token 0
  const int32_t* rp;         // CSR row pointers of packed token 0 (vm without key outliers)
  const uint32_t* ent;       // CSR entries
  const uint32_t* vout;      // value-outlier entries of packed token 0 (NULL: none)
  int32_t csr_cap;           // at most INT32_MAX (checked by the host)
  int rp_step;               // 1; 0 without key outliers (both row loads read vm)
  int v_kv;                  // value outliers per token
  float scale_log2;
};

// 2B consecutive code words of a lane's channel pair.
template <int B>
__device__ __forceinline__ void load_words(uint32_t* dst, const uint32_t* p) {
  if constexpr (B == 3) {
    const uint2 x = ld_stream2(p);
    const uint4 y = ld_stream4(p + 2);
    dst[0] = x.x; dst[1] = x.y; dst[2] = y.x; dst[3] = y.y; dst[4] = y.z; dst[5] = y.w;
  } else {
#pragma unroll
    for (int i = 0; i < B / 2; ++i) {
      const uint4 x = ld_stream4(p + 4 * i);
      dst[4 * i] = x.x; dst[4 * i + 1] = x.y; dst[4 * i + 2] = x.z; dst[4 * i + 3] = x.w;
    }
  }
}

template <int B>
__device__ __forceinline__ void load_nuq_block(NuqBlockRegs<B>& r, const NuqStreams& S,
                                               int64_t blk, int lane) {
  load_words<B>(r.kw, S.kc + blk * (kHeadDim * B) + 2 * lane * B);
  load_words<B>(r.vw, S.vc + blk * (kHeadDim * B) + 2 * lane * B);
  r.vmeta = S.vm[blk * kGroup + (lane >> 1)];
}

// Row pointers of the block: the even lane of token t loads the start of its row, the odd
// lane the end.  Unconditional (without key outliers it reads a value-metadata word,
// ignored by load_block_entries), so that no register copy of a conditionally loaded
// value makes the wave wait for the loads just issued.
__device__ __forceinline__ int32_t load_rows(const NuqStreams& S, int64_t blk, int lane) {
  return S.rp[blk * kGroup + (lane >> 1) + (lane & 1) * S.rp_step];
}

__device__ __forceinline__ NuqBlockEntries load_block_entries(const NuqStreams& S, int64_t blk,
                                                              int32_t rp, int lane) {
  NuqBlockEntries e;
  e.e_begin = e.n = 0;
  e.rows = 0;
  if (S.rp_step) {
    const int32_t other = __builtin_amdgcn_update_dpp(0, rp, 0xB1, 0xF, 0xF, false);
    const int32_t r0 = (lane & 1) ? other : rp, r1 = (lane & 1) ? rp : other;
    KVQ_CHECK(r0 >= 0 && r0 <= r1 && r1 <= S.csr_cap, kDbgCsr);
    const int32_t b0 = max(__builtin_amdgcn_readlane(rp, 0), 0);
    const int32_t b1 = min(__builtin_amdgcn_readlane(rp, 63), S.csr_cap);
    e.e_begin = b0;
    e.n = min(max(b1 - b0, 0), kGroup * kHeadDim);
    // relative to b0 in unsigned arithmetic (wraps, never traps), clamped to [0, n]
    const int lo = min(max((int)((uint32_t)r0 - (uint32_t)b0), 0), e.n);
    const int hi = min(max((int)((uint32_t)r1 - (uint32_t)b0), 0), e.n);
    e.rows = (uint32_t)lo | ((uint32_t)hi << 16);
  }
  e.ent = 0;
  if (lane < e.n) e.ent = (S.ent + e.e_begin)[lane];
  e.vent = 0;
  if (S.vout != nullptr && lane < kGroup * S.v_kv) e.vent = S.vout[blk * kGroup * S.v_kv + lane];
  return e;
}

template <int GQ, int B>
__device__ void process_nuq_block(const NuqStreams& S, int64_t blk, const NuqBlockRegs<B>& r, const NuqBlockEntries& be,
                                  const PairConsts& pc,
                                  float2 base,   // e^(-i t0 theta); q e^(-i t0 theta) if GQ == 1
                                  const Lut<B>& lk, NuqState<GQ>& st,
                                  const NuqShared<GQ>& sh, NuqWaveScratch<GQ, B>& ws, int lane) {
  const int t = lane >> 1;                  // this lane's token after the reduction
  const uint32_t* kw0 = r.kw;
  const uint32_t* kw1 = r.kw + B;
  const uint32_t* vw0 = r.vw;
  const uint32_t* vw1 = r.vw + B;

  // The block's CSR entries [e_begin, e_begin + n_ent) (the first 64 already requested) and
  // value outliers: v_kv per token, 32 * v_kv entries from vbase.
  const int32_t e_begin = be.e_begin, n_ent = be.n;
  const int v_ne = S.vout != nullptr ? kGroup * S.v_kv : 0;
  const int64_t vbase = blk * kGroup * S.v_kv;

  // ---- keys: dequantize this lane's pair for the 32 tokens, then per head the
  // rotated-query partial scores and their sum across lanes
  float s[GQ];
  float2 qb[GQ];
  if constexpr (GQ == 1) {
    // one head: the key metadata ride in the chains (u, v, w), and the lookups of each
    // chain step are used at once
    float part[32];
    qb[0] = base;                                    // q e^(-i t0 theta), see the caller
    {
      // one chain over the 32 tokens; the pair-table entries of tokens 4 m4 .. 4 m4 + 3
      // are requested one group ahead of their use
      Uvw c0 = uvw_of(qb[0], pc), c1 = uvw_of(cmul(qb[0], pc.step), pc);   // tokens k, k + 1
      uint32_t eb[2][4];
      auto fetch = [&](uint32_t (&e)[4], int m4) {
        const uint32_t x = key_pair_idx<B>(kw0, kw1, m4);
        e[0] = pair_entry<0>(sh.tk, x);
        e[1] = pair_entry<1>(sh.tk, x);
        e[2] = pair_entry<2>(sh.tk, x);
        e[3] = pair_entry<3>(sh.tk, x);
      };
      fetch(eb[0], 0);
#pragma unroll
      for (int m4 = 0; m4 < 8; ++m4) {
        if (m4 < 7) fetch(eb[(m4 + 1) & 1], m4 + 1);
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
          const int k = 4 * m4 + kk;
          const uint32_t e = eb[m4 & 1][kk];
          part[k] = fmaf(c0.u, lo_f16(e), fmaf(c0.v, hi_f16(e), c0.w));
          if (k < 31) {
            Uvw n = c1;
            if (k < 30) n = cheb_next(pc.tc, c1, c0);
            c0 = c1;
            c1 = n;
          }
        }
      }
    }
    s[0] = transpose_sum32(part, lane);
  } else {
    float kd0[32], kd1[32];
#pragma unroll
    for (int m4 = 0; m4 < 8; ++m4) {
      uint32_t a01, a23, b01, b23;
      lut4<B>(lk, codes_of<B>(kw0, m4), a01, a23);
      lut4<B>(lk, codes_of<B>(kw1, m4), b01, b23);
      kd0[4 * m4 + 0] = fmaf(lo_f16(a01), pc.ks0, pc.km0);
      kd0[4 * m4 + 1] = fmaf(hi_f16(a01), pc.ks0, pc.km0);
      kd0[4 * m4 + 2] = fmaf(lo_f16(a23), pc.ks0, pc.km0);
      kd0[4 * m4 + 3] = fmaf(hi_f16(a23), pc.ks0, pc.km0);
      kd1[4 * m4 + 0] = fmaf(lo_f16(b01), pc.ks1, pc.km1);
      kd1[4 * m4 + 1] = fmaf(hi_f16(b01), pc.ks1, pc.km1);
      kd1[4 * m4 + 2] = fmaf(lo_f16(b23), pc.ks1, pc.km1);
      kd1[4 * m4 + 3] = fmaf(hi_f16(b23), pc.ks1, pc.km1);
    }
#pragma unroll
    for (int j = 0; j < GQ; ++j) {
      float part[32];
      qb[j] = cmul(pc.q[j], base);
      pair_scores(part, qb[j], pc, kd0, kd1);
      s[j] = transpose_sum32(part, lane);
    }
  }

  // ---- outliers: token t's CSR entries replace the dequantized code by the exact value.
  // Entries are taken in windows of 64, one per lane: every entry lane computes its
  // correction comp(q e^(-i (t0 + te) theta)) * (x - dequant(0)) (an outlier's position
  // stores code 0; the real part for an even channel, the imaginary part for an odd one;
  // te is the token's place in the block, stored in the entry), and the two lanes of
  // token t add the corrections of its row, every other entry each in row order, then
  // exchange their sums.
  if (n_ent > 0) {
#pragma unroll
    for (int j = 0; j < GQ; ++j) ws.qb[j][lane] = qb[j];
    __builtin_amdgcn_wave_barrier();
    // this lane's token row relative to e_begin (within [0, n_ent]; the clamps below
    // keep every LDS index inside the window)
    const int rlo = (int)(be.rows & 0xFFFFu);
    const int rhi = (int)(be.rows >> 16);
    auto window = [&](int off, uint32_t ent) {
      if (off + lane < n_ent) {
        KVQ_CHECK(((ent >> 8) & 0xFFu) < (uint32_t)kGroup && (ent & 0xFFu) < (uint32_t)kHeadDim,
                  kDbgEntry);
        const int te = (int)((ent >> 8) & (kGroup - 1));
        const int col = (int)(ent & (kHeadDim - 1));
        const int pr = col >> 1;
        const float x = f16_bits_to_f32((uint16_t)(ent >> 16));
        const float khat = fmaf(sh.lutk[0], sh.ks[col], sh.km[col]);
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
      const int lo = max(rlo, off) - off;
      const int hi = min(rhi, min(n_ent, off + 64)) - off;
      float acc[GQ];
#pragma unroll
      for (int j = 0; j < GQ; ++j) acc[j] = 0.f;
      for (int e = lo + (lane & 1); e < hi; e += 2) {
#pragma unroll
        for (int j = 0; j < GQ; ++j) acc[j] += ws.corr[j][e];
      }
#pragma unroll
      for (int j = 0; j < GQ; ++j) s[j] += acc[j] + dpp<0xB1>(0.f, acc[j]);
      __builtin_amdgcn_wave_barrier();
    };
    // the first window from the entries already in registers; more than 64 entries in
    // a block (rare) are loaded window by window
    window(0, be.ent);
    for (int off = 64; off < n_ent; off += 64)
      window(off, off + lane < n_ent ? (S.ent + e_begin)[off + lane] : 0u);
  }

  // ---- softmax (lanes 2t and 2t+1 both carry the corrected score of token t)
  float p[GQ], alpha[GQ];
#pragma unroll
  for (int j = 0; j < GQ; ++j) s[j] *= S.scale_log2;
  softmax_block<GQ>(st, s, p, alpha);

  // ---- values: fp16 weights p * scale * 2^-e per token into LDS, p * min per lane
  const float vs = lo_f16(r.vmeta), vm = hi_f16(r.vmeta);
#pragma unroll
  for (int j = 0; j < GQ; ++j) {
    const float w = p[j] * vs;
    float wsc = ldexpf(w, -st.e[j]);
    float o0 = st.o[j][0] * alpha[j], o1 = st.o[j][1] * alpha[j];
    if (__any(wsc >= 32768.0f)) {
      // a weight would reach 2^15: raise e so that the block's largest weight lands in
      // [2^14, 2^15), and rescale the sums (powers of two: exact)
      int x;
      (void)frexpf(wave_max(w), &x);
      const int e1 = x - 15;
      o0 = ldexpf(o0, st.e[j] - e1);
      o1 = ldexpf(o1, st.e[j] - e1);
      st.e[j] = e1;
      wsc = ldexpf(w, -e1);
    }
    // the value pair tables pair tokens 8q + k and 8q + 4 + k: token t = 8q + 4h + k
    // goes to half h of pair 4q + k
    const int slot = (t & ~7) | ((t & 3) << 1) | ((t >> 2) & 1);
    ws.psh[j][slot] = __builtin_bit_cast(uint16_t, (_Float16)wsc);
    st.mv[j] = fmaf(p[j], vm, st.mv[j] * alpha[j]);     // every token counted twice
    st.o[j][0] = o0;
    st.o[j][1] = o1;
  }
#pragma unroll
  for (int j = 0; j < GQ; ++j) {
    float o0 = st.o[j][0], o1 = st.o[j][1];
    const uint4* pp = reinterpret_cast<const uint4*>(&ws.psh[j][0]);
#pragma unroll
    for (int i = 0; i < 4; ++i) {                // tokens 8i..8i+7
      const uint4 w8 = pp[i];
      const uint32_t x0 = value_pair_idx<B>(vw0, i), x1 = value_pair_idx<B>(vw1, i);
      const uint32_t wk[4] = {w8.x, w8.y, w8.z, w8.w};
#pragma unroll
      for (int k = 0; k < 4; ++k) {              // tokens 8i + k, 8i + 4 + k
        const uint32_t e0 = k == 0   ? pair_entry<0>(sh.tv, x0)
                            : k == 1 ? pair_entry<1>(sh.tv, x0)
                            : k == 2 ? pair_entry<2>(sh.tv, x0)
                                     : pair_entry<3>(sh.tv, x0);
        const uint32_t e1 = k == 0   ? pair_entry<0>(sh.tv, x1)
                            : k == 1 ? pair_entry<1>(sh.tv, x1)
                            : k == 2 ? pair_entry<2>(sh.tv, x1)
                                     : pair_entry<3>(sh.tv, x1);
        o0 = __builtin_amdgcn_fdot2(as_h2(wk[k]), as_h2(e0), o0, false);
        o1 = __builtin_amdgcn_fdot2(as_h2(wk[k]), as_h2(e1), o1, false);
      }
    }
    st.o[j][0] = o0;
    st.o[j][1] = o1;
  }

  // ---- value outliers: each token's entries replace the dequantized value (of code 0,
  // the code stored at an outlier) by the exact one.  One lane per entry adds
  // p_t * (x - v_hat) for its channel into LDS; each lane then takes its two channels'
  // sums.
  if (v_ne > 0) {
    if (!(lane & 1)) {
      ws.vmeta[t] = r.vmeta;
#pragma unroll
      for (int j = 0; j < GQ; ++j) ws.pv[j][t] = p[j];
    }
    __builtin_amdgcn_wave_barrier();
    for (int e0 = 0; e0 < v_ne; e0 += 64) {
      const int e = e0 + lane;
      if (e < v_ne) {
        const uint32_t ent = e0 == 0 ? be.vent : S.vout[vbase + e];
        const int te = (e / S.v_kv) & (kGroup - 1);
        KVQ_CHECK((ent & 0xFFFFu) < (uint32_t)kHeadDim, kDbgEntry);
        const int d = (int)(ent & (kHeadDim - 1));
        const float x = f16_bits_to_f32((uint16_t)(ent >> 16));
        const uint32_t vmw = ws.vmeta[te];
        const float vhat = sh.lutv[0] * lo_f16(vmw) + hi_f16(vmw);
#pragma unroll
        for (int j = 0; j < GQ; ++j) atomicAdd(&ws.vcorr[j][d], ws.pv[j][te] * (x - vhat));
      }
    }
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int j = 0; j < GQ; ++j) {
      const float2 cv = *reinterpret_cast<const float2*>(&ws.vcorr[j][2 * lane]);
      st.o[j][0] += ldexpf(cv.x, -st.e[j]);
      st.o[j][1] += ldexpf(cv.y, -st.e[j]);
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
  const float2 base = to_f32(rot_at64(pos0, pc.theta));
  float k0[32], k1[32];
#pragma unroll
  for (int k = 0; k < 32; ++k) {
    k0[k] = lo_f16(kv[k]);
    k1[k] = hi_f16(kv[k]);
  }
  float s[GQ], p[GQ], alpha[GQ];
#pragma unroll
  for (int j = 0; j < GQ; ++j) {
    float part[32];
    pair_scores(part, cmul(pc.q[j], base), pc, k0, k1);
    s[j] = transpose_sum32(part, lane) * a.scale_log2;
    if (t >= nvalid) s[j] = kNegInf;
  }
  softmax_block<GQ>(st, s, p, alpha);
#pragma unroll
  for (int j = 0; j < GQ; ++j) {
    psL[j][t] = ldexpf(p[j], -st.e[j]);      // the sums are kept scaled by 2^-e
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

// One query head: 4 waves per SIMD (at most 128 VGPRs) for nuq2 and nuq3; nuq4, whose
// 16-entry lookups need more registers, spills at that bound and runs at 3 (150 VGPRs:
// 386 against 438 us on a 256K-token context; nuq2 at 3 waves measured 2 % slower).
template <int GQ, int NW, int B>
__global__ __launch_bounds__(NW * kWave, GQ == 1 ? 4 : 1) void decode_nuq_kernel(
    DecodeArgs a) {
  constexpr int NT = NW * kWave;
  __shared__ NuqShared<GQ> sh;
  __shared__ __align__(16) NuqWaveScratch<GQ, B> wsc[NW];
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
  const double2 step64 = rot_at64(1, pc.theta);
  pc.step = to_f32(step64);
  pc.tc = (float)(2.0 * step64.x);
  pc.r16 = to_f32(rot_at64(16, pc.theta));
  pc.step32 = rot_at64(kGroup, pc.theta);
  if (a.n_blocks > 0) {
    const uint2 km = *reinterpret_cast<const uint2*>(a.k_meta + bh * kHeadDim + 2 * lane);
    pc.ks0 = lo_f16(km.x); pc.km0 = hi_f16(km.x);
    pc.ks1 = lo_f16(km.y); pc.km1 = hi_f16(km.y);
  } else {
    pc.ks0 = pc.km0 = pc.ks1 = pc.km1 = 0.f;
  }
  const Lut<B> lk = load_lut<B>(a.lut_k);
  for (int j = wave; j < kGroup; j += NW) sh.rot[j][lane] = to_f32(rot_at64(j, pc.theta));
  if (wave == 0) {
    sh.ks[2 * lane] = pc.ks0; sh.km[2 * lane] = pc.km0;
    sh.ks[2 * lane + 1] = pc.ks1; sh.km[2 * lane + 1] = pc.km1;
    if (lane < (1 << B)) sh.lutk[lane] = lut_value(a.lut_k, lane);
    if (lane < (1 << B)) sh.lutv[lane] = lut_value(a.lut_v, lane);
    if constexpr (B == 3) {
      sh.tk[lane] = a.lut_k[lane & 7] | ((uint32_t)a.lut_k[lane >> 3] << 16);
      sh.tv[lane] = a.lut_v[lane & 7] | ((uint32_t)a.lut_v[lane >> 3] << 16);
    } else if constexpr (B == 2) {
      if (lane < 16) {
        sh.tk[lane] = a.lut_k[lane & 3] | ((uint32_t)a.lut_k[lane >> 2] << 16);
        sh.tv[lane] = a.lut_v[lane & 3] | ((uint32_t)a.lut_v[lane >> 2] << 16);
      }
    } else {
      for (int i = lane; i < 256; i += kWave) {
        sh.tk[i] = a.lut_k[i & 15] | ((uint32_t)a.lut_k[i >> 4] << 16);
        sh.tv[i] = a.lut_v[i & 15] | ((uint32_t)a.lut_v[i >> 4] << 16);
      }
    }
  }
  __syncthreads();

  NuqState<GQ> st;
#pragma unroll
  for (int j = 0; j < GQ; ++j) {
    st.m[j] = kNegInf;
    st.l[j] = 0.f;
    st.o[j][0] = st.o[j][1] = 0.f;
    st.mv[j] = 0.f;
    st.e[j] = -24;
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
  KVQ_CHECK(a.n_blocks <= a.cap_blocks && s1 <= units, kDbgSplit);
  if (b0 < b1) {
    // One block in flight ahead of the one being processed (clamped index, unrolled by
    // two so no register copy waits on the loads just issued).
    const int last = b1 - 1;
    NuqStreams S;
    const int64_t bt = bh * (a.cap_blocks * kGroup);      // this head's first token slot
    S.kc = a.k_codes + bh * a.cap_blocks * (kHeadDim * B);
    S.vc = a.v_codes + bh * a.cap_blocks * (kHeadDim * B);
    S.vm = a.v_meta + bt;
    S.rp = a.csr_rowptr ? a.csr_rowptr + bh * (a.cap_blocks * kGroup + 1)
                        : reinterpret_cast<const int32_t*>(S.vm);
    S.rp_step = a.csr_rowptr ? 1 : 0;
    S.ent = a.csr_ent + bh * a.csr_capacity;
    S.csr_cap = (int32_t)a.csr_capacity;
    S.vout = a.v_out ? a.v_out + bt * a.v_kv : nullptr;
    S.v_kv = a.v_kv;
    S.scale_log2 = a.scale_log2;
    // Code words one block ahead of their use; row pointers two blocks ahead, so that the
    // entries they locate can be requested one block ahead.
    NuqBlockRegs<B> r0, r1;
    int32_t rp0 = load_rows(S, b0, lane);
    int32_t rp1 = load_rows(S, min(b0 + 1, last), lane);
    load_nuq_block<B>(r0, S, b0, lane);
    NuqBlockEntries e0 = load_block_entries(S, b0, rp0, lane), e1;
    // e^(-i t0 theta) of the current block, in fp64 from block to block; with one query
    // head the query is folded in (the block then starts from q e^(-i t0 theta) itself)
    double2 base = rot_at64(a.n_sink + (int64_t)b0 * kGroup, pc.theta);
    if constexpr (GQ == 1) base = cmul64(base, make_double2(pc.q[0].x, pc.q[0].y));
    for (int i = b0; i < b1; i += 2) {
      // block i: entries e0 and codes r0 requested one block ago; now the entries of block
      // i + 1 (its rows arrived), the rows of block i + 2, the codes of block i + 1
      e1 = load_block_entries(S, min(i + 1, last), rp1, lane);
      rp0 = load_rows(S, min(i + 2, last), lane);
      load_nuq_block<B>(r1, S, min(i + 1, last), lane);
      process_nuq_block<GQ, B>(S, i, r0, e0, pc, to_f32(base), lk, st, sh, wsc[wave], lane);
      base = cmul64(base, pc.step32);
      if (i + 1 >= b1) break;
      e0 = load_block_entries(S, min(i + 2, last), rp0, lane);
      rp1 = load_rows(S, min(i + 3, last), lane);
      load_nuq_block<B>(r0, S, min(i + 2, last), lane);
      process_nuq_block<GQ, B>(S, i + 1, r1, e1, pc, to_f32(base), lk, st, sh, wsc[wave],
                               lane);
      base = cmul64(base, pc.step32);
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
        make_float2(ldexpf(st.o[j][0], st.e[j]) + mvall, ldexpf(st.o[j][1], st.e[j]) + mvall);
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

hipError_t launch_decode_nuq(const DecodeArgs& a, int gq, int bits, hipStream_t s) {
  const int64_t wgs = (int64_t)a.batch * a.kv_heads * a.splits;
  const int nw = a.waves_per_group;
  dim3 grid((unsigned)wgs), block((unsigned)(nw * kWave));
#define KVQ_DN(G_, NW_, B_)                                               \
  if (gq == G_ && nw == NW_ && bits == B_) {                              \
    decode_nuq_kernel<G_, NW_, B_><<<grid, block, 0, s>>>(a);             \
    hipError_t e_ = hipGetLastError();                                    \
    if (e_ != hipSuccess || a.splits == 1) return e_;                     \
    return launch_merge_splits(a, s);                                     \
  }
#define KVQ_DNB(B_) KVQ_DN(1, 4, B_) KVQ_DN(2, 4, B_) KVQ_DN(4, 4, B_) KVQ_DN(8, 4, B_)
  KVQ_DNB(2) KVQ_DNB(3) KVQ_DNB(4)
#undef KVQ_DNB
#undef KVQ_DN
  return hipErrorInvalidValue;
}

const void* decode_nuq_fn(int gq, int nw, int bits) {
#define KVQ_DF(G_, B_)                                                    \
  if (nw == 4 && gq == G_ && bits == B_)                                  \
    return reinterpret_cast<const void*>(&decode_nuq_kernel<G_, 4, B_>);
#define KVQ_DFB(B_) KVQ_DF(1, B_) KVQ_DF(2, B_) KVQ_DF(4, B_) KVQ_DF(8, B_)
  KVQ_DFB(2) KVQ_DFB(3) KVQ_DFB(4)
#undef KVQ_DFB
#undef KVQ_DF
  return nullptr;
}

uint32_t debug_take_decode_nuq() { return debug_take_local(); }

}  // namespace kvq
