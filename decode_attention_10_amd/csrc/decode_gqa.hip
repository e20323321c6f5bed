// Decode attention for grouped queries (several query heads per kv head) on the matrix
// cores.
//
// With g query heads sharing a kv head, the scores S = Q K_hat^T and the output
// O = P V_hat are small dense products (g rows against the block's 32 tokens and 128
// channels) - the case where the dequantized dot products stop being HBM-bound and the
// vector ALUs become the limit ("The KV cache has a geometry problem", section on
// grouped-query attention; KIVI post, "Experiments").  The scores run on
// v_mfma_f32_16x16x32_bf16 and the value products on v_mfma_f32_16x16x32_f16; the codes
// never leave their packed form except for one AND-OR per pair:
//
//   * a 2-bit (4-bit) code field masked into the low mantissa bits of a bf16 (fp16) 1.0
//     is the exact value 1 + c * 2^(p - 7) (1 + c * 2^(p - 10)), p = the field's bit
//     position, so one v_and_or_b32 turns two codes into two matrix elements;
//   * the key weights q * scale are fp32, each split into bf16 hi + lo (about 16
//     significant bits), both rows of the A operand, the factor 2^(7 - p) folded in;
//   * the value weights p * scale enter as fp16, scaled by 2^-e with e the wave's
//     exponent, raised (and the sums rescaled by an exact power of two) whenever a weight
//     would reach 2^15; one rounding per weight, at most 2^-11 relative;
//   * the constant 1 of every element is removed with one more product against a
//     constant matrix (-1 for the scores, +1 for the value weights' column sums), with
//     the same rounded weights, so it cancels exactly.
//
// Keys: rows = (head, hi/lo), K = channels (4 steps of 32), columns = 16 tokens; the
// weights reach the A operand through LDS in matrix order.  Values: rows = 16 channel
// octets (one channel of each per product, 8 products per block), K = the block's 32
// tokens, columns = (head, value group); weights p * scale are formed directly in the
// B operand registers.  Softmax, the q . min and p . min terms and the window chunks
// (fp16, through the vector path) follow the vector kernel.  One workgroup of 8 waves
// (4 from four heads per CU on) handles one (batch, kv head) and a range of blocks dealt
// round-robin to its waves (8-wave groups: 33.9 us on the llama3_8b GQA shape against
// 34.5 us with 4-wave groups),
// streamed with nontemporal loads, one block in flight per wave (measured on the
// llama3_8b GQA shape: 34.5-35.1 us against 36.6-37.1 us with two blocks in flight and
// plain loads); each wave leaves a packed-block partial and a window partial, merged in
// LDS.
#include "decode_common.h"

namespace kvq {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr uint32_t kOne2 = 0x3F803F80u;        // (1.0, 1.0) as bf16
constexpr uint32_t kMinusOne2 = 0xBF80BF80u;   // (-1.0, -1.0)
constexpr int kARow = 136;                     // bf16 per weight row in LDS (128 + pad)
constexpr int kPRow = 36;                      // floats per p / value-meta row (32 + pad)

// Constants of the AND-OR unpacking kept in registers (SGPR masks, VGPR one): the
// 3-operand v_and_or_b32 cannot take two 32-bit literals, so with both constants as
// literals the compiler would emit a separate AND and OR.
struct Unpack {
  uint32_t one;                 // (1.0, 1.0) bf16, VGPR
  uint32_t one_h;               // (1.0, 1.0) fp16, VGPR
  uint32_t m2[3];               // 2-bit field masks at positions 0, 2, 4 of each half
  uint32_t m4;                  // 4-bit field mask at position 0 of each half
};

__device__ __forceinline__ uint32_t opaque_sgpr(uint32_t x) {
  return __builtin_amdgcn_readfirstlane(__builtin_amdgcn_mov_dpp(x, 0xE4, 0xF, 0xF, true));
}

__device__ __forceinline__ Unpack make_unpack() {
  Unpack u;
  u.one = __builtin_amdgcn_mov_dpp(kOne2, 0xE4, 0xF, 0xF, true);
  u.one_h = __builtin_amdgcn_mov_dpp(0x3C003C00u, 0xE4, 0xF, 0xF, true);
  u.m2[0] = opaque_sgpr(0x00030003u);
  u.m2[1] = opaque_sgpr(0x000C000Cu);
  u.m2[2] = opaque_sgpr(0x00300030u);
  u.m4 = opaque_sgpr(0x000F000Fu);
  return u;
}

__device__ __forceinline__ uint32_t and_or(uint32_t w, uint32_t mask, uint32_t one) {
  return (w & mask) | one;
}

__device__ __forceinline__ f32x4 mfma16(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
__device__ __forceinline__ f32x4 mfma16h(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}
__device__ __forceinline__ uint32_t pack_f16(float x0, float x1) {
  const h2_t v = {(_Float16)x0, (_Float16)x1};
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ uint32_t pack_bf16(float x0, float x1) {
  const bf16x2 v = {(__bf16)x0, (__bf16)x1};
  return __builtin_bit_cast(uint32_t, v);
}

// x = hi + lo + r with hi, lo bf16 (round to nearest) and |r| <= 2^-17 |x|.
__device__ __forceinline__ void split_bf16(float x0, float x1, uint32_t& hi, uint32_t& lo) {
  hi = pack_bf16(x0, x1);
  const float h0 = __builtin_bit_cast(float, hi << 16);
  const float h1 = __builtin_bit_cast(float, hi & 0xFFFF0000u);
  lo = pack_bf16(x0 - h0, x1 - h1);
}

// Bit position (0, 2 or 4) of pair j's 2-bit fields after the shift that brings them
// into bits 0..5 of each half: pairs 0-2 unshifted, 3-5 shifted by 6, 6-7 by 12.
__host__ __device__ constexpr int pair_pos2(int j) { return 2 * (j % 3); }
__device__ __forceinline__ float pair_factor(int bits, int j) {   // 2^(7 - p)
  return bits == 2 ? (float)(1 << (7 - pair_pos2(j))) : 128.0f;
}

// The four bf16 pairs of K-step ks from this lane's key words (see key_pair_channel).
template <int KB>
__device__ __forceinline__ u32x4 key_step_pairs(const uint32_t* k, int ks, const Unpack& u) {
  if constexpr (KB == 2) {
    const uint32_t w = k[ks >> 1];
    if ((ks & 1) == 0)
      return u32x4{and_or(w, u.m2[0], u.one), and_or(w, u.m2[1], u.one),
                   and_or(w, u.m2[2], u.one), and_or(w >> 6, u.m2[0], u.one)};
    const uint32_t w6 = w >> 6, w12 = w >> 12;
    return u32x4{and_or(w6, u.m2[1], u.one), and_or(w6, u.m2[2], u.one),
                 and_or(w12, u.m2[0], u.one), and_or(w12, u.m2[1], u.one)};
  } else {
    const uint32_t w = k[ks];
    return u32x4{and_or(w, u.m4, u.one), and_or(w >> 4, u.m4, u.one),
                 and_or(w >> 8, u.m4, u.one), and_or(w >> 12, u.m4, u.one)};
  }
}

// Pair T (tile T: channel T of the octet) of the four token-pair words of a value tile.
template <int VB>
__device__ __forceinline__ u32x4 value_tile_pairs(const uint32_t* vc, int t, const Unpack& u,
                                                  uint32_t one) {
  if constexpr (VB == 2) {
    const int sh = t < 3 ? 0 : t < 6 ? 6 : 12;
    const uint32_t m = u.m2[t % 3];
    return u32x4{and_or(vc[0] >> sh, m, one), and_or(vc[1] >> sh, m, one),
                 and_or(vc[2] >> sh, m, one), and_or(vc[3] >> sh, m, one)};
  } else {
    const int base = 4 * (t >> 2), sh = 4 * (t & 3);
    return u32x4{and_or(vc[base] >> sh, u.m4, one), and_or(vc[base + 1] >> sh, u.m4, one),
                 and_or(vc[base + 2] >> sh, u.m4, one), and_or(vc[base + 3] >> sh, u.m4, one)};
  }
}

// Channels of the key pair (ks, kg, i): the two channels whose codes form element pair
// i of this lane group's K-step ks (see key_operands).
template <int KB>
__device__ __forceinline__ int key_pair_channel(int ks, int kg, int i) {
  if constexpr (KB == 2) return 32 * kg + 16 * (ks >> 1) + 4 * (ks & 1) + i;   // and + 8
  else return 32 * kg + 8 * ks + i;                                            // and + 4
}

template <int KB, int VB>
struct GqRegs {
  uint32_t k0[KB];     // token n (column) of the block, channel quarter kg
  uint32_t k1[KB];     // token n + 16
  uint32_t km[2];      // key meta of this lane's channel pair
  uint32_t vc[2 * VB]; // value tile (token octet kg, channel octet n)
  uint32_t vm[2];      // value meta words lane and lane + 64
};

template <int KB, int VB>
__device__ __forceinline__ void gq_load(GqRegs<KB, VB>& r, const uint32_t* kc, const uint32_t* km,
                                        const uint32_t* vc, const uint32_t* vm, int blk, int lane,
                                        int kch0, int kch1) {
  constexpr int WK = kHeadDim * KB / 32;
  const int n = lane & 15, kg = lane >> 4;
  const uint32_t* kp = kc + (uint32_t)blk * (kGroup * WK) + (uint32_t)(n * WK + kg * KB);
  if constexpr (KB == 2) {
    const uint2 x = ld_stream2(kp);
    const uint2 y = ld_stream2(kp + 16 * WK);
    r.k0[0] = x.x; r.k0[1] = x.y; r.k1[0] = y.x; r.k1[1] = y.y;
  } else {
    const uint4 x = ld_stream4(kp);
    const uint4 y = ld_stream4(kp + 16 * WK);
    r.k0[0] = x.x; r.k0[1] = x.y; r.k0[2] = x.z; r.k0[3] = x.w;
    r.k1[0] = y.x; r.k1[1] = y.y; r.k1[2] = y.z; r.k1[3] = y.w;
  }
  const uint32_t* mp = km + (uint32_t)blk * kHeadDim;
  // The two key-meta loads each read half of the same four 128-byte lines (the lanes'
  // channel pairs interleave), so they stay plain loads: the lines must survive in L2
  // from the first to the second (measured 34.2-34.8 us against 34.8-36.6 us with the
  // streaming hint on the llama3_8b GQA shape).
  r.km[0] = mp[(uint32_t)kch0];
  r.km[1] = mp[(uint32_t)kch1];
  const uint4* vp = reinterpret_cast<const uint4*>(vc + (uint32_t)blk * (kHeadDim * VB) +
                                                   (uint32_t)(lane * 2 * VB));
#pragma unroll
  for (int i = 0; i < VB / 2; ++i) {
    const uint4 u = ld_stream4(vp + i);
    r.vc[4 * i] = u.x; r.vc[4 * i + 1] = u.y; r.vc[4 * i + 2] = u.z; r.vc[4 * i + 3] = u.w;
  }
  const uint32_t* mv = vm + (uint32_t)blk * (kGroup * 4);
  r.vm[0] = ld_stream(mv + (uint32_t)lane);
  r.vm[1] = ld_stream(mv + (uint32_t)lane + 64);
}

// Per-wave LDS of the packed-block path.
template <int GQ>
struct GqShared {
  uint16_t aw[16][kARow];      // key weights, rows (head, hi/lo), K order (kg, ks, e)
  float pl[GQ][kPRow];         // softmax p of the block per head and token
  uint32_t vml[4][kPRow];      // value meta words per group and token
  float alpha[GQ];             // rescale factors of a max update
};

// Sum over the wave of GQ values per lane (GQ = 2 or 4), returned in SGPR-uniform form.
template <int GQ>
__device__ __forceinline__ void wave_sums(const float* x, float* out, int lane) {
  float v;
  if constexpr (GQ == 4) {
    const bool odd = lane & 1, hi2 = lane & 2;
    const float ka = odd ? x[1] : x[0], sa = odd ? x[0] : x[1];
    const float kb = odd ? x[3] : x[2], sb = odd ? x[2] : x[3];
    const float ya = ka + dpp<kQuadSwap1>(0.f, sa);   // even lanes: x0 pairs, odd: x1
    const float yb = kb + dpp<kQuadSwap1>(0.f, sb);   // even lanes: x2 pairs, odd: x3
    const float kz = hi2 ? yb : ya, sz = hi2 ? ya : yb;
    v = kz + dpp<kQuadSwap2>(0.f, sz);                // lane holds x[lane & 3] over its quad
  } else {
    const bool odd = lane & 1;
    const float k = odd ? x[1] : x[0], s = odd ? x[0] : x[1];
    v = k + dpp<kQuadSwap1>(0.f, s);                  // x[lane & 1] over the lane pair
    v += dpp<kQuadSwap2>(0.f, v);
  }
  v += dpp<kRowRor4>(0.f, v);                         // lanes of equal (lane & 3) in a row
  v += dpp<kRowRor8>(0.f, v);
  v += __shfl_xor(v, 16);
  v += __shfl_xor(v, 32);
#pragma unroll
  for (int j = 0; j < GQ; ++j)
    out[j] = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), j));
}

__device__ __forceinline__ float row_max(float x) {   // over the 16 lanes of a row
  x = fmaxf(x, dpp<kQuadSwap1>(kNegInf, x));
  x = fmaxf(x, dpp<kQuadSwap2>(kNegInf, x));
  x = fmaxf(x, dpp<kRowHalfMirror>(kNegInf, x));
  x = fmaxf(x, dpp<kRowMirror>(kNegInf, x));
  return x;
}
__device__ __forceinline__ float row_sum(float x) {
  x += dpp<kQuadSwap1>(0.f, x);
  x += dpp<kQuadSwap2>(0.f, x);
  x += dpp<kRowHalfMirror>(0.f, x);
  x += dpp<kRowMirror>(0.f, x);
  return x;
}

template <int GQ>
struct GqState {
  float m[2];          // running max of this lane group's heads 2u, 2u + 1 (score lanes)
  float l[2];          // p sums of those heads over this lane's tokens
  float mv;            // p * min over this lane's tokens, column (head, group)
  f32x4 acc[8];        // value products: tile T, rows = channel octets, cols = (head, group)
  f32x4 corr;          // column sums of the value weights (the constant-1 part)
  int e;               // fp16 value weights: acc and corr are kept scaled by 2^-e
};

template <int KB, int VB, int GQ>
__device__ __forceinline__ void gq_block(const GqRegs<KB, VB>& r, GqState<GQ>& st,
                                         GqShared<GQ>& sh, const float (*qf)[2],
                                         const uint32_t* qpair, float cscale, const Unpack& up,
                                         int lane, int kg_w, int ks_w, int i_w) {
  const int n = lane & 15, u = lane >> 4;

  // ---- key weights w = q * scale (fp32) -> bf16 hi/lo rows of the A operand in LDS;
  // q . min per head summed over the wave
  const uint32_t kmin2 = __builtin_amdgcn_perm(r.km[1], r.km[0], 0x07060302u);
  float cm[GQ];
#pragma unroll
  for (int j = 0; j < GQ; ++j) {
    uint32_t hi, lo;
    split_bf16(qf[j][0] * lo_f16(r.km[0]), qf[j][1] * lo_f16(r.km[1]), hi, lo);
    const int col = 32 * kg_w + 8 * ks_w + 2 * i_w;
    *reinterpret_cast<uint32_t*>(&sh.aw[2 * j][col]) = hi;
    *reinterpret_cast<uint32_t*>(&sh.aw[2 * j + 1][col]) = lo;
    cm[j] = __builtin_amdgcn_fdot2(as_h2(qpair[j]), as_h2(kmin2), 0.0f, false);
  }
  float cmin[GQ];
  wave_sums<GQ>(cm, cmin, lane);
#pragma unroll
  for (int j = 0; j < GQ; ++j) cmin[j] *= cscale;           // log2 units, like the products

  // ---- scores: C = -rowsum(A) + A * codes, two 16-token halves
  u32x4 aop[4];
  {
    const uint4* ap = reinterpret_cast<const uint4*>(&sh.aw[n][32 * u]);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const uint4 x = ap[ks];
      aop[ks] = u32x4{x.x, x.y, x.z, x.w};
    }
  }
  f32x4 off = {0.f, 0.f, 0.f, 0.f};
  const u32x4 mone = {kMinusOne2, kMinusOne2, kMinusOne2, kMinusOne2};
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) off = mfma16(aop[ks], mone, off);
  f32x4 s0 = off, s1 = off;
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    s0 = mfma16(aop[ks], key_step_pairs<KB>(r.k0, ks, up), s0);
    s1 = mfma16(aop[ks], key_step_pairs<KB>(r.k1, ks, up), s1);
  }

  // ---- softmax: lane group u holds heads 2u, 2u+1 (rows 4u..4u+3 = (head, hi/lo))
  const bool valid = 2 * u < GQ;
  const int jA = valid ? 2 * u : 0;
  const float cA = GQ == 4 ? (u == 0 ? cmin[0] : cmin[GQ == 4 ? 2 : 0]) : cmin[0];
  const float cB = GQ == 4 ? (u == 0 ? cmin[1] : cmin[GQ == 4 ? 3 : 1]) : cmin[1];
  const float sA0 = valid ? s0[0] + s0[1] + cA : kNegInf;
  const float sA1 = valid ? s1[0] + s1[1] + cA : kNegInf;
  const float sB0 = valid ? s0[2] + s0[3] + cB : kNegInf;
  const float sB1 = valid ? s1[2] + s1[3] + cB : kNegInf;
  const float mxA = fmaxf(sA0, sA1), mxB = fmaxf(sB0, sB1);
  if (__any(mxA > st.m[0] + kMaxSlack || mxB > st.m[1] + kMaxSlack)) {
    const float nA = fmaxf(st.m[0], row_max(mxA)), nB = fmaxf(st.m[1], row_max(mxB));
    const float aA = fast_exp2(st.m[0] - nA), aB = fast_exp2(st.m[1] - nB);
    st.m[0] = nA; st.m[1] = nB;
    st.l[0] *= aA; st.l[1] *= aB;
    if (valid && n == 0) {
      sh.alpha[jA] = aA;
      sh.alpha[jA + 1] = aB;
    }
    // value accumulators of column (head, group) = (n / 4, n % 4)
    const float al = sh.alpha[min(n >> 2, GQ - 1)];
    st.mv *= al;
#pragma unroll
    for (int t = 0; t < 8; ++t) st.acc[t] *= al;
    st.corr *= al;
  }
  const float pA0 = fast_exp2(sA0 - st.m[0]), pA1 = fast_exp2(sA1 - st.m[0]);
  const float pB0 = fast_exp2(sB0 - st.m[1]), pB1 = fast_exp2(sB1 - st.m[1]);
  st.l[0] += pA0 + pA1;
  st.l[1] += pB0 + pB1;
  if (valid) {
    sh.pl[jA][n] = pA0;
    sh.pl[jA][n + 16] = pA1;
    sh.pl[jA + 1][n] = pB0;
    sh.pl[jA + 1][n + 16] = pB1;
  }
  // value meta of the block, transposed to [group][token]
  sh.vml[lane & 3][lane >> 2] = r.vm[0];
  sh.vml[lane & 3][16 + (lane >> 2)] = r.vm[1];

  // ---- value weights p * scale for column (head n/4, group n%4), tokens 8u .. 8u+7
  const int jc = min(n >> 2, GQ - 1), gc = n & 3;
  float pw[8];
  uint32_t vw[8];
  {
    const float4* pp = reinterpret_cast<const float4*>(&sh.pl[jc][8 * u]);
    const float4 a0 = pp[0], a1 = pp[1];
    pw[0] = a0.x; pw[1] = a0.y; pw[2] = a0.z; pw[3] = a0.w;
    pw[4] = a1.x; pw[5] = a1.y; pw[6] = a1.z; pw[7] = a1.w;
    const uint4* mp = reinterpret_cast<const uint4*>(&sh.vml[gc][8 * u]);
    const uint4 b0 = mp[0], b1 = mp[1];
    vw[0] = b0.x; vw[1] = b0.y; vw[2] = b0.z; vw[3] = b0.w;
    vw[4] = b1.x; vw[5] = b1.y; vw[6] = b1.z; vw[7] = b1.w;
  }
  // fp16 weights p * scale * 2^-e, e the wave's exponent: raised (and the sums rescaled
  // by an exact power of two) whenever a weight would reach 2^15
  float w8[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) w8[i] = pw[i] * lo_f16(vw[i]);
#pragma unroll
  for (int i = 0; i < 4; ++i)
    st.mv = fmaf(pw[2 * i], hi_f16(vw[2 * i]), fmaf(pw[2 * i + 1], hi_f16(vw[2 * i + 1]), st.mv));
  float wmax = w8[0];
#pragma unroll
  for (int i = 1; i < 8; ++i) wmax = fmaxf(wmax, w8[i]);
  if (__any(ldexpf(wmax, -st.e) >= 32768.0f)) {
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) wmax = fmaxf(wmax, __shfl_xor(wmax, o));
    int x;
    (void)frexpf(wmax, &x);
    const int e1 = __builtin_amdgcn_readfirstlane(x - 15);
#pragma unroll
    for (int t = 0; t < 8; ++t)
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) st.acc[t][rr] = ldexpf(st.acc[t][rr], st.e - e1);
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) st.corr[rr] = ldexpf(st.corr[rr], st.e - e1);
    st.e = e1;
  }
  u32x4 bw;
#pragma unroll
  for (int i = 0; i < 4; ++i) bw[i] = pack_f16(ldexpf(w8[2 * i], -st.e), ldexpf(w8[2 * i + 1], -st.e));
  const u32x4 ones = {up.one_h, up.one_h, up.one_h, up.one_h};
  st.corr = mfma16h(ones, bw, st.corr);
#pragma unroll
  for (int t = 0; t < 8; ++t)
    st.acc[t] = mfma16h(value_tile_pairs<VB>(r.vc, t, up, up.one_h), bw, st.acc[t]);
}

template <int KB, int VB, int GQ, int NW>
__global__ __launch_bounds__(NW * kWave) void decode_gqa_kernel(DecodeArgs a) {
  constexpr int CPW = 32 / KB;
  __shared__ __align__(16) uint32_t qh[GQ][64];
  __shared__ __align__(16) GqShared<GQ> shw[NW];
  __shared__ __align__(16) float winp[NW][GQ][4][kRow];
  __shared__ float wm[2 * NW][GQ], wl[2 * NW][GQ];
  __shared__ __align__(16) float wo[2 * NW][GQ][kHeadDim];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int split = blockIdx.x % a.splits;
  const int64_t bh = blockIdx.x / a.splits;
  const int b = (int)(bh / a.kv_heads);
  const int hkv = (int)(bh % a.kv_heads);
  const int hq0 = hkv * GQ;
  GqShared<GQ>& sh = shw[wave];
  const Unpack up = make_unpack();

  // this lane's key pair for the weight rows: (kg, ks, i) and its two channels
  const int kg_w = lane >> 4, ks_w = (lane >> 2) & 3, i_w = lane & 3;
  const int kch0 = key_pair_channel<KB>(ks_w, kg_w, i_w);
  const int kch1 = kch0 + (KB == 2 ? 8 : 4);
  const float fp = pair_factor(KB, KB == 2 ? 4 * (ks_w & 1) + i_w : i_w);
  float qf[GQ][2];
  uint32_t qpair[GQ];
  const uint16_t* qb = a.q + ((int64_t)b * a.q_heads + hq0) * kHeadDim;
#pragma unroll
  for (int j = 0; j < GQ; ++j) {
    const uint16_t q0 = qb[j * kHeadDim + kch0], q1 = qb[j * kHeadDim + kch1];
    qf[j][0] = f16_bits_to_f32(q0) * fp * a.scale_log2;
    qf[j][1] = f16_bits_to_f32(q1) * fp * a.scale_log2;
    qpair[j] = (uint32_t)q0 | ((uint32_t)q1 << 16);
    if (wave == 0) qh[j][lane] = *reinterpret_cast<const uint32_t*>(qb + j * kHeadDim + 2 * lane);
  }
  // zero weight rows beyond the heads (never written again)
  for (int i = lane; i < (16 - 2 * GQ) * (kARow / 2); i += kWave)
    reinterpret_cast<uint32_t*>(&sh.aw[2 * GQ][0])[i] = 0u;
  __syncthreads();

  const int nchunks = fp16_chunks(a);
  const int units = a.n_blocks + kWindowUnits * nchunks;
  const int s0 = (int)((int64_t)units * split / a.splits);
  const int s1 = (int)((int64_t)units * (split + 1) / a.splits);
  const int bend = min(s1, a.n_blocks);
  KVQ_CHECK(a.n_blocks <= a.cap_blocks && s1 <= units, kDbgSplit);
  const int first = s0 + wave;
  const int cnt = first < bend ? (bend - first + NW - 1) / NW : 0;

  // ---- window chunks through the vector path, as their own partial
  {
    WaveState<GQ> ws;
    init_wave_state<GQ>(ws);
    for (int c = 0; c < nchunks; ++c) {
      const int u = a.n_blocks + kWindowUnits * c;
      if (u >= s0 && u < s1 && NW - 1 - (c % NW) == wave)
        process_window<GQ, VB>(a, bh, c, ws, qh, reinterpret_cast<float(*)[kGroup]>(winp[wave]), lane);
    }
    finish_wave_state<GQ, VB>(ws, wm[NW + wave], wl[NW + wave], wo[NW + wave], lane);
  }

  // ---- packed blocks on the matrix cores
  GqState<GQ> st;
  st.m[0] = st.m[1] = kNegInf;
  if (2 * (lane >> 4) >= GQ) st.m[0] = st.m[1] = 0.f;   // lane groups without heads
  st.l[0] = st.l[1] = 0.f;
  st.mv = 0.f;
#pragma unroll
  for (int t = 0; t < 8; ++t) st.acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  st.corr = f32x4{0.f, 0.f, 0.f, 0.f};
  st.e = -24;
  if (cnt > 0) {
    const int64_t seg = bh * a.cap_blocks;
    const uint32_t* kc = a.k_codes + seg * (kGroup * kHeadDim * KB / 32);
    const uint32_t* km = a.k_meta + seg * kHeadDim;
    const uint32_t* vc = a.v_codes + seg * (kHeadDim * VB);
    const uint32_t* vm = a.v_meta + seg * (kGroup * 4);
    const int last = cnt - 1;
    GqRegs<KB, VB> r0, r1;
    gq_load<KB, VB>(r0, kc, km, vc, vm, first, lane, kch0, kch1);
    for (int k = 0; k < cnt; k += 2) {
      gq_load<KB, VB>(r1, kc, km, vc, vm, first + min(k + 1, last) * NW, lane, kch0, kch1);
      gq_block<KB, VB, GQ>(r0, st, sh, qf, qpair, a.scale_log2, up, lane, kg_w, ks_w, i_w);
      if (k + 1 >= cnt) break;
      gq_load<KB, VB>(r0, kc, km, vc, vm, first + min(k + 2, last) * NW, lane, kch0, kch1);
      gq_block<KB, VB, GQ>(r1, st, sh, qf, qpair, a.scale_log2, up, lane, kg_w, ks_w, i_w);
    }
  }

  // ---- packed partial: m, l per head; outputs of the lanes whose column group matches
  // their rows' group
  {
    const int n = lane & 15, u = lane >> 4;
    const float lA = row_sum(st.l[0]), lB = row_sum(st.l[1]);
    if (2 * u < GQ && n == 0) {
      wm[wave][2 * u] = st.m[0];
      wm[wave][2 * u + 1] = st.m[1];
      wl[wave][2 * u] = lA;
      wl[wave][2 * u + 1] = lB;
    }
    float mv = st.mv;
    mv += __shfl_xor(mv, 16);
    mv += __shfl_xor(mv, 32);
    const int j = n >> 2, g = n & 3;
    if (j < GQ && g == u) {
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        // fp16 elements 1 + c 2^(p - 10), sums scaled by 2^-e
        const float f = ldexpf(VB == 2 ? pair_factor(2, t) * 8.0f : 1024.0f, st.e);
#pragma unroll
        for (int rr = 0; rr < 4; ++rr)
          wo[wave][j][8 * (4 * u + rr) + t] = (st.acc[t][rr] - st.corr[rr]) * f + mv;
      }
    }
  }
  __syncthreads();
  merge_partials<GQ, 2 * NW>(a, wm, wl, wo, b, hq0, split);
}

}  // namespace

hipError_t launch_decode_gqa(const DecodeArgs& a, int k_bits, int v_bits, int gq,
                             hipStream_t s) {
  const int64_t wgs = (int64_t)a.batch * a.kv_heads * a.splits;
  const int nw = a.waves_per_group;
  dim3 grid((unsigned)wgs), block((unsigned)(nw * kWave));
#define KVQ_GL(KB_, VB_, G_, NW_)                                                   \
  if (k_bits == KB_ && v_bits == VB_ && gq == G_ && nw == NW_) {                    \
    decode_gqa_kernel<KB_, VB_, G_, NW_><<<grid, block, 0, s>>>(a);                 \
    hipError_t e_ = hipGetLastError();                                              \
    if (e_ != hipSuccess || a.splits == 1) return e_;                               \
    return launch_merge_splits(a, s);                                               \
  }
#define KVQ_GLB(G_, NW_) KVQ_GL(2, 2, G_, NW_) KVQ_GL(2, 4, G_, NW_) KVQ_GL(4, 2, G_, NW_) \
  KVQ_GL(4, 4, G_, NW_)
  KVQ_GLB(2, 4) KVQ_GLB(4, 4) KVQ_GLB(2, 8) KVQ_GLB(4, 8)
#undef KVQ_GLB
#undef KVQ_GL
  return hipErrorInvalidValue;
}

const void* decode_gqa_fn(int k_bits, int v_bits, int gq, int nw) {
#define KVQ_GF(KB_, VB_, G_, NW_)                                                   \
  if (k_bits == KB_ && v_bits == VB_ && gq == G_ && nw == NW_)                      \
    return reinterpret_cast<const void*>(&decode_gqa_kernel<KB_, VB_, G_, NW_>);
#define KVQ_GFB(G_, NW_) KVQ_GF(2, 2, G_, NW_) KVQ_GF(2, 4, G_, NW_) KVQ_GF(4, 2, G_, NW_) \
  KVQ_GF(4, 4, G_, NW_)
  KVQ_GFB(2, 4) KVQ_GFB(4, 4) KVQ_GFB(2, 8) KVQ_GFB(4, 8)
#undef KVQ_GFB
#undef KVQ_GF
  return nullptr;
}

uint32_t debug_take_decode_gqa() { return debug_take_local(); }

}  // namespace kvq
