// Non-uniform 2-, 3- and 4-bit quantizers with per-vector dense-and-sparse outliers.
//
// KVQuant review ("KVQuant: Towards 10 Million Context Length LLM Inference with KV
// Cache Quantization"), abstract items (i)-(iv): keys are quantized per channel and
// before RoPE, with a non-uniform datatype, and in each vector the largest-magnitude
// entries are kept in full precision in a sparse matrix; values are quantized per
// token.  Readings (shared with the oracle): (min, scale) over the dense entries
// exactly as the uniform quantizer with B bits; the normalized value (x - min) * inv
// goes to the nearest code-book level (ties to the even index); a key channel's
// outliers are its ceil(n * bp / 1e4) largest fp16 magnitudes, ties to lower tokens.
//
// Keys (one shot over the whole context, per (batch, head, channel)):
//   1. magnitude histogram of the top 8 of the 15 magnitude bits, per channel
//   2. the bin that holds the k-th largest magnitude
//   3. histogram of the low 7 bits inside that bin  ->  exact threshold T and the
//      number of elements equal to T that are outliers (the earliest tokens); the same
//      read gathers, per chunk of tokens, the dense min/max below that bin, the count
//      above it, and a list of the bin's own entries
//   4. per chunk of tokens: ties to T, magnitudes above T, the last positive/negative
//      tie, dense min/max (from the lists of step 3; a chunk whose list overflowed is
//      read again)
//   5. per channel: tie prefix of every chunk, dense min/max -> (scale, min), and each
//      chunk's outlier count (above T plus the ties ranked below the tie quota)
//   6. per (batch, head): scan of the chunk counts -> each chunk's first CSR entry
//   7. codes for every element; the rows of the CSR (row pointers and entries, exact
//      values from the tile) written in token order by the same pass
// Steps 1, 3 and 7 read the keys with coalesced rows; histograms live in LDS and only
// their non-zero bins reach global memory.
#include "kvq_common.h"

namespace kvq {
namespace {

constexpr int kThreads = 256;

// Midpoints between consecutive code-book levels (2^B - 1 of them).
template <int B>
struct Mids {
  float m[(1 << B) - 1];
};

template <int B>
__device__ __forceinline__ Mids<B> load_mids(const uint16_t* lut) {
  Mids<B> r;
#pragma unroll
  for (int i = 0; i < (1 << B) - 1; ++i)
    r.m[i] = (f16_bits_to_f32(lut[i]) + f16_bits_to_f32(lut[i + 1])) * 0.5f;
  return r;
}

// Index of the nearest code-book level (ties to the even index): the number of
// midpoints below xn, plus one for a midpoint equal to xn above an odd level (the tie
// then goes to the even level above).  The code book ascends strictly, so its midpoints
// do too (each is the exact fp32 half-sum of two fp16 levels) and the count is the code.
template <int B>
__device__ __forceinline__ uint32_t nuq_code(float xn, const Mids<B>& md) {
  uint32_t c = 0;
#pragma unroll
  for (int i = 0; i < (1 << B) - 1; ++i) c += (i & 1) ? (xn >= md.m[i]) : (xn > md.m[i]);
  return c;
}

// The same search in one comparison.  The level axis [0, 2^B) is cut into cells of half a
// level; a cell holds at most one midpoint of a code book whose levels lie in [0, 2^B - 1]
// at least half a level apart (checked when the cells are built: otherwise the counting
// search above is used).  Cell i keeps the number of midpoints below it and twice its
// own midpoint (+inf if none), the midpoint one ulp lower above an odd level so that
// xn > it settles a tie toward the even level.  The search takes xn2 = 2 xn, formed as
// (x - min) * (2 inv): scaling by two commutes with rounding, so xn2 is exactly twice the
// normalized value, its integer part is the cell that holds it, and xn2 > 2 m exactly
// when xn > m.
template <int B>
struct CodeCells {
  static constexpr int N = 2 << B;
  float2 e[N];                      // (2 x threshold, code below the cell as float bits)
};

// Built by the first N threads; returns, to every thread of the block (a barrier), whether
// the cells decide every code.
template <int B>
__device__ bool build_code_cells(CodeCells<B>& cc, const Mids<B>& md, int tid) {
  constexpr int NM = (1 << B) - 1;
  int bad = 0;
  if (tid < CodeCells<B>::N) {
    const float lo = 0.5f * (float)tid, hi = 0.5f * (float)(tid + 1);
    uint32_t below = 0;
    int inside = 0;
    float thr = __builtin_inff();
#pragma unroll
    for (int j = 0; j < NM; ++j) {
      const float m = md.m[j];
      if (m < lo) {
        ++below;
      } else if (m < hi) {
        ++inside;
        thr = (j & 1) ? __builtin_bit_cast(float, __builtin_bit_cast(uint32_t, m) - 1u) : m;
      }
    }
    bad = inside > 1 || (tid == 0 && (below > 0 || (inside == 1 && thr <= 0.0f))) ||
          (tid == CodeCells<B>::N - 1 && md.m[NM - 1] >= hi);
    cc.e[tid] = make_float2(2.0f * thr, __builtin_bit_cast(float, below));
  }
  return !__syncthreads_or(bad);
}

// Float to unsigned with the hardware's saturation (negative and NaN to 0, too large to
// the maximum).  Arithmetic only.
__device__ __forceinline__ uint32_t cvt_u32_sat(float x) {
  uint32_t r;
  asm("v_cvt_u32_f32 %0, %1" : "=v"(r) : "v"(x));
  return r;
}

// Codes of 16 values, one per byte (value jj in byte jj % 4 of cb[jj / 4]), ORed into
// cb, from xn2_of(jj): twice the normalized value, or -inf for a value that takes code 0
// (-inf lands in cell 0, whose code below is 0, under its threshold; and under every
// midpoint of the counting search).  Branch-free, in groups of G values whose cell reads
// are all issued before the first of them is used.  CELLS selects the search at compile
// time (see CellsTag).
template <int B, int G, bool CELLS, class Xn2Of>
__device__ __forceinline__ void nuq_code16(uint32_t (&cb)[4], Xn2Of xn2_of,
                                           const CodeCells<B>& cc, const Mids<B>& md) {
#pragma unroll
  for (int g = 0; g < 16; g += G) {
    float xn2[G];
    uint32_t c[G];
#pragma unroll
    for (int jj = 0; jj < G; ++jj) xn2[jj] = xn2_of(g + jj);
    if constexpr (CELLS) {
      float2 e[G];
#pragma unroll
      for (int jj = 0; jj < G; ++jj)
        e[jj] = cc.e[min(cvt_u32_sat(xn2[jj]), (uint32_t)(CodeCells<B>::N - 1))];
#pragma unroll
      for (int jj = 0; jj < G; ++jj)
        c[jj] = __builtin_bit_cast(uint32_t, e[jj].y) + (xn2[jj] > e[jj].x ? 1u : 0u);
    } else {
#pragma unroll
      for (int jj = 0; jj < G; ++jj) c[jj] = nuq_code<B>(xn2[jj] * 0.5f, md);
    }
#pragma unroll
    for (int jj = 0; jj < G; ++jj) cb[(g + jj) >> 2] |= c[jj] << (8 * ((g + jj) & 3));
  }
}

// The search as a type, so that a workgroup's whole tile loop is compiled once per search
// and the uniform choice between them is one branch before the loop (a choice per group
// of values lets the compiler compute the counting search beside the cell lookups).
template <bool V>
struct CellsTag {
  static constexpr bool value = V;
};

// (scale, min) of a dense range for B-bit codes: scale = (max - min) / (2^B - 1).
__device__ __forceinline__ void params_nuq(float mn, float mx, int bits, uint32_t* meta,
                                           float* mn_o, float* inv_o) {
  mn = mn + 0.0f;
  mx = mx + 0.0f;
  const uint16_t min_h = f32_to_f16_bits(mn);
  const uint16_t scale_h = f32_to_f16_bits((mx - mn) / (float)((1 << bits) - 1));
  const float s = f16_bits_to_f32(scale_h);
  *mn_o = mn;
  *inv_o = (s == 0.0f) ? 0.0f : 1.0f / s;
  *meta = (uint32_t)scale_h | ((uint32_t)min_h << 16);
}

// Exact sums for Q-Norm.  An fp16 value is an integer multiple of 2^-24 with
// |x| * 2^24 < 2^40, so sum x is an integer in units of 2^-24 and sum x^2 a 128-bit
// integer in units of 2^-48.  Both are exact in any order of addition and are rounded
// once to fp64 at the end (nearest, ties to even), which makes the moments independent
// of how the tokens are split over chunks, lanes and workgroups.
struct ExactSums {
  uint64_t x_lo;   // sum of x * 2^24, 128-bit two's complement
  int64_t x_hi;
  uint64_t q_lo;   // sum of (x * 2^24)^2, 128-bit unsigned
  uint64_t q_hi;
};

__device__ __forceinline__ void exact_zero(ExactSums& s) { s.x_lo = s.q_lo = s.q_hi = 0; s.x_hi = 0; }

// x * 2^24 of the fp16 value with bits h (finite): (1024 + m) << (e - 1), or m if e = 0.
__device__ __forceinline__ int64_t f16_units(uint32_t h) {
  const uint32_t e = (h >> 10) & 31u, m = h & 1023u;
  const uint64_t mag = e ? (uint64_t)(m | 1024u) << (e - 1) : (uint64_t)m;
  return (h & 0x8000u) ? -(int64_t)mag : (int64_t)mag;
}

__device__ __forceinline__ void exact_add_parts(ExactSums& s, uint64_t xl, int64_t xh,
                                                uint64_t ql, uint64_t qh) {
  const uint64_t a = s.x_lo + xl;
  s.x_hi += xh + (a < s.x_lo ? 1 : 0);
  s.x_lo = a;
  const uint64_t b = s.q_lo + ql;
  s.q_hi += qh + (b < s.q_lo ? 1u : 0u);
  s.q_lo = b;
}

// one fp16 value
__device__ __forceinline__ void exact_add(ExactSums& s, uint32_t h) {
  const int64_t x = f16_units(h);
  const uint64_t mag = (uint64_t)(x < 0 ? -x : x);
  exact_add_parts(s, (uint64_t)x, x < 0 ? -1 : 0, mag * mag, __umul64hi(mag, mag));
}

__device__ __forceinline__ void exact_merge(ExactSums& s, const ExactSums& o) {
  exact_add_parts(s, o.x_lo, o.x_hi, o.q_lo, o.q_hi);
}

// the sums of the lane `mask` apart added in (all lanes of the pattern take part)
__device__ __forceinline__ void exact_merge_xor(ExactSums& s, int mask) {
  ExactSums o;
  o.x_lo = __shfl_xor(s.x_lo, mask);
  o.x_hi = __shfl_xor(s.x_hi, mask);
  o.q_lo = __shfl_xor(s.q_lo, mask);
  o.q_hi = __shfl_xor(s.q_hi, mask);
  exact_merge(s, o);
}

// Nearest fp64 (ties to even) of the 128-bit unsigned (hi, lo): the top 64 bits with
// every lower bit folded into bit 0 (a sticky bit below the 53 kept bits), converted,
// then scaled by the power of two shifted out.
__device__ __forceinline__ double u128_to_f64(uint64_t lo, uint64_t hi) {
  if (hi == 0) return (double)lo;
  const int lz = __clzll((long long)hi);
  const int sh = 64 - lz;
  uint64_t v = lz ? (hi << lz) | (lo >> sh) : hi;
  const uint64_t rest = lz ? (lo << lz) : lo;
  v |= rest != 0 ? 1u : 0u;
  return ldexp((double)v, sh);
}

// (sum x, sum x^2) in fp64, each the exact sum rounded once.
__device__ __forceinline__ void exact_to_f64(const ExactSums& s, double* sx, double* sxx) {
  uint64_t lo = s.x_lo, hi = (uint64_t)s.x_hi;
  const bool neg = s.x_hi < 0;
  if (neg) {
    lo = ~lo + 1u;
    hi = ~hi + (lo == 0 ? 1u : 0u);
  }
  const double m = u128_to_f64(lo, hi);
  *sx = ldexp(neg ? -m : m, -24);
  *sxx = ldexp(u128_to_f64(s.q_lo, s.q_hi), -48);
}

// Q-Norm of one vector ("KVQuant" review, "Proposed method": the dequantized
// distribution matched to the statistics before quantization): from the dense
// entries' sum and sum of squares (fp64) and their code histogram, the metadata
// (a * scale, a * min + b) that give the dequantized entries the original mean and
// variance; a = sqrt(var / var_hat) (1 if var_hat = 0), b = mean - a * mean_hat, the
// moments of the dequantized entries taken level by level (ascending) in fp64 from
// the fp32 level values lut[c] * scale + min.  The old metadata stand if n = 0.
__device__ uint32_t qnorm_meta(uint32_t meta, double sx, double sxx, const uint32_t* hist,
                               uint32_t n, const uint16_t* lut, int bits) {
  if (n == 0) return meta;
  const double dn = (double)n;
  const double mean = sx / dn;
  double var = sxx / dn - mean * mean;
  if (var < 0.0) var = 0.0;
  const float s = f16_bits_to_f32((uint16_t)(meta & 0xFFFFu));
  const float m = f16_bits_to_f32((uint16_t)(meta >> 16));
  double m1 = 0.0, m2 = 0.0;
  for (int c = 0; c < (1 << bits); ++c) {
    const double lev = (double)(f16_bits_to_f32(lut[c]) * s + m);
    const double cnt = (double)hist[c];
    m1 += cnt * lev;
    m2 += cnt * lev * lev;
  }
  const double mean_hat = m1 / dn;
  double var_hat = m2 / dn - mean_hat * mean_hat;
  if (var_hat < 0.0) var_hat = 0.0;
  const double a = var_hat > 0.0 ? sqrt(var / var_hat) : 1.0;
  const double b = mean - a * mean_hat;
  const uint16_t s_h = f32_to_f16_bits((float)(a * (double)s));
  const uint16_t m_h = f32_to_f16_bits((float)(a * (double)m + b));
  return (uint32_t)s_h | ((uint32_t)m_h << 16);
}

__device__ __forceinline__ const uint16_t* key_row(const NuqKeysArgs& a, int64_t bh,
                                                   int64_t t) {
  const int64_t b = bh / a.kv_heads, h = bh % a.kv_heads;
  return a.k + b * a.sb + h * a.sh + t * a.st;
}

__global__ void fill_u32_kernel(uint32_t* p, int64_t n, uint32_t v) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x)
    p[i] = v;
}

typedef short s16x2 __attribute__((ext_vector_type(2)));

// Per-half fp16 max / min of two pairs (finite inputs), without the canonicalizing
// multiplies the compiler would add around the generic min / max.
__device__ __forceinline__ uint32_t pk_max_f16(uint32_t x, uint32_t y) {
  uint32_t r;
  asm("v_pk_max_f16 %0, %1, %2" : "=v"(r) : "v"(x), "v"(y));
  return r;
}
__device__ __forceinline__ uint32_t pk_min_f16(uint32_t x, uint32_t y) {
  uint32_t r;
  asm("v_pk_min_f16 %0, %1, %2" : "=v"(r) : "v"(x), "v"(y));
  return r;
}
// Bits of a where mask is set, of b elsewhere (one v_bfi_b32; written out, the compiler
// turns a per-half mask back into compares and selects).
__device__ __forceinline__ uint32_t bitsel(uint32_t mask, uint32_t a, uint32_t b) {
  uint32_t r;
  asm("v_bfi_b32 %0, %1, %2, %3" : "=v"(r) : "v"(mask), "v"(a), "v"(b));
  return r;
}

// ---- 1/3: magnitude histograms (LDS counts are u16 pairs packed in u32) ------------
// A lane owns two adjacent channels (one 4-byte load per token).  The high-bin pass keeps
// 256 bins per channel, so a workgroup takes half of the channels (64): its LDS (33 KB)
// then lets four workgroups share a CU, where 128 channels (66 KB) allowed two; half-wave
// lane groups take different tokens.  The low-bin pass (128 bins) takes all 128.  Each
// channel's row of counters is padded by one word so that the rows of different channels
// start on different LDS banks: key magnitudes crowd into a few bins, and unpadded rows
// put a wave's atomics on the same few banks.  Sixteen tokens' loads are issued before
// their atomics.
//
// The low-bin pass also gathers what the chunk statistics need once the threshold T
// inside the high bin is known: per chunk and channel the min / max of the entries below
// the high bin (dense whatever T is), the count of those above it (outliers whatever T
// is), and the entries of the high bin itself, as (fp16 bits << 16 | token in the
// chunk), at most kNuqListCap per channel.  The count is stored even when it exceeds the
// list; such a chunk is read again by the statistics pass.  (Lists per token row with
// counters in registers instead of one LDS counter per channel measured slower: 2.46 ms
// against 2.37 ms on the 1M-token keys.)
template <bool LOW>
__global__ __launch_bounds__(kThreads) void nuq_hist_kernel(NuqKeysArgs a) {
  constexpr int NB = LOW ? 128 : 256;
  constexpr int CH = LOW ? kHeadDim : kHeadDim / 2;       // channels per workgroup
  constexpr int LPT = CH / 2;                             // lanes per token
  constexpr int RW = NB / 2 + 1;                          // words per channel row
  constexpr int TW = kThreads / LPT;                      // token rows of a pass
  __shared__ uint32_t h[CH][RW];
  __shared__ uint32_t lcnt[LOW ? kHeadDim : 1];
  __shared__ float rmin[LOW ? TW : 1][LOW ? kHeadDim : 1], rmax[LOW ? TW : 1][LOW ? kHeadDim : 1];
  __shared__ uint32_t rab[LOW ? TW : 1][LOW ? kHeadDim : 1];
  constexpr int PARTS = kHeadDim / CH;
  const int64_t job = blockIdx.x / PARTS;
  const int c0 = (int)(blockIdx.x % PARTS) * CH;          // first channel of this group
  const int64_t bh = job / a.nchunks;
  const int chunk = (int)(job % a.nchunks);
  const int tid = threadIdx.x;
  for (int i = tid; i < CH * RW; i += kThreads) (&h[0][0])[i] = 0;
  if (LOW && tid < kHeadDim) lcnt[tid] = 0;
  const int cp = tid % LPT;                               // channels c0 + 2cp, c0 + 2cp + 1
  // low pass: magnitudes below lo are dense, from hi on outliers, in between the high
  // bin; without a high bin (no outliers, or all) lo = hi = T.  A lane tests its two
  // channels at once on 16-bit halves: lo - 1 - m and hi - 1 - m lie in [-2^15, 2^15)
  // and are negative exactly where m >= lo (not dense) and m >= hi (above).
  s16x2 lom1 = {0, 0}, him1 = {0, 0};
  if (LOW) {
    auto bounds = [&](int ch, int& lo, int& hi) {
      const int32_t* th = a.thr + (bh * kHeadDim + ch) * 4;
      const int hb = th[2];
      if (hb >= 0) {
        lo = hb << 7;
        hi = (hb + 1) << 7;
      } else {
        lo = hi = th[0] < 0 ? 0 : 0x8000;
      }
    };
    int lo0, hi0, lo1, hi1;
    bounds(c0 + 2 * cp, lo0, hi0);
    bounds(c0 + 2 * cp + 1, lo1, hi1);
    lom1 = s16x2{(short)(lo0 - 1), (short)(lo1 - 1)};
    him1 = s16x2{(short)(hi0 - 1), (short)(hi1 - 1)};
  }
  uint32_t amin = 0x7C007C00u, amax = 0xFC00FC00u;        // fp16 pairs: dense min / max
  s16x2 nabove = {0, 0};                                  // minus the counts above
  __syncthreads();
  const int64_t t0 = (int64_t)chunk * kNuqChunk;
  const int64_t t1 = min((int64_t)a.n_tokens, t0 + kNuqChunk);
  // this lane's lists: channels 2cp and 2cp + 1
  uint32_t* list0 = LOW ? a.lists + ((bh * a.nchunks + chunk) * kHeadDim + 2 * cp) * kNuqListCap
                        : nullptr;
  // x: the entry's fp16 bits in the high half, m: its magnitude
  auto in_bin = [&](int k, uint32_t x, uint32_t m, int64_t t) {
    atomicAdd(&h[2 * cp + k][(m & 127u) >> 1], m & 1u ? 0x10000u : 1u);
    const uint32_t slot = atomicAdd(&lcnt[2 * cp + k], 1u);
    if (slot < (uint32_t)kNuqListCap)
      list0[k * kNuqListCap + slot] = x | (uint32_t)(t - t0);
  };
  // low pass, every word: dense min / max and the count above; returns the word's
  // high-bin mask (0xFFFF in each half that holds an entry of the high bin)
  auto classify = [&](uint32_t w) -> uint32_t {
    const uint32_t m = w & 0x7FFF7FFFu;
    const s16x2 ms = __builtin_bit_cast(s16x2, m);
    const uint32_t nd = __builtin_bit_cast(uint32_t, (s16x2)((lom1 - ms) >> 15));
    const s16x2 abm = (him1 - ms) >> 15;
    nabove += abm;
    amax = pk_max_f16(amax, bitsel(nd, 0xFC00FC00u, w));
    amin = pk_min_f16(amin, bitsel(nd, 0x7C007C00u, w));
    return nd & ~__builtin_bit_cast(uint32_t, abm);
  };
  auto count = [&](uint32_t w, int64_t t) {
    if (!LOW) {
      const uint32_t m0 = w & 0x7FFFu, m1 = (w >> 16) & 0x7FFFu;
      atomicAdd(&h[2 * cp][(m0 >> 7) >> 1], (m0 >> 7) & 1u ? 0x10000u : 1u);
      atomicAdd(&h[2 * cp + 1][(m1 >> 7) >> 1], (m1 >> 7) & 1u ? 0x10000u : 1u);
    } else {
      const uint32_t mid = classify(w);
      if (mid) {
        if (mid & 0xFFFFu) in_bin(0, w << 16, w & 0x7FFFu, t);
        if (mid >> 16) in_bin(1, w & 0xFFFF0000u, (w >> 16) & 0x7FFFu, t);
      }
    }
  };
  constexpr int U = 16;                                   // tokens in flight per lane
  int64_t t = t0 + tid / LPT;
  for (; t + (int64_t)(U - 1) * TW < t1; t += (int64_t)U * TW) {
    const uint16_t* p0 = key_row(a, bh, t) + c0 + 2 * cp;
    uint32_t w[U];
#pragma unroll
    for (int u = 0; u < U; ++u)
      w[u] = *reinterpret_cast<const uint32_t*>(p0 + (int64_t)u * TW * a.st);
    if (!LOW) {
#pragma unroll
      for (int u = 0; u < U; ++u) count(w[u], t + u * TW);
    } else {
      // A wave holds a high-bin entry in about half of its words, so a branch per word
      // would run on half of them.  Instead the words' high-bin halves are marked (bit
      // 2u + k: half k of word u) and taken afterwards one per round, each word requested
      // again (it has just been read: the request is served from the cache).
      uint32_t midm = 0u;
#pragma unroll
      for (int u = 0; u < U; ++u) midm |= ((classify(w[u]) >> 15) & 3u) << (2 * u);
      while (midm) {
        const int j = __builtin_ctz(midm);
        midm &= midm - 1u;
        const int u = j >> 1, k = j & 1;
        const uint32_t x = *reinterpret_cast<const uint32_t*>(p0 + (int64_t)u * TW * a.st);
        const uint32_t xh = k ? x & 0xFFFF0000u : x << 16;
        in_bin(k, xh, (xh >> 16) & 0x7FFFu, t + u * TW);
      }
    }
  }
  for (; t < t1; t += TW)
    count(*reinterpret_cast<const uint32_t*>(key_row(a, bh, t) + c0 + 2 * cp), t);
  if (LOW) {
    const int r = tid / LPT;
    rmin[r][2 * cp] = f16_bits_to_f32((uint16_t)amin);
    rmin[r][2 * cp + 1] = f16_bits_to_f32((uint16_t)(amin >> 16));
    rmax[r][2 * cp] = f16_bits_to_f32((uint16_t)amax);
    rmax[r][2 * cp + 1] = f16_bits_to_f32((uint16_t)(amax >> 16));
    rab[r][2 * cp] = (uint32_t)(uint16_t)(-nabove[0]);
    rab[r][2 * cp + 1] = (uint32_t)(uint16_t)(-nabove[1]);
  }
  __syncthreads();
  if (LOW && tid < kHeadDim) {
    float mn = __builtin_inff(), mx = -__builtin_inff();
    uint32_t ab = 0u;
#pragma unroll
    for (int r = 0; r < TW; ++r) {
      mn = fminf(mn, rmin[r][tid]);
      mx = fmaxf(mx, rmax[r][tid]);
      ab += rab[r][tid];
    }
    uint32_t* cs = a.chunk_stats + ((bh * a.nchunks + chunk) * kHeadDim + tid) * 8;
    cs[3] = __builtin_bit_cast(uint32_t, mn);
    cs[4] = __builtin_bit_cast(uint32_t, mx);
    cs[5] = ab;
    cs[7] = lcnt[tid];
  }
  uint32_t* g = LOW ? a.hist_lo : a.hist_hi;
  for (int i = tid; i < CH * NB / 2; i += kThreads) {
    const int d = i / (NB / 2), b2 = i % (NB / 2);
    const uint32_t v = h[d][b2];
    if (v == 0) continue;
    uint32_t* row = g + (bh * kHeadDim + c0 + d) * NB;
    if (v & 0xFFFFu) atomicAdd(&row[2 * b2], v & 0xFFFFu);
    if (v >> 16) atomicAdd(&row[2 * b2 + 1], v >> 16);
  }
}

// ---- 2/3: thresholds.  thr[(bh*D + d)*4 + {0: T, 1: need, 2: high bin, 3: count above}]
// T = -1: every element is an outlier; T = 0x8000: none is.
__global__ void nuq_select_kernel(NuqKeysArgs a, int pass) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (int64_t)a.bh_count * kHeadDim) return;
  int32_t* th = a.thr + i * 4;
  const int64_t k = a.k_out;
  if (pass == 0) {
    th[2] = -1;
    th[3] = 0;
    if (k <= 0) { th[0] = 0x8000; th[1] = 0; return; }
    if (k >= a.n_tokens) { th[0] = -1; th[1] = 0; return; }
    const uint32_t* hh = a.hist_hi + i * 256;
    int64_t cum = 0;
    for (int b = 255; b >= 0; --b) {
      const int64_t c = hh[b];
      if (cum + c >= k) { th[2] = b; th[3] = (int32_t)cum; break; }
      cum += c;
    }
  } else {
    if (th[2] < 0) return;
    const uint32_t* hl = a.hist_lo + i * 128;
    int64_t cum = th[3];
    for (int b = 127; b >= 0; --b) {
      const int64_t c = hl[b];
      if (cum + c >= k) {
        th[0] = (th[2] << 7) | b;
        th[1] = (int32_t)(k - cum);
        break;
      }
      cum += c;
    }
  }
}

// A 32-token block of keys, staged in LDS: this thread's two 16-byte pieces (fetched into
// registers a block ahead of their store).
struct KeyPieces {
  uint4 u0, u1;
};
__device__ __forceinline__ KeyPieces fetch_key_tile(const NuqKeysArgs& a, int64_t bh,
                                                    int64_t t0) {
  const int t = threadIdx.x >> 3, c = (threadIdx.x & 7) * 16;
  const uint4* p = reinterpret_cast<const uint4*>(key_row(a, bh, t0 + t) + c);
  return KeyPieces{p[0], p[1]};
}
__device__ __forceinline__ void store_key_tile(uint16_t (*tile)[kHeadDim], const KeyPieces& k) {
  const int t = threadIdx.x >> 3, c = (threadIdx.x & 7) * 16;
  uint4* d = reinterpret_cast<uint4*>(&tile[t][c]);
  d[0] = k.u0;
  d[1] = k.u1;
}

// ---- 4: per chunk: ties, last positive / negative tie, dense min / max ----------------
// From the low-bin pass's gathering when every channel's high-bin entries of the chunk
// fit its list: the entries below T add to the dense min / max, those above to the count
// above T, and the ties are ranked in token order by their token offsets.  Otherwise the
// chunk is read again: two threads per channel (tokens 0..15 and 16..31 of each 32-token
// tile); a chunk's ties are numbered in token order, the second half's after the first
// half's of the same tile.  Tiles are double-buffered in LDS and each is requested into
// registers while the one before it is read.
__global__ __launch_bounds__(kThreads) void nuq_chunk_stats_kernel(NuqKeysArgs a) {
  __shared__ __align__(16) uint16_t tiles[2][kGroup][kHeadDim];
  const int64_t bh = blockIdx.x / a.nchunks;
  const int chunk = blockIdx.x % a.nchunks;
  const int tid = threadIdx.x;
  const int ch = tid >> 1, half = tid & 1;
  const int T = a.thr[(bh * kHeadDim + ch) * 4];
  uint32_t* cs = a.chunk_stats + ((bh * a.nchunks + chunk) * kHeadDim + ch) * 8;
  const uint32_t n_list = cs[7];
  if (!__syncthreads_or(n_list > (uint32_t)kNuqListCap)) {
    // every listed entry lies in T's high bin (none without one); this thread takes
    // entries 16 half .. 16 half + 15, all requested at once
    const uint4* lp = reinterpret_cast<const uint4*>(
        a.lists + ((bh * a.nchunks + chunk) * kHeadDim + ch) * kNuqListCap + 16 * half);
    uint32_t ent[16];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint4 u = lp[q];
      ent[4 * q] = u.x; ent[4 * q + 1] = u.y; ent[4 * q + 2] = u.z; ent[4 * q + 3] = u.w;
    }
    const int nmine = min(max((int)n_list - 16 * half, 0), 16);
    const uint32_t tbits = (uint32_t)T;                   // T's magnitude bits
    uint32_t run = 0u, above = 0u;
    int32_t pos_tok = -1, neg_tok = -1;
    float dmin = __builtin_inff(), dmax = -__builtin_inff();
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      if (i < nmine) {
        const uint32_t x = ent[i] >> 16, mag = x & 0x7FFFu;
        const int tok = (int)(ent[i] & 2047u);
        if (mag < tbits) {
          const float v = f16_bits_to_f32((uint16_t)x);
          dmin = fminf(dmin, v);
          dmax = fmaxf(dmax, v);
        } else if (mag > tbits) {
          above += 1u;
        } else {
          run += 1u;
          if (x >> 15) neg_tok = max(neg_tok, tok);
          else pos_tok = max(pos_tok, tok);
        }
      }
    }
    pos_tok = max(pos_tok, __shfl_xor(pos_tok, 1));
    neg_tok = max(neg_tok, __shfl_xor(neg_tok, 1));
    // rank of the last positive (negative) tie: the ties at earlier tokens
    uint32_t rp = 0u, rn = 0u;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      if (i < nmine && ((ent[i] >> 16) & 0x7FFFu) == tbits) {
        const int tok = (int)(ent[i] & 2047u);
        rp += tok < pos_tok ? 1u : 0u;
        rn += tok < neg_tok ? 1u : 0u;
      }
    }
    run += __shfl_xor(run, 1);
    above += __shfl_xor(above, 1);
    rp += __shfl_xor(rp, 1);
    rn += __shfl_xor(rn, 1);
    dmin = fminf(dmin, __shfl_xor(dmin, 1));
    dmax = fmaxf(dmax, __shfl_xor(dmax, 1));
    if (half == 0) {
      cs[0] = run;
      cs[1] = pos_tok >= 0 ? rp : 0xFFFFFFFFu;
      cs[2] = neg_tok >= 0 ? rn : 0xFFFFFFFFu;
      cs[3] = __builtin_bit_cast(uint32_t, fminf(__builtin_bit_cast(float, cs[3]), dmin));
      cs[4] = __builtin_bit_cast(uint32_t, fmaxf(__builtin_bit_cast(float, cs[4]), dmax));
      cs[5] += above;
    }
    return;
  }
  uint32_t run = 0, above = 0;              // ties so far in the chunk; values above T
  int32_t last_pos = -1, last_neg = -1;
  float dmin = __builtin_inff(), dmax = -__builtin_inff();
  const int64_t t0 = (int64_t)chunk * kNuqChunk;
  const int64_t t1 = min((int64_t)a.n_tokens, t0 + kNuqChunk);
  const int lt = tid >> 3, lc = (tid & 7) * 16;           // loader: token row, 16 channels
  uint4 u0 = make_uint4(0u, 0u, 0u, 0u), u1 = u0;
  if (t0 < t1) {
    const uint4* p = reinterpret_cast<const uint4*>(key_row(a, bh, t0 + lt) + lc);
    u0 = p[0];
    u1 = p[1];
  }
  for (int64_t tb = t0; tb < t1; tb += kGroup) {
    const int buf = (int)(((tb - t0) / kGroup) & 1);
    uint4* d = reinterpret_cast<uint4*>(&tiles[buf][lt][lc]);
    d[0] = u0;
    d[1] = u1;
    if (tb + kGroup < t1) {
      const uint4* p = reinterpret_cast<const uint4*>(key_row(a, bh, tb + kGroup + lt) + lc);
      u0 = p[0];
      u1 = p[1];
    }
    __syncthreads();
    uint32_t tiebits = 0u, posbits = 0u;
#pragma unroll
    for (int jj = 0; jj < 16; ++jj) {
      const uint32_t x = tiles[buf][16 * half + jj][ch];
      const int mag = (int)(x & 0x7FFFu);
      const float v = f16_bits_to_f32((uint16_t)x);
      const bool dense = mag < T;
      dmin = dense ? fminf(dmin, v) : dmin;
      dmax = dense ? fmaxf(dmax, v) : dmax;
      above += mag > T ? 1u : 0u;
      const uint32_t eq = mag == T ? 1u : 0u;
      tiebits |= eq << jj;
      posbits |= (eq & ((x >> 15) ^ 1u)) << jj;
    }
    const uint32_t my = (uint32_t)__builtin_popcount(tiebits);
    const uint32_t other = __shfl_xor(my, 1);
    if (tiebits) {
      // chunk-level number of this half's first tie, then of its last positive / negative
      const uint32_t base = run + (half ? other : 0u);
      const uint32_t negbits = tiebits & ~posbits;
      if (posbits) {
        const int j = 31 - __builtin_clz(posbits);
        last_pos = (int32_t)(base + __builtin_popcount(tiebits & ((2u << j) - 1u)) - 1u);
      }
      if (negbits) {
        const int j = 31 - __builtin_clz(negbits);
        last_neg = (int32_t)(base + __builtin_popcount(tiebits & ((2u << j) - 1u)) - 1u);
      }
    }
    run += my + other;
  }
  dmin = fminf(dmin, __shfl_xor(dmin, 1));
  dmax = fmaxf(dmax, __shfl_xor(dmax, 1));
  above += __shfl_xor(above, 1);
  last_pos = max(last_pos, __shfl_xor(last_pos, 1));
  last_neg = max(last_neg, __shfl_xor(last_neg, 1));
  if (half == 0) {
    cs[0] = run;
    cs[1] = (uint32_t)last_pos;
    cs[2] = (uint32_t)last_neg;
    cs[3] = __builtin_bit_cast(uint32_t, dmin);
    cs[4] = __builtin_bit_cast(uint32_t, dmax);
    cs[5] = above;
  }
}

// ---- 5: per channel: tie prefix of each chunk, dense min / max, (scale, min) ----------
// One wave per channel: lane l takes chunks l, l + 64, ...; the tie counts are scanned
// across the wave, the last-tie ranks and dense min / max reduced across it.
__global__ __launch_bounds__(kThreads) void nuq_finalize_kernel(NuqKeysArgs a) {
  const int lane = threadIdx.x & 63;
  const int64_t i = (int64_t)blockIdx.x * (kThreads / kWave) + (threadIdx.x >> 6);
  if (i >= (int64_t)a.bh_count * kHeadDim) return;     // uniform over the wave
  const int64_t bh = i / kHeadDim;
  const int d = (int)(i % kHeadDim);
  const int T = a.thr[i * 4];
  const int64_t need = a.thr[i * 4 + 1];
  int64_t base = 0, last_pos = -1, last_neg = -1;
  float dmin = __builtin_inff(), dmax = -__builtin_inff();
  for (int c0 = 0; c0 < a.nchunks; c0 += kWave) {
    const int c = c0 + lane;
    uint32_t* cs = a.chunk_stats + ((bh * a.nchunks + c) * kHeadDim + d) * 8;
    uint32_t ties = 0u, above = 0u;
    int32_t lp = -1, ln = -1;
    if (c < a.nchunks) {
      ties = cs[0];
      lp = (int32_t)cs[1];
      ln = (int32_t)cs[2];
      dmin = fminf(dmin, __builtin_bit_cast(float, cs[3]));
      dmax = fmaxf(dmax, __builtin_bit_cast(float, cs[4]));
      above = cs[5];
    }
    uint32_t incl = ties;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
      const uint32_t x = __shfl_up(incl, o);
      if (lane >= o) incl += x;
    }
    const int64_t prefix = base + (int64_t)(incl - ties);     // ties of the earlier chunks
    if (c < a.nchunks) {
      a.tie_prefix[(bh * a.nchunks + c) * kHeadDim + d] = (uint32_t)prefix;
      if (a.rowptr != nullptr) {
        // this channel's outliers in chunk c: the magnitudes above T and the ties ranked
        // below need (ranks prefix .. prefix + ties - 1 fall in this chunk)
        const int64_t taken = min(max(need - prefix, (int64_t)0), (int64_t)ties);
        cs[6] = above + (uint32_t)taken;
      }
      if (lp >= 0) last_pos = max(last_pos, prefix + lp);
      if (ln >= 0) last_neg = max(last_neg, prefix + ln);
    }
    base += __shfl(incl, kWave - 1);
  }
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    last_pos = max(last_pos, (int64_t)__shfl_xor((long long)last_pos, o));
    last_neg = max(last_neg, (int64_t)__shfl_xor((long long)last_neg, o));
    dmin = fminf(dmin, __shfl_xor(dmin, o));
    dmax = fmaxf(dmax, __shfl_xor(dmax, o));
  }
  if (lane != 0) return;
  if (T >= 0 && T < 0x8000) {          // ties ranked need.. are dense
    const float tv = f16_bits_to_f32((uint16_t)T);
    if (last_pos >= need) { dmin = fminf(dmin, tv); dmax = fmaxf(dmax, tv); }
    if (last_neg >= need) { dmin = fminf(dmin, -tv); dmax = fmaxf(dmax, -tv); }
  }
  if (!(dmin <= dmax)) { dmin = 0.0f; dmax = 0.0f; }     // no dense entry
  uint32_t meta;
  float mn, inv;
  params_nuq(dmin, dmax, a.bits, &meta, &mn, &inv);
  a.k_meta[bh * kHeadDim + d] = meta;
  a.norm[i * 2] = mn;
  a.norm[i * 2 + 1] = inv;
}


// The B code words of a channel's 32-token block from its codes one per byte: this lane
// holds tokens 16 * half + 4mm + k in byte k of cb[mm], its partner lane (lane ^ 1) the
// other half (the layout of nuq_code_fields).  Both lanes of the pair must call it.
template <int B>
__device__ __forceinline__ void store_code_words(uint32_t* kw, const uint32_t (&cb)[4],
                                                 int half) {
  if constexpr (B == 4) {
    // word 2 half + i holds tokens 8i..8i+7 of the half, token 4mm + k at 8k + 4(mm % 2)
    kw[2 * half] = cb[0] | (cb[1] << 4);
    kw[2 * half + 1] = cb[2] | (cb[3] << 4);
  } else if constexpr (B == 2) {
    kw[half] = cb[0] | (cb[1] << 2) | (cb[2] << 4) | (cb[3] << 6);
  } else {
    // half 0: m = mm, words 0 and 1 (m = 0..3).  Half 1: m = 4 + mm, word 2 (m = 4, 5) and
    // the m = 6, 7 fields split over words 0 / 1 (low bits at 8k + 6) and word 2 (high bit
    // at 8k + m).  The halves' fields are disjoint: OR them.
    const uint32_t p01 = cb[0] | (cb[1] << 3), p23 = cb[2] | (cb[3] << 3);
    const uint32_t h6 = ((cb[2] >> 2) & 0x01010101u) << 6;
    const uint32_t h7 = ((cb[3] >> 2) & 0x01010101u) << 7;
    const uint32_t w0 = half ? (cb[2] & 0x03030303u) << 6 : p01;
    const uint32_t w1 = half ? (cb[3] & 0x03030303u) << 6 : p23;
    const uint32_t w2 = half ? p01 | h6 | h7 : 0u;
    const uint32_t x0 = w0 | __shfl_xor(w0, 1);
    const uint32_t x1 = w1 | __shfl_xor(w1, 1);
    const uint32_t x2 = w2 | __shfl_xor(w2, 1);
    if (half == 0) {
      kw[0] = x0;
      kw[1] = x1;
    } else {
      kw[2] = x2;
    }
  }
}

// ---- 7: codes and CSR rows ---------------------------------------------------------
// Four waves per SIMD (at most 128 registers, cell reads in groups of eight): 3.22 ms on
// the 1M-token keys against 3.68 ms at the three the compiler picks by itself with groups
// of sixteen.  Compiled apart with and without Q-Norm (QN): without it the exact moment
// sums and the per-channel code counts are not kept across the tile loop (105 registers
// for nuq3 against 128).
template <int B, bool QN>
__global__ __launch_bounds__(kThreads, 4) void nuq_quant_keys_kernel(NuqKeysArgs a) {
  // two tiles and outlier masks: the CSR rows of one tile are written while the next is
  // loaded and coded
  __shared__ __align__(16) uint16_t tiles[2][kGroup][kHeadDim];
  __shared__ uint32_t oms[2][kGroup][4];
  __shared__ uint32_t qh[kHeadDim][16];     // Q-Norm: dense code counts per channel
  __shared__ CodeCells<B> cells;
  const int64_t bh = blockIdx.x / a.nchunks;
  const int chunk = blockIdx.x % a.nchunks;
  const int tid = threadIdx.x;
  const Mids<B> md = load_mids<B>(a.lut);
  const bool by_cells = build_code_cells<B>(cells, md, tid);
  ExactSums qs;
  exact_zero(qs);
  if constexpr (QN)
    for (int i = tid; i < kHeadDim * 16; i += kThreads) (&qh[0][0])[i] = 0u;
  // per-channel state of this lane's channel (two lanes per channel)
  int cT, cneed;
  uint32_t crank;
  float cmn, cinv2;
  {
    const int ch = tid >> 1;
    const int64_t i = bh * kHeadDim + ch;
    cT = a.thr[i * 4];
    cneed = a.thr[i * 4 + 1];
    crank = a.tie_prefix[(bh * a.nchunks + chunk) * kHeadDim + ch];
    cmn = a.norm[i * 2];
    cinv2 = 2.0f * a.norm[i * 2 + 1];
  }
  const int64_t t0 = (int64_t)chunk * kNuqChunk;
  const int64_t t1 = min((int64_t)a.n_tokens, t0 + kNuqChunk);
  // CSR: this chunk's first entry (the scan of the per-chunk counts), kept by every wave
  int64_t run = a.rowptr != nullptr ? (int64_t)a.chunk_off[bh * a.nchunks + chunk] : 0;
  auto tile_loop = [&](auto cells_tag) {
    constexpr bool CELLS = decltype(cells_tag)::value;
    KeyPieces kp = t0 < t1 ? fetch_key_tile(a, bh, t0) : KeyPieces{};
    for (int64_t tb = t0; tb < t1; tb += kGroup) {
      const int buf = (int)(((tb - t0) / kGroup) & 1);
      uint16_t (*tile)[kHeadDim] = tiles[buf];
      uint32_t (*om)[4] = oms[buf];
      store_key_tile(tile, kp);
      if (tb + kGroup < t1) kp = fetch_key_tile(a, bh, tb + kGroup);
      if (tid < kGroup * 4) om[tid >> 2][tid & 3] = 0;
      __syncthreads();
      {
        // Two lanes of one wave per channel, tokens 0..15 and 16..31.  The outlier rank of
        // ties at the threshold runs in token order: the second half's continues from the
        // first half's count.  Codes are gathered one per byte (token 4mm + k of the half
        // in byte k of cb[mm]) and turned into the channel's B code words at the end.
        const int ch = tid >> 1, half = tid & 1;
        uint32_t xs[16];
        float xn2[16];
        uint32_t outbits = 0u, my_ties = 0u;
#pragma unroll
        for (int jj = 0; jj < 16; ++jj) {
          const uint32_t x = tile[16 * half + jj][ch];
          xs[jj] = x;
          const int mag = (int)(x & 0x7FFFu);
          const bool out = mag > cT;                 // ties at cT: below
          my_ties += mag == cT ? 1u : 0u;
          outbits |= (uint32_t)out << jj;
          // an outlier's position stores code 0 (its exact value replaces the dequantized
          // one), and so does every position of a channel without a dense range
          xn2[jj] = out || cinv2 == 0.0f ? -__builtin_inff()
                                         : (f16_bits_to_f32((uint16_t)x) - cmn) * cinv2;
        }
        const uint32_t other_ties = __shfl_xor(my_ties, 1);
        uint32_t cb[4] = {0u, 0u, 0u, 0u};
        nuq_code16<B, B == 4 ? 4 : 8, CELLS>(cb, [&](int jj) { return xn2[jj]; }, cells, md);
        if (__any(my_ties != 0u)) {
          // ties at the threshold, in token order: the first cneed of the channel's ties
          // (counted from crank, the ties of the earlier chunks) are outliers
          uint32_t r = crank + (half ? other_ties : 0u);
          uint32_t tbits = 0u;
#pragma unroll
          for (int jj = 0; jj < 16; ++jj) tbits |= (uint32_t)((int)(xs[jj] & 0x7FFFu) == cT) << jj;
          while (tbits) {
            const int jj = __builtin_ctz(tbits);
            tbits &= tbits - 1u;
            if (r < (uint32_t)cneed) {
              outbits |= 1u << jj;
              cb[jj >> 2] &= ~(0xFFu << (8 * (jj & 3)));
            }
            ++r;
          }
        }
        crank += my_ties + other_ties;
        for (uint32_t ob = outbits; ob != 0u; ob &= ob - 1u) {
          const int jj = __builtin_ctz(ob);
          atomicOr(&om[16 * half + jj][ch >> 5], 1u << (ch & 31));
        }
        if constexpr (QN) {
#pragma unroll
          for (int jj = 0; jj < 16; ++jj) {
            if (!((outbits >> jj) & 1u)) {
              exact_add(qs, xs[jj]);
              atomicAdd(&qh[ch][(cb[jj >> 2] >> (8 * (jj & 3))) & 0xFFu], 1u);
            }
          }
        }
        KVQ_CHECK(tb / kGroup < a.cap_blocks, kDbgWrite);
        uint32_t* kw = a.k_codes + (bh * a.cap_blocks + tb / kGroup) * (kHeadDim * B) + ch * B;
        store_code_words<B>(kw, cb, half);
      }
      __syncthreads();
      if (a.rowptr != nullptr) {
        // each token's first entry: every wave scans the 32 row lengths itself (lane j: token
        // j), so no barrier separates the scan from the writes; then thread (token j,
        // sixteenth e) writes the entries of channels 16e..16e+15 (ascending, the exact fp16
        // value from the tile) and e = 0 the row pointer.  No barrier after: the next tile
        // goes to the other buffers.
        const int l = tid & (kWave - 1);
        const uint32_t cnt = l < kGroup ? (uint32_t)(__popc(om[l][0]) + __popc(om[l][1]) +
                                                     __popc(om[l][2]) + __popc(om[l][3]))
                                        : 0u;
        uint32_t incl = cnt;
#pragma unroll
        for (int o = 1; o < kGroup; o <<= 1) {
          const uint32_t x = __shfl_up(incl, o);
          if (l >= o) incl += x;
        }
        const int j = tid >> 3, e = tid & 7, w = e >> 1;
        const uint32_t word = om[j][w];
        const uint32_t bits0 = (e & 1) ? word >> 16 : word & 0xFFFFu;
        int64_t pos = run + (int64_t)__shfl(incl - cnt, j);
        for (int i = 0; i < w; ++i) pos += __popc(om[j][i]);
        if (e & 1) pos += __popc(word & 0xFFFFu);
        if (e == 0) a.rowptr[bh * (a.cap_tokens + 1) + tb + j] = (int32_t)pos;
        uint32_t* ent = a.ent + bh * a.csr_capacity;
        for (uint32_t bits = bits0; bits != 0u; bits &= bits - 1u) {
          const int d = 16 * e + __builtin_ctz(bits);
          KVQ_CHECK(pos < a.csr_capacity, kDbgCsr);
          if (pos < a.csr_capacity)
            ent[pos] = (uint32_t)d | ((uint32_t)j << 8) | ((uint32_t)tile[j][d] << 16);
          ++pos;
        }
        run += __shfl(incl, kGroup - 1);
      }
    }
  };
  if (by_cells) tile_loop(CellsTag<true>{});
  else tile_loop(CellsTag<false>{});
  if constexpr (QN) {
    // the two lanes of a channel combine their sums; the block's atomics on qh are done
    exact_merge_xor(qs, 1);
    __syncthreads();
    if ((tid & 1) == 0) {
      const int ch = tid >> 1;
      const int64_t q = (bh * a.nchunks + chunk) * kHeadDim + ch;
      a.qn_sum[q * 4] = qs.x_lo;
      a.qn_sum[q * 4 + 1] = (uint64_t)qs.x_hi;
      a.qn_sum[q * 4 + 2] = qs.q_lo;
      a.qn_sum[q * 4 + 3] = qs.q_hi;
#pragma unroll
      for (int c = 0; c < 16; ++c) a.qn_hist[q * 16 + c] = qh[ch][c];
    }
  }
}

// Q-Norm of the key channels: the chunks' sums and counts combined in chunk order.
__global__ void nuq_qnorm_keys_kernel(NuqKeysArgs a) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (int64_t)a.bh_count * kHeadDim) return;
  const int64_t bh = i / kHeadDim;
  const int d = (int)(i % kHeadDim);
  ExactSums es;
  exact_zero(es);
  uint32_t hist[16];
#pragma unroll
  for (int c = 0; c < 16; ++c) hist[c] = 0u;
  for (int ch = 0; ch < a.nchunks; ++ch) {
    const int64_t q = (bh * a.nchunks + ch) * kHeadDim + d;
    exact_add_parts(es, a.qn_sum[q * 4], (int64_t)a.qn_sum[q * 4 + 1], a.qn_sum[q * 4 + 2],
                    a.qn_sum[q * 4 + 3]);
#pragma unroll
    for (int c = 0; c < 16; ++c) hist[c] += a.qn_hist[q * 16 + c];
  }
  uint32_t n = 0;
#pragma unroll
  for (int c = 0; c < 16; ++c) n += hist[c];
  double sx, sxx;
  exact_to_f64(es, &sx, &sxx);
  uint32_t* meta = a.k_meta + bh * kHeadDim + d;
  *meta = qnorm_meta(*meta, sx, sxx, hist, n, a.lut, a.bits);
}

// ---- 6: CSR chunk offsets -----------------------------------------------------------
// One workgroup of kHeadDim threads per (batch, head, chunk): the chunk's outlier count,
// summed over its channels.
__global__ __launch_bounds__(kHeadDim) void csr_chunk_count_kernel(NuqKeysArgs a) {
  __shared__ uint32_t part[kHeadDim / kWave];
  const int64_t q = blockIdx.x;                 // bh * nchunks + chunk
  uint32_t v = a.chunk_stats[(q * kHeadDim + threadIdx.x) * 8 + 6];
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = v;
  __syncthreads();
  if (threadIdx.x == 0) a.chunk_cnt[q] = part[0] + part[1];
}

// One workgroup per (batch, head): exclusive scan of the chunk counts.
__global__ __launch_bounds__(kThreads) void csr_scan_kernel(NuqKeysArgs a) {
  const int64_t bh = blockIdx.x;
  if (threadIdx.x != 0) return;
  uint32_t run = 0;
  for (int c = 0; c < a.nchunks; ++c) {
    const uint32_t v = a.chunk_cnt[bh * a.nchunks + c];
    a.chunk_off[bh * a.nchunks + c] = run;
    run += v;
  }
  a.rowptr[bh * (a.cap_tokens + 1) + a.n_tokens] = (int32_t)run;
}

// Outliers of one token's vector ("KVQuant" review, abstract item (iv): the largest
// magnitudes of each vector are kept exactly): the kv channels of largest fp16
// magnitude, ties to the lower channel.  Eight threads (consecutive lanes) hold 16
// channels each.  Up to six outliers are taken one at a time, largest magnitude first
// (lower channel first among equals).  Otherwise a binary search finds the threshold T,
// the largest magnitude with at least kv channels at or above it; channels above T are
// outliers, and so are the first kv - count(> T) channels equal to T (in channel
// order).  Returns this thread's flags (bit j: channel 16 * part + j).
__device__ __forceinline__ uint32_t count8(uint32_t x) {
#pragma unroll
  for (int o = 1; o < 8; o <<= 1) x += __shfl_xor(x, o);
  return x;
}

__device__ uint32_t value_outliers(const uint32_t (&xw)[8], int part, int kv) {
  uint32_t mag[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) mag[j] = (xw[j >> 1] >> (16 * (j & 1))) & 0x7FFFu;
  if (kv <= 6) {
    // Few outliers: take the largest remaining (magnitude, lower channel first) kv times.
    // The key (magnitude << 8 | 255 - channel) is unique per channel and at least 128.
    uint32_t flags = 0;
    for (int r = 0; r < kv; ++r) {
      uint32_t best = 0;
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const uint32_t key = (mag[j] << 8) | (uint32_t)(255 - (part * 16 + j));
        if (!((flags >> j) & 1u)) best = max(best, key);
      }
#pragma unroll
      for (int o = 1; o < 8; o <<= 1) best = max(best, (uint32_t)__shfl_xor(best, o));
      const int ch = 255 - (int)(best & 255u);
      if ((ch >> 4) == part) flags |= 1u << (ch & 15);
    }
    return flags;
  }
  uint32_t lo = 0, hi = 0x7FFF;
  for (int it = 0; it < 15; ++it) {                // hi - lo + 1 halves from 2^15 to 1
    const uint32_t mid = (lo + hi + 1) >> 1;
    uint32_t c = 0;
#pragma unroll
    for (int j = 0; j < 16; ++j) c += mag[j] >= mid ? 1u : 0u;
    if (count8(c) >= (uint32_t)kv) lo = mid;
    else hi = mid - 1;
  }
  uint32_t above = 0, ties = 0, tie_mask = 0, flags = 0;
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    if (mag[j] > lo) { above += 1; flags |= 1u << j; }
    if (mag[j] == lo) { ties += 1; tie_mask |= 1u << j; }
  }
  const uint32_t need = (uint32_t)kv - count8(above);
  uint32_t ties_before = ties;                      // ties in lower parts (exclusive scan)
#pragma unroll
  for (int o = 1; o < 8; o <<= 1) {
    const uint32_t x = __shfl_up(ties_before, o, 8);
    if (part >= o) ties_before += x;
  }
  ties_before -= ties;
  uint32_t m = tie_mask;
  for (uint32_t i = ties_before; m != 0u && i < need; ++i) {
    flags |= m & (0u - m);                          // lowest remaining tie
    m &= m - 1u;
  }
  return flags;
}

// ---- values: per token over all channels --------------------------------------------
// VOUT: the cache keeps per-token value outliers (an instance of its own, so that the
// search's registers do not lower the occupancy of the plain case).
// Values: per token over its D channels (with VOUT, dense-and-sparse: the token's kv
// largest magnitudes kept exactly).  A workgroup takes kValueTiles consecutive 32-token
// blocks of one head.  Per block, eight threads per token (16 channels each) gather the
// token's outliers, dense min / max and metadata and code their channels straight from
// registers, one code per byte into an LDS tile; then two threads per channel (16 tokens
// each) gather the channel's codes and write its code words.  The code tiles are
// double-buffered, so one barrier per block separates the two roles; everything else a
// token needs (its Q-Norm counts included) stays within the wave that holds it.
constexpr int kValueTiles = 16;

// Four waves per SIMD (at most 128 registers): measured 2.43 ms on the 1M-token values
// against 2.72 ms at the three the compiler picks by itself, and 3.91 ms at five (spills).
// Compiled apart with and without Q-Norm (QN): without it, and without value outliers,
// nuq3 takes 66 registers instead of 128 with spills.
template <int B, bool VOUT, bool QN>
__global__ __launch_bounds__(kThreads, 4) void nuq_quant_values_kernel(NuqValuesArgs a) {
  __shared__ __align__(16) uint8_t codes[2][kGroup][kHeadDim];   // per token, per channel
  __shared__ uint32_t qh[kGroup][16];       // Q-Norm: dense code counts per token
  __shared__ CodeCells<B> cells;
  const int groups = (a.n_blocks + kValueTiles - 1) / kValueTiles;
  const int64_t bh = blockIdx.x / groups;
  const int grp = (int)(blockIdx.x % groups);
  const int64_t b = bh / a.kv_heads, h = bh % a.kv_heads;
  const int tid = threadIdx.x;
  const Mids<B> md = load_mids<B>(a.lut);
  const bool by_cells = build_code_cells<B>(cells, md, tid);
  const int t = tid >> 3, part = tid & 7;   // token role
  const int ch = tid >> 1, half = tid & 1;  // channel role
  const int blk0 = grp * kValueTiles, blk1 = min(a.n_blocks, blk0 + kValueTiles);
  auto block_loop = [&](auto cells_tag) {
    constexpr bool CELLS = decltype(cells_tag)::value;
    for (int blk = blk0; blk < blk1; ++blk) {
      const int buf = (blk - blk0) & 1;
      const int64_t tok = a.tok0 + (int64_t)blk * kGroup + t;
      // ---- token role: this thread's 16 channels, straight from HBM into registers
      uint32_t xw[8];
      {
        const uint4* p = reinterpret_cast<const uint4*>(
            a.v + b * a.sb + h * a.sh + ((int64_t)blk * kGroup + t) * a.st + part * 16);
        const uint4 u0 = p[0], u1 = p[1];
        xw[0] = u0.x; xw[1] = u0.y; xw[2] = u0.z; xw[3] = u0.w;
        xw[4] = u1.x; xw[5] = u1.y; xw[6] = u1.z; xw[7] = u1.w;
      }
      const uint32_t outm = VOUT ? value_outliers(xw, part, a.kv) : 0u;
      float mn = __builtin_inff(), mx = -__builtin_inff();
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        if (!((outm >> j) & 1u)) {
          const float x = (j & 1) ? hi_f16(xw[j >> 1]) : lo_f16(xw[j >> 1]);
          mn = fminf(mn, x);
          mx = fmaxf(mx, x);
        }
      }
#pragma unroll
      for (int o = 1; o < 8; o <<= 1) {
        mn = fminf(mn, __shfl_xor(mn, o));
        mx = fmaxf(mx, __shfl_xor(mx, o));
      }
      if (mn > mx) mn = mx = 0.0f;            // every channel an outlier
      if (VOUT) {
        // this thread's outliers, channels ascending, after those of the lower parts
        const uint32_t mine = (uint32_t)__builtin_popcount(outm);
        uint32_t before = mine;
#pragma unroll
        for (int o = 1; o < 8; o <<= 1) {
          const uint32_t x = __shfl_up(before, o, 8);
          if (part >= o) before += x;
        }
        before -= mine;
        uint32_t* dst = a.v_out + (bh * a.cap_tokens + tok) * a.kv + before;
        uint32_t m = outm;
        for (int i = 0; m != 0u; ++i) {
          const int j = __builtin_ctz(m);
          m &= m - 1u;
          dst[i] = (uint32_t)(part * 16 + j) | (((xw[j >> 1] >> (16 * (j & 1))) & 0xFFFFu) << 16);
        }
      }
      uint32_t meta;
      float m0, inv;
      params_nuq(mn, mx, a.bits, &meta, &m0, &inv);
      // codes of the 16 channels (an outlier's position, and every position of a token
      // without a dense range, takes code 0), into the token's row of the code tile
      const float inv2 = 2.0f * inv;
      uint32_t cw[4] = {0u, 0u, 0u, 0u};
      nuq_code16<B, 16, CELLS>(
          cw,
          [&](int j) {
            const float x = (j & 1) ? hi_f16(xw[j >> 1]) : lo_f16(xw[j >> 1]);
            return ((outm >> j) & 1u) || inv2 == 0.0f ? -__builtin_inff() : (x - m0) * inv2;
          },
          cells, md);
      *reinterpret_cast<uint4*>(&codes[buf][t][part * 16]) = make_uint4(cw[0], cw[1], cw[2], cw[3]);
      if constexpr (!QN) {
        if (part == 0) a.v_meta[bh * a.cap_tokens + tok] = meta;
      } else {
        // Q-Norm: the token's dense sums and code counts (the token's eight threads share a
        // wave, whose LDS operations run in order), then its metadata
        ExactSums es;
        exact_zero(es);
#pragma unroll
        for (int j = 0; j < 16; ++j)
          if (!((outm >> j) & 1u)) exact_add(es, (xw[j >> 1] >> (16 * (j & 1))) & 0xFFFFu);
#pragma unroll
        for (int o = 1; o < 8; o <<= 1) exact_merge_xor(es, o);
        qh[t][2 * part] = qh[t][2 * part + 1] = 0u;
        __builtin_amdgcn_wave_barrier();
#pragma unroll
        for (int j = 0; j < 16; ++j)
          if (!((outm >> j) & 1u)) atomicAdd(&qh[t][(cw[j >> 2] >> (8 * (j & 3))) & 0xFFu], 1u);
        __builtin_amdgcn_wave_barrier();
        if (part == 0) {
          double sx, sxx;
          exact_to_f64(es, &sx, &sxx);
          uint32_t n = 0;
#pragma unroll
          for (int c = 0; c < 16; ++c) n += qh[t][c];
          a.v_meta[bh * a.cap_tokens + tok] = qnorm_meta(meta, sx, sxx, qh[t], n, a.lut, a.bits);
        }
        __builtin_amdgcn_wave_barrier();
      }
      __syncthreads();
      // ---- channel role: channel ch of tokens 16 half .. 16 half + 15, codes one per byte
      {
        uint32_t cb[4] = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int jj = 0; jj < 16; ++jj)
          cb[jj >> 2] |= (uint32_t)codes[buf][16 * half + jj][ch] << (8 * (jj & 3));
        KVQ_CHECK(a.tok0 / kGroup + blk < a.cap_blocks, kDbgWrite);
        uint32_t* kw = a.v_codes + (bh * a.cap_blocks + a.tok0 / kGroup + blk) * (kHeadDim * B) +
                       ch * B;
        store_code_words<B>(kw, cb, half);
      }
    }
  };
  if (by_cells) block_loop(CellsTag<true>{});
  else block_loop(CellsTag<false>{});
}

inline unsigned grid1(int64_t n) { return (unsigned)((n + kThreads - 1) / kThreads); }

}  // namespace

hipError_t launch_nuq_keys(const NuqKeysArgs& a, hipStream_t s) {
  const int64_t bhd = (int64_t)a.bh_count * kHeadDim;
  const unsigned jobs = (unsigned)((int64_t)a.bh_count * a.nchunks);
  fill_u32_kernel<<<dim3(1024), dim3(kThreads), 0, s>>>(a.hist_hi, bhd * 256, 0u);
  fill_u32_kernel<<<dim3(1024), dim3(kThreads), 0, s>>>(a.hist_lo, bhd * 128, 0u);
  nuq_hist_kernel<false><<<dim3(2 * jobs), dim3(kThreads), 0, s>>>(a);   // two channel halves
  nuq_select_kernel<<<dim3(grid1(bhd)), dim3(kThreads), 0, s>>>(a, 0);
  nuq_hist_kernel<true><<<dim3(jobs), dim3(kThreads), 0, s>>>(a);
  nuq_select_kernel<<<dim3(grid1(bhd)), dim3(kThreads), 0, s>>>(a, 1);
  nuq_chunk_stats_kernel<<<dim3(jobs), dim3(kThreads), 0, s>>>(a);
  nuq_finalize_kernel<<<dim3((unsigned)((bhd + 3) / 4)), dim3(kThreads), 0, s>>>(a);
  if (a.rowptr != nullptr) {
    csr_chunk_count_kernel<<<dim3(jobs), dim3(kHeadDim), 0, s>>>(a);
    csr_scan_kernel<<<dim3((unsigned)a.bh_count), dim3(kThreads), 0, s>>>(a);
  }
#define KVQ_QK(B_)                                                                   \
  (a.qnorm ? nuq_quant_keys_kernel<B_, true><<<dim3(jobs), dim3(kThreads), 0, s>>>(a)      \
           : nuq_quant_keys_kernel<B_, false><<<dim3(jobs), dim3(kThreads), 0, s>>>(a))
  if (a.bits == 2) KVQ_QK(2);
  else if (a.bits == 3) KVQ_QK(3);
  else KVQ_QK(4);
#undef KVQ_QK
  if (a.qnorm) nuq_qnorm_keys_kernel<<<dim3(grid1(bhd)), dim3(kThreads), 0, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_nuq_values(const NuqValuesArgs& a, hipStream_t s) {
  const int64_t jobs = (int64_t)a.bh_count * ((a.n_blocks + kValueTiles - 1) / kValueTiles);
  if (jobs == 0) return hipSuccess;
  const dim3 grid((unsigned)jobs), block(kThreads);
  const bool vout = a.kv > 0;
#define KVQ_QV(B_, VO_)                                                              \
  (a.qnorm ? nuq_quant_values_kernel<B_, VO_, true><<<grid, block, 0, s>>>(a)        \
           : nuq_quant_values_kernel<B_, VO_, false><<<grid, block, 0, s>>>(a))
  if (a.bits == 2 && vout) KVQ_QV(2, true);
  else if (a.bits == 2) KVQ_QV(2, false);
  else if (a.bits == 3 && vout) KVQ_QV(3, true);
  else if (a.bits == 3) KVQ_QV(3, false);
  else if (vout) KVQ_QV(4, true);
  else KVQ_QV(4, false);
#undef KVQ_QV
  return hipGetLastError();
}

uint32_t debug_take_quant_nuq() { return debug_take_local(); }

}  // namespace kvq
