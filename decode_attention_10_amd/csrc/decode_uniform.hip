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
// Work split: a workgroup of 4 or 8 waves handles one (batch, kv head) and a
// range of work units (split-K over the context, as in flash-decoding); a wave
// streams one 32-token block at a time (keys: a lane covers two tokens x 32
// channels; values: one 8-token x 8-channel tile), with the next block's loads in
// flight (the next two in 4-wave split plans).  Blocks are dealt to the waves in rounds
// and the fp16 window chunks go to the last waves, which take correspondingly fewer
// blocks.  Waves merge in LDS.
// With one split per (batch, kv head) the workgroup writes the output; otherwise it
// writes a (max, sum, output) partial and a second small launch merges the splits.
#include "decode_common.h"

namespace kvq {
namespace {

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
template <int KB, int VB, bool NT>
__device__ __forceinline__ void load_block(BlockRegs<KB, VB>& r, const HeadPtrs& hp, int blk,
                                           int lane) {
  constexpr int WK = kHeadDim * KB / 32;            // words per token row
  const int tp = lane >> 2, q = lane & 3;
  const uint32_t* kp = hp.kc + (uint32_t)blk * (kGroup * WK);
  const uint32_t ka_off = (uint32_t)(tp * WK + q * KB), kb_off = ka_off + 16 * WK;
  if constexpr (KB == 2) {
    const uint2 x = ld_cache2<NT>(kp + ka_off);
    const uint2 y = ld_cache2<NT>(kp + kb_off);
    r.ka[0] = x.x; r.ka[1] = x.y; r.kb[0] = y.x; r.kb[1] = y.y;
  } else {
    const uint4 x = ld_cache4<NT>(kp + ka_off);
    const uint4 y = ld_cache4<NT>(kp + kb_off);
    r.ka[0] = x.x; r.ka[1] = x.y; r.ka[2] = x.z; r.ka[3] = x.w;
    r.kb[0] = y.x; r.kb[1] = y.y; r.kb[2] = y.z; r.kb[3] = y.w;
  }
  const uint2 km = ld_cache2<NT>(hp.km + (uint32_t)blk * kHeadDim + (uint32_t)(2 * lane));
  r.km[0] = km.x; r.km[1] = km.y;
  const uint32_t* vp = hp.vc + (uint32_t)blk * (kHeadDim * VB) + (uint32_t)(lane * 2 * VB);
#pragma unroll
  for (int i = 0; i < VB / 2; ++i) {
    const uint4 u = ld_cache4<NT>(vp + 4 * i);
    r.vc[4 * i] = u.x; r.vc[4 * i + 1] = u.y; r.vc[4 * i + 2] = u.z; r.vc[4 * i + 3] = u.w;
  }
  const uint32_t* vm = hp.vm + (uint32_t)blk * (kGroup * 4);
  r.vm[0] = ld_cache<NT>(vm + (uint32_t)lane);
  r.vm[1] = ld_cache<NT>(vm + (uint32_t)lane + 64);
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

// Work units: packed block i is unit i (0 <= i < n_blocks); window chunk c (32 fp16
// tokens) is units [n_blocks + kWindowUnits*c, n_blocks + kWindowUnits*(c+1)), weighted
// by its larger byte count.  A split covers a contiguous unit range: the packed blocks
// in it and every window chunk whose first unit falls in it.
template <int KB, int VB, int GQ, int NW, bool NT>
__global__ __launch_bounds__(NW * kWave) void decode_uniform_kernel(DecodeArgs a) {
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
  init_wave_state<GQ>(st);

  const int nchunks = fp16_chunks(a);
  const int units = a.n_blocks + kWindowUnits * nchunks;
  const int s0 = (int)((int64_t)units * split / a.splits);
  const int s1 = (int)((int64_t)units * (split + 1) / a.splits);
  // Window chunks of the split go to the waves from the last one down, cyclically;
  // packed blocks are dealt in rounds so that every wave ends with about the same
  // work: in round k the waves with more than k blocks take the next consecutive
  // blocks (the workgroup streams one contiguous stretch of each cache array).
  const int bend = min(s1, a.n_blocks);
  const int nb = max(bend - s0, 0);
  const int c_first = max(s0 - a.n_blocks + kWindowUnits - 1, 0) / kWindowUnits;
  const int c_end = min(nchunks, max(s1 - a.n_blocks + kWindowUnits - 1, 0) / kWindowUnits);
  KVQ_CHECK(a.n_blocks <= a.cap_blocks && s1 <= units && c_end <= nchunks, kDbgSplit);
  const Deal deal = deal_blocks(nb, max(c_end - c_first, 0), NW);
  const int cnt = __builtin_amdgcn_readfirstlane(deal.count(wave));

  // ---- window chunks first (their loads are short), then the packed blocks
  for (int c = c_first; c < c_end; ++c)
    if (NW - 1 - ((c - c_first) % NW) == wave)
      process_window<GQ, VB>(a, bh, c, st, qh, reinterpret_cast<float(*)[kGroup]>(psL[wave]), lane);
  if (cnt > 0) {
    const int64_t seg = bh * a.cap_blocks;
    const HeadPtrs hp = {a.k_codes + seg * (kGroup * kHeadDim * KB / 32),
                         a.k_meta + seg * kHeadDim, a.v_codes + seg * (kHeadDim * VB),
                         a.v_meta + seg * (kGroup * 4)};
    // PF blocks in flight ahead of the one being processed: one with streaming loads (a
    // workgroup per head), two otherwise.  The prefetch index is clamped rather than
    // guarded so every iteration issues the same loads, and the loop is unrolled by PF + 1
    // with rotating register sets so no register copy has to wait for the loads just
    // issued.
    constexpr int PF = NT ? 1 : 2;
    constexpr int RS = PF + 1;
    const int last = cnt - 1;
    BlockRegs<KB, VB> r[RS];
#pragma unroll
    for (int i = 0; i < PF; ++i)
      load_block<KB, VB, NT>(r[i], hp, block_of(deal, s0, i, last, wave), lane);
    for (int k = 0; k < cnt; k += RS) {
#pragma unroll
      for (int d = 0; d < RS; ++d) {
        if (k + d >= cnt) break;
        load_block<KB, VB, NT>(r[(d + PF) % RS], hp, block_of(deal, s0, k + d + PF, last, wave),
                               lane);
        process_block<KB, VB, GQ>(r[d], st, qreg, qf, cscale, qsL[wave], psL[wave], lane);
      }
    }
  }

  // ---- finish the wave, then the workgroup merge
  finish_wave_state<GQ, VB>(st, wm[wave], wl[wave], wo[wave], lane);
  __syncthreads();
  merge_partials<GQ, NW>(a, wm, wl, wo, b, hq0, split);
}

// Combines the per-split (max, sum, output) partials of one (batch, query head) row.
// A separate launch: the kernel boundary makes every split's stores visible, which
// costs far less than device-scope fences in each workgroup of the main kernel.  Each
// thread owns one output channel and every 8th split; it issues the loads of a chunk of
// splits at once and folds them into a running (max, sum, output) (one memory round
// per chunk, so 64 splits take one round); the eight split classes are combined in LDS.
constexpr int kMergeParts = 8;
constexpr int kMergeThreads = kMergeParts * kHeadDim;
constexpr int kMergeChunk = 8;

__global__ __launch_bounds__(kMergeThreads) void merge_splits_kernel(const float* partials,
                                                                    float* out, int splits) {
  __shared__ float pm[kMergeParts], pl[kMergeParts];
  __shared__ float po[kMergeParts][kHeadDim];
  const int64_t row = blockIdx.x;
  const int d = threadIdx.x & (kHeadDim - 1), part = threadIdx.x >> 7;
  KVQ_CHECK(splits >= 1 && splits <= kMaxSplits, kDbgSplit);
  const float* P = partials + row * splits * kPartialStride;
  float M = kNegInf, L = 0.f, O = 0.f;
  for (int s0 = part; s0 < splits; s0 += kMergeParts * kMergeChunk) {
    float m[kMergeChunk], l[kMergeChunk], o[kMergeChunk];
#pragma unroll
    for (int c = 0; c < kMergeChunk; ++c) {
      const int sp = min(s0 + c * kMergeParts, splits - 1);   // clamped: loads stay uniform
      const float* p = P + (int64_t)sp * kPartialStride;
      m[c] = p[kHeadDim];
      l[c] = p[kHeadDim + 1];
      o[c] = p[d];
    }
    float cm = M;
#pragma unroll
    for (int c = 0; c < kMergeChunk; ++c)
      if (s0 + c * kMergeParts < splits) cm = fmaxf(cm, m[c]);
    if (cm == kNegInf) continue;                  // nothing but empty splits so far
    const float sc = exp2f(M - cm);               // 0 while M = -inf
    L *= sc;
    O *= sc;
#pragma unroll
    for (int c = 0; c < kMergeChunk; ++c) {
      if (s0 + c * kMergeParts < splits) {
        const float e = exp2f(m[c] - cm);
        L = fmaf(l[c], e, L);
        O = fmaf(o[c], e, O);
      }
    }
    M = cm;
  }
  if (d == 0) {
    pm[part] = M;
    pl[part] = L;
  }
  po[part][d] = O;
  __syncthreads();
  if (part == 0) {
    float Mt = kNegInf;
#pragma unroll
    for (int q = 0; q < kMergeParts; ++q) Mt = fmaxf(Mt, pm[q]);
    float Lt = 0.f, Ot = 0.f;
    if (Mt != kNegInf) {
#pragma unroll
      for (int q = 0; q < kMergeParts; ++q) {
        const float e = exp2f(pm[q] - Mt);
        Lt = fmaf(pl[q], e, Lt);
        Ot = fmaf(po[q][d], e, Ot);
      }
    }
    out[row * kHeadDim + d] = Lt > 0.f ? Ot / Lt : 0.f;
  }
}

}  // namespace

// Streaming (nontemporal) cache loads and one block in flight per wave for 8-wave
// workgroups and when one workgroup covers each (batch, kv head); plain loads and two
// blocks in flight for 4-wave split plans.  Measured on MI355X: the hint took the
// one-workgroup-per-head llama2_7b shapes from 26.3 to 25.1 us (27.8 to 27.0 with a
// 32-token sink), but llama2_13b split over 4-wave workgroups from 124.0 to 138.9 us;
// one block in flight instead of two took llama2_7b from 26.2 to 25.7 us and that
// llama2_13b plan from 124.8 to 125.4 us.  llama2_13b over 8-wave workgroups with both:
// 119.0 us.
hipError_t launch_decode_uniform(const DecodeArgs& a, int k_bits, int v_bits, int gq,
                                 hipStream_t s) {
  const int64_t wgs = (int64_t)a.batch * a.kv_heads * a.splits;
  const int nw = a.waves_per_group;
  const bool nt = a.splits == 1 || nw == 8;
  dim3 grid((unsigned)wgs), block((unsigned)(nw * kWave));
#define KVQ_DL(KB_, VB_, G_, NW_, NT_)                                              \
  if (k_bits == KB_ && v_bits == VB_ && gq == G_ && nw == NW_ && nt == NT_) {       \
    decode_uniform_kernel<KB_, VB_, G_, NW_, NT_><<<grid, block, 0, s>>>(a);        \
    hipError_t e_ = hipGetLastError();                                              \
    if (e_ != hipSuccess || a.splits == 1) return e_;                               \
    return launch_merge_splits(a, s);                                               \
  }
#define KVQ_DLB(G_, NW_, NT_) KVQ_DL(2, 2, G_, NW_, NT_) KVQ_DL(2, 4, G_, NW_, NT_) \
  KVQ_DL(4, 2, G_, NW_, NT_) KVQ_DL(4, 4, G_, NW_, NT_)
  // 2 and 4 query heads per kv head run on the matrix cores (decode_gqa.hip); split
  // plans use 8-wave workgroups for one query head per kv head, 4-wave ones for eight
  KVQ_DLB(1, 4, true) KVQ_DLB(8, 4, true) KVQ_DLB(1, 8, true)
  KVQ_DLB(8, 4, false)
#undef KVQ_DLB
#undef KVQ_DL
  return hipErrorInvalidValue;
}

// The kernel a split plan of nw-wave workgroups launches (for occupancy queries).
const void* decode_uniform_fn(int k_bits, int v_bits, int gq, int nw) {
#define KVQ_DF(KB_, VB_, G_, NW_, NT_)                                              \
  if (k_bits == KB_ && v_bits == VB_ && gq == G_ && nw == NW_)                      \
    return reinterpret_cast<const void*>(&decode_uniform_kernel<KB_, VB_, G_, NW_, NT_>);
#define KVQ_DFB(G_, NW_, NT_) KVQ_DF(2, 2, G_, NW_, NT_) KVQ_DF(2, 4, G_, NW_, NT_) \
  KVQ_DF(4, 2, G_, NW_, NT_) KVQ_DF(4, 4, G_, NW_, NT_)
  KVQ_DFB(1, 4, true) KVQ_DFB(8, 4, false) KVQ_DFB(1, 8, true)
#undef KVQ_DFB
#undef KVQ_DF
  return nullptr;
}

hipError_t launch_merge_splits(const DecodeArgs& a, hipStream_t s) {
  const int64_t rows = (int64_t)a.batch * a.q_heads;
  merge_splits_kernel<<<dim3((unsigned)rows), dim3(kMergeThreads), 0, s>>>(a.partials, a.out,
                                                                           a.splits);
  return hipGetLastError();
}

uint32_t debug_take_decode_uniform() { return debug_take_local(); }

}  // namespace kvq
