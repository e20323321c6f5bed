// Internal declarations shared by the library's translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kvq.h"

namespace kvq {

constexpr int kGroup = 32;        // tokens per packed block, channels per value group
constexpr int kHeadDim = 128;     // the GPU kernels are built for D = 128
constexpr int kWave = 64;

typedef _Float16 h2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ h2_t as_h2(uint32_t w) { return __builtin_bit_cast(h2_t, w); }
__device__ __forceinline__ float lo_f16(uint32_t w) { return (float)as_h2(w)[0]; }
__device__ __forceinline__ float hi_f16(uint32_t w) { return (float)as_h2(w)[1]; }
__device__ __forceinline__ float f16_bits_to_f32(uint16_t b) {
  return (float)__builtin_bit_cast(_Float16, b);
}
// fp32 -> fp16 bits, round to nearest even (v_cvt_f16_f32 under the default mode).
__device__ __forceinline__ uint16_t f32_to_f16_bits(float x) {
  return __builtin_bit_cast(uint16_t, (_Float16)x);
}

// ---- debug builds (compiled with -DKVQ_DEBUG) -------------------------------------------
// Device-side bounds checks.  A failed check does not trap: it sets a bit in its
// translation unit's flag word (a global atomic), the kernel goes on (every checked access
// is also guarded or clamped), and the host entry point, which in these builds waits for
// its stream after launching, reads and clears the words of all translation units and
// returns KVQ_ERR_HIP naming the bits.  Release builds compile the checks away.
enum DebugBit : uint32_t {
  kDbgBlock = 1u << 0,    // a packed block or window chunk beyond the cache
  kDbgCsr = 1u << 1,      // a CSR row range or entry index beyond csr_capacity
  kDbgEntry = 1u << 2,    // a CSR or value-outlier entry with a field out of range
  kDbgWrite = 1u << 3,    // a quantizer write beyond the buffers' capacity
  kDbgSplit = 1u << 4,    // a split's unit range or a merge index beyond the plan
};
#ifdef KVQ_DEBUG
static __device__ uint32_t kvq_debug_word;
#define KVQ_CHECK(cond, bit)                                                    \
  do {                                                                          \
    if (!(cond)) atomicOr(&::kvq::kvq_debug_word, (uint32_t)(bit));             \
  } while (0)
// This translation unit's flag word, read and cleared (host; the caller synchronized).
static inline uint32_t debug_take_local() {
  uint32_t v = 0, z = 0;
  if (hipMemcpyFromSymbol(&v, HIP_SYMBOL(kvq_debug_word), sizeof v) != hipSuccess) return ~0u;
  if (hipMemcpyToSymbol(HIP_SYMBOL(kvq_debug_word), &z, sizeof z) != hipSuccess) return ~0u;
  return v;
}
#else
#define KVQ_CHECK(cond, bit) ((void)0)
static inline uint32_t debug_take_local() { return 0u; }
#endif
// Each kernel translation unit defines one: its flag word (0 in release builds).
uint32_t debug_take_decode_uniform();
uint32_t debug_take_decode_gqa();
uint32_t debug_take_decode_nuq();
uint32_t debug_take_quant_uniform();
uint32_t debug_take_quant_nuq();

// Streaming loads: global loads with the nontemporal hint, for data read once per decode
// (packed codes, metadata, fp16 windows).  Measured on a 117 MB read by one workgroup
// per CU: 6.5 TB/s with the hint against 5.8 TB/s without.  Pointers must be aligned to
// the load width.
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint32_t ld_stream(const uint32_t* p) {
  return __builtin_nontemporal_load(p);
}
__device__ __forceinline__ uint2 ld_stream2(const void* p) {
  const u32x2_t t = __builtin_nontemporal_load(reinterpret_cast<const u32x2_t*>(p));
  return make_uint2(t.x, t.y);
}
__device__ __forceinline__ uint4 ld_stream4(const void* p) {
  const u32x4_t t = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  return make_uint4(t.x, t.y, t.z, t.w);
}
// Cache loads with the hint chosen at compile time (NT = true: streaming loads).
template <bool NT>
__device__ __forceinline__ uint32_t ld_cache(const uint32_t* p) {
  if constexpr (NT) return ld_stream(p); else return *p;
}
template <bool NT>
__device__ __forceinline__ uint2 ld_cache2(const void* p) {
  if constexpr (NT) return ld_stream2(p); else return *reinterpret_cast<const uint2*>(p);
}
template <bool NT>
__device__ __forceinline__ uint4 ld_cache4(const void* p) {
  if constexpr (NT) return ld_stream4(p); else return *reinterpret_cast<const uint4*>(p);
}

// ---- launch parameter blocks (host fills, kernels read) ----------------------
struct QuantArgs {
  const uint16_t* k;        // source keys (NULL: skip keys)
  const uint16_t* v;        // source values (NULL: skip values)
  int64_t ks_b, ks_h, ks_t; // element strides of the key source
  int64_t vs_b, vs_h, vs_t;
  uint32_t* k_codes;
  uint32_t* k_meta;
  uint32_t* v_codes;
  uint32_t* v_meta;
  int32_t kv_heads;
  int32_t n_blocks;         // blocks of 32 tokens to quantize per (b, h)
  int64_t blk0;             // destination block index of the first block
  int64_t cap_blocks;       // capacity_tokens / 32
};

struct AppendArgs {
  const uint16_t* k_new;
  const uint16_t* v_new;
  uint16_t* k_resid;
  uint16_t* v_resid;
  int32_t rows;             // batch * kv_heads
  int32_t residual_len;
  int32_t slot;
};

struct DecodeArgs {
  const uint32_t* k_codes;
  const uint32_t* k_meta;
  const uint32_t* v_codes;
  const uint32_t* v_meta;
  const uint16_t* k_resid;
  const uint16_t* v_resid;
  const uint16_t* k_sink;   // attention-sink window (the sequence's first tokens, fp16)
  const uint16_t* v_sink;
  const uint16_t* q;
  float* out;
  float* partials;          // [batch][q_heads][splits][kPartialStride]
  // nuq extras
  const uint16_t* lut_k;
  const uint16_t* lut_v;
  const int32_t* csr_rowptr;
  const uint32_t* csr_ent;
  int64_t csr_capacity;
  const uint32_t* v_out;    // value outliers [bh][cap_tokens][v_kv] (NULL: none)
  int32_t v_kv;
  float rope_theta;
  int32_t batch, kv_heads, q_heads;
  int32_t residual_len;
  int32_t sink_len, n_sink;
  int64_t cap_blocks;
  int32_t n_blocks;         // packed blocks (n_packed / 32)
  int32_t n_resid;
  int32_t splits;           // workgroups per (batch, kv head)
  int32_t waves_per_group;  // 4 or 8
  float scale_log2;         // sm_scale * log2(e)
};

// fp16 tokens of a decode come in chunks of 32: the sink's chunks first (positions
// 0 .. n_sink-1), then the window's (positions n_sink + n_packed ..).
__device__ __forceinline__ int fp16_chunks(const DecodeArgs& a) {
  return (a.n_sink + kGroup - 1) / kGroup + (a.n_resid + kGroup - 1) / kGroup;
}

struct Fp16Chunk {
  const uint16_t* k;        // token 0 of the chunk, channel 0 (rows of kHeadDim)
  const uint16_t* v;
  int nvalid;               // tokens present, 1..32
  int64_t pos0;             // sequence position of token 0
};

__device__ __forceinline__ Fp16Chunk fp16_chunk(const DecodeArgs& a, int64_t bh, int c) {
  const int sink_chunks = (a.n_sink + kGroup - 1) / kGroup;
  Fp16Chunk r;
  if (c < sink_chunks) {
    const int tok0 = c * kGroup;
    r.k = a.k_sink + (bh * a.sink_len + tok0) * kHeadDim;
    r.v = a.v_sink + (bh * a.sink_len + tok0) * kHeadDim;
    r.nvalid = min(kGroup, a.n_sink - tok0);
    r.pos0 = tok0;
    KVQ_CHECK(r.nvalid >= 1 && a.n_sink <= a.sink_len, kDbgBlock);
  } else {
    const int tok0 = (c - sink_chunks) * kGroup;
    r.k = a.k_resid + (bh * a.residual_len + tok0) * kHeadDim;
    r.v = a.v_resid + (bh * a.residual_len + tok0) * kHeadDim;
    r.nvalid = min(kGroup, a.n_resid - tok0);
    r.pos0 = a.n_sink + (int64_t)a.n_blocks * kGroup + tok0;
    KVQ_CHECK(r.nvalid >= 1 && a.n_resid <= a.residual_len, kDbgBlock);
  }
  return r;
}

constexpr int kPartialStride = kHeadDim + 4;   // o[128], m, l, pad
constexpr int kMaxSplits = 2048;               // workgroups per (batch, kv head) at most
constexpr int kNuqChunk = 2048;                // tokens per chunk in the nuq key passes
constexpr int kNuqListCap = 32;                // threshold-bin entries kept per chunk and channel
constexpr int64_t kMaxCapacityTokens = (int64_t)1 << 28;   // packed tokens per (batch, head)

struct NuqKeysArgs {
  const uint16_t* k;        // keys of token 0: element (b, h, t, d) at b*sb + h*sh + t*st + d
  int64_t sb, sh, st;
  const uint16_t* lut;      // fp16[2^bits]
  int32_t bits;             // 2, 3 or 4
  int32_t qnorm;            // 1: Q-Norm the per-channel metadata
  int32_t kv_heads;
  int32_t bh_count;         // batch * kv_heads
  int64_t n_tokens;         // tokens quantized (multiple of 32)
  int32_t nchunks;          // ceil(n_tokens / kNuqChunk)
  int64_t k_out;            // outliers per channel
  int64_t cap_tokens, cap_blocks, csr_capacity;
  uint32_t* k_codes;
  uint32_t* k_meta;
  int32_t* rowptr;          // NULL: no outliers
  uint32_t* ent;
  // workspace
  uint32_t* hist_hi;        // [bh][D][256]
  uint32_t* hist_lo;        // [bh][D][128]
  int32_t* thr;             // [bh][D][4]: T, need, high bin, count above
  float* norm;              // [bh][D][2]: min, 1/scale
  uint32_t* chunk_stats;    // [bh][nchunks][D][8]
  uint32_t* lists;          // [bh][nchunks][D][kNuqListCap]: threshold-bin entries
  uint32_t* tie_prefix;     // [bh][nchunks][D]
  uint32_t* chunk_cnt;      // [bh][nchunks]
  uint32_t* chunk_off;      // [bh][nchunks]
  uint64_t* qn_sum;         // [bh][nchunks][D][4]: exact sum x (128-bit, 2^-24 units) and
                            // sum x^2 (128-bit, 2^-48 units) of the dense entries (Q-Norm)
  uint32_t* qn_hist;        // [bh][nchunks][D][16]: dense code counts (Q-Norm)
};

struct NuqValuesArgs {
  const uint16_t* v;        // values of token tok0
  int64_t sb, sh, st;
  const uint16_t* lut;
  int32_t bits;             // 2, 3 or 4
  int32_t qnorm;            // 1: Q-Norm the per-token metadata
  int32_t kv_heads, bh_count;
  int32_t n_blocks;
  int64_t tok0;
  int64_t cap_tokens, cap_blocks;
  uint32_t* v_codes;
  uint32_t* v_meta;
  uint32_t* v_out;          // outlier entries [bh][cap_tokens][kv] (NULL: none)
  int32_t kv;               // outliers per token
};

// ---- launchers (defined in the .hip files) ------------------------------------
hipError_t launch_quant_uniform(const QuantArgs& a, int batch, int k_bits, int v_bits,
                                hipStream_t s);
hipError_t launch_append(const AppendArgs& a, hipStream_t s);
hipError_t launch_decode_uniform(const DecodeArgs& a, int k_bits, int v_bits, int gq,
                                 hipStream_t s);
hipError_t launch_decode_gqa(const DecodeArgs& a, int k_bits, int v_bits, int gq,
                             hipStream_t s);
hipError_t launch_merge_splits(const DecodeArgs& a, hipStream_t s);
hipError_t launch_nuq_keys(const NuqKeysArgs& a, hipStream_t s);
hipError_t launch_nuq_values(const NuqValuesArgs& a, hipStream_t s);
hipError_t launch_decode_nuq(const DecodeArgs& a, int gq, int bits, hipStream_t s);
// The kernel a launcher above would run (for occupancy queries); NULL if none.
const void* decode_uniform_fn(int k_bits, int v_bits, int gq, int nw);
const void* decode_gqa_fn(int k_bits, int v_bits, int gq, int nw);
const void* decode_nuq_fn(int gq, int nw, int bits);

}  // namespace kvq
