/*
 * kvq.h - packed low-bit KV cache and decode attention over it, for AMD
 * Instinct MI355X (gfx950).  C ABI; every device buffer is allocated and owned
 * by the caller, the library never allocates device memory.
 *
 * What is computed (sources, by title and section):
 *  - "The KV cache has a geometry problem, not a bits problem" (unite.ai):
 *      section "Quantization error in practice" - uniform asymmetric B-bit
 *      quantization of a group: the minimum is the zero point, the step is the
 *      range divided by 2^B - 1, every element is rounded to the nearest step;
 *      sections on keys and values - keys grouped per channel, values per
 *      token; section "The systems tax" - the newest tokens (up to 128) stay
 *      in full precision and are quantized as a group once the window fills;
 *      section on rotary embeddings - quantize keys before RoPE and rotate
 *      them after dequantization.
 *  - "KIVI: A Tuning-Free Asymmetric 2bit Quantization for KV Cache"
 *      (Telegram post): "Method" - per-channel keys, per-token values, a
 *      full-precision window of 128 recent tokens quantized when full;
 *      "Experiments" - group size 32 with a floating-point zero point.
 *  - "KVQuant: Towards 10 Million Context Length LLM Inference with KV Cache
 *      Quantization" (paper review): abstract items (ii) pre-RoPE keys,
 *      (iii) non-uniform datatype nuqX, (iv) per-vector dense-and-sparse
 *      quantization with the outliers kept in full precision.
 *  - "Quantize What Counts: More for Keys, Less for Values": more bits for
 *      keys than for values (4-bit keys with 2-bit values).
 *
 * Readings where the sources are silent (one rule on every call):
 *  - Code of an element x of a group: with mn = min + 0 and mx = max + 0 of the
 *    group (fp32, -0 becomes +0), scale_h = fp16_rne((mx - mn) / (2^B - 1)),
 *    s = (float)scale_h, inv = (s == 0 ? 0 : 1.0f / s), code =
 *    (s == 0 ? 0 : clamp(rint((x - mn) * inv), 0, 2^B - 1)), every operation an
 *    IEEE fp32 operation with round-to-nearest-even and no fused multiply-add.
 *    Dequantized value: code * s + min.
 *  - nuq (KVQ_NUQ, B = 2, 3 or 4): the same (mn, scale, inv) over the
 *    vector's dense entries; xn = (x - mn) * inv; the code is the index of the
 *    nearest level of the caller's 2^B-entry fp16 code book (levels in "level
 *    units", 0..2^B - 1, strictly ascending; ties go to the even index).
 *    Dequantized value: lut[code] * s + mn.  The identity code book
 *    {0, ..., 2^B - 1} reproduces the uniform B-bit quantizer exactly.
 *  - Outliers (nuq keys, outlier_bp > 0): per (batch, head, channel) the
 *    ceil(n * outlier_bp / 10000) entries of largest fp16 magnitude over the
 *    n quantized tokens (ties: lower token first) are kept exactly in a CSR
 *    matrix and excluded from the channel's min/max.  Their positions store
 *    code 0; attention uses the exact value.  (Value outliers likewise.)
 *  - Q-Norm (nuq, qnorm = 1; KVQuant review, "Proposed method": the dequantized
 *    distribution is matched to the statistics taken before quantization): per
 *    vector, after its codes, (scale, min) become (a * scale, a * min + b) with
 *    a = sqrt(var / var_hat) (1 if var_hat = 0) and b = mean - a * mean_hat, so
 *    that the dequantized dense entries get the mean and variance of the original
 *    ones; each result rounded to fp32, then fp16.  mean and var of the original
 *    dense entries in fp64 (E[x^2] - E[x]^2), where sum x and sum x^2 are the
 *    exact sums rounded once to fp64 (independent of the order of addition);
 *    mean_hat and var_hat from the code
 *    histogram, level values lut[c] * scale + min in fp32, summed in fp64 over c
 *    ascending.  Codes are unchanged.
 *  - Value outliers (nuq values, outlier_bp > 0): per (batch, head, token) the
 *    kv = ceil(D * outlier_bp / 10000) channels of largest fp16 magnitude (ties:
 *    lower channel first), handled like the key outliers (KVQuant review,
 *    abstract item (iv): outliers isolated for each vector, keys and values).
 *  - Sequence order: the attention-sink tokens (positions 0..n_sink-1, fp16;
 *    "The KV cache has a geometry problem", section on where research goes:
 *    full-precision windows for the recent tokens and for the attention-sink
 *    tokens), then the packed tokens (positions n_sink..n_sink+n_packed-1), then
 *    the window (the next n_resid positions, fp16).  The sink fills first.
 *  - Attention: s_t = sm_scale * q . k_t over every cached token (sink and
 *    window in fp16, packed tokens dequantized), softmax over all of them,
 *    out = sum_t p_t v_t / sum_t p_t, fp32.  With rope_theta > 0 (nuq caches
 *    only) key t is rotated by RoPE at its position t (interleaved pairs
 *    (2i, 2i+1), frequency theta^(-2i/D)); the query is passed already rotated.
 *    GQA: query head h reads kv head h / (Hq / Hkv).
 *
 * Packed layouts (little-endian 32-bit words, codes least-significant first;
 * G = 32 tokens per block, D = head_dim, nb = capacity_tokens / 32):
 *  UNIFORM keys, bits Bk (2 or 4), per-channel groups of 32 tokens:
 *    k_codes [batch][kv_heads][nb][32 tokens][D*Bk/32 words]: channel d of a
 *      token at bit (Bk*d) % 32 of word (Bk*d) / 32 of that token's row.
 *    k_meta  [batch][kv_heads][nb][D] words: scale_h | min_h << 16 of (block, d).
 *  UNIFORM values, bits Bv (2 or 4), per-token groups of 32 channels:
 *    v_codes [batch][kv_heads][nb][D*Bv words]: each block is cut into tiles of
 *      8 tokens x 8 channels, stored in (token octet, channel octet) order with
 *      2*Bv words per tile.  Token pair i of a tile (tokens 2i, 2i+1 of the octet)
 *      owns word i (Bv = 2) or words i and i + 4 (Bv = 4: channels 0..3 of the
 *      octet, then 4..7); the even token fills bits 0..15 and the odd token bits
 *      16..31, the channels Bv bits apart from bit 0 of each half.
 *    v_meta  [batch][kv_heads][nb*32 tokens][D/32] words.
 *  NUQ codes (B = 2, 3 or 4 bits), keys and values alike:
 *    [batch][kv_heads][nb][D][B words] per block and channel.  B = 3: word 0
 *      holds the low two bits of tokens 0..15 and word 1 those of tokens 16..31
 *      (token j of its half at bit 8*(j%4) + 2*(j/4)); word 2 holds the high bits
 *      of all 32 tokens (token j at bit 8*(j%4) + j/4).  B = 2: words 0 and 1 as
 *      for B = 3.  B = 4: word i holds tokens 8i..8i+7, token j of its octet at
 *      bit 8*(j%4) + 4*(j/4).
 *  NUQ keys (per channel over all quantized tokens):
 *    k_meta  [batch][kv_heads][D] words (one scale/min per channel).
 *    k_csr_rowptr [batch][kv_heads][capacity_tokens + 1] int32, rows = tokens,
 *      offsets relative to the head's segment of k_csr_ent;
 *    k_csr_ent [batch][kv_heads][csr_capacity] uint32: channel in bits 0..7, the
 *      row's token modulo 32 (its place in its 32-token block) in bits 8..12, fp16
 *      value in bits 16..31, channels ascending within a row.
 *  NUQ value outliers: v_out [batch][kv_heads][capacity_tokens][kv] uint32,
 *      entries as for the keys, channels ascending (a CSR whose rows all hold kv).
 *  NUQ values (per token over all D channels):
 *    v_meta  [batch][kv_heads][capacity_tokens] words.
 *  Window: k_resid, v_resid [batch][kv_heads][residual_len][D] fp16.
 *  Sink: k_sink, v_sink [batch][kv_heads][sink_len][D] fp16.
 *
 * Conventions:
 *  - fp16 values travel as uint16_t bit patterns.
 *  - Every device pointer must be 16-byte aligned (KVQ_ERR_ALIGNMENT).
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream).  Work
 *    is enqueued on it; no call synchronizes the host.
 *  - Arguments are checked on the host before anything is enqueued; a call
 *    that returns an error has changed nothing.  KVQ_ERR_HIP reports a failed
 *    launch; faults inside kernels surface at the caller's next synchronization.
 *  - kvq_last_error() returns a thread-local message for the last non-OK
 *    status of the calling thread.
 *  - Calls that share a cache or a workspace on one stream are ordered; calls
 *    on different streams that touch the same buffers race.
 *  - Calls enqueue kernel launches only (no memsets, copies or allocations), so
 *    they can be captured into a HIP graph.  A captured call keeps the pointers
 *    and the counters (n_packed, n_resid, n_sink) it saw at capture: each replay
 *    repeats that step on the buffers' current contents.
 *  - Debug build (libkvq_debug.so, compiled with -DKVQ_DEBUG; same ABI): the
 *    kernels also check every block index, CSR row range, outlier entry, append
 *    slot and split range they derive, setting a flag instead of trapping, and
 *    every call then waits for the device and returns KVQ_ERR_HIP, naming the
 *    flags, if a check failed.  Those calls synchronize, so they cannot be
 *    captured into a graph.
 */
#ifndef KVQ_H
#define KVQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  KVQ_OK = 0,
  KVQ_ERR_INVALID_ARG = 1,  /* null pointer, bad size or inconsistent descriptor */
  KVQ_ERR_UNSUPPORTED = 2,  /* valid for the method, not built for the GPU here */
  KVQ_ERR_CAPACITY = 3,     /* token range or outliers exceed the buffers */
  KVQ_ERR_ALIGNMENT = 4,    /* a device pointer is not 16-byte aligned */
  KVQ_ERR_HIP = 5           /* the HIP runtime reported an error */
} kvq_status;

enum { KVQ_AXIS_CHANNEL = 0, KVQ_AXIS_TOKEN = 1 };
enum { KVQ_UNIFORM = 0, KVQ_NUQ = 1 };

/* Buffer slots reported by kvq_layout_bytes. */
enum {
  KVQ_BUF_K_CODES = 0, KVQ_BUF_K_META = 1, KVQ_BUF_V_CODES = 2, KVQ_BUF_V_META = 3,
  KVQ_BUF_K_RESID = 4, KVQ_BUF_V_RESID = 5, KVQ_BUF_K_CSR_ROWPTR = 6,
  KVQ_BUF_K_CSR_ENT = 7, KVQ_BUF_K_SINK = 8, KVQ_BUF_V_SINK = 9, KVQ_BUF_V_OUT = 10,
  KVQ_NUM_BUFS = 11
};

/* Operations for kvq_workspace_bytes. */
enum { KVQ_OP_QUANTIZE_KEYS = 0, KVQ_OP_DECODE_ATTN = 1 };

/* Quantization settings of one tensor (K or V). */
typedef struct {
  int32_t kind;        /* KVQ_UNIFORM or KVQ_NUQ (K and V must agree) */
  int32_t bits;        /* UNIFORM: 2 or 4; NUQ: 2, 3 or 4 (K and V alike) */
  int32_t axis;        /* K: KVQ_AXIS_CHANNEL, V: KVQ_AXIS_TOKEN; the swapped
                          axes are valid for the method but KVQ_ERR_UNSUPPORTED */
  int32_t group_size;  /* UNIFORM: 32; NUQ: 0 (the whole vector) */
  const uint16_t* lut; /* NUQ: device fp16[2^bits], ascending, level units
                          [0, 2^bits - 1]; else NULL */
  int32_t outlier_bp;  /* NUQ: outliers per vector in basis points (100 = 1 %),
                          0..10000 - keys: of each channel's quantized tokens,
                          values: of each token's D channels; UNIFORM: 0 */
  int32_t qnorm;       /* NUQ: 1 = Q-Norm the metadata (see above), 0 = off;
                          UNIFORM: 0 */
} kvq_qparams;

/* The cache descriptor.  Caller-owned; the library reads it and only
 * kvq_append_flush writes it (n_packed, n_resid). */
typedef struct {
  int32_t batch;           /* >= 1 */
  int32_t kv_heads;        /* >= 1 */
  int32_t head_dim;        /* 128 on the GPU (the layouts allow any multiple of 32) */
  int32_t residual_len;    /* fp16 window R: 0 or a multiple of 32, <= 1024 */
  int64_t capacity_tokens; /* packed capacity, a multiple of 32, <= 2^28 */
  kvq_qparams kq, vq;
  void* k_codes;           /* device buffers, sizes from kvq_layout_bytes */
  void* k_meta;
  void* v_codes;
  void* v_meta;
  uint16_t* k_resid;       /* window buffers (NULL when residual_len == 0) */
  uint16_t* v_resid;
  int32_t* k_csr_rowptr;   /* NUQ keys with outlier_bp > 0, else NULL */
  uint32_t* k_csr_ent;
  int64_t csr_capacity;    /* entries per (batch, head) segment of k_csr_ent, < 2^31
                              (the row pointers are int32) */
  uint32_t* v_out;         /* NUQ values with vq.outlier_bp > 0, else NULL */
  int64_t n_packed;        /* tokens in the packed part (multiple of 32) */
  int32_t n_resid;         /* tokens in the window, 0..residual_len */
  int32_t sink_len;        /* attention-sink window: the sequence's first sink_len
                              tokens stay in fp16 and are never quantized; 0..1024 */
  uint16_t* k_sink;        /* [batch][kv_heads][sink_len][D] fp16 (NULL when sink_len
                              == 0); written by kvq_append_flush or by the caller */
  uint16_t* v_sink;
  int32_t n_sink;          /* tokens in the sink, 0..sink_len */
  int32_t reserved;        /* 0 */
} kvq_cache;

/* Passage: the bit budgets of KIVI "Experiments" (2-bit codes, group 32, fp zero
 * point) and of the KVQuant review's results table (KV-cache size per width).
 * Bytes of each buffer slot for the descriptor's shape and settings (0 for slots
 * the settings do not use).  Reads no pointer.  The CSR entry slot is sized for
 * c->csr_capacity entries per head. */
kvq_status kvq_layout_bytes(const kvq_cache* c, size_t sizes_out[KVQ_NUM_BUFS]);

/* Passage: KVQuant review, abstract item (iv) (per-vector dense-and-sparse, 1 %).
 * Smallest csr_capacity that holds the outliers of a full cache:
 * head_dim * ceil(capacity_tokens * outlier_bp / 10000); 0 without outliers, -1
 * for an invalid descriptor. */
int64_t kvq_csr_entries_needed(const kvq_cache* c);

/* No passage: the split-K partials and the nuq select passes are this library's
 * design.  Device scratch bytes that `op` needs for this descriptor (decode: for any
 * n_packed <= capacity_tokens and n_resid <= residual_len; q_heads is ignored by
 * the quantize op).  The decode workspace holds per-split partial results; its
 * contents need no initialization and are overwritten by every call.  Returns 0
 * if the op needs none or on invalid input. */
size_t kvq_workspace_bytes(const kvq_cache* c, int32_t q_heads, int32_t op);

/* Passage: KIVI "Method" and "The KV cache has a geometry problem", section on keys
 * (keys per channel); KVQuant review, abstract items (i)-(iv) for NUQ.
 * Quantize keys of tokens [token_offset, token_offset + n_tokens) into the packed
 * part (k_codes, k_meta and, for NUQ, the CSR).  k points at the key of token
 * token_offset: element (b, h, t, d) is k[b*stride_b + h*stride_h + t*stride_t + d]
 * (fp16, channels contiguous).  UNIFORM: offset and count are multiples of 32,
 * workspace unused.  NUQ: one shot over the whole context (offset 0), workspace of
 * kvq_workspace_bytes(c, 0, KVQ_OP_QUANTIZE_KEYS) bytes; KVQ_ERR_CAPACITY if the
 * outliers exceed csr_capacity.  Does not move n_packed. */
kvq_status kvq_quantize_keys(const kvq_cache* c, const uint16_t* k, int64_t stride_b,
                             int64_t stride_h, int64_t stride_t, int64_t token_offset,
                             int64_t n_tokens, void* workspace, size_t ws_bytes,
                             void* stream);

/* Passage: KIVI "Method" and "The KV cache has a geometry problem", section on values
 * (values per token); KVQuant review, abstract items (iii)-(iv) for NUQ.
 * Quantize values of tokens [token_offset, token_offset + n_tokens) into v_codes and
 * v_meta; arguments as for kvq_quantize_keys (no workspace). */
kvq_status kvq_quantize_values(const kvq_cache* c, const uint16_t* v, int64_t stride_b,
                               int64_t stride_h, int64_t stride_t, int64_t token_offset,
                               int64_t n_tokens, void* stream);

/* Passage: KIVI "Method" (the newest tokens, up to 128, stay in full precision and are
 * quantized together when the window fills); "The KV cache has a geometry problem",
 * section "The systems tax".
 * Append one token per (batch, kv head): k_new, v_new are fp16 [batch][kv_heads][D],
 * contiguous.  While the sink has room (n_sink < sink_len) the token goes to sink
 * slot n_sink and n_sink += 1; nothing else changes.  Otherwise, if the window is
 * full (n_resid == residual_len) it is first
 * quantized into the packed part at token n_packed (KVQ_ERR_CAPACITY if that
 * would pass capacity_tokens) and n_packed += residual_len, n_resid = 0; then the
 * token is written at window slot n_resid and n_resid += 1.  UNIFORM only, and
 * residual_len > 0 once the sink is full.  The counters are updated on the host
 * when the work is enqueued.  A prefill that starts with a sink copies the first
 * sink tokens into k_sink/v_sink itself, sets n_sink, and quantizes the following
 * tokens with the calls above (their token offsets count from the first packed
 * token). */
kvq_status kvq_append_flush(kvq_cache* c, const uint16_t* k_new, const uint16_t* v_new,
                            void* stream);

/* Passage: "The KV cache has a geometry problem", section "Why the KV cache is a
 * problem" (each generated token reads the whole cache) and its section on rotary
 * embeddings with KVQuant review abstract item (ii) (RoPE after dequantization).
 * Decode attention of one query token per (batch, query head) over the whole
 * cache: q fp16 [batch][q_heads][D], out fp32 [batch][q_heads][D], both contiguous.
 * q_heads is a multiple of kv_heads (at most 8 query heads per kv head).
 * rope_theta: 0 = no rotation; > 0 (NUQ caches only) rotates key t at position t.
 * workspace: kvq_workspace_bytes(c, q_heads, KVQ_OP_DECODE_ATTN) bytes; its
 * contents need no initialization.  A cache with no tokens (no sink, packed or
 * window tokens) gives out = 0. */
kvq_status kvq_decode_attn(const kvq_cache* c, const uint16_t* q, int32_t q_heads,
                           float sm_scale, float rope_theta, float* out, void* workspace,
                           size_t ws_bytes, void* stream);

/* For callers that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc): kvq_decode_attn without a workspace.
 * The split partials go to a file-scope device array of the library, 8 MiB per GPU (a
 * copy on every GPU the library runs on, held until the process ends); its address is
 * taken once per device, on the first call there.  Arguments, results and errors as for
 * kvq_decode_attn, plus KVQ_ERR_CAPACITY when the decode's split plan needs more than
 * 8 MiB of partials (batch * q_heads * splits * 528 bytes; such a call changes nothing).
 * Calls on one GPU share the array: calls that overlap in time on one GPU (different
 * streams, or host threads without ordering) race and may return wrong results.  The
 * array needs no initialization: every split writes its partial before the merge reads
 * it.  Allocates nothing and calls no allocating routine. */
kvq_status kvq_decode_attn_noalloc(const kvq_cache* c, const uint16_t* q, int32_t q_heads,
                                   float sm_scale, float rope_theta, float* out, void* stream);

/* No passage (error reporting).  Message for the calling thread's last non-OK status
 * ("" if none). */
const char* kvq_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* KVQ_H */
