// Host-side argument checks of the C ABI under AddressSanitizer and UBSan, without a GPU:
// every call below must be rejected by the library's host validation before anything is
// enqueued.  Prints one "name status" line per call; device pointers are fake addresses
// that are never dereferenced.
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "kvq.h"

static const uintptr_t kFake = 0x7F0000000000ull;

static void* fake(int i) { return (void*)(kFake + 0x100000ull * (uintptr_t)(i + 1)); }

static kvq_cache desc(int kind, int kb, int vb, int B, int H, int64_t cap, int R) {
  kvq_cache c;
  memset(&c, 0, sizeof c);
  c.batch = B;
  c.kv_heads = H;
  c.head_dim = 128;
  c.residual_len = R;
  c.capacity_tokens = cap;
  const uint16_t* lut = kind == KVQ_NUQ ? (const uint16_t*)fake(40) : NULL;
  c.kq.kind = kind; c.kq.bits = kb; c.kq.axis = KVQ_AXIS_CHANNEL;
  c.kq.group_size = kind == KVQ_UNIFORM ? 32 : 0; c.kq.lut = lut;
  c.vq.kind = kind; c.vq.bits = vb; c.vq.axis = KVQ_AXIS_TOKEN;
  c.vq.group_size = kind == KVQ_UNIFORM ? 32 : 0; c.vq.lut = lut;
  return c;
}

static void buffers(kvq_cache* c) {
  c->k_codes = fake(1); c->k_meta = fake(2); c->v_codes = fake(3); c->v_meta = fake(4);
  c->k_resid = (uint16_t*)fake(5); c->v_resid = (uint16_t*)fake(6);
}

static void report(const char* name, kvq_status s) {
  printf("%s %d\n", name, (int)s);
  // the message buffer is read in full: a missing terminator or an overrun shows here
  const char* m = kvq_last_error();
  if (s != KVQ_OK && (m == NULL || strlen(m) == 0)) printf("%s no-message\n", name);
}

int main(void) {
  size_t sizes[KVQ_NUM_BUFS];
  kvq_cache c;

  c = desc(KVQ_UNIFORM, 3, 2, 2, 3, 256, 128);
  report("layout_bits3", kvq_layout_bytes(&c, sizes));
  c = desc(KVQ_UNIFORM, 2, 2, 2, 3, 100, 128);
  report("layout_cap100", kvq_layout_bytes(&c, sizes));
  c = desc(KVQ_UNIFORM, 2, 2, 2, 3, ((int64_t)1 << 28) + 32, 128);
  report("layout_cap_over", kvq_layout_bytes(&c, sizes));
  c = desc(KVQ_UNIFORM, 2, 2, 0, 3, 256, 128);
  report("layout_batch0", kvq_layout_bytes(&c, sizes));
  c = desc(KVQ_UNIFORM, 2, 2, 2, 3, 256, 100);
  report("layout_resid100", kvq_layout_bytes(&c, sizes));
  c = desc(KVQ_UNIFORM, 2, 2, 2, 3, 256, 128);
  c.sink_len = 1025;
  report("layout_sink", kvq_layout_bytes(&c, sizes));
  report("layout_null", kvq_layout_bytes(NULL, sizes));
  c = desc(KVQ_UNIFORM, 2, 2, 2, 3, 256, 128);
  c.csr_capacity = (int64_t)1 << 31;
  report("layout_csr_over", kvq_layout_bytes(&c, sizes));

  // quantize: null, misaligned, bad offsets, capacity, strides
  c = desc(KVQ_UNIFORM, 2, 2, 2, 3, 256, 128);
  buffers(&c);
  report("qk_null", kvq_quantize_keys(&c, NULL, 0, 0, 128, 0, 32, NULL, 0, NULL));
  report("qk_align", kvq_quantize_keys(&c, (const uint16_t*)((uintptr_t)fake(9) + 8), 0, 0, 128,
                                       0, 32, NULL, 0, NULL));
  report("qk_off16", kvq_quantize_keys(&c, (const uint16_t*)fake(9), 0, 0, 128, 16, 32, NULL, 0,
                                       NULL));
  report("qk_cap", kvq_quantize_keys(&c, (const uint16_t*)fake(9), 0, 0, 128, 224, 64, NULL, 0,
                                     NULL));
  report("qk_stride", kvq_quantize_keys(&c, (const uint16_t*)fake(9), 0, 0, 64, 0, 32, NULL, 0,
                                        NULL));
  report("qv_n48", kvq_quantize_values(&c, (const uint16_t*)fake(9), 0, 0, 128, 0, 48, NULL));

  // append: full window with no room to flush; counters out of range
  c = desc(KVQ_UNIFORM, 2, 2, 2, 3, 128, 128);
  buffers(&c);
  c.n_packed = 128; c.n_resid = 128;
  report("append_full", kvq_append_flush(&c, (const uint16_t*)fake(9), (const uint16_t*)fake(10),
                                         NULL));
  printf("append_state %lld %d\n", (long long)c.n_packed, c.n_resid);
  c.n_resid = 129;
  report("append_resid", kvq_append_flush(&c, (const uint16_t*)fake(9),
                                          (const uint16_t*)fake(10), NULL));

  // decode: bad query-head counts, RoPE on a uniform cache, scales, pointers
  c = desc(KVQ_UNIFORM, 2, 2, 2, 3, 256, 128);
  buffers(&c);
  c.n_packed = 64; c.n_resid = 5;
  const uint16_t* q = (const uint16_t*)fake(11);
  float* out = (float*)fake(12);
  report("dec_hq4", kvq_decode_attn(&c, q, 4, 0.1f, 0.f, out, fake(13), 1 << 20, NULL));
  report("dec_hq15", kvq_decode_attn(&c, q, 15, 0.1f, 0.f, out, fake(13), 1 << 20, NULL));
  report("dec_rope", kvq_decode_attn(&c, q, 3, 0.1f, 1e4f, out, fake(13), 1 << 20, NULL));
  report("dec_scale", kvq_decode_attn(&c, q, 3, 1.0f / 0.0f, 0.f, out, fake(13), 1 << 20, NULL));
  report("dec_qalign", kvq_decode_attn(&c, (const uint16_t*)((uintptr_t)q + 4), 3, 0.1f, 0.f,
                                       out, fake(13), 1 << 20, NULL));
  report("dec_out", kvq_decode_attn(&c, q, 3, 0.1f, 0.f, NULL, fake(13), 1 << 20, NULL));
  report("noalloc_hq4", kvq_decode_attn_noalloc(&c, q, 4, 0.1f, 0.f, out, NULL));
  report("noalloc_theta", kvq_decode_attn_noalloc(&c, q, 3, 0.1f, -1.f, out, NULL));

  // nuq keys: outliers beyond the int32 row pointers
  c = desc(KVQ_NUQ, 3, 3, 1, 1, (int64_t)1 << 28, 0);
  buffers(&c);
  c.kq.outlier_bp = 700;
  c.csr_capacity = ((int64_t)1 << 31) - 1;
  c.k_csr_rowptr = (int32_t*)fake(20);
  c.k_csr_ent = (uint32_t*)fake(21);
  report("nuq_csr_int32", kvq_quantize_keys(&c, (const uint16_t*)fake(9), 0, 0, 128, 0,
                                            (int64_t)1 << 28, fake(22), (size_t)1 << 40, NULL));
  printf("csr_needed %lld\n", (long long)kvq_csr_entries_needed(&c));
  printf("ws_bad %zu\n", kvq_workspace_bytes(NULL, 1, KVQ_OP_DECODE_ATTN));
  return 0;
}
