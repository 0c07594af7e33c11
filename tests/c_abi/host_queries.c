/* A plain C caller of the library's host-only entry points (no GPU needed):
 * builds the INT2 pre-RoPE 32K cache config, sizes its arena and workspace,
 * reads the layout, and checks that an invalid config is rejected.  Prints one
 * line of key=value pairs for the test that compiles and runs it. */
#include <stdio.h>
#include <string.h>
#include "kvq.h"

int main(void) {
  kvq_config c;
  memset(&c, 0, sizeof c);
  c.batch = 32; c.num_q_heads = 32; c.num_kv_heads = 8; c.head_dim = 128;
  c.max_tokens = 32832; c.in_dtype = KVQ_BF16; c.out_dtype = KVQ_F32;
  c.k.scheme = KVQ_INT_ASYM; c.k.bits = 2; c.k.axis = KVQ_PER_CHANNEL; c.k.group = 32;
  c.v.scheme = KVQ_INT_ASYM; c.v.bits = 2; c.v.axis = KVQ_PER_TOKEN; c.v.group = 32;
  c.residual = 32; c.pre_rope_k = 1; c.rope_base = 10000.0f; c.meta_dtype = KVQ_F32;
  if (kvq_validate_config(&c) != KVQ_OK) { printf("validate failed\n"); return 1; }
  size_t arena = 0, ws = 0;
  kvq_layout lay;
  kvq_attn_options opt;
  memset(&opt, 0, sizeof opt);
  if (kvq_arena_bytes(&c, &arena) != KVQ_OK || kvq_arena_layout(&c, &lay) != KVQ_OK ||
      kvq_workspace_bytes(&c, 32769, &opt, &ws) != KVQ_OK) { printf("sizing failed\n"); return 1; }
  c.meta_dtype = KVQ_F16;
  size_t arena16 = 0;
  if (kvq_arena_bytes(&c, &arena16) != KVQ_OK) { printf("fp16 sizing failed\n"); return 1; }
  kvq_config bad = c;
  bad.num_q_heads = 30;                      /* not a multiple of the kv heads */
  const int st = kvq_validate_config(&bad);
  printf("abi=%d arena=%zu arena16=%zu ws=%zu tq=%lld ring_slots=%d bad=%d msg=%s\n",
         kvq_abi_version(), arena, arena16, ws, (long long)kvq_quantized_tokens(&c, 32769),
         lay.ring_slots, st, kvq_status_string(st));
  return lay.total_bytes == arena ? 0 : 1;
}
