// Launchers of the device kernels (internal interface between kvq_api.hip and
// the kernel translation units).
#pragma once
#include "kvq_internal.h"

namespace kvq {

// Page ids of one token split that the MFMA kernel keeps in LDS (paged caches).
constexpr int kMaxSplitPages = 256;

// Plan of one decode-attention call.
struct AttnPlan {
  int32_t kernel;          // 1 generic, 2 MFMA
  int32_t splits;          // token splits per (b, kv head)
  // MFMA kernel: the query heads of a kv head are taken in groups of hg by
  // ngroups work-groups per (b, kv head, split) (the last group may be short)
  int32_t hg, ngroups;
  int64_t chunk;           // tokens per split (multiple of 64)
  int64_t T, Tq;
  uint64_t ws_o, ws_ml;    // workspace offsets: o [B][Hq][S][D], (m, l) [B][Hq][S][2]
  uint64_t workspace_bytes;
};

int make_attn_plan(const Plan& p, int64_t T, const kvq_attn_options* opt, AttnPlan* ap);

// One token per sequence appended by the attention launch itself (decode
// step): mode 1 writes it into the fp16 window, mode 2 encodes it as FP8 (no
// window); the work-group whose token range holds position t writes it before
// it streams the cache.
struct StepAppend {
  const void* k;   // [B][Hkv][1][D] in in_dtype
  const void* v;
  int64_t t;
  int32_t mode;    // 0: none
};
bool mfma_supported(const Plan& p);
// query heads per MFMA work-group (the kernel's PV rows hold at most 16
// (value group, head) pairs, or 32 with two A operands)
int mfma_head_group(const Plan& p);

hipError_t launch_rope_tables(const Plan& p, void* arena, hipStream_t s);
hipError_t launch_fp8_setup(const Plan& p, void* arena, const void* k_new, const void* v_new,
                            int n_new, const float* k_scale, const float* v_scale, bool calibrate,
                            hipStream_t s, const int32_t* new_lens = nullptr);
hipError_t launch_quantize_range(const Plan& p, void* arena, int64_t t0, int n_new, int64_t q_lo,
                                 int64_t q_hi, const void* k_new, const void* v_new, hipStream_t s);
hipError_t launch_ring_write(const Plan& p, void* arena, int64_t t0, int n_new, int64_t w_lo,
                             const void* k_new, const void* v_new, hipStream_t s);
hipError_t launch_dequantize(const Plan& p, const void* arena, int64_t T, float* k_out,
                             float* v_out, hipStream_t s);
// Per-sequence lengths of a ragged (paged) attention call: sequence b holds
// seq_lens[b] + lens_add tokens, clamped to [0, AttnPlan::T].
struct Ragged {
  PageMap pm;
  const int32_t* seq_lens;
  int32_t lens_add;
};

hipError_t launch_attention(const Plan& p, const AttnPlan& ap, const void* arena, const void* q,
                            void* out, float sm_scale, void* ws, hipStream_t s,
                            const StepAppend* app = nullptr, const Ragged* rg = nullptr);

// One-pass append (kvq_append.hip): tokens [t0_b, t0_b + n_b) of every
// sequence, t0_b = seq_lens[b] (t0 when seq_lens is null), n_b = new_lens[b]
// (n when null); quantized units and window slots in one launch.
bool append_fused_supported(const Plan& p);
hipError_t launch_append_fused(const Plan& p, void* arena, const PageMap& pm, const int32_t* seq_lens,
                               const int32_t* new_lens, int64_t t0, int n, int64_t cap, const void* k_new,
                               const void* v_new, hipStream_t s);
// Work-groups per (kv head, side) of the FP8 calibration kernels: each lane
// takes about four 16-byte loads of every sequence (n tokens of D values).
inline unsigned fp8_absmax_blocks(const Plan& p, int64_t n) {
  const int64_t per = p.in_dtype == KVQ_F32 ? 4 : 8;
  int64_t blocks = (n * p.D / per + 4 * 256 - 1) / (4 * 256);
  if (blocks > 512) blocks = 512;
  if (blocks < 1) blocks = 1;
  return (unsigned)blocks;
}
hipError_t launch_fp8_absmax_lens(const Plan& p, const void* k_new, const void* v_new, int n,
                                  const int32_t* new_lens, uint32_t* amax, hipStream_t s);
hipError_t launch_fp8_finalize(const Plan& p, void* arena, const float* k_scale, const float* v_scale,
                               bool calibrate, hipStream_t s);
hipError_t launch_dequantize_paged(const Plan& p, const void* arena, const PageMap& pm,
                                   const int32_t* seq_lens, int64_t max_T, float* k_out, float* v_out,
                                   hipStream_t s);

}  // namespace kvq
