// Launchers of the device kernels (internal interface between kvq_api.hip and
// the kernel translation units).
#pragma once
#include "kvq_internal.h"

namespace kvq {

// Plan of one decode-attention call.
struct AttnPlan {
  int32_t kernel;          // 1 generic, 2 MFMA
  int32_t splits;          // token splits per (b, kv head)
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

hipError_t launch_rope_tables(const Plan& p, void* arena, hipStream_t s);
hipError_t launch_fp8_setup(const Plan& p, void* arena, const void* k_new, const void* v_new,
                            int n_new, const float* k_scale, const float* v_scale, bool calibrate,
                            hipStream_t s);
hipError_t launch_quantize_range(const Plan& p, void* arena, int64_t t0, int n_new, int64_t q_lo,
                                 int64_t q_hi, const void* k_new, const void* v_new, hipStream_t s);
hipError_t launch_ring_write(const Plan& p, void* arena, int64_t t0, int n_new, int64_t w_lo,
                             const void* k_new, const void* v_new, hipStream_t s);
hipError_t launch_dequantize(const Plan& p, const void* arena, int64_t T, float* k_out,
                             float* v_out, hipStream_t s);
hipError_t launch_attention(const Plan& p, const AttnPlan& ap, const void* arena, const void* q,
                            void* out, float sm_scale, void* ws, hipStream_t s,
                            const StepAppend* app = nullptr);

}  // namespace kvq
