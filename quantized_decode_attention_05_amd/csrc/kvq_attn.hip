// Split-K decode attention over the quantized cache: pass 1 (per token split)
// and pass 2 (merge of the splits).
//
// Per query head h (kv head h / n_rep), over tokens j of one split:
//   logit_j = (q . k_hat_j) * sm_scale      [k_hat rotated by RoPE at position j
//                                             when keys are cached pre-RoPE]
//   running max m, running sum l = sum exp(logit - m), o = sum exp(logit - m) v_hat_j
// ("FP8 KV Cache Quantization: Why Keys Break Before Values", section "Why does
// the K cache break before the V cache?").  Logits are kept in log2 units
// (pre-multiplied by log2 e) so the exponentials are exp2.  Pass 2 combines
// splits with M = max m_s, out = sum_s 2^(m_s - M) o_s / sum_s 2^(m_s - M) l_s.
//
// This file holds the generic kernel: it dequantizes 64-token tiles of any
// supported format into LDS (fp32) and does the dot products on the vector
// ALUs.  The MFMA kernel for the hot formats lives in kvq_attn_mfma.hip.
#include "kvq_internal.h"
#include "kvq_launch.h"
#include "kvq_device.h"

namespace kvq {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kNegBig = -1.0e30f;     // logit of masked / absent tokens
constexpr int kTile = 64;

struct AttnArgs {
  const uint8_t* arena;
  const void* q;
  float* ws_o;
  float* ws_ml;
  int64_t T, Tq, chunk;
  int32_t S;
  float qscale;            // sm_scale * log2(e)
  // ragged / paged calls: sequence b holds seq_lens[b] + lens_add tokens
  // (clamped to [0, T]); tokens are read through the block table
  PageMap pm;
  const int32_t* seq_lens;
  int32_t lens_add;
  // query heads in groups of hg (at most 16) per work-group, ngroups per kv
  // head (grid y = kv head * ngroups + group)
  int32_t hg, ngroups;
};

// Tokens of sequence b and how many of them are quantized.
__device__ __forceinline__ void seq_extent(const Plan& p, const int32_t* seq_lens, int32_t lens_add, int b,
                                           int64_t T_all, int64_t Tq_all, int64_t* T, int64_t* Tq) {
  if (!seq_lens) { *T = T_all; *Tq = Tq_all; return; }
  int64_t t = (int64_t)seq_lens[b] + lens_add;
  t = t < 0 ? 0 : (t > T_all ? T_all : t);
  *T = t;
  *Tq = quantized_tokens(p, t);
}

// cos/sin of position * theta_i from the two-level table (fine: pos mod 32,
// coarse: 32 * floor(pos / 32)), combined with the angle-addition formula.
__device__ __forceinline__ float2 rope_cs(const Plan& p, const float2* tab, int64_t pos, int pair) {
  const int half = p.D >> 1;
  const float2 f = tab[(pos & 31) * half + pair];
  const float2 c = tab[(kVBlock + (pos >> 5)) * half + pair];
  return make_float2(c.x * f.x - c.y * f.y, c.y * f.x + c.x * f.y);
}

template <int D>
__global__ void __launch_bounds__(256) attn_generic(Plan p, AttnArgs a) {
  __shared__ float q_s[16][D];
  __shared__ float kv_s[kTile][D + 1];
  __shared__ float p_s[16][kTile];
  __shared__ float m_s[16], l_s[16], alpha_s[16];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int split = blockIdx.x, kvh = blockIdx.y / a.ngroups, b = blockIdx.z;
  // this work-group's query heads: hb .. hb + n_rep - 1 of the kv head's p.n_rep
  const int hb = (blockIdx.y - kvh * a.ngroups) * a.hg;
  const int n_rep = a.hg < p.n_rep - hb ? a.hg : p.n_rep - hb;
  const int64_t hq0 = (int64_t)b * p.Hq + (int64_t)kvh * p.n_rep + hb;   // first query head
  int64_t T, Tq;
  seq_extent(p, a.seq_lens, a.lens_add, b, a.T, a.Tq, &T, &Tq);
  const int64_t t_begin = (int64_t)split * a.chunk;
  int64_t t_end = t_begin + a.chunk;
  if (t_end > T) t_end = T;

  for (int e = tid; e < n_rep * D; e += 256) {
    const int r = e / D, c = e % D;
    const int64_t qi = (hq0 + r) * D + c;
    q_s[r][c] = load_in(a.q, qi, p.in_dtype) * a.qscale;
  }
  if (tid < 16) { m_s[tid] = kNegBig; l_s[tid] = 0.0f; }

  constexpr int kOut = 16 * D / 256;       // (head, channel) outputs per thread, max
  float o_acc[kOut];
#pragma unroll
  for (int j = 0; j < kOut; ++j) o_acc[j] = 0.0f;
  const float2* rtab = p.pre_rope ? (const float2*)(a.arena + p.rope) : nullptr;
  __syncthreads();

  for (int64_t t0 = t_begin; t0 < t_end; t0 += kTile) {
    // 1. keys of the tile -> LDS (dequantized, rotated)
    for (int e = tid; e < kTile * (D / 2); e += 256) {
      const int tt = e / (D / 2), pr = e % (D / 2);
      const int64_t t = t0 + tt;
      float k0 = 0.0f, k1 = 0.0f;
      if (t < t_end) {
        k0 = dequant_elem<SIDE_K>(p, a.arena, b, kvh, t, 2 * pr, Tq, a.pm);
        k1 = dequant_elem<SIDE_K>(p, a.arena, b, kvh, t, 2 * pr + 1, Tq, a.pm);
        if (rtab) {
          const float2 cs = rope_cs(p, rtab, t, pr);
          const float r0 = k0 * cs.x - k1 * cs.y;
          const float r1 = k0 * cs.y + k1 * cs.x;
          k0 = r0; k1 = r1;
        }
      }
      kv_s[tt][2 * pr] = k0;
      kv_s[tt][2 * pr + 1] = k1;
    }
    __syncthreads();
    // 2. logits
    for (int e = tid; e < n_rep * kTile; e += 256) {
      const int r = e / kTile, tt = e % kTile;
      float acc = 0.0f;
#pragma unroll 8
      for (int c = 0; c < D; ++c) acc += q_s[r][c] * kv_s[tt][c];
      p_s[r][tt] = (t0 + tt < t_end) ? acc : kNegBig;
    }
    __syncthreads();
    // 3. online softmax, one wave per head (heads strided over the 4 waves)
    for (int r = wave; r < n_rep; r += 4) {
      const float x = p_s[r][lane];
      float mx = x;
      for (int off = 32; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off, 64));
      const float m_old = m_s[r];
      const float m_new = fmaxf(m_old, mx);
      const float pv = (x <= kNegBig) ? 0.0f : exp2f(x - m_new);
      float sum = pv;
      for (int off = 32; off > 0; off >>= 1) sum += __shfl_xor(sum, off, 64);
      p_s[r][lane] = pv;
      if (lane == 0) {
        const float alpha = exp2f(m_old - m_new);
        alpha_s[r] = alpha;
        l_s[r] = l_s[r] * alpha + sum;
        m_s[r] = m_new;
      }
    }
    // 4. values of the tile -> LDS (reuses the key buffer)
    __syncthreads();
    for (int e = tid; e < kTile * D; e += 256) {
      const int tt = e / D, c = e % D;
      const int64_t t = t0 + tt;
      kv_s[tt][c] = (t < t_end) ? dequant_elem<SIDE_V>(p, a.arena, b, kvh, t, c, Tq, a.pm) : 0.0f;
    }
    __syncthreads();
    // 5. o = alpha * o + p . V
#pragma unroll
    for (int j = 0; j < kOut; ++j) {
      const int e = tid + 256 * j;
      const int r = e / D, c = e % D;
      if (r < n_rep) {
        float acc = o_acc[j] * alpha_s[r];
#pragma unroll 8
        for (int tt = 0; tt < kTile; ++tt) acc += p_s[r][tt] * kv_s[tt][c];
        o_acc[j] = acc;
      }
    }
    __syncthreads();
  }

  // partials of this split
#pragma unroll
  for (int j = 0; j < kOut; ++j) {
    const int e = tid + 256 * j;
    const int r = e / D, c = e % D;
    if (r < n_rep) {
      const int64_t hq = hq0 + r;
      a.ws_o[(hq * a.S + split) * D + c] = o_acc[j];
    }
  }
  if (tid < n_rep) {
    const int64_t hq = hq0 + tid;
    a.ws_ml[(hq * a.S + split) * 2 + 0] = m_s[tid];
    a.ws_ml[(hq * a.S + split) * 2 + 1] = l_s[tid];
  }
}

// Pass 2: one work-group of four wavefronts per (query head, sequence).
// Wavefront w takes the splits s = w (mod 4) in one pass over their partials,
// keeping a running maximum m, mass l and weighted sum (two channels per lane
// when D = 128) that it rescales whenever the maximum rises, with several
// splits' loads in flight; the four wavefronts' states meet in LDS, rescaled
// to the common maximum.  (Each partial is read once: no separate passes for
// the maximum and the mass.)
__global__ void __launch_bounds__(256) attn_merge(Plan p, const float* ws_o, const float* ws_ml, int S,
                                                  void* out) {
  __shared__ float part[4][128];
  __shared__ float wml[4][2];
  const int hq = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6;
  const int64_t row = (int64_t)b * p.Hq + hq;
  const float* ml = ws_ml + row * S * 2;
  const float* o = ws_o + row * S * p.D;
  const bool d128 = p.D == 128;
  float m = kNegBig, l = 0.0f, a0 = 0.0f, a1 = 0.0f;
#pragma unroll 4
  for (int s = w; s < S; s += 4) {
    const float ms = ml[2 * s], ls = ml[2 * s + 1];
    float v0, v1 = 0.0f;
    if (d128) {
      const float2 v = ((const float2*)(o + (int64_t)s * 128))[lane];
      v0 = v.x;
      v1 = v.y;
    } else {   // D = 64: one channel per lane
      v0 = o[(int64_t)s * 64 + lane];
    }
    const float mn = fmaxf(m, ms);
    const float f0 = exp2f(m - mn), f1 = exp2f(ms - mn);
    l = l * f0 + ls * f1;
    a0 = a0 * f0 + v0 * f1;
    a1 = a1 * f0 + v1 * f1;
    m = mn;
  }
  if (d128) {
    part[w][2 * lane] = a0;
    part[w][2 * lane + 1] = a1;
  } else {
    part[w][lane] = a0;
  }
  if (lane == 0) {
    wml[w][0] = m;
    wml[w][1] = l;
  }
  __syncthreads();
  if (tid < p.D) {
    const float M = fmaxf(fmaxf(wml[0][0], wml[1][0]), fmaxf(wml[2][0], wml[3][0]));
    float L = 0.0f, acc = 0.0f;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const float f = exp2f(wml[k][0] - M);
      L += wml[k][1] * f;
      acc += part[k][tid] * f;
    }
    // a sequence with no tokens (ragged batches) has no mass: output 0
    const float v = L > 0.0f ? acc / L : 0.0f;
    const int64_t oi = row * p.D + tid;
    if (p.out_dtype == KVQ_F32) ((float*)out)[oi] = v;
    else if (p.out_dtype == KVQ_F16) ((_Float16*)out)[oi] = (_Float16)v;
    else {
      const uint32_t u = __float_as_uint(v);
      ((uint16_t*)out)[oi] = (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
    }
  }
}

// ---- planning and launch ----------------------------------------------------------

static int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

int make_attn_plan(const Plan& p, int64_t T, const kvq_attn_options* opt, AttnPlan* ap) {
  int kernel = 0, splits = 0;
  if (opt) {
    for (int i = 0; i < 6; ++i) if (opt->reserved[i]) return KVQ_ERR_INVALID_ARG;
    kernel = opt->kernel;
    splits = opt->num_splits;
    if (kernel < 0 || kernel > 2 || splits < 0) return KVQ_ERR_INVALID_ARG;
  }
  if (kernel == 2 && !mfma_supported(p)) return KVQ_ERR_UNSUPPORTED;
  if (kernel == 0) kernel = mfma_supported(p) ? 2 : 1;
  const int64_t unit = 64;
  const int64_t max_splits = cdiv(T, unit);
  if (kernel == 2) {
    ap->hg = mfma_head_group(p);
  } else {   // the generic kernel holds up to 16 query rows
    const int ng = (int)cdiv(p.n_rep, 16);
    ap->hg = (int)cdiv(p.n_rep, ng);
  }
  ap->ngroups = (int32_t)cdiv(p.n_rep, ap->hg);
  if (splits == 0) {
    // about two work-groups per CU (the MFMA kernel runs at two waves per
    // SIMD), each with a long run of tokens per wavefront
    const int64_t bh = (int64_t)p.B * p.Hkv * ap->ngroups;
    const int64_t want = cdiv(kernel == 2 ? 512 : 1024, bh);
    const int64_t min_tokens = (kernel == 2) ? 512 : 128;
    const int64_t by_len = cdiv(T, min_tokens);
    splits = (int)(want < by_len ? want : by_len);
  }
  if (splits > max_splits) splits = (int)max_splits;
  if (splits < 1) splits = 1;
  if (p.paged) {
    // a split's page ids sit in the MFMA kernel's LDS (kMaxSplitPages entries)
    // (a chunk of c tokens, rounded up to 64, spans at most c / P + 3 pages)
    const int64_t need = cdiv(T, (int64_t)(kMaxSplitPages - 4) * p.P);
    if (splits < need) splits = (int)need;
  }
  // The workspace is sized for the target split count, which never decreases
  // with T; rounding the chunk to whole 64-token units can only lower the count.
  const int64_t target = splits;
  int64_t chunk = cdiv(cdiv(T, splits), unit) * unit;
  splits = (int)cdiv(T, chunk);
  ap->kernel = kernel;
  ap->splits = splits;
  ap->chunk = chunk;
  ap->T = T;
  ap->Tq = quantized_tokens(p, T);
  const uint64_t rows = (uint64_t)p.B * p.Hq * target;
  ap->ws_o = 0;
  ap->ws_ml = (rows * p.D * 4 + 255) & ~(uint64_t)255;
  ap->workspace_bytes = ap->ws_ml + ((rows * 2 * 4 + 255) & ~(uint64_t)255);
  return KVQ_OK;
}

hipError_t launch_attention_mfma(const Plan& p, const AttnPlan& ap, const void* arena, const void* q,
                                 float sm_scale, void* ws, hipStream_t s, const StepAppend* app,
                                 const Ragged* rg);

hipError_t launch_attention(const Plan& p, const AttnPlan& ap, const void* arena, const void* q,
                            void* out, float sm_scale, void* ws, hipStream_t s, const StepAppend* app,
                            const Ragged* rg) {
  if (app && app->mode != 0 && ap.kernel != 2) return hipErrorInvalidValue;   // MFMA kernel only
  if (app && app->mode != 0 && rg) return hipErrorInvalidValue;               // contiguous only
  if (app && app->mode != 0 && ap.ngroups != 1) return hipErrorInvalidValue;   // one writer per (b, kv head)
  float* ws_o = (float*)((uint8_t*)ws + ap.ws_o);
  float* ws_ml = (float*)((uint8_t*)ws + ap.ws_ml);
  if (ap.kernel == 2) {
    hipError_t e = launch_attention_mfma(p, ap, arena, q, sm_scale, ws, s, app, rg);
    if (e != hipSuccess) return e;
  } else {
    AttnArgs a{(const uint8_t*)arena, q, ws_o, ws_ml, ap.T, ap.Tq, ap.chunk, ap.splits,
               sm_scale * kLog2e, rg ? rg->pm : PageMap{nullptr, 0}, rg ? rg->seq_lens : nullptr,
               rg ? rg->lens_add : 0, ap.hg, ap.ngroups};
    dim3 grid(ap.splits, p.Hkv * ap.ngroups, p.B);
    if (p.D == 128) hipLaunchKernelGGL(attn_generic<128>, grid, dim3(256), 0, s, p, a);
    else hipLaunchKernelGGL(attn_generic<64>, grid, dim3(256), 0, s, p, a);
  }
  hipLaunchKernelGGL(attn_merge, dim3(p.Hq, p.B), dim3(256), 0, s, p, (const float*)ws_o,
                     (const float*)ws_ml, ap.splits, out);
  return hipGetLastError();
}

}  // namespace kvq
