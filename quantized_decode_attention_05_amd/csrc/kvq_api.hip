// Host side of the C ABI: config validation, arena layout, and the order of
// kernel launches for append / attention / dequantize.  Everything here runs
// on the host; validation finishes before the first HIP call.
#include <mutex>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "kvq_internal.h"
#include "kvq_launch.h"

namespace kvq {

static int64_t gcd64(int64_t a, int64_t b) { while (b) { int64_t t = a % b; a = b; b = t; } return a; }
static int64_t round_up(int64_t x, int64_t m) { return (x + m - 1) / m * m; }
static uint64_t align256(uint64_t x) { return (x + 255) & ~(uint64_t)255; }

static bool is_int(int s) { return s == KVQ_INT_ASYM || s == KVQ_INT_SYM; }

static int check_spec(const kvq_tensor_spec& s, int D) {
  switch (s.scheme) {
    case KVQ_NONE:
      if (s.bits != 16 && s.bits != 32) return KVQ_ERR_INVALID_ARG;
      return KVQ_OK;
    case KVQ_FP8_E4M3:
    case KVQ_FP8_E5M2:
      if (s.bits != 8) return KVQ_ERR_INVALID_ARG;
      return KVQ_OK;
    case KVQ_INT_SYM:
      if (s.bits != 8) return KVQ_ERR_INVALID_ARG;
      break;
    case KVQ_INT_ASYM:
      if (s.bits != 2 && s.bits != 4 && s.bits != 8) return KVQ_ERR_INVALID_ARG;
      break;
    default:
      return KVQ_ERR_INVALID_ARG;
  }
  if (s.axis < KVQ_PER_TENSOR || s.axis > KVQ_PER_TOKEN) return KVQ_ERR_INVALID_ARG;
  if (s.group < 0) return KVQ_ERR_INVALID_ARG;
  if (s.axis == KVQ_PER_CHANNEL && s.group > 65536) return KVQ_ERR_INVALID_ARG;
  if (s.axis == KVQ_PER_TOKEN && s.group != 0) {
    int g = s.group;
    if (g < 8 || g > D || (g & (g - 1)) || D % g) return KVQ_ERR_INVALID_ARG;
  }
  if (s.axis == KVQ_PER_TENSOR && s.group != 0) return KVQ_ERR_INVALID_ARG;
  return KVQ_OK;
}

static int code_bits(const kvq_tensor_spec& s) {
  if (s.scheme == KVQ_NONE) return s.bits;
  return (s.scheme == KVQ_INT_ASYM) ? s.bits : 8;
}

static bool spec_one_shot(const kvq_tensor_spec& s) {
  return is_int(s.scheme) && (s.axis == KVQ_PER_TENSOR || (s.axis == KVQ_PER_CHANNEL && s.group == 0));
}

static int spec_token_group(const kvq_tensor_spec& s) {
  return (is_int(s.scheme) && s.axis == KVQ_PER_CHANNEL && s.group > 0) ? s.group : 1;
}

static void side_meta(const kvq_tensor_spec& s, int D, int64_t Tc, int Hkv, SideFmt* f) {
  f->scheme = s.scheme;
  f->bits = code_bits(s);
  f->axis = s.axis;
  f->group = s.group;
  f->meta_cols = 0;
  f->meta_rows = 0;
  if (is_fp8(s.scheme)) {
    f->meta_rows = 1;
    f->meta_cols = 1;
  } else if (is_int(s.scheme)) {
    if (s.axis == KVQ_PER_TENSOR) { f->meta_rows = 1; f->meta_cols = 1; }
    else if (s.axis == KVQ_PER_CHANNEL) { f->meta_rows = s.group ? Tc / s.group : 1; f->meta_cols = D; }
    else { f->group = s.group ? s.group : D; f->meta_rows = Tc; f->meta_cols = D / f->group; }
  }
  (void)Hkv;
}

int make_plan(const kvq_config* cfg, Plan* p) {
  if (!cfg || !p) return KVQ_ERR_NULL;
  memset(p, 0, sizeof(*p));
  const int D = cfg->head_dim;
  if (cfg->batch < 1 || cfg->num_kv_heads < 1 || cfg->num_q_heads < cfg->num_kv_heads) return KVQ_ERR_INVALID_ARG;
  if (cfg->num_q_heads % cfg->num_kv_heads) return KVQ_ERR_INVALID_ARG;
  if (cfg->num_q_heads / cfg->num_kv_heads > kMaxHeadsPerKv) return KVQ_ERR_INVALID_ARG;
  if (D != 64 && D != 128) return KVQ_ERR_INVALID_ARG;
  if (cfg->max_tokens < 1 || cfg->max_tokens > ((int64_t)1 << 31)) return KVQ_ERR_INVALID_ARG;
  if (cfg->in_dtype < KVQ_F32 || cfg->in_dtype > KVQ_BF16) return KVQ_ERR_INVALID_ARG;
  if (cfg->out_dtype < KVQ_F32 || cfg->out_dtype > KVQ_BF16) return KVQ_ERR_INVALID_ARG;
  if (cfg->meta_dtype != KVQ_F32 && cfg->meta_dtype != KVQ_F16) return KVQ_ERR_INVALID_ARG;
  if (cfg->residual < 0 || cfg->pre_rope_k < 0 || cfg->pre_rope_k > 1) return KVQ_ERR_INVALID_ARG;
  if (cfg->pre_rope_k && !(cfg->rope_base > 0.0f)) return KVQ_ERR_INVALID_ARG;
  int st;
  if ((st = check_spec(cfg->k, D)) != KVQ_OK) return st;
  if ((st = check_spec(cfg->v, D)) != KVQ_OK) return st;
  const int gk = spec_token_group(cfg->k), gv = spec_token_group(cfg->v);
  if (gk > 1 && gv > 1 && gk != gv) return KVQ_ERR_INVALID_ARG;
  const int Gt = gk > 1 ? gk : gv;
  const bool one_shot = spec_one_shot(cfg->k) || spec_one_shot(cfg->v);
  if (one_shot && (cfg->residual != 0 || Gt > 1)) return KVQ_ERR_INVALID_ARG;
  if (cfg->residual % Gt) return KVQ_ERR_INVALID_ARG;
  if (cfg->page_tokens < 0 || cfg->num_pages < 0) return KVQ_ERR_INVALID_ARG;
  const bool paged = cfg->page_tokens > 0;
  if (!paged && cfg->num_pages != 0) return KVQ_ERR_INVALID_ARG;

  p->B = cfg->batch; p->Hq = cfg->num_q_heads; p->Hkv = cfg->num_kv_heads; p->D = D;
  p->n_rep = p->Hq / p->Hkv;
  p->in_dtype = cfg->in_dtype; p->out_dtype = cfg->out_dtype;
  p->R = cfg->residual; p->Gt = Gt;
  p->one_shot = one_shot;
  p->window = (cfg->residual > 0 || Gt > 1);
  p->Rs = p->window ? (int)round_up(cfg->residual + Gt, kRingAlign) : 0;
  p->pre_rope = cfg->pre_rope_k; p->rope_base = cfg->rope_base;
  p->max_tokens = cfg->max_tokens;
  const int64_t lcm = (int64_t)kVBlock / gcd64(kVBlock, Gt) * Gt;
  p->Tc = round_up(cfg->max_tokens, lcm);
  side_meta(cfg->k, D, p->Tc, p->Hkv, &p->k);
  side_meta(cfg->v, D, p->Tc, p->Hkv, &p->v);
  p->k.meta16 = cfg->meta_dtype == KVQ_F16 && is_int(cfg->k.scheme);
  p->v.meta16 = cfg->meta_dtype == KVQ_F16 && is_int(cfg->v.scheme);
  p->k_row_bytes = D * p->k.bits / 8;
  p->v_block_bytes = kVBlock * D * p->v.bits / 8;
  p->v_nblk = p->Tc / kVBlock;

  // the one-pass append kernel: key groups of up to 128 tokens (or none),
  // value groups along channels, no whole-axis / per-tensor group
  const auto fused_side = [&](const kvq_tensor_spec& sp, bool is_v) {
    if (sp.scheme == KVQ_NONE || is_fp8(sp.scheme)) return true;
    if (sp.axis == KVQ_PER_TOKEN) return true;
    return !is_v && sp.axis == KVQ_PER_CHANNEL && sp.group > 0;
  };
  const bool fused_ok = !one_shot && fused_side(cfg->k, false) && fused_side(cfg->v, true) &&
                        (Gt == 1 || (Gt % kVBlock == 0 && Gt <= 128));
  p->unit = fused_ok ? (Gt > kVBlock ? Gt : kVBlock) : 0;

  // token sections: pages of P tokens ([pages][H][P] token rows)
  if (paged) {
    const int P = cfg->page_tokens;
    if (P % kVBlock || P % Gt || P > (1 << 20) || cfg->num_pages < 1) return KVQ_ERR_INVALID_ARG;
    if (!fused_ok) return KVQ_ERR_INVALID_ARG;   // append-only groups within pages
    p->paged = 1;
    p->P = P;
    p->pages = cfg->num_pages;
  } else {
    p->paged = 0;
    p->P = p->Tc;
    p->pages = p->B;
  }
  const uint64_t rows = (uint64_t)p->pages * p->Hkv * p->P;   // token rows of the token sections

  const uint64_t BH = (uint64_t)p->B * p->Hkv;
  uint64_t off = 0;
  auto take = [&](uint64_t bytes) { uint64_t o = off; off = align256(off + bytes); return o; };
  const uint64_t NA = UINT64_MAX;
  p->k.codes = take(rows * p->k_row_bytes);
  auto meta_bytes = [&](const SideFmt& f) -> uint64_t {
    const uint64_t esz = f.meta16 ? 2 : 4;
    if (is_fp8(f.scheme)) return (uint64_t)p->Hkv * 4;
    if (f.axis == KVQ_PER_CHANNEL && f.group > 0) return rows / f.group * f.meta_cols * esz;
    if (f.axis == KVQ_PER_TOKEN) return rows * f.meta_cols * esz;
    return BH * f.meta_rows * f.meta_cols * esz;    // one row per (sequence, head)
  };
  p->k.scale = (p->k.scheme == KVQ_NONE) ? NA : take(meta_bytes(p->k));
  p->k.zero = (p->k.scheme == KVQ_INT_ASYM) ? take(meta_bytes(p->k)) : NA;
  p->v.codes = take(rows / kVBlock * p->v_block_bytes);
  p->v.scale = (p->v.scheme == KVQ_NONE) ? NA : take(meta_bytes(p->v));
  p->v.zero = (p->v.scheme == KVQ_INT_ASYM) ? take(meta_bytes(p->v)) : NA;
  p->ring_k = p->window ? take(BH * p->Rs * D * 2) : NA;
  p->ring_v = p->window ? take(BH * p->Rs * D * 2) : NA;
  p->rope_rows = p->Tc / kVBlock + 1;
  p->rope = p->pre_rope ? take((uint64_t)(kVBlock + p->rope_rows) * (D / 2) * 2 * 4) : NA;
  const bool fp8 = is_fp8(p->k.scheme) || is_fp8(p->v.scheme);
  p->fp8_calib = fp8 ? take((uint64_t)2 * p->Hkv * 4) : NA;
  p->total = off;
  return KVQ_OK;
}

static bool aligned(const void* ptr, uintptr_t a) { return ((uintptr_t)ptr & (a - 1)) == 0; }

static bool log_enabled() {
  static int v = -1;
  if (v < 0) { const char* e = getenv("KVQ_LOG"); v = (e && e[0] == '1') ? 1 : 0; }
  return v == 1;
}

static int hip_status(hipError_t e, const char* where) {
  if (e == hipSuccess) return KVQ_OK;
  if (log_enabled()) fprintf(stderr, "[kvq] %s: HIP error %s (%s)\n", where, hipGetErrorName(e),
                             hipGetErrorString(e));
  return KVQ_ERR_HIP;
}

// Split-K partials of kvq_decode_attention_static: a file-scope device array
// (one copy per GPU, alive until the process ends) in place of a caller
// workspace.  Host code never passes `scratch` itself to a kernel (in host
// code the name is a stand-in, not a device address): each device's address
// is taken once with hipGetSymbolAddress, with that device current, and kept.
static __device__ __align__(256) uint8_t scratch[KVQ_STATIC_WORKSPACE_BYTES];

constexpr int kMaxDevices = 64;
static std::mutex g_scratch_mu;
static void* g_scratch_ptr[kMaxDevices];

// Device address of the current device's scratch array (looked up on the
// first call on that device).
static int scratch_ptr(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e, "kvq_decode_attention_static: hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return KVQ_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr) return hip_status(e == hipSuccess ? hipErrorInvalidSymbol : e,
                                                   "kvq_decode_attention_static: hipGetSymbolAddress");
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return KVQ_OK;
}

}  // namespace kvq

using namespace kvq;

extern "C" {

int kvq_abi_version(void) { return 5; }

const char* kvq_status_string(int s) {
  switch (s) {
    case KVQ_OK: return "ok";
    case KVQ_ERR_INVALID_ARG: return "invalid argument";
    case KVQ_ERR_UNSUPPORTED: return "unsupported operation for this cache format";
    case KVQ_ERR_CAPACITY: return "token capacity exceeded";
    case KVQ_ERR_ALIGN: return "pointer not aligned";
    case KVQ_ERR_NULL: return "required pointer is NULL";
    case KVQ_ERR_WORKSPACE: return "workspace too small";
    case KVQ_ERR_HIP: return "HIP launch failed";
    default: return "unknown status";
  }
}

int kvq_validate_config(const kvq_config* cfg) {
  Plan p;
  return make_plan(cfg, &p);
}

int kvq_arena_layout(const kvq_config* cfg, kvq_layout* out) {
  if (!out) return KVQ_ERR_NULL;
  Plan p;
  int st = make_plan(cfg, &p);
  if (st != KVQ_OK) return st;
  auto sz = [](uint64_t o) { return o == UINT64_MAX ? (size_t)SIZE_MAX : (size_t)o; };
  out->k_codes = sz(p.k.codes); out->k_scale = sz(p.k.scale); out->k_zero = sz(p.k.zero);
  out->v_codes = sz(p.v.codes); out->v_scale = sz(p.v.scale); out->v_zero = sz(p.v.zero);
  out->ring_k = sz(p.ring_k); out->ring_v = sz(p.ring_v);
  out->rope = sz(p.rope); out->fp8_calib = sz(p.fp8_calib);
  out->total_bytes = p.total;
  out->token_capacity = p.Tc;
  out->k_row_bytes = p.k_row_bytes;
  out->v_block_bytes = p.v_block_bytes;
  out->ring_slots = p.Rs;
  out->token_group = p.Gt;
  out->k_meta_cols = p.k.meta_cols;
  out->v_meta_cols = p.v.meta_cols;
  out->page_tokens = p.P;
  out->pages = p.pages;
  return KVQ_OK;
}

int kvq_arena_bytes(const kvq_config* cfg, size_t* bytes) {
  if (!bytes) return KVQ_ERR_NULL;
  Plan p;
  int st = make_plan(cfg, &p);
  if (st != KVQ_OK) return st;
  *bytes = p.total;
  return KVQ_OK;
}

int64_t kvq_quantized_tokens(const kvq_config* cfg, int64_t T) {
  Plan p;
  int st = make_plan(cfg, &p);
  if (st != KVQ_OK) return st;
  if (T < 0 || T > p.max_tokens) return KVQ_ERR_CAPACITY;
  return quantized_tokens(p, T);
}

int kvq_quantize_append(const kvq_config* cfg, void* arena, int64_t t0, int32_t n_new,
                        const void* k_new, const void* v_new, const float* k_scale,
                        const float* v_scale, uint32_t flags, hipStream_t stream) {
  Plan p;
  int st = make_plan(cfg, &p);
  if (st != KVQ_OK) return st;
  if (p.paged) return KVQ_ERR_UNSUPPORTED;                // kvq_paged_quantize_append
  if (flags & ~KVQ_CALIBRATE) return KVQ_ERR_INVALID_ARG;
  if (t0 < 0 || n_new < 0) return KVQ_ERR_INVALID_ARG;
  if (t0 + n_new > p.max_tokens) return KVQ_ERR_CAPACITY;
  const bool fp8 = is_fp8(p.k.scheme) || is_fp8(p.v.scheme);
  if ((flags & KVQ_CALIBRATE) && (!fp8 || t0 != 0)) return KVQ_ERR_INVALID_ARG;
  if ((k_scale || v_scale) && (!fp8 || t0 != 0 || (flags & KVQ_CALIBRATE))) return KVQ_ERR_INVALID_ARG;
  // E5M2 takes no scale
  if ((k_scale && p.k.scheme != KVQ_FP8_E4M3) || (v_scale && p.v.scheme != KVQ_FP8_E4M3))
    return KVQ_ERR_INVALID_ARG;
  if (p.one_shot && t0 != 0) return KVQ_ERR_UNSUPPORTED;
  if (n_new == 0) return KVQ_OK;
  if (!arena || !k_new || !v_new) return KVQ_ERR_NULL;
  if (!aligned(arena, 256) || !aligned(k_new, 16) || !aligned(v_new, 16)) return KVQ_ERR_ALIGN;
  if ((k_scale && !aligned(k_scale, 4)) || (v_scale && !aligned(v_scale, 4))) return KVQ_ERR_ALIGN;

  const int64_t T_old = t0, T_new = t0 + n_new;
  const int64_t q_lo = quantized_tokens(p, T_old), q_hi = quantized_tokens(p, T_new);
  const int64_t w_lo = q_hi > T_old ? q_hi : T_old;
  if (log_enabled())
    fprintf(stderr, "[kvq] append t0=%lld n=%d quantize [%lld,%lld) window [%lld,%lld)\n",
            (long long)t0, n_new, (long long)q_lo, (long long)q_hi, (long long)w_lo, (long long)T_new);
  (void)hipGetLastError();   // drop a sticky error left by unrelated earlier calls
  hipError_t e = hipSuccess;
  if (t0 == 0) {
    if (p.pre_rope && e == hipSuccess) e = launch_rope_tables(p, arena, stream);
    if (fp8 && e == hipSuccess)
      e = launch_fp8_setup(p, arena, k_new, v_new, n_new, k_scale, v_scale,
                           (flags & KVQ_CALIBRATE) != 0, stream);
  }
  if (p.unit) {
    // one pass: quantized units and window slots in one launch
    if ((q_hi > q_lo || T_new > w_lo) && e == hipSuccess)
      e = launch_append_fused(p, arena, PageMap{nullptr, 0}, nullptr, nullptr, t0, n_new, p.max_tokens,
                              k_new, v_new, stream);
  } else {
    if (q_hi > q_lo && e == hipSuccess)
      e = launch_quantize_range(p, arena, t0, n_new, q_lo, q_hi, k_new, v_new, stream);
    if (T_new > w_lo && e == hipSuccess)
      e = launch_ring_write(p, arena, t0, n_new, w_lo, k_new, v_new, stream);
  }
  if (e == hipSuccess) e = hipGetLastError();
  return hip_status(e, "kvq_quantize_append");
}

int kvq_workspace_bytes(const kvq_config* cfg, int64_t T, const kvq_attn_options* opt,
                        size_t* bytes) {
  if (!bytes) return KVQ_ERR_NULL;
  Plan p;
  int st = make_plan(cfg, &p);
  if (st != KVQ_OK) return st;
  if (T < 1 || T > p.max_tokens) return KVQ_ERR_CAPACITY;
  AttnPlan ap;
  st = make_attn_plan(p, T, opt, &ap);
  if (st != KVQ_OK) return st;
  *bytes = ap.workspace_bytes;
  return KVQ_OK;
}

int kvq_decode_attention(const kvq_config* cfg, const void* arena, int64_t T, const void* q,
                         void* out, float sm_scale, void* workspace, size_t workspace_bytes,
                         const kvq_attn_options* opt, hipStream_t stream) {
  Plan p;
  int st = make_plan(cfg, &p);
  if (st != KVQ_OK) return st;
  if (p.paged) return KVQ_ERR_UNSUPPORTED;                // the kvq_paged_ entry points
  if (T < 1 || T > p.max_tokens) return KVQ_ERR_CAPACITY;
  if (!(sm_scale > 0.0f) || sm_scale > 1e30f) return KVQ_ERR_INVALID_ARG;
  AttnPlan ap;
  st = make_attn_plan(p, T, opt, &ap);
  if (st != KVQ_OK) return st;
  if (!arena || !q || !out || (ap.workspace_bytes && !workspace)) return KVQ_ERR_NULL;
  if (!aligned(arena, 256) || !aligned(q, 16) || !aligned(out, 16) ||
      (workspace && !aligned(workspace, 256)))
    return KVQ_ERR_ALIGN;
  if (workspace_bytes < ap.workspace_bytes) return KVQ_ERR_WORKSPACE;
  if (log_enabled())
    fprintf(stderr, "[kvq] attention T=%lld Tq=%lld kernel=%d splits=%d chunk=%lld\n",
            (long long)T, (long long)ap.Tq, ap.kernel, ap.splits, (long long)ap.chunk);
  (void)hipGetLastError();
  hipError_t e = launch_attention(p, ap, arena, q, out, sm_scale, workspace, stream);
  if (e == hipSuccess) e = hipGetLastError();
  return hip_status(e, "kvq_decode_attention");
}

int kvq_decode_attention_static(const kvq_config* cfg, const void* arena, int64_t T, const void* q,
                                void* out, float sm_scale, const kvq_attn_options* opt,
                                hipStream_t stream) {
  Plan p;
  int st = make_plan(cfg, &p);
  if (st != KVQ_OK) return st;
  if (p.paged) return KVQ_ERR_UNSUPPORTED;                // the kvq_paged_ entry points
  if (T < 1 || T > p.max_tokens) return KVQ_ERR_CAPACITY;
  if (!(sm_scale > 0.0f) || sm_scale > 1e30f) return KVQ_ERR_INVALID_ARG;
  AttnPlan ap;
  st = make_attn_plan(p, T, opt, &ap);
  if (st != KVQ_OK) return st;
  if (ap.workspace_bytes > KVQ_STATIC_WORKSPACE_BYTES) return KVQ_ERR_WORKSPACE;
  if (!arena || !q || !out) return KVQ_ERR_NULL;
  if (!aligned(arena, 256) || !aligned(q, 16) || !aligned(out, 16)) return KVQ_ERR_ALIGN;
  void* ws = nullptr;
  if ((st = scratch_ptr(&ws)) != KVQ_OK) return st;
  if (log_enabled())
    fprintf(stderr, "[kvq] attention (static scratch) T=%lld kernel=%d splits=%d bytes=%llu\n",
            (long long)T, ap.kernel, ap.splits, (unsigned long long)ap.workspace_bytes);
  (void)hipGetLastError();
  hipError_t e = launch_attention(p, ap, arena, q, out, sm_scale, ws, stream);
  if (e == hipSuccess) e = hipGetLastError();
  return hip_status(e, "kvq_decode_attention_static");
}

// How a decode step at t0 runs: 1 = new token into the fp16 window inside the
// attention launch, 2 = FP8 codes of the new token inside the attention
// launch, 0 = a separate append first (a fold, or a shape the MFMA kernel
// does not serve).
static int step_mode(const Plan& p, const AttnPlan& ap, int64_t t0) {
  // the appending work-group must be the only reader of its (b, kv head)'s
  // split: not with several head groups
  if (ap.kernel != 2 || ap.ngroups != 1) return 0;
  const int64_t q_lo = quantized_tokens(p, t0), q_hi = quantized_tokens(p, t0 + 1);
  if (q_hi == q_lo) return 1;
  if (is_fp8(p.k.scheme) && is_fp8(p.v.scheme) && !p.window && q_hi == q_lo + 1) return 2;
  return 0;
}

int kvq_decode_step_fused(const kvq_config* cfg, int64_t t0, const kvq_attn_options* opt) {
  Plan p;
  int st = make_plan(cfg, &p);
  if (st != KVQ_OK) return st;
  if (p.paged) return KVQ_ERR_UNSUPPORTED;                // the kvq_paged_ entry points
  if (t0 < 1) return KVQ_ERR_INVALID_ARG;
  if (t0 + 1 > p.max_tokens) return KVQ_ERR_CAPACITY;
  if (p.one_shot) return KVQ_ERR_UNSUPPORTED;
  AttnPlan ap;
  st = make_attn_plan(p, t0 + 1, opt, &ap);
  if (st != KVQ_OK) return st;
  return step_mode(p, ap, t0) != 0 ? 1 : 0;
}

int kvq_decode_step(const kvq_config* cfg, void* arena, int64_t t0, const void* k_new,
                    const void* v_new, const void* q, void* out, float sm_scale, void* workspace,
                    size_t workspace_bytes, const kvq_attn_options* opt, hipStream_t stream) {
  Plan p;
  int st = make_plan(cfg, &p);
  if (st != KVQ_OK) return st;
  if (p.paged) return KVQ_ERR_UNSUPPORTED;                // the kvq_paged_ entry points
  if (t0 < 1) return KVQ_ERR_INVALID_ARG;                 // a cache is started by quantize_append
  if (t0 + 1 > p.max_tokens) return KVQ_ERR_CAPACITY;
  if (p.one_shot) return KVQ_ERR_UNSUPPORTED;
  if (!(sm_scale > 0.0f) || sm_scale > 1e30f) return KVQ_ERR_INVALID_ARG;
  const int64_t T = t0 + 1;
  AttnPlan ap;
  st = make_attn_plan(p, T, opt, &ap);
  if (st != KVQ_OK) return st;
  if (!arena || !k_new || !v_new || !q || !out || (ap.workspace_bytes && !workspace)) return KVQ_ERR_NULL;
  if (!aligned(arena, 256) || !aligned(k_new, 16) || !aligned(v_new, 16) || !aligned(q, 16) ||
      !aligned(out, 16) || (workspace && !aligned(workspace, 256)))
    return KVQ_ERR_ALIGN;
  if (workspace_bytes < ap.workspace_bytes) return KVQ_ERR_WORKSPACE;
  // one launch when the new token needs no fold: it goes to the fp16 window,
  // or (FP8, no window) it is encoded alone with the stored scales
  const int mode = step_mode(p, ap, t0);
  if (log_enabled())
    fprintf(stderr, "[kvq] decode step t0=%lld mode=%d kernel=%d splits=%d\n", (long long)t0, mode,
            ap.kernel, ap.splits);
  if (mode == 0) {
    st = kvq_quantize_append(cfg, arena, t0, 1, k_new, v_new, nullptr, nullptr, 0, stream);
    if (st != KVQ_OK) return st;
    return kvq_decode_attention(cfg, arena, T, q, out, sm_scale, workspace, workspace_bytes, opt, stream);
  }
  (void)hipGetLastError();
  StepAppend app{k_new, v_new, t0, mode};
  hipError_t e = launch_attention(p, ap, arena, q, out, sm_scale, workspace, stream, &app);
  if (e == hipSuccess) e = hipGetLastError();
  return hip_status(e, "kvq_decode_step");
}

int kvq_dequantize(const kvq_config* cfg, const void* arena, int64_t T, float* k_out,
                   float* v_out, hipStream_t stream) {
  Plan p;
  int st = make_plan(cfg, &p);
  if (st != KVQ_OK) return st;
  if (p.paged) return KVQ_ERR_UNSUPPORTED;                // the kvq_paged_ entry points
  if (T < 0 || T > p.max_tokens) return KVQ_ERR_CAPACITY;
  if (T == 0 || (!k_out && !v_out)) return KVQ_OK;
  if (!arena) return KVQ_ERR_NULL;
  if (!aligned(arena, 256) || (k_out && !aligned(k_out, 16)) || (v_out && !aligned(v_out, 16)))
    return KVQ_ERR_ALIGN;
  (void)hipGetLastError();
  hipError_t e = launch_dequantize(p, arena, T, k_out, v_out, stream);
  if (e == hipSuccess) e = hipGetLastError();
  return hip_status(e, "kvq_dequantize");
}

// ---- paged caches --------------------------------------------------------------

static int check_paged(const Plan& p, const int32_t* bt, int32_t max_blocks, const int32_t* lens) {
  if (!p.paged) return KVQ_ERR_UNSUPPORTED;             // the contiguous entry points
  if (!bt || !lens) return KVQ_ERR_NULL;
  if (max_blocks < 1) return KVQ_ERR_INVALID_ARG;
  if (!aligned(bt, 4) || !aligned(lens, 4)) return KVQ_ERR_ALIGN;
  return KVQ_OK;
}

int kvq_paged_quantize_append(const kvq_config* cfg, void* arena, const int32_t* block_table,
                              int32_t max_blocks, const int32_t* seq_lens, const int32_t* new_lens,
                              int32_t n_max, const void* k_new, const void* v_new, const float* k_scale,
                              const float* v_scale, uint32_t flags, hipStream_t stream) {
  Plan p;
  int st = make_plan(cfg, &p);
  if (st != KVQ_OK) return st;
  if ((st = check_paged(p, block_table, max_blocks, seq_lens)) != KVQ_OK) return st;
  if (flags & ~(KVQ_CALIBRATE | KVQ_INIT)) return KVQ_ERR_INVALID_ARG;
  if (n_max < 0 || (int64_t)n_max > p.max_tokens) return KVQ_ERR_INVALID_ARG;
  const bool init = (flags & KVQ_INIT) != 0;
  const bool fp8 = is_fp8(p.k.scheme) || is_fp8(p.v.scheme);
  if ((flags & KVQ_CALIBRATE) && (!fp8 || !init)) return KVQ_ERR_INVALID_ARG;
  if ((k_scale || v_scale) && (!fp8 || !init || (flags & KVQ_CALIBRATE))) return KVQ_ERR_INVALID_ARG;
  if ((k_scale && p.k.scheme != KVQ_FP8_E4M3) || (v_scale && p.v.scheme != KVQ_FP8_E4M3))
    return KVQ_ERR_INVALID_ARG;
  if (!arena) return KVQ_ERR_NULL;
  if (n_max > 0 && (!k_new || !v_new)) return KVQ_ERR_NULL;
  if (!aligned(arena, 256) || (k_new && !aligned(k_new, 16)) || (v_new && !aligned(v_new, 16)) ||
      (new_lens && !aligned(new_lens, 4)) || (k_scale && !aligned(k_scale, 4)) ||
      (v_scale && !aligned(v_scale, 4)))
    return KVQ_ERR_ALIGN;
  int64_t cap = (int64_t)max_blocks * p.P;
  if (cap > p.max_tokens) cap = p.max_tokens;
  if (log_enabled())
    fprintf(stderr, "[kvq] paged append n_max=%d init=%d cap=%lld\n", n_max, (int)init, (long long)cap);
  (void)hipGetLastError();
  hipError_t e = hipSuccess;
  if (init) {
    if (p.pre_rope) e = launch_rope_tables(p, arena, stream);
    if (fp8 && e == hipSuccess)
      e = launch_fp8_setup(p, arena, k_new, v_new, n_max, k_scale, v_scale, (flags & KVQ_CALIBRATE) != 0,
                           stream, new_lens ? new_lens : nullptr);
  }
  if (n_max > 0 && e == hipSuccess)
    e = launch_append_fused(p, arena, PageMap{block_table, max_blocks}, seq_lens, new_lens, 0, n_max, cap,
                            k_new, v_new, stream);
  if (e == hipSuccess) e = hipGetLastError();
  return hip_status(e, "kvq_paged_quantize_append");
}

static int paged_attention(const kvq_config* cfg, const void* arena, const int32_t* block_table,
                           int32_t max_blocks, const int32_t* seq_lens, int64_t max_seq_len, int32_t lens_add,
                           const void* q, void* out, float sm_scale, void* workspace, size_t workspace_bytes,
                           const kvq_attn_options* opt, hipStream_t stream, const char* where) {
  Plan p;
  int st = make_plan(cfg, &p);
  if (st != KVQ_OK) return st;
  if ((st = check_paged(p, block_table, max_blocks, seq_lens)) != KVQ_OK) return st;
  if (max_seq_len < 1 || max_seq_len > p.max_tokens) return KVQ_ERR_CAPACITY;
  if (max_seq_len > (int64_t)max_blocks * p.P) return KVQ_ERR_INVALID_ARG;
  if (!(sm_scale > 0.0f) || sm_scale > 1e30f) return KVQ_ERR_INVALID_ARG;
  AttnPlan ap;
  st = make_attn_plan(p, max_seq_len, opt, &ap);
  if (st != KVQ_OK) return st;
  if (!arena || !q || !out || (ap.workspace_bytes && !workspace)) return KVQ_ERR_NULL;
  if (!aligned(arena, 256) || !aligned(q, 16) || !aligned(out, 16) ||
      (workspace && !aligned(workspace, 256)))
    return KVQ_ERR_ALIGN;
  if (workspace_bytes < ap.workspace_bytes) return KVQ_ERR_WORKSPACE;
  if (log_enabled())
    fprintf(stderr, "[kvq] %s max_T=%lld kernel=%d splits=%d chunk=%lld\n", where, (long long)max_seq_len,
            ap.kernel, ap.splits, (long long)ap.chunk);
  (void)hipGetLastError();
  const Ragged rg{PageMap{block_table, max_blocks}, seq_lens, lens_add};
  hipError_t e = launch_attention(p, ap, arena, q, out, sm_scale, workspace, stream, nullptr, &rg);
  if (e == hipSuccess) e = hipGetLastError();
  return hip_status(e, where);
}

int kvq_paged_decode_attention(const kvq_config* cfg, const void* arena, const int32_t* block_table,
                               int32_t max_blocks, const int32_t* seq_lens, int64_t max_seq_len,
                               const void* q, void* out, float sm_scale, void* workspace,
                               size_t workspace_bytes, const kvq_attn_options* opt, hipStream_t stream) {
  return paged_attention(cfg, arena, block_table, max_blocks, seq_lens, max_seq_len, 0, q, out, sm_scale,
                         workspace, workspace_bytes, opt, stream, "kvq_paged_decode_attention");
}

int kvq_paged_decode_step(const kvq_config* cfg, void* arena, const int32_t* block_table, int32_t max_blocks,
                          const int32_t* seq_lens, int64_t max_seq_len, const void* k_new, const void* v_new,
                          const void* q, void* out, float sm_scale, void* workspace, size_t workspace_bytes,
                          const kvq_attn_options* opt, hipStream_t stream) {
  Plan p;
  int st = make_plan(cfg, &p);
  if (st != KVQ_OK) return st;
  if ((st = check_paged(p, block_table, max_blocks, seq_lens)) != KVQ_OK) return st;
  if (max_seq_len < 1 || max_seq_len > p.max_tokens) return KVQ_ERR_CAPACITY;
  if (!k_new || !v_new || !q || !out) return KVQ_ERR_NULL;
  // validate the attention half before anything is launched
  AttnPlan ap;
  st = make_attn_plan(p, max_seq_len, opt, &ap);
  if (st != KVQ_OK) return st;
  if (max_seq_len > (int64_t)max_blocks * p.P) return KVQ_ERR_INVALID_ARG;
  if (!(sm_scale > 0.0f) || sm_scale > 1e30f) return KVQ_ERR_INVALID_ARG;
  if (ap.workspace_bytes && !workspace) return KVQ_ERR_NULL;
  if (workspace_bytes < ap.workspace_bytes) return KVQ_ERR_WORKSPACE;
  if (!aligned(q, 16) || !aligned(out, 16) || (workspace && !aligned(workspace, 256))) return KVQ_ERR_ALIGN;
  st = kvq_paged_quantize_append(cfg, arena, block_table, max_blocks, seq_lens, nullptr, 1, k_new, v_new,
                                 nullptr, nullptr, 0, stream);
  if (st != KVQ_OK) return st;
  return paged_attention(cfg, arena, block_table, max_blocks, seq_lens, max_seq_len, 1, q, out, sm_scale,
                         workspace, workspace_bytes, opt, stream, "kvq_paged_decode_step");
}

int kvq_paged_dequantize(const kvq_config* cfg, const void* arena, const int32_t* block_table, int32_t max_blocks,
                         const int32_t* seq_lens, int64_t max_seq_len, float* k_out, float* v_out,
                         hipStream_t stream) {
  Plan p;
  int st = make_plan(cfg, &p);
  if (st != KVQ_OK) return st;
  if ((st = check_paged(p, block_table, max_blocks, seq_lens)) != KVQ_OK) return st;
  if (max_seq_len < 0 || max_seq_len > p.max_tokens) return KVQ_ERR_CAPACITY;
  if (max_seq_len > (int64_t)max_blocks * p.P) return KVQ_ERR_INVALID_ARG;
  if (max_seq_len == 0 || (!k_out && !v_out)) return KVQ_OK;
  if (!arena) return KVQ_ERR_NULL;
  if (!aligned(arena, 256) || (k_out && !aligned(k_out, 16)) || (v_out && !aligned(v_out, 16)))
    return KVQ_ERR_ALIGN;
  (void)hipGetLastError();
  hipError_t e = launch_dequantize_paged(p, arena, PageMap{block_table, max_blocks}, seq_lens, max_seq_len,
                                         k_out, v_out, stream);
  if (e == hipSuccess) e = hipGetLastError();
  return hip_status(e, "kvq_paged_dequantize");
}

}  // extern "C"
