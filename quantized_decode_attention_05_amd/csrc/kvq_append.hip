// One-pass quantize-append: the tokens an append call quantizes are read
// once, reduced to their scales and zero-points, encoded and packed by the
// same work-group, in contiguous and paged caches alike.
//
// What is computed is the pages' recipe, element for element as the
// two-kernel path and the oracle do it:
//  - keys per channel over groups of Gt tokens and values per token over
//    groups of channels ("KV Cache Quantization: Why Keys and Values Need
//    Different Axes", section "Why does per-token key quantization destroy
//    accuracy?": min-max with scale = max(max-min, 1e-8)/(2^b-1), code =
//    clamp(rint((x-min)/scale)), zero-point = min), symmetric absmax INT8
//    ("FP8 KV Cache Quantization: Why Keys Break Before Values", section "Why
//    does the K cache break before the V cache?"), FP8 with per-head scales
//    (same page, "Why do per-tensor scales waste bits on the K cache?");
//  - the most recent tokens kept in an fp16 window and folded into the
//    quantized cache a block of Gt tokens at a time ("...Need Different
//    Axes", section "What should I actually turn on in production?"); the
//    key groups of a paged cache sit inside its fixed-size pages ("FP8 KV
//    Cache Quantization...", section "Should you quantize keys pre-RoPE or
//    post-RoPE?").
//
// Work split.  A quantize unit is one key group of one (sequence, kv head)
// (U = Gt tokens; 32 when keys have no token groups), a ring unit is up to 32
// window tokens.  Each sequence's range comes from device data (the lengths
// of a ragged batch) or from the call's uniform t0, so units a sequence does
// not need exit at once.  Three kernels share the work items and outputs:
//  - append_kivi_h<W> (fp16-staged caches, per-channel INT keys, per-token
//    INT values, D = 128): W = U / 32 wavefronts per unit, each holding 32
//    tokens as packed fp16 pairs (lane: 8 channels of 8 tokens), key-channel
//    min / max across the lane's tokens, the token rows (permlane swaps) and,
//    for W > 1, the unit's wavefronts (LDS); value groups within the lane's
//    channels and its neighbours; codes by a division-free exact rule;
//  - append_wave<KS, VS, KAX> (32-token units of other formats, D = 128): the
//    same lane layout in fp32, one instance per scheme;
//  - append_units<D, U> (everything else): one 256-thread work-group per
//    unit, a thread owning 16-byte granules; key channels reduce across the
//    four wavefronts through LDS, value codes go through LDS so that each
//    thread assembles whole words of the 32-token value block layout.
// In every kernel a value word (8 tokens of one channel) has one writer, so
// no two threads write one byte; whole units of new tokens issue all their
// loads before using any.
//
// Built with -ffp-contract=off: every step rounds once, in the listings' order.
#include "kvq_internal.h"
#include "kvq_launch.h"
#include "kvq_device.h"

namespace kvq {

struct AppendArgs {
  uint8_t* arena;
  const void* k_in;          // [B][Hkv][n][D] in in_dtype
  const void* v_in;
  PageMap pm;
  const int32_t* seq_lens;   // device [B]: tokens held before the call (nullptr: t0 for all)
  const int32_t* new_lens;   // device [B]: tokens appended (nullptr: n for all)
  int64_t t0;
  int32_t n;                 // tokens per sequence in the input rows
  int64_t cap;               // a sequence's range must end at or before this
  int32_t units_q;           // work-groups per (sequence, head) that take quantize units
  int32_t phases;            // bit 0: quantize units run, bit 1: ring units run
  int32_t x0;                // index of the launch's first work item (unit, or wavefront slot of append_kivi_h)
  float one;                 // 1.0f (an operand the compiler cannot fold)
};

constexpr int kAppendThreads = 256;

// 8 staged values of channels c0..c0+7 of token t of (b, h): from the fp16
// ring for tokens appended by earlier calls (t < t0), else from the input,
// rounded through fp16 when the cache keeps a window.
template <int SIDE, int D>
__device__ __forceinline__ void load_granule(const Plan& p, const AppendArgs& a, int b, int h, int64_t t,
                                             int64_t t0, int c0, float* x) {
  const int64_t bh = (int64_t)b * p.Hkv + h;
  if (t < t0) {
    const int64_t slot = t % p.Rs;
    if (SIDE == SIDE_K) {
      const uint4 r = *(const uint4*)(a.arena + p.ring_k + ((bh * p.Rs + slot) * D + c0) * 2);
      const uint32_t w[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        x[2 * j] = (float)__builtin_bit_cast(_Float16, (uint16_t)(w[j] & 0xFFFFu));
        x[2 * j + 1] = (float)__builtin_bit_cast(_Float16, (uint16_t)(w[j] >> 16));
      }
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) x[j] = ring_v_elem(p, a.arena, bh, slot, c0 + j);
    }
    return;
  }
  const void* in = SIDE == SIDE_K ? a.k_in : a.v_in;
  const int64_t e = (bh * a.n + (t - t0)) * D + c0;
  if (p.in_dtype == KVQ_F32) {
    const float4 u = ((const float4*)in)[e / 4], v = ((const float4*)in)[e / 4 + 1];
    x[0] = u.x; x[1] = u.y; x[2] = u.z; x[3] = u.w; x[4] = v.x; x[5] = v.y; x[6] = v.z; x[7] = v.w;
  } else {
    const uint4 r = ((const uint4*)in)[e / 8];
    const uint32_t w[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (p.in_dtype == KVQ_F16) {
        x[2 * j] = (float)__builtin_bit_cast(_Float16, (uint16_t)(w[j] & 0xFFFFu));
        x[2 * j + 1] = (float)__builtin_bit_cast(_Float16, (uint16_t)(w[j] >> 16));
      } else {
        x[2 * j] = __uint_as_float(w[j] << 16);
        x[2 * j + 1] = __uint_as_float(w[j] & 0xFFFF0000u);
      }
    }
  }
  if (p.window) {
#pragma unroll
    for (int j = 0; j < 8; ++j) x[j] = stage_f16(x[j]);
  }
}

// 1 / s within one ulp (the hardware reciprocal) where that is a normal
// number, else NaN (then every quotient by s takes the division).
__device__ __forceinline__ float recip_or_nan(float s) {
  return fabsf(s) < 0x1p125f ? __builtin_amdgcn_rcpf(s) : __builtin_nanf("");
}

// rint of the correctly rounded quotient d / s, given rs = recip_or_nan(s)
// and m = (qmax + 1) * 2^-20 for codes clamped to [-qmax, qmax] or [0, qmax].
// q = d * rs lies within |d / s| * 1.5 * 2^-23 of d / s (rs within one ulp,
// the product rounded once) and the rounded quotient within |d / s| * 2^-24,
// so where |d / s| <= qmax + 1 the two lie within m / 2 of each other and
// round to the same integer unless a half-integer lies within m of q.  The
// test is exact there (fract(q) and its distance to 1/2 round no bits) and
// false for NaN and infinity; beyond qmax + 1 both clamp alike.  Only the
// rare quotients the test rejects are divided; the division sits behind a
// side effect so that it is never evaluated speculatively.
__device__ __forceinline__ float rint_quot(float d, float s, float rs, float m) {
  const float q = d * rs;
  if (__builtin_expect(fabsf(__builtin_amdgcn_fractf(q) - 0.5f) > m, 1)) return __builtin_rintf(q);
  asm volatile("" ::: "memory");
  return __builtin_rintf(d / s);
}

// Keys and values of N granules (channels c0 .. c0 + 7 of tokens t1 + ts i,
// i < N), all from the input (t1 >= t0), staged as load_granule stages them.
// Every load is issued before any value is used, so the memory latency is
// waited for once per batch, not once per granule.
template <int D, int N>
__device__ __forceinline__ void load_kv_granules(const Plan& p, const AppendArgs& a, int b, int h, int64_t t1, int ts,
                                                 int64_t t0, int c0, float (&xk)[N][8], float (&xv)[N][8]) {
  const int64_t bh = (int64_t)b * p.Hkv + h;
  const int64_t e0 = (bh * a.n + (t1 - t0)) * D + c0;
  if (p.in_dtype == KVQ_F32) {
    const float4* kp = (const float4*)a.k_in + e0 / 4;
    const float4* vp = (const float4*)a.v_in + e0 / 4;
    float4 fk[2 * N], fv[2 * N];
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int64_t o = (int64_t)i * ts * (D / 4);
      fk[2 * i] = kp[o]; fk[2 * i + 1] = kp[o + 1];
      fv[2 * i] = vp[o]; fv[2 * i + 1] = vp[o + 1];
    }
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const float ck[8] = {fk[2 * i].x, fk[2 * i].y, fk[2 * i].z, fk[2 * i].w,
                           fk[2 * i + 1].x, fk[2 * i + 1].y, fk[2 * i + 1].z, fk[2 * i + 1].w};
      const float cv[8] = {fv[2 * i].x, fv[2 * i].y, fv[2 * i].z, fv[2 * i].w,
                           fv[2 * i + 1].x, fv[2 * i + 1].y, fv[2 * i + 1].z, fv[2 * i + 1].w};
#pragma unroll
      for (int j = 0; j < 8; ++j) { xk[i][j] = ck[j]; xv[i][j] = cv[j]; }
    }
  } else {
    const uint4* kp = (const uint4*)a.k_in + e0 / 8;
    const uint4* vp = (const uint4*)a.v_in + e0 / 8;
    uint4 rk[N], rv[N];
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int64_t o = (int64_t)i * ts * (D / 8);
      rk[i] = kp[o];
      rv[i] = vp[o];
    }
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const uint32_t wk[4] = {rk[i].x, rk[i].y, rk[i].z, rk[i].w}, wv[4] = {rv[i].x, rv[i].y, rv[i].z, rv[i].w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (p.in_dtype == KVQ_F16) {
          xk[i][2 * j] = (float)__builtin_bit_cast(_Float16, (uint16_t)(wk[j] & 0xFFFFu));
          xk[i][2 * j + 1] = (float)__builtin_bit_cast(_Float16, (uint16_t)(wk[j] >> 16));
          xv[i][2 * j] = (float)__builtin_bit_cast(_Float16, (uint16_t)(wv[j] & 0xFFFFu));
          xv[i][2 * j + 1] = (float)__builtin_bit_cast(_Float16, (uint16_t)(wv[j] >> 16));
        } else {
          xk[i][2 * j] = __uint_as_float(wk[j] << 16);
          xk[i][2 * j + 1] = __uint_as_float(wk[j] & 0xFFFF0000u);
          xv[i][2 * j] = __uint_as_float(wv[j] << 16);
          xv[i][2 * j + 1] = __uint_as_float(wv[j] & 0xFFFF0000u);
        }
      }
    }
  }
  if (p.window) {
#pragma unroll
    for (int i = 0; i < N; ++i)
#pragma unroll
      for (int j = 0; j < 8; ++j) { xk[i][j] = stage_f16(xk[i][j]); xv[i][j] = stage_f16(xv[i][j]); }
  }
}

// 1 / s rounded once for an FP8 per-head scale s in [2^-80, 2^80], else NaN
// (then fp8_quot divides).
__device__ __forceinline__ float fp8_recip(float s) {
  return fabsf(s) >= 0x1p-80f && fabsf(s) <= 0x1p80f ? 1.0f / s : __builtin_nanf("");
}

// x / s rounded once, given ys = fp8_recip(s): x is first clamped to
// +-2^17 s (exact; every FP8 code saturates beyond 2^17), then q0 = x ys,
// r = x - s q0 (exact by FMA) and q0 + r ys rounded once is the correctly
// rounded quotient (the correction step of Markstein's division).  With s in
// [2^-80, 2^80] every step stays in the normal range wherever the quotient
// reaches an FP8 rounding boundary (|x / s| >= 2^-17); below that the code
// is a signed zero whatever the last bits.  The correction never changes the
// quotient's sign, but for x = -0 it yields +0 (r = +0, +0 + -0 = +0), so the
// sign is taken from x: FP8 codes keep the sign of zero.  ys = NaN (a scale
// outside that range, uniform per head) divides.
__device__ __forceinline__ float fp8_quot(float x, float s, float ys) {
  if (ys != ys) return x / s;
  const float lim = s * 0x1p17f;
  const float xc = fminf(fmaxf(x, -lim), lim);
  const float q0 = xc * ys;
  const float r = __builtin_fmaf(-q0, s, xc);
  return __builtin_copysignf(__builtin_fmaf(r, ys, q0), xc);
}

// FP8 codes of four values x0..x3 under a per-head scale s whose reciprocal
// ys = fp8_recip(s) is finite, packed in one dword (value k in byte k): the
// quotient of fp8_quot without its division fallback, saturated at the
// format's largest finite value by a median (which keeps the sign, also of
// zero), then converted two at a time by the instruction that rounds to
// nearest, ties to even (the rounding of e4m3_encode / e5m2_encode).
template <bool E5>
__device__ __forceinline__ float fp8_sat_quot(float x, float s, float ys) {
  const float lim = s * 0x1p17f;
  const float xc = __builtin_amdgcn_fmed3f(x, -lim, lim);
  const float q0 = xc * ys;
  const float r = __builtin_fmaf(-q0, s, xc);
  const float q = __builtin_copysignf(__builtin_fmaf(r, ys, q0), xc);
  const float mx = E5 ? kE5M2Max : kE4M3Max;
  return __builtin_amdgcn_fmed3f(q, -mx, mx);
}
template <bool E5>
__device__ __forceinline__ uint32_t fp8_pack4(float x0, float x1, float x2, float x3, float s, float ys) {
  const float q0 = fp8_sat_quot<E5>(x0, s, ys), q1 = fp8_sat_quot<E5>(x1, s, ys);
  const float q2 = fp8_sat_quot<E5>(x2, s, ys), q3 = fp8_sat_quot<E5>(x3, s, ys);
  if constexpr (E5) {
    const int w = __builtin_amdgcn_cvt_pk_bf8_f32(q0, q1, 0, false);
    return (uint32_t)__builtin_amdgcn_cvt_pk_bf8_f32(q2, q3, w, true);
  } else {
    const int w = __builtin_amdgcn_cvt_pk_fp8_f32(q0, q1, 0, false);
    return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(q2, q3, w, true);
  }
}

// Code field (masked to the format's bits) of value x under scale s (rs =
// recip_or_nan(s) for INT schemes, fp8_recip(s) for FP8) and zero z; S >= 0
// fixes the scheme at compile time.
template <int S>
__device__ __forceinline__ uint32_t code_t(const SideFmt& f, float x, float s, float rs, float z) {
  switch (S >= 0 ? S : f.scheme) {
    case KVQ_NONE:
      if (f.bits == 16) { const _Float16 hv = (_Float16)x; return (uint32_t)__builtin_bit_cast(uint16_t, hv); }
      return __float_as_uint(x);
    case KVQ_FP8_E4M3: return e4m3_encode(fp8_quot(x, s, rs));
    case KVQ_FP8_E5M2: return e5m2_encode(fp8_quot(x, s, rs));
    case KVQ_INT_SYM: {
      const float r = fminf(fmaxf(rint_quot(x, s, rs, 128.0f * 0x1p-20f), -127.0f), 127.0f);
      return (uint32_t)(int32_t)r & 0xFFu;
    }
    default: {
      const float qmax = (float)((1 << f.bits) - 1);
      const float r = fminf(fmaxf(rint_quot(x - z, s, rs, (qmax + 1.0f) * 0x1p-20f), 0.0f), qmax);
      return (uint32_t)r;
    }
  }
}

// Min / max (absmax in mx for symmetric groups) of the lanes l ^ m for masks
// m in [from, to) (powers of two): lanes of one group of channels.
__device__ __forceinline__ void lane_minmax(float& mn, float& mx, int from, int to) {
  for (int m = from; m < to; m <<= 1) {
    mn = fminf(mn, __shfl_xor(mn, m, 64));
    mx = fmaxf(mx, __shfl_xor(mx, m, 64));
  }
}

// Write the 8 codes of one granule (channels 8 cb .. 8 cb + 7) into a key row.
__device__ __forceinline__ void write_k_granule(uint8_t* row, int cb, int bits, const uint32_t* c) {
  // 2- and 4-bit codes come from the asymmetric encoders, clamped to
  // [0, 2^bits - 1]: no mask before they are shifted into place
  if (bits == 2) {
    uint32_t v = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) v |= c[j] << (2 * j);
    ((uint16_t*)row)[cb] = (uint16_t)v;
  } else if (bits == 4) {
    uint32_t v = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) v |= c[j] << (4 * j);
    ((uint32_t*)row)[cb] = v;
  } else if (bits == 8) {
    uint32_t lo = 0, hi = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) { lo |= (c[j] & 255u) << (8 * j); hi |= (c[j + 4] & 255u) << (8 * j); }
    ((uint2*)row)[cb] = make_uint2(lo, hi);
  } else if (bits == 16) {
    ((uint4*)row)[cb] = make_uint4(c[0] | (c[1] << 16), c[2] | (c[3] << 16), c[4] | (c[5] << 16),
                                   c[6] | (c[7] << 16));
  } else {
    ((uint4*)row)[2 * cb] = make_uint4(c[0], c[1], c[2], c[3]);
    ((uint4*)row)[2 * cb + 1] = make_uint4(c[4], c[5], c[6], c[7]);
  }
}

// Store a value word (8 codes of `bits` bits, tokens 0..7 of the word in
// lo | hi) at wp; codes of tokens outside `valid` keep the bits already there.
__device__ __forceinline__ void store_vword(uint8_t* wp, int bits, uint32_t valid, uint32_t lo, uint32_t hi) {
  if (bits == 2) {
    if (valid != 0xFFu) {
      uint32_t keep = 0;
#pragma unroll
      for (int i = 0; i < 8; ++i) if (!((valid >> i) & 1u)) keep |= 3u << (2 * i);
      lo |= (uint32_t)*(const uint16_t*)wp & keep;
    }
    *(uint16_t*)wp = (uint16_t)lo;
  } else if (bits == 4) {
    if (valid != 0xFFu) {
      uint32_t keep = 0;
#pragma unroll
      for (int i = 0; i < 8; ++i) if (!((valid >> i) & 1u)) keep |= 15u << (4 * i);
      lo |= *(const uint32_t*)wp & keep;
    }
    *(uint32_t*)wp = lo;
  } else {
    if (valid != 0xFFu) {
      const uint2 old = *(const uint2*)wp;
      uint32_t klo = 0, khi = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (!((valid >> i) & 1u)) klo |= 0xFFu << (8 * i);
        if (!((valid >> (i + 4)) & 1u)) khi |= 0xFFu << (8 * i);
      }
      lo |= old.x & klo;
      hi |= old.y & khi;
    }
    *(uint2*)wp = make_uint2(lo, hi);
  }
}

// A 16-byte granule of a 16-bit input (8 values) as fp32, staged as
// load_granule stages it.
__device__ __forceinline__ void unpack16(const Plan& p, const uint4& r, float (&x)[8]) {
  const uint32_t w[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    if (p.in_dtype == KVQ_F16) {
      x[2 * j] = (float)__builtin_bit_cast(_Float16, (uint16_t)(w[j] & 0xFFFFu));
      x[2 * j + 1] = (float)__builtin_bit_cast(_Float16, (uint16_t)(w[j] >> 16));
    } else {
      x[2 * j] = __uint_as_float(w[j] << 16);
      x[2 * j + 1] = __uint_as_float(w[j] & 0xFFFF0000u);
    }
  }
  if (p.window) {
#pragma unroll
    for (int j = 0; j < 8; ++j) x[j] = stage_f16(x[j]);
  }
}

template <int D>
struct AppendShared {
  float red_mn[4][D], red_mx[4][D];   // per-wavefront partial min / max of key channels
  float ks[D], kz[D], kr[D];           // the key group's stored scale / zero-point, recip_or_nan(scale)
  uint32_t vt[D][33];                  // value codes of a 32-token block, channel-major
};

// Tokens [v_lo, v_hi) of the unit [u0, u0 + U): keys then values.
template <int D, int U>
__device__ __forceinline__ void quantize_unit(const Plan& p, const AppendArgs& a, AppendShared<D>& sh, int b, int h,
                              int64_t t0, int64_t u0, int64_t v_lo, int64_t v_hi) {
  constexpr int CB = D / 8, TPP = kAppendThreads / CB;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int cb = tid % CB, tq = tid / CB;
  const int64_t bh = (int64_t)b * p.Hkv + h;
  const SideFmt& fk = p.k;
  const bool k_int = fk.scheme == KVQ_INT_ASYM || fk.scheme == KVQ_INT_SYM;
  const bool k_sym = fk.scheme == KVQ_INT_SYM;

  // A whole unit of new tokens of a 16-bit input (every unit of such a
  // prefill) issues all its key and value loads at once; the value granules
  // are the same tokens as the key granules (value block sb, granule i is
  // key granule sb * (32 / TPP) + i) and wait as raw words.
  constexpr int NG = U / TPP;              // granules per thread
  const bool batch = u0 >= t0 && v_lo == u0 && v_hi == u0 + U && p.in_dtype != KVQ_F32;
  uint4 rv[NG];

  // ---- keys --------------------------------------------------------------------
  {
    float x[NG][8];
    if (batch) {
      const int64_t e0 = (bh * a.n + (u0 + tq - t0)) * D + 8 * cb;
      const uint4* kp = (const uint4*)a.k_in + e0 / 8;
      const uint4* vp = (const uint4*)a.v_in + e0 / 8;
      uint4 rk[NG];
#pragma unroll
      for (int i = 0; i < NG; ++i) {
        rk[i] = kp[(int64_t)i * TPP * (D / 8)];
        rv[i] = vp[(int64_t)i * TPP * (D / 8)];
      }
#pragma unroll
      for (int i = 0; i < NG; ++i) unpack16(p, rk[i], x[i]);
    } else {
#pragma unroll
      for (int i = 0; i < NG; ++i) {
        const int64_t t = u0 + tq + TPP * i;
        if (t >= v_lo && t < v_hi) load_granule<SIDE_K, D>(p, a, b, h, t, t0, 8 * cb, x[i]);
        else {
#pragma unroll
          for (int j = 0; j < 8; ++j) x[i][j] = 0.0f;
        }
      }
    }
    const bool per_channel = k_int && fk.axis == KVQ_PER_CHANNEL;
    if (per_channel) {
      // the unit is one whole key group: every token is valid
      float mn[8], mx[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) { mn[j] = INFINITY; mx[j] = -INFINITY; }
#pragma unroll
      for (int i = 0; i < NG; ++i) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          if (k_sym) mx[j] = fmaxf(mx[j], fabsf(x[i][j]));
          else { mn[j] = fminf(mn[j], x[i][j]); mx[j] = fmaxf(mx[j], x[i][j]); }
        }
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) lane_minmax(mn[j], mx[j], CB, 64);
      if (lane < CB) {
#pragma unroll
        for (int j = 0; j < 8; ++j) { sh.red_mn[wave][8 * cb + j] = mn[j]; sh.red_mx[wave][8 * cb + j] = mx[j]; }
      }
      __syncthreads();
      if (tid < D) {
        float m0 = sh.red_mn[0][tid], m1 = sh.red_mx[0][tid];
#pragma unroll
        for (int w = 1; w < 4; ++w) { m0 = fminf(m0, sh.red_mn[w][tid]); m1 = fmaxf(m1, sh.red_mx[w][tid]); }
        float s, z;
        meta_values(fk, m0, m1, &s, &z);
        sh.ks[tid] = s;
        sh.kz[tid] = z;
        sh.kr[tid] = recip_or_nan(s);
        const int32_t pg = page_of(p, a.pm, b, u0);
        if (pg >= 0) store_meta_values(fk, a.arena, meta_index_row(p, fk, bh, h, row_of(p, pg, h, u0), tid), s, z);
      }
      __syncthreads();
    }
    const float fp8s = is_fp8(fk.scheme) ? ((const float*)(a.arena + fk.scale))[h] : 1.0f;
    const float fp8r = fp8_recip(fp8s);
#pragma unroll
    for (int i = 0; i < NG; ++i) {
      const int64_t t = u0 + tq + TPP * i;
      const bool ok = t >= v_lo && t < v_hi;
      float s[8], z[8], rs[8];
      if (per_channel) {
#pragma unroll
        for (int j = 0; j < 8; ++j) { s[j] = sh.ks[8 * cb + j]; z[j] = sh.kz[8 * cb + j]; rs[j] = sh.kr[8 * cb + j]; }
      } else if (k_int) {
        // per-token groups of Gc channels: Gc / 8 neighbouring lanes
        float mn = INFINITY, mx = -INFINITY;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          if (k_sym) mx = fmaxf(mx, fabsf(x[i][j]));
          else { mn = fminf(mn, x[i][j]); mx = fmaxf(mx, x[i][j]); }
        }
        lane_minmax(mn, mx, 1, fk.group / 8);
        float sv, zv;
        meta_values(fk, mn, mx, &sv, &zv);
        const float rv = recip_or_nan(sv);
#pragma unroll
        for (int j = 0; j < 8; ++j) { s[j] = sv; z[j] = zv; rs[j] = rv; }
        if (ok && (cb % (fk.group / 8)) == 0) {
          const int32_t pg = page_of(p, a.pm, b, t);
          if (pg >= 0) store_meta_values(fk, a.arena, meta_index_row(p, fk, bh, h, row_of(p, pg, h, t), 8 * cb), sv, zv);
        }
      } else {
#pragma unroll
        for (int j = 0; j < 8; ++j) { s[j] = fp8s; z[j] = 0.0f; rs[j] = fp8r; }
      }
      if (!ok) continue;
      const int32_t pg = page_of(p, a.pm, b, t);
      if (pg < 0) continue;
      uint32_t c[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) c[j] = code_t<-1>(fk, x[i][j], s[j], rs[j], z[j]);
      write_k_granule(a.arena + fk.codes + row_of(p, pg, h, t) * p.k_row_bytes, cb, fk.bits, c);
    }
  }

  // ---- values, 32-token blocks -----------------------------------------------------
  const SideFmt& fv = p.v;
  const bool v_int = fv.scheme == KVQ_INT_ASYM || fv.scheme == KVQ_INT_SYM;
  const bool v_sym = fv.scheme == KVQ_INT_SYM;
  const float vfp8s = is_fp8(fv.scheme) ? ((const float*)(a.arena + fv.scale))[h] : 1.0f;
  const uint32_t vmask = fv.bits >= 32 ? 0xFFFFFFFFu : ((1u << fv.bits) - 1);
#pragma unroll
  for (int sb = 0; sb < U / 32; ++sb) {
    const int64_t ts = u0 + 32 * sb;
    if (ts + 32 <= v_lo || ts >= v_hi) continue;
    constexpr int NVG = 32 / TPP;          // granules per thread per block
#pragma unroll
    for (int i = 0; i < NVG; ++i) {
      const int tk = tq + TPP * i;          // token within the block
      const int64_t t = ts + tk;
      const bool ok = t >= v_lo && t < v_hi;
      float x[8];
      if (batch) unpack16(p, rv[sb * NVG + i], x);
      else if (ok) load_granule<SIDE_V, D>(p, a, b, h, t, t0, 8 * cb, x);
      else {
#pragma unroll
        for (int j = 0; j < 8; ++j) x[j] = 0.0f;
      }
      float sv = vfp8s, zv = 0.0f;
      if (v_int) {
        float mn = INFINITY, mx = -INFINITY;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          if (v_sym) mx = fmaxf(mx, fabsf(x[j]));
          else { mn = fminf(mn, x[j]); mx = fmaxf(mx, x[j]); }
        }
        lane_minmax(mn, mx, 1, fv.group / 8);
        meta_values(fv, mn, mx, &sv, &zv);
        if (ok && (cb % (fv.group / 8)) == 0) {
          const int32_t pg = page_of(p, a.pm, b, t);
          if (pg >= 0) store_meta_values(fv, a.arena, meta_index_row(p, fv, bh, h, row_of(p, pg, h, t), 8 * cb), sv, zv);
        }
      }
      const float rv = v_int ? recip_or_nan(sv) : fp8_recip(sv);
#pragma unroll
      for (int j = 0; j < 8; ++j) sh.vt[8 * cb + j][tk] = ok ? (code_t<-1>(fv, x[j], sv, rv, zv) & vmask) : 0u;
    }
    __syncthreads();
    // words of the block: word (lane L = 16 g + n, i) = channel 16 i + n, tokens 8 g .. 8 g + 7
    const int32_t pg = page_of(p, a.pm, b, ts);
    if (pg >= 0) {
      uint8_t* blk = a.arena + fv.codes + (row_of(p, pg, h, ts) >> 5) * p.v_block_bytes;
      constexpr int NW = 64 * (D / 16);
      for (int w = tid; w < NW; w += kAppendThreads) {
        const int L = w / (D / 16), i = w % (D / 16);
        const int g = L >> 4, nn = L & 15, c = 16 * i + nn;
        uint32_t valid = 0;
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          const int64_t t = ts + 8 * g + k;
          valid |= (t >= v_lo && t < v_hi ? 1u : 0u) << k;
        }
        if (!valid) continue;
        uint8_t* wp = blk + (int64_t)w * fv.bits;
        const uint32_t* cv = &sh.vt[c][8 * g];
        if (fv.bits <= 4) {
          uint32_t v = 0, keep = 0;
#pragma unroll
          for (int k = 0; k < 8; ++k) {
            v |= cv[k] << (k * fv.bits);
            if (!((valid >> k) & 1u)) keep |= vmask << (k * fv.bits);
          }
          if (fv.bits == 2) {
            if (keep) v |= (uint32_t)*(const uint16_t*)wp & keep;
            *(uint16_t*)wp = (uint16_t)v;
          } else {
            if (keep) v |= *(const uint32_t*)wp & keep;
            *(uint32_t*)wp = v;
          }
        } else if (fv.bits == 8) {
          uint32_t lo = 0, hi = 0;
#pragma unroll
          for (int k = 0; k < 4; ++k) { lo |= cv[k] << (8 * k); hi |= cv[k + 4] << (8 * k); }
          if (valid != 0xFFu) {
            const uint2 old = *(const uint2*)wp;
            uint32_t klo = 0, khi = 0;
#pragma unroll
            for (int k = 0; k < 4; ++k) {
              if (!((valid >> k) & 1u)) klo |= 0xFFu << (8 * k);
              if (!((valid >> (k + 4)) & 1u)) khi |= 0xFFu << (8 * k);
            }
            lo |= old.x & klo;
            hi |= old.y & khi;
          }
          *(uint2*)wp = make_uint2(lo, hi);
        } else {
          // 16- and 32-bit values: element stores of the valid tokens
#pragma unroll
          for (int k = 0; k < 8; ++k) {
            if (!((valid >> k) & 1u)) continue;
            if (fv.bits == 16) ((uint16_t*)wp)[k] = (uint16_t)cv[k];
            else ((uint32_t*)wp)[k] = cv[k];
          }
        }
      }
    }
    __syncthreads();
  }
}

// Window tokens [w0, w1) (inside one 32-token block, all from this call's
// input) into their ring slots t mod Rs, as fp16.
template <int D>
__device__ __forceinline__ void ring_unit(const Plan& p, const AppendArgs& a, int b, int h, int64_t t0, int64_t w0,
                          int64_t w1) {
  constexpr int CB = D / 8, TPP = kAppendThreads / CB;
  const int tid = threadIdx.x, cb = tid % CB, tq = tid / CB;
  const int64_t bh = (int64_t)b * p.Hkv + h;
  const int64_t blk = w0 & ~(int64_t)31;
  const int rblock = kVBlock * D * 2;
#pragma unroll
  for (int i = 0; i < 32 / TPP; ++i) {
    const int64_t t = blk + tq + TPP * i;
    if (t < w0 || t >= w1) continue;
    const int64_t slot = t % p.Rs;
    float xk[8], xv[8];
    load_granule<SIDE_K, D>(p, a, b, h, t, t0, 8 * cb, xk);
    load_granule<SIDE_V, D>(p, a, b, h, t, t0, 8 * cb, xv);
    uint32_t u[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const _Float16 lo = (_Float16)xk[2 * j], hi = (_Float16)xk[2 * j + 1];
      u[j] = (uint32_t)__builtin_bit_cast(uint16_t, lo) | ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
    }
    *(uint4*)(a.arena + p.ring_k + ((bh * p.Rs + slot) * D + 8 * cb) * 2) = make_uint4(u[0], u[1], u[2], u[3]);
    uint8_t* base = a.arena + p.ring_v + (uint64_t)bh * (p.Rs / kVBlock) * rblock;
#pragma unroll
    for (int j = 0; j < 8; ++j)
      ((_Float16*)(base + vblock_word_byte(slot, 8 * cb + j, D, 16, rblock)))[slot & 7] = (_Float16)xv[j];
  }
}

template <int D, int U>
__global__ void __launch_bounds__(kAppendThreads) append_units(Plan p, AppendArgs a) {
  __shared__ AppendShared<D> sh;
  const int h = blockIdx.y, b = blockIdx.z;
  const int64_t t0 = a.seq_lens ? (int64_t)a.seq_lens[b] : a.t0;
  int64_t nb = a.new_lens ? (int64_t)a.new_lens[b] : (int64_t)a.n;
  if (nb > a.n) nb = a.n;
  if (t0 < 0 || nb <= 0 || t0 + nb > a.cap) return;    // nothing, or a range past the capacity
  const int64_t q_lo = quantized_tokens(p, t0), q_hi = quantized_tokens(p, t0 + nb);
  const int64_t u_first = (q_lo / U) * U;
  const int64_t n_qu = q_hi > q_lo ? (q_hi - u_first + U - 1) / U : 0;
  const int64_t x = (int64_t)blockIdx.x + a.x0;
  if (x < a.units_q) {
    if (x >= n_qu || !(a.phases & 1)) return;
    const int64_t u0 = u_first + x * U;
    quantize_unit<D, U>(p, a, sh, b, h, t0, u0, u0 > q_lo ? u0 : q_lo, u0 + U < q_hi ? u0 + U : q_hi);
  } else {
    if (!(a.phases & 2)) return;
    const int64_t w_lo = q_hi > t0 ? q_hi : t0, w_hi = t0 + nb;
    const int64_t r0 = (w_lo & ~(int64_t)31) + 32 * (x - a.units_q);
    if (w_hi <= w_lo || r0 >= w_hi) return;
    ring_unit<D>(p, a, b, h, t0, r0 > w_lo ? r0 : w_lo, r0 + 32 < w_hi ? r0 + 32 : w_hi);
  }
}

// ---- one wavefront per 32-token unit ---------------------------------------------
// Units of 32 tokens (key groups of 32, or no key groups) with D = 128 and
// value codes of at most 8 bits: a wavefront owns a whole unit, lane (cb, r)
// the 8 channels 8 cb .. 8 cb + 7 of the 8 consecutive tokens 8 r .. 8 r + 7.
// Key-channel min / max: the lane's 8 tokens, then lanes l ^ 16 and l ^ 32
// (the other token rows) through permlane swaps; per-token groups: the lanes
// holding the group's channels (neighbours).  A value word (8 consecutive
// tokens of one channel) forms inside one lane, so nothing goes through LDS
// and the wavefronts of a work-group never wait for each other.

// min / max over lanes n, n ^ 16, n ^ 32, n ^ 48 (the swaps return the
// partner's value in one half and the lane's own in the other)
__device__ __forceinline__ void rows_minmax(float& mn, float& mx) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(mn), __float_as_uint(mn), false, false);
  mn = fminf(__uint_as_float(r[0]), __uint_as_float(r[1]));
  r = __builtin_amdgcn_permlane16_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
  mx = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
  r = __builtin_amdgcn_permlane32_swap(__float_as_uint(mn), __float_as_uint(mn), false, false);
  mn = fminf(__uint_as_float(r[0]), __uint_as_float(r[1]));
  r = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
  mx = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// Scale / zero-point (and recip_or_nan of the scale) of per-token groups of
// Gc channels for the 8 tokens of a lane: min / max over its 8 channels, then
// over the Gc / 8 neighbouring lanes.
template <int S>
__device__ __forceinline__ void token_groups(const SideFmt& f, const float (&x)[8][8], float (&s)[8],
                                             float (&z)[8], float (&rs)[8]) {
  const bool sym = (S >= 0 ? S : f.scheme) == KVQ_INT_SYM;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    float mn = INFINITY, mx = -INFINITY;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (sym) mx = fmaxf(mx, fabsf(x[i][j]));
      else { mn = fminf(mn, x[i][j]); mx = fmaxf(mx, x[i][j]); }
    }
    lane_minmax(mn, mx, 1, f.group / 8);
    meta_values(f, mn, mx, &s[i], &z[i]);
    rs[i] = recip_or_nan(s[i]);
  }
}

// Window tokens of one 32-token block (ring unit xr of (b, h)) into their
// ring slots: lane (cb, r) moves channels 8 cb .. 8 cb + 7 of tokens 8 r ..
// 8 r + 7 of the block.
__device__ __forceinline__ void wave_ring_block(const Plan& p, const AppendArgs& a, int b, int h, int64_t t0,
                                                int64_t nb, int64_t q_hi, int64_t xr, int cb, int r) {
  constexpr int D = 128;
  const int64_t bh = (int64_t)b * p.Hkv + h;
  const int64_t w_lo = q_hi > t0 ? q_hi : t0, w_hi = t0 + nb;
  const int64_t blk = (w_lo & ~(int64_t)31) + 32 * xr;
  if (w_hi <= w_lo || blk >= w_hi) return;
  const int rblock = kVBlock * D * 2;
  uint8_t* vbase = a.arena + p.ring_v + (uint64_t)bh * (p.Rs / kVBlock) * rblock;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int64_t t = blk + 8 * r + i;
    if (t < w_lo || t >= w_hi) continue;
    const int64_t slot = t % p.Rs;
    float xk[8], xv[8];
    load_granule<SIDE_K, D>(p, a, b, h, t, t0, 8 * cb, xk);
    load_granule<SIDE_V, D>(p, a, b, h, t, t0, 8 * cb, xv);
    uint32_t u[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const _Float16 lo = (_Float16)xk[2 * j], hi = (_Float16)xk[2 * j + 1];
      u[j] = (uint32_t)__builtin_bit_cast(uint16_t, lo) | ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
    }
    *(uint4*)(a.arena + p.ring_k + ((bh * p.Rs + slot) * D + 8 * cb) * 2) = make_uint4(u[0], u[1], u[2], u[3]);
#pragma unroll
    for (int j = 0; j < 8; ++j)
      ((_Float16*)(vbase + vblock_word_byte(slot, 8 * cb + j, D, 16, rblock)))[slot & 7] = (_Float16)xv[j];
  }
}

// KS / VS >= 0 fix the key / value scheme and KAX >= 0 the key axis at
// compile time, so that an instance holds only its own encoder (the whole
// unrolled body then stays in the instruction cache).
// FP8 key rows of a wavefront's unit: token 8 r + i of lane (cb, r), channels
// 8 cb .. 8 cb + 7 (byte j of the row's 8-byte granule cb is channel 8 cb + j).
template <bool E5>
__device__ __forceinline__ void fp8_rows(const float (&x)[8][8], const bool (&ok)[8], float s, float ys,
                                         uint8_t* row0, int64_t row_bytes, int cb) {
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    if (!ok[i]) continue;
    const uint32_t lo = fp8_pack4<E5>(x[i][0], x[i][1], x[i][2], x[i][3], s, ys);
    const uint32_t hi = fp8_pack4<E5>(x[i][4], x[i][5], x[i][6], x[i][7], s, ys);
    ((uint2*)(row0 + i * row_bytes))[cb] = make_uint2(lo, hi);
  }
}

// FP8 value words of a wavefront's unit: channel 8 cb + j of tokens 8 r ..
// 8 r + 7 (byte i of the word is token 8 r + i), in the 32-token block layout
// (store_vword keeps the bytes of tokens outside `valid`).
template <bool E5, int D>
__device__ __forceinline__ void fp8_vwords(const float (&x)[8][8], uint32_t valid, float s, float ys, uint8_t* blk,
                                           int cb, int r) {
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int c = 8 * cb + j, n = c & 15, iw = c >> 4;
    uint8_t* wp = blk + (int64_t)((16 * r + n) * (D / 16) + iw) * 8;
    const uint32_t lo = fp8_pack4<E5>(x[0][j], x[1][j], x[2][j], x[3][j], s, ys);
    const uint32_t hi = fp8_pack4<E5>(x[4][j], x[5][j], x[6][j], x[7][j], s, ys);
    store_vword(wp, 8, valid, lo, hi);
  }
}

template <int KS, int VS, int KAX>
__global__ void __launch_bounds__(256) append_wave(Plan p, AppendArgs a) {
  constexpr int D = 128;
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int h = blockIdx.y, b = blockIdx.z;
  const int cb = lane & 15, r = lane >> 4;        // channels 8 cb.., tokens 8 r..
  const int64_t t0 = a.seq_lens ? (int64_t)a.seq_lens[b] : a.t0;
  int64_t nb = a.new_lens ? (int64_t)a.new_lens[b] : (int64_t)a.n;
  if (nb > a.n) nb = a.n;
  if (t0 < 0 || nb <= 0 || t0 + nb > a.cap) return;
  const int64_t q_lo = quantized_tokens(p, t0), q_hi = quantized_tokens(p, t0 + nb);
  const int64_t u_first = q_lo & ~(int64_t)31;
  const int64_t n_qu = q_hi > q_lo ? (q_hi - u_first + 31) / 32 : 0;
  const int64_t x = (int64_t)blockIdx.x * 4 + wave + a.x0;
  const int64_t bh = (int64_t)b * p.Hkv + h;

  if (x >= a.units_q) {
    if (a.phases & 2) wave_ring_block(p, a, b, h, t0, nb, q_hi, x - a.units_q, cb, r);
    return;
  }
  if (!(a.phases & 1) || x >= n_qu) return;
  const int64_t u0 = u_first + 32 * x;
  const int64_t v_lo = u0 > q_lo ? u0 : q_lo, v_hi = u0 + 32 < q_hi ? u0 + 32 : q_hi;
  const int32_t pg = page_of(p, a.pm, b, u0);     // the unit's page (units never straddle pages)
  bool ok[8];
  float xk[8][8], xv[8][8];
  if (u0 >= t0 && v_lo == u0 && v_hi == u0 + 32) {
    // a whole unit of new tokens (every unit of a prefill)
#pragma unroll
    for (int i = 0; i < 8; ++i) ok[i] = true;
    load_kv_granules<D, 8>(p, a, b, h, u0 + 8 * r, 1, t0, 8 * cb, xk, xv);
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int64_t t = u0 + 8 * r + i;
      ok[i] = t >= v_lo && t < v_hi;
      if (ok[i]) {
        load_granule<SIDE_K, D>(p, a, b, h, t, t0, 8 * cb, xk[i]);
        load_granule<SIDE_V, D>(p, a, b, h, t, t0, 8 * cb, xv[i]);
      } else {
#pragma unroll
        for (int j = 0; j < 8; ++j) { xk[i][j] = 0.0f; xv[i][j] = 0.0f; }
      }
    }
  }

  // ---- keys ----
  const SideFmt& fk = p.k;
  const int ksch = KS >= 0 ? KS : fk.scheme, kax = KAX >= 0 ? KAX : fk.axis;
  const bool k_int = ksch == KVQ_INT_ASYM || ksch == KVQ_INT_SYM;
  uint8_t* krow0 = pg >= 0 ? a.arena + fk.codes + row_of(p, pg, h, u0 + 8 * r) * p.k_row_bytes : nullptr;
  if (k_int && kax == KVQ_PER_CHANNEL) {
    // one whole key group of 32 tokens: every token valid
    const bool sym = ksch == KVQ_INT_SYM;
    float sc[8], zc[8], rc[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      float mn = INFINITY, mx = -INFINITY;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        if (sym) mx = fmaxf(mx, fabsf(xk[i][j]));
        else { mn = fminf(mn, xk[i][j]); mx = fmaxf(mx, xk[i][j]); }
      }
      rows_minmax(mn, mx);
      meta_values(fk, mn, mx, &sc[j], &zc[j]);
      rc[j] = recip_or_nan(sc[j]);
      if (r == 0 && pg >= 0)
        store_meta_values(fk, a.arena, meta_index_row(p, fk, bh, h, row_of(p, pg, h, u0), 8 * cb + j), sc[j], zc[j]);
    }
    if (pg >= 0) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        uint32_t c[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) c[j] = code_t<KS>(fk, xk[i][j], sc[j], rc[j], zc[j]);
        write_k_granule(krow0 + i * p.k_row_bytes, cb, fk.bits, c);
      }
    }
  } else {
    float st[8], zt[8], rt[8];
    if (k_int) {
      token_groups<KS>(fk, xk, st, zt, rt);
    } else {
      const float s8 = is_fp8(ksch) ? ((const float*)(a.arena + fk.scale))[h] : 1.0f;
      const float r8 = fp8_recip(s8);
#pragma unroll
      for (int i = 0; i < 8; ++i) { st[i] = s8; zt[i] = 0.0f; rt[i] = r8; }
    }
    if (pg >= 0 && is_fp8(ksch) && rt[0] == rt[0]) {
      // FP8 under an in-range scale (uniform per head): eight codes per token
      // row from four conversions, no division
      if (ksch == KVQ_FP8_E5M2) fp8_rows<true>(xk, ok, st[0], rt[0], krow0, p.k_row_bytes, cb);
      else fp8_rows<false>(xk, ok, st[0], rt[0], krow0, p.k_row_bytes, cb);
    } else if (pg >= 0) {
      // per-token key groups: the first lane of each group stores its
      // metadata; the lane's tokens are consecutive token rows
      const int gl = k_int ? fk.group / 8 : 1;
      const bool klane = k_int && (cb % gl) == 0;
      const int64_t kmi0 = klane ? row_of(p, pg, h, u0 + 8 * r) * fk.meta_cols + cb / gl : 0;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        if (!ok[i]) continue;
        if (klane) store_meta_values(fk, a.arena, kmi0 + i * fk.meta_cols, st[i], zt[i]);
        uint32_t c[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) c[j] = code_t<KS>(fk, xk[i][j], st[i], rt[i], zt[i]);
        write_k_granule(krow0 + i * p.k_row_bytes, cb, fk.bits, c);
      }
    }
  }

  // ---- values: per-token groups, words of 8 tokens formed in the lane ----
  const SideFmt& fv = p.v;
  const int vsch = VS >= 0 ? VS : fv.scheme;
  const bool v_int = vsch == KVQ_INT_ASYM || vsch == KVQ_INT_SYM;
  float vs[8], vz[8], vr[8];
  if (v_int) {
    token_groups<VS>(fv, xv, vs, vz, vr);
    const int gl = fv.group / 8;
    if (pg >= 0 && (cb % gl) == 0) {
      const int64_t vmi0 = row_of(p, pg, h, u0 + 8 * r) * fv.meta_cols + cb / gl;
#pragma unroll
      for (int i = 0; i < 8; ++i)
        if (ok[i]) store_meta_values(fv, a.arena, vmi0 + i * fv.meta_cols, vs[i], vz[i]);
    }
  } else {
    const float s8 = is_fp8(vsch) ? ((const float*)(a.arena + fv.scale))[h] : 1.0f;
    const float r8 = fp8_recip(s8);
#pragma unroll
    for (int i = 0; i < 8; ++i) { vs[i] = s8; vz[i] = 0.0f; vr[i] = r8; }
  }
  if (pg < 0) return;
  uint32_t valid = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) valid |= (ok[i] ? 1u : 0u) << i;
  if (!valid) return;
  const int bits = fv.bits;
  const uint32_t mask = (1u << bits) - 1;
  uint8_t* blk = a.arena + fv.codes + (row_of(p, pg, h, u0) >> 5) * p.v_block_bytes;
  if (is_fp8(vsch) && vr[0] == vr[0]) {
    // FP8 under an in-range scale: a word of eight tokens from four conversions
    if (vsch == KVQ_FP8_E5M2) fp8_vwords<true, D>(xv, valid, vs[0], vr[0], blk, cb, r);
    else fp8_vwords<false, D>(xv, valid, vs[0], vr[0], blk, cb, r);
    return;
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int c = 8 * cb + j, n = c & 15, iw = c >> 4;
    uint8_t* wp = blk + (int64_t)((16 * r + n) * (D / 16) + iw) * bits;
    uint32_t lo = 0, hi = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t code = code_t<VS>(fv, xv[i][j], vs[i], vr[i], vz[i]) & mask;
      const int bit = i * bits;
      if (bit < 32) lo |= code << bit;
      else hi |= code << (bit - 32);
    }
    store_vword(wp, bits, valid, lo, hi);
  }
}

// ---- fp16-staged caches: keys per channel, values per token ------------------
// When every value is rounded to fp16 before it is quantized (caches with an
// fp16 window, or fp16 inputs), a wavefront holds its unit as packed fp16
// pairs: half the registers of fp32 values, so twice the wavefronts fit per
// SIMD, and min / max take one packed instruction per two values.  x - z is
// taken from the fp16 value by one mixed-precision FMA (x * 1 - z rounds
// once, as the subtraction does), and the correctly rounded quotient comes
// from a correctly rounded reciprocal and one FMA correction (asym_codes8_h).
// Same lane layout, work split and outputs as append_wave.

typedef _Float16 h2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ h2_t as_h2(uint32_t u) { return __builtin_bit_cast(h2_t, u); }
__device__ __forceinline__ uint32_t as_u32(h2_t v) { return __builtin_bit_cast(uint32_t, v); }
__device__ __forceinline__ uint32_t pk_h(float lo, float hi) {
  const h2_t v = {(_Float16)lo, (_Float16)hi};
  return as_u32(v);
}

// Channels c0 .. c0 + 7 of token t as four fp16 pairs: from the ring for
// tokens appended by earlier calls (t < t0), else the input rounded to fp16.
template <int SIDE>
__device__ __forceinline__ void load_granule_h(const Plan& p, const AppendArgs& a, int b, int h, int64_t t,
                                               int64_t t0, int c0, uint32_t (&w)[4]) {
  constexpr int D = 128;
  const int64_t bh = (int64_t)b * p.Hkv + h;
  if (t < t0) {
    const int64_t slot = t % p.Rs;
    if (SIDE == SIDE_K) {
      const uint4 r = *(const uint4*)(a.arena + p.ring_k + ((bh * p.Rs + slot) * D + c0) * 2);
      w[0] = r.x; w[1] = r.y; w[2] = r.z; w[3] = r.w;
    } else {
      const int rblock = kVBlock * D * 2;
      const uint8_t* base = a.arena + p.ring_v + (uint64_t)bh * (p.Rs / kVBlock) * rblock;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t lo = ((const uint16_t*)(base + vblock_word_byte(slot, c0 + 2 * j, D, 16, rblock)))[slot & 7];
        const uint32_t hi = ((const uint16_t*)(base + vblock_word_byte(slot, c0 + 2 * j + 1, D, 16, rblock)))[slot & 7];
        w[j] = lo | (hi << 16);
      }
    }
    return;
  }
  const void* in = SIDE == SIDE_K ? a.k_in : a.v_in;
  const int64_t e = (bh * a.n + (t - t0)) * D + c0;
  if (p.in_dtype == KVQ_F16) {
    const uint4 r = ((const uint4*)in)[e / 8];
    w[0] = r.x; w[1] = r.y; w[2] = r.z; w[3] = r.w;
  } else if (p.in_dtype == KVQ_F32) {
    const float4 u = ((const float4*)in)[e / 4], v = ((const float4*)in)[e / 4 + 1];
    w[0] = pk_h(u.x, u.y); w[1] = pk_h(u.z, u.w); w[2] = pk_h(v.x, v.y); w[3] = pk_h(v.z, v.w);
  } else {
    const uint4 r = ((const uint4*)in)[e / 8];
    const uint32_t q[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) w[j] = pk_h(__uint_as_float(q[j] << 16), __uint_as_float(q[j] & 0xFFFF0000u));
  }
}

// Tokens u0 + 8 r + i (i = 0..7), channels 8 cb .. 8 cb + 7, all from the
// input (u0 >= t0), as fp16 pairs.  Every load is issued before any value is
// used, so a wavefront waits for its unit's memory once, not once per granule.
__device__ __forceinline__ void load_unit_h(const Plan& p, const AppendArgs& a, int b, int h, int64_t u0, int64_t t0,
                                            int cb, int r, uint32_t (&hk)[8][4], uint32_t (&hv)[8][4]) {
  constexpr int D = 128;
  const int64_t bh = (int64_t)b * p.Hkv + h;
  const int64_t e0 = (bh * a.n + (u0 + 8 * r - t0)) * D + 8 * cb;   // element of (token u0 + 8 r, channel 8 cb)
  if (p.in_dtype == KVQ_F32) {
    // two 16-byte loads per granule: keys, then values
#pragma unroll
    for (int side = 0; side < 2; ++side) {
      const float4* src = (const float4*)(side ? a.v_in : a.k_in) + e0 / 4;
      float4 f[16];
#pragma unroll
      for (int i = 0; i < 8; ++i) { f[2 * i] = src[i * (D / 4)]; f[2 * i + 1] = src[i * (D / 4) + 1]; }
      uint32_t (&w)[8][4] = side ? hv : hk;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        w[i][0] = pk_h(f[2 * i].x, f[2 * i].y);
        w[i][1] = pk_h(f[2 * i].z, f[2 * i].w);
        w[i][2] = pk_h(f[2 * i + 1].x, f[2 * i + 1].y);
        w[i][3] = pk_h(f[2 * i + 1].z, f[2 * i + 1].w);
      }
    }
    return;
  }
  const uint4* ks = (const uint4*)a.k_in + e0 / 8;
  const uint4* vs = (const uint4*)a.v_in + e0 / 8;
  uint4 rk[8], rv[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) { rk[i] = ks[i * (D / 8)]; rv[i] = vs[i * (D / 8)]; }
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint32_t qk[4] = {rk[i].x, rk[i].y, rk[i].z, rk[i].w}, qv[4] = {rv[i].x, rv[i].y, rv[i].z, rv[i].w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (p.in_dtype == KVQ_F16) {
        hk[i][j] = qk[j];
        hv[i][j] = qv[j];
      } else {
        hk[i][j] = pk_h(__uint_as_float(qk[j] << 16), __uint_as_float(qk[j] & 0xFFFF0000u));
        hv[i][j] = pk_h(__uint_as_float(qv[j] << 16), __uint_as_float(qv[j] & 0xFFFF0000u));
      }
    }
  }
}

// Asymmetric codes of eight fp16 values xh[k] under scales s[k] and zero-
// points z[k], given ys[k] = 1 / s[k] rounded once (the IEEE division).
// d = x - z is one mixed-precision FMA from the fp16 value (one = 1.0 from the
// host, kept opaque so that the FMA is not turned back into a conversion and
// a subtraction); both rounding steps of the quotient are exact-rounding
// steps: q0 = d * y, r = d - s q0 (exact by FMA), q = q0 + r y rounded once is
// the correctly rounded d / s (the correction step of Markstein's division,
// valid for a correctly rounded reciprocal).  For fp16-staged groups d is 0
// or at least 2^-24, s lies in [1e-8 / 255, 2^16] and d = 0 whenever s is at
// the floor, so no step leaves the normal range.  No branch, no division per
// element.
__device__ __forceinline__ void asym_codes8_h(const _Float16 (&xh)[8], const float (&s)[8], const float (&ys)[8],
                                              const float (&z)[8], float one, float qmax, uint32_t (&c)[8]) {
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const float d = __builtin_fmaf((float)xh[k], one, -z[k]);
    const float q0 = d * ys[k];
    const float r = __builtin_fmaf(-q0, s[k], d);
    const float q = __builtin_fmaf(r, ys[k], q0);
    c[k] = (uint32_t)__builtin_amdgcn_fmed3f(__builtin_rintf(q), 0.0f, qmax);
  }
}

// Group metadata of fp16-staged values without an IEEE division.  A group's
// range d lies in [1e-8, 2^17] (fp16 magnitudes are at most 65504; the floor
// is 1e-8) unless the input overflowed fp16 (then it is infinite or NaN):
//   s = RN(d / qmax) by the correction step with yq = RN(1 / qmax), which
//   gives the correctly rounded quotient for every fp32 d in [1e-8, 2^17]
//   and qmax in {3, 15, 127, 255} (checked exhaustively against the
//   division); an infinite or NaN d takes d * yq, which equals d / qmax there;
//   1 / s by the hardware reciprocal and one Newton step with FMA, the
//   correctly rounded reciprocal for every s in [2^-40, 2^21) (checked for
//   every significand; the scales here lie in [2^-35, 2^16]); beyond, the
//   bare reciprocal (1 / inf = 0).
__device__ __forceinline__ float div_qmax(float d, float qm, float yq) {
  const float q0 = d * yq;
  const float r = __builtin_fmaf(-q0, qm, d);
  const float q = __builtin_fmaf(r, yq, q0);
  return d <= 0x1p17f ? q : q0;
}
__device__ __forceinline__ float recip_rn(float s) {
  const float y0 = __builtin_amdgcn_rcpf(s);
  const float e = __builtin_fmaf(-s, y0, 1.0f);
  const float y1 = __builtin_fmaf(e, y0, y0);
  return s < 0x1p21f ? y1 : y0;
}
// meta_values for fp16-staged groups (same results), yq = RN(1 / qmax) of
// the side (1 / 127 for symmetric groups).
__device__ __forceinline__ void meta_values_h(const SideFmt& f, float mn, float mx, float yq, float* s, float* z) {
  if (f.scheme == KVQ_INT_ASYM) {
    const float qm = (float)((1 << f.bits) - 1);
    if (f.meta16) {
      const _Float16 zh = f16_directed(mn, false);
      const float sc = div_qmax(fmaxf(mx - (float)zh, 1e-8f), qm, yq);
      *s = (float)f16_directed(sc, true);
      *z = (float)zh;
    } else {
      *s = div_qmax(fmaxf(mx - mn, 1e-8f), qm, yq);
      *z = mn;
    }
  } else {
    const float sc = div_qmax(fmaxf(mx, 1e-8f), 127.0f, yq);
    *s = f.meta16 ? (float)f16_directed(sc, true) : sc;
    *z = 0.0f;
  }
}

__device__ __forceinline__ void rows_minmax_h(uint32_t& mn, uint32_t& mx) {
  auto r = __builtin_amdgcn_permlane16_swap(mn, mn, false, false);
  mn = as_u32(__builtin_elementwise_min(as_h2(r[0]), as_h2(r[1])));
  r = __builtin_amdgcn_permlane16_swap(mx, mx, false, false);
  mx = as_u32(__builtin_elementwise_max(as_h2(r[0]), as_h2(r[1])));
  r = __builtin_amdgcn_permlane32_swap(mn, mn, false, false);
  mn = as_u32(__builtin_elementwise_min(as_h2(r[0]), as_h2(r[1])));
  r = __builtin_amdgcn_permlane32_swap(mx, mx, false, false);
  mx = as_u32(__builtin_elementwise_max(as_h2(r[0]), as_h2(r[1])));
}

// W = Gt / 32 wavefronts share one key group (unit) of Gt tokens; wavefront
// s of a unit takes its tokens 32 s .. 32 s + 31.  With W > 1 the key
// channels' min / max combine across the unit's wavefronts through LDS, and
// every wavefront of the work-group (ring units and idle ones too) reaches
// that one barrier.  Launch slots count wavefronts: units_q * W quantize
// slots, then one slot per ring unit.
template <int W>
__global__ void __launch_bounds__(256) append_kivi_h(Plan p, AppendArgs a) {
  constexpr int D = 128;
  static_assert(W == 1 || W == 2 || W == 4, "units of 32, 64 or 128 tokens");
  __shared__ uint32_t red[W > 1 ? 4 : 1][2][64];   // per wavefront: channel-pair min / max (packed fp16)
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int h = blockIdx.y, b = blockIdx.z;
  const int cb = lane & 15, r = lane >> 4;        // channels 8 cb.., tokens 8 r..
  const int64_t t0 = a.seq_lens ? (int64_t)a.seq_lens[b] : a.t0;
  int64_t nb = a.new_lens ? (int64_t)a.new_lens[b] : (int64_t)a.n;
  if (nb > a.n) nb = a.n;
  if (t0 < 0 || nb <= 0 || t0 + nb > a.cap) return;   // uniform over the work-group
  const int64_t U = 32 * W;
  const int64_t q_lo = quantized_tokens(p, t0), q_hi = quantized_tokens(p, t0 + nb);
  const int64_t u_first = (q_lo / U) * U;
  const int64_t n_qu = q_hi > q_lo ? (q_hi - u_first + U - 1) / U : 0;
  const int64_t slot = (int64_t)blockIdx.x * 4 + wave + a.x0;
  const int64_t q_slots = (int64_t)a.units_q * W;
  const int64_t bh = (int64_t)b * p.Hkv + h;
  const bool ring = slot >= q_slots;
  const int64_t x = slot / W;                      // unit
  const int s = (int)(slot % W);                   // the wavefront's 32 tokens in it
  const bool active = !ring && (a.phases & 1) && x < n_qu;
  if (ring && (a.phases & 2)) wave_ring_block(p, a, b, h, t0, nb, q_hi, slot - q_slots, cb, r);
  if (W == 1 && !active) return;
  const int64_t u0 = u_first + U * x;              // the unit (key group)
  const int64_t us = u0 + 32 * s;                  // this wavefront's tokens
  const int64_t v_lo = us > q_lo ? us : q_lo, v_hi = us + 32 < q_hi ? us + 32 : q_hi;
  const int32_t pg = active ? page_of(p, a.pm, b, u0) : -1;   // units never straddle pages
  bool ok[8];
  uint32_t hk[8][4], hv[8][4];
  if (active && us >= t0 && v_lo == us && v_hi == us + 32) {
    // 32 new tokens (every wavefront of a prefill)
#pragma unroll
    for (int i = 0; i < 8; ++i) ok[i] = true;
    load_unit_h(p, a, b, h, us, t0, cb, r, hk, hv);
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int64_t t = us + 8 * r + i;
      ok[i] = active && t >= v_lo && t < v_hi;
      if (ok[i]) {
        load_granule_h<SIDE_K>(p, a, b, h, t, t0, 8 * cb, hk[i]);
        load_granule_h<SIDE_V>(p, a, b, h, t, t0, 8 * cb, hv[i]);
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) { hk[i][j] = 0u; hv[i][j] = 0u; }
      }
    }
  }
  const float one = a.one;

  // ---- keys: one whole key group of U tokens (every token valid) ----
  {
    const SideFmt& fk = p.k;
    const float qmax = (float)((1 << fk.bits) - 1);
    const float yqk = 1.0f / (fk.scheme == KVQ_INT_ASYM ? qmax : 127.0f);   // once per wavefront
    uint32_t umn[4], umx[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      h2_t mn = as_h2(hk[0][m]), mx = mn;
#pragma unroll
      for (int i = 1; i < 8; ++i) {
        mn = __builtin_elementwise_min(mn, as_h2(hk[i][m]));
        mx = __builtin_elementwise_max(mx, as_h2(hk[i][m]));
      }
      umn[m] = as_u32(mn);
      umx[m] = as_u32(mx);
      rows_minmax_h(umn[m], umx[m]);
    }
    if constexpr (W > 1) {
      if (r == 0) {
#pragma unroll
        for (int m = 0; m < 4; ++m) { red[wave][0][4 * cb + m] = umn[m]; red[wave][1][4 * cb + m] = umx[m]; }
      }
      __syncthreads();
      if (!active) return;
      const int w0 = (wave / W) * W;               // the unit's first wavefront in the work-group
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        h2_t mn = as_h2(red[w0][0][4 * cb + m]), mx = as_h2(red[w0][1][4 * cb + m]);
#pragma unroll
        for (int k = 1; k < W; ++k) {
          mn = __builtin_elementwise_min(mn, as_h2(red[w0 + k][0][4 * cb + m]));
          mx = __builtin_elementwise_max(mx, as_h2(red[w0 + k][1][4 * cb + m]));
        }
        umn[m] = as_u32(mn);
        umx[m] = as_u32(mx);
      }
    }
    float sc[8], zc[8], rc[8];
#pragma unroll
    for (int m = 0; m < 4; ++m) {
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const int j = 2 * m + e;
        meta_values_h(fk, (float)as_h2(umn[m])[e], (float)as_h2(umx[m])[e], yqk, &sc[j], &zc[j]);
        rc[j] = recip_rn(sc[j]);
      }
    }
    if (pg >= 0) {
      if (r == 0 && s == 0) {
        const int64_t mi = meta_index_row(p, fk, bh, h, row_of(p, pg, h, u0), 8 * cb);   // 8 consecutive entries
        if (fk.meta16) {
          *(uint4*)((_Float16*)(a.arena + fk.scale) + mi) =
              make_uint4(pk_h(sc[0], sc[1]), pk_h(sc[2], sc[3]), pk_h(sc[4], sc[5]), pk_h(sc[6], sc[7]));
          *(uint4*)((_Float16*)(a.arena + fk.zero) + mi) =
              make_uint4(pk_h(zc[0], zc[1]), pk_h(zc[2], zc[3]), pk_h(zc[4], zc[5]), pk_h(zc[6], zc[7]));
        } else {
          float4* ps = (float4*)((float*)(a.arena + fk.scale) + mi);
          float4* pz = (float4*)((float*)(a.arena + fk.zero) + mi);
          ps[0] = make_float4(sc[0], sc[1], sc[2], sc[3]);
          ps[1] = make_float4(sc[4], sc[5], sc[6], sc[7]);
          pz[0] = make_float4(zc[0], zc[1], zc[2], zc[3]);
          pz[1] = make_float4(zc[4], zc[5], zc[6], zc[7]);
        }
      }
      uint8_t* krow0 = a.arena + fk.codes + row_of(p, pg, h, us + 8 * r) * p.k_row_bytes;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        _Float16 xh[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) xh[j] = as_h2(hk[i][j >> 1])[j & 1];
        uint32_t c[8];
        asym_codes8_h(xh, sc, rc, zc, one, qmax, c);
        write_k_granule(krow0 + i * p.k_row_bytes, cb, fk.bits, c);
      }
    }
  }

  // ---- values: per-token groups of Gc channels, words of 8 tokens formed in the lane ----
  const SideFmt& fv = p.v;
  const float qmax = (float)((1 << fv.bits) - 1);
  const float yqv = 1.0f / (fv.scheme == KVQ_INT_ASYM ? qmax : 127.0f);
  // the first lane of each value group stores the group's metadata; the
  // lane's eight tokens are consecutive token rows (a unit never straddles a
  // page), so their metadata indices step by the row's group count
  const int gl = fv.group / 8;                       // lanes per value group
  const bool vlane = pg >= 0 && (cb % gl) == 0;
  const int64_t vmi0 = vlane ? row_of(p, pg, h, us + 8 * r) * fv.meta_cols + cb / gl : 0;
  float vs[8], vz[8], vr[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    h2_t mn = __builtin_elementwise_min(__builtin_elementwise_min(as_h2(hv[i][0]), as_h2(hv[i][1])),
                                        __builtin_elementwise_min(as_h2(hv[i][2]), as_h2(hv[i][3])));
    h2_t mx = __builtin_elementwise_max(__builtin_elementwise_max(as_h2(hv[i][0]), as_h2(hv[i][1])),
                                        __builtin_elementwise_max(as_h2(hv[i][2]), as_h2(hv[i][3])));
    float fmn = fminf((float)mn[0], (float)mn[1]), fmx = fmaxf((float)mx[0], (float)mx[1]);
    lane_minmax(fmn, fmx, 1, fv.group / 8);
    meta_values_h(fv, fmn, fmx, yqv, &vs[i], &vz[i]);
    vr[i] = recip_rn(vs[i]);
    if (ok[i] && vlane) store_meta_values(fv, a.arena, vmi0 + i * fv.meta_cols, vs[i], vz[i]);
  }
  if (pg < 0) return;
  uint32_t valid = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) valid |= (ok[i] ? 1u : 0u) << i;
  if (!valid) return;
  const int bits = fv.bits;
  uint8_t* blk = a.arena + fv.codes + (row_of(p, pg, h, us) >> 5) * p.v_block_bytes;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int c = 8 * cb + j, n = c & 15, iw = c >> 4;
    uint8_t* wp = blk + (int64_t)((16 * r + n) * (D / 16) + iw) * bits;
    _Float16 xh[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) xh[i] = as_h2(hv[i][j >> 1])[j & 1];
    uint32_t code[8];
    asym_codes8_h(xh, vs, vr, vz, one, qmax, code);
    uint32_t lo = 0, hi = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int bit = i * bits;
      if (bit < 32) lo |= code[i] << bit;
      else hi |= code[i] << (bit - 32);
    }
    store_vword(wp, bits, valid, lo, hi);
  }
}

// FP8 calibration over the valid tokens of every sequence (new_lens), for
// paged calls: absmax per (kv head, side) into amax (u32 bit patterns).
template <int DT, bool WIN>
__global__ void __launch_bounds__(256) fp8_absmax_lens(Plan p, const void* kin, const void* vin, int n,
                                                        const int32_t* new_lens, uint32_t* amax) {
  const int h = blockIdx.y, side = blockIdx.z;
  const void* in = side ? vin : kin;
  // each sequence's first new_lens[b] tokens (n * D values per run, 16-byte aligned)
  const int64_t per_seq = (int64_t)n * p.D;
  const int64_t gid = blockIdx.x * (int64_t)blockDim.x + threadIdx.x, stride = (int64_t)gridDim.x * blockDim.x;
  const int D = p.D;
  float m = absmax_runs<DT, WIN>(in, p.B, p.Hkv, h, per_seq, gid, stride, [=](int b) {
    int64_t nl = new_lens ? (int64_t)new_lens[b] : n;
    nl = nl < 0 ? 0 : (nl > n ? n : nl);
    return nl * D;
  });
  for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, 64));
  __shared__ float sm[4];
  if ((threadIdx.x & 63) == 0) sm[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int w = 1; w < 4; ++w) m = fmaxf(m, sm[w]);
    atomicMax(&amax[side * p.Hkv + h], __float_as_uint(m));   // non-negative floats order as uints
  }
}

bool append_fused_supported(const Plan& p) { return p.unit > 0; }

hipError_t launch_append_fused(const Plan& p, void* arena, const PageMap& pm, const int32_t* seq_lens,
                               const int32_t* new_lens, int64_t t0, int n, int64_t cap, const void* k_new,
                               const void* v_new, hipStream_t s) {
  AppendArgs a;
  a.arena = (uint8_t*)arena;
  a.k_in = k_new;
  a.v_in = v_new;
  a.pm = pm;
  a.seq_lens = seq_lens;
  a.new_lens = new_lens;
  a.t0 = t0;
  a.n = n;
  a.cap = cap;
  a.one = 1.0f;
  // quantize units a sequence can need: the call's tokens plus the window it
  // already held (< Rs), from a group-aligned start; ring units: one per
  // 32-token block of window tokens
  const int64_t U = p.unit;
  const int64_t w = p.Rs > 0 ? p.Rs : 0;
  a.units_q = (int32_t)((n + w + U - 1) / U + 2);
  const int64_t units_r = p.window ? ((n < w ? n : w) + 31) / 32 + 1 : 0;
  const dim3 blk(kAppendThreads);
  // A fold reads window tokens [q_lo, t0) from the ring while the call writes
  // its own window tokens [w_lo, t0 + n) into slots t mod Rs.  Two such tokens
  // share a slot only if they lie Rs or more apart, i.e. when t0 + n - 1 -
  // q_lo >= Rs, which needs n + R + Gt - 2 >= Rs (q_lo >= t0 - R - Gt + 1):
  // then the ring writes run in a second launch, after every fold's reads.
  // A decode step (n = 1) never gets there.
  const bool split = p.window && (int64_t)n + p.R + p.Gt - 2 >= p.Rs;
  // one wavefront per 32-token unit where the format allows (D = 128, value
  // codes of at most 8 bits): four units per work-group
  const bool wave_units = U == 32 && p.D == 128 && p.v.bits <= 8;
  // keys per channel and values per token, both asymmetric integers (the
  // recipe of the "Different Axes" page)
  const bool kivi = p.k.scheme == KVQ_INT_ASYM && p.k.axis == KVQ_PER_CHANNEL && p.v.scheme == KVQ_INT_ASYM;
  // fp16-staged caches of that recipe: W = U / 32 wavefronts per unit
  const bool kivi_h = kivi && (p.window || p.in_dtype == KVQ_F16) && p.D == 128 && p.v.bits <= 8 &&
                      (U == 32 || U == 64 || U == 128);
  // a launch of one phase covers only that phase's units (work items: units,
  // or wavefront slots for the fp16-staged kernel)
  auto go = [&](int phases) {
    a.phases = phases;
    if (kivi_h) {
      const int64_t W = U / 32, q_slots = a.units_q * W;
      const int64_t first = phases == 2 ? q_slots : 0;
      const int64_t last = phases == 1 ? q_slots : q_slots + units_r;
      a.x0 = (int32_t)first;
      const dim3 grid_s((unsigned)((last - first + 3) / 4), p.Hkv, p.B);
      if (W == 4) hipLaunchKernelGGL(append_kivi_h<4>, grid_s, blk, 0, s, p, a);
      else if (W == 2) hipLaunchKernelGGL(append_kivi_h<2>, grid_s, blk, 0, s, p, a);
      else hipLaunchKernelGGL(append_kivi_h<1>, grid_s, blk, 0, s, p, a);
      return;
    }
    const int64_t first = phases == 2 ? a.units_q : 0;
    const int64_t last = phases == 1 ? a.units_q : a.units_q + units_r;
    a.x0 = (int32_t)first;
    const dim3 grid((unsigned)(last - first), p.Hkv, p.B);
    const dim3 grid_w((unsigned)((last - first + 3) / 4), p.Hkv, p.B);
    if (wave_units) {
      if (kivi)
        hipLaunchKernelGGL((append_wave<KVQ_INT_ASYM, KVQ_INT_ASYM, KVQ_PER_CHANNEL>), grid_w, blk, 0, s, p, a);
      else if (p.k.scheme == KVQ_FP8_E4M3 && p.v.scheme == KVQ_FP8_E4M3)
        hipLaunchKernelGGL((append_wave<KVQ_FP8_E4M3, KVQ_FP8_E4M3, -1>), grid_w, blk, 0, s, p, a);
      else if (p.k.scheme == KVQ_FP8_E5M2 && p.v.scheme == KVQ_FP8_E5M2)
        hipLaunchKernelGGL((append_wave<KVQ_FP8_E5M2, KVQ_FP8_E5M2, -1>), grid_w, blk, 0, s, p, a);
      else
        hipLaunchKernelGGL((append_wave<-1, -1, -1>), grid_w, blk, 0, s, p, a);
    } else if (p.D == 128) {
      if (U == 128) hipLaunchKernelGGL((append_units<128, 128>), grid, blk, 0, s, p, a);
      else if (U == 64) hipLaunchKernelGGL((append_units<128, 64>), grid, blk, 0, s, p, a);
      else hipLaunchKernelGGL((append_units<128, 32>), grid, blk, 0, s, p, a);
    } else {
      if (U == 128) hipLaunchKernelGGL((append_units<64, 128>), grid, blk, 0, s, p, a);
      else if (U == 64) hipLaunchKernelGGL((append_units<64, 64>), grid, blk, 0, s, p, a);
      else hipLaunchKernelGGL((append_units<64, 32>), grid, blk, 0, s, p, a);
    }
  };
  if (split) {
    go(1);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    go(2);
  } else {
    go(3);
  }
  return hipGetLastError();
}

hipError_t launch_fp8_absmax_lens(const Plan& p, const void* k_new, const void* v_new, int n,
                                  const int32_t* new_lens, uint32_t* amax, hipStream_t s) {
  const dim3 grid(fp8_absmax_blocks(p, n), p.Hkv, 2);
  const bool win = p.window != 0;
#define KVQ_ABSMAX_LENS(DT, W) \
  hipLaunchKernelGGL((fp8_absmax_lens<DT, W>), grid, dim3(256), 0, s, p, k_new, v_new, n, new_lens, amax)
  if (p.in_dtype == KVQ_F32) { if (win) KVQ_ABSMAX_LENS(KVQ_F32, true); else KVQ_ABSMAX_LENS(KVQ_F32, false); }
  else if (p.in_dtype == KVQ_F16) { if (win) KVQ_ABSMAX_LENS(KVQ_F16, true); else KVQ_ABSMAX_LENS(KVQ_F16, false); }
  else { if (win) KVQ_ABSMAX_LENS(KVQ_BF16, true); else KVQ_ABSMAX_LENS(KVQ_BF16, false); }
#undef KVQ_ABSMAX_LENS
  return hipGetLastError();
}

}  // namespace kvq
