// Device helpers shared by the quantize and attention kernels: staged source
// values, scale/zero addressing, the E4M3 codec and element dequantization.
#pragma once
#include "kvq_internal.h"

namespace kvq {

enum Side { SIDE_K = 0, SIDE_V = 1 };

// Staged value of token t, channel c of (b, h): from the fp16 ring when the
// token was appended by an earlier call (t < t0), else from this call's input.
struct Src {
  const uint8_t* arena;
  const void* in;
  int64_t t0;
  int32_t n;
};

__device__ __forceinline__ float ring_v_elem(const Plan& p, const uint8_t* arena, int64_t bh,
                                             int64_t slot, int c) {
  const int rblock = kVBlock * p.D * 2;
  const uint8_t* base = arena + p.ring_v + (uint64_t)bh * (p.Rs / kVBlock) * rblock;
  int64_t wb = vblock_word_byte(slot, c, p.D, 16, rblock);
  return (float)((const _Float16*)(base + wb))[slot & 7];
}

template <int SIDE>
__device__ __forceinline__ float src_val(const Plan& p, const Src& s, int b, int h, int64_t t, int c) {
  const int64_t bh = (int64_t)b * p.Hkv + h;
  if (t < s.t0) {
    const int64_t slot = t % p.Rs;
    if (SIDE == SIDE_K)
      return (float)((const _Float16*)(s.arena + p.ring_k))[(bh * p.Rs + slot) * p.D + c];
    return ring_v_elem(p, s.arena, bh, slot, c);
  }
  float x = load_in(s.in, (bh * s.n + (t - s.t0)) * p.D + c, p.in_dtype);
  return p.window ? stage_f16(x) : x;
}

__device__ __forceinline__ int64_t meta_index(const Plan& p, const SideFmt& f, int b, int h,
                                              int64_t t, int c) {
  const int64_t bh = (int64_t)b * p.Hkv + h;
  if (is_fp8(f.scheme)) return h;
  if (f.axis == KVQ_PER_TENSOR) return bh;
  if (f.axis == KVQ_PER_CHANNEL) {
    const int64_t g = f.group ? t / f.group : 0;
    return (bh * f.meta_rows + g) * p.D + c;
  }
  return (bh * p.Tc + t) * f.meta_cols + c / f.group;
}

// ---- fp16 scale / zero-point metadata ----------------------------------------

// fp16 rounding of finite x toward +inf (up) or -inf (down): the RNE
// conversion, moved one fp16 step when it landed on the wrong side; results
// beyond the fp16 range saturate at +-65504.
__device__ __forceinline__ _Float16 f16_directed(float x, bool up) {
  _Float16 h = (_Float16)x;
  const float hf = (float)h;
  if (up ? hf < x : hf > x) {
    uint16_t b = __builtin_bit_cast(uint16_t, h);
    const bool neg = b & 0x8000u;
    if (up) b = neg ? (b == 0x8000u ? 0x0001u : b - 1) : b + 1;
    else b = neg ? b + 1 : (b == 0 ? 0x8001u : b - 1);
    h = __builtin_bit_cast(_Float16, b);
  }
  const float r = (float)h;
  if (r > 65504.0f) h = (_Float16)65504.0f;
  if (r < -65504.0f) h = (_Float16)-65504.0f;
  return h;
}

__device__ __forceinline__ float load_meta(const uint8_t* base, int64_t i, bool m16) {
  return m16 ? (float)((const _Float16*)base)[i] : ((const float*)base)[i];
}

// ---- encodings ---------------------------------------------------------------

__device__ __forceinline__ void asym_params(float mn, float mx, int bits, float* s) {
  float d = mx - mn;
  d = fmaxf(d, 1e-8f);
  *s = d / (float)((1 << bits) - 1);
}

__device__ __forceinline__ uint32_t asym_code(float x, float s, float z, int bits) {
  float t = (x - z) / s;
  float r = __builtin_rintf(t);
  r = fminf(fmaxf(r, 0.0f), (float)((1 << bits) - 1));
  return (uint32_t)r;
}

__device__ __forceinline__ uint32_t sym_code(float x, float s) {
  float r = __builtin_rintf(x / s);
  r = fminf(fmaxf(r, -127.0f), 127.0f);
  return (uint32_t)(int32_t)r & 0xFFu;
}

// E5M2 encode with saturation: nearest representable, ties to even (the
// code's parity is its last mantissa bit's).
__device__ __forceinline__ uint32_t e5m2_encode(float y) {
  const uint32_t sign = (__float_as_uint(y) >> 24) & 0x80u;
  const float a = fminf(fabsf(y), kE5M2Max);
  uint32_t code;
  if (a < 6.103515625e-05f) {                // below 2^-14: quantum 2^-16
    code = (uint32_t)__builtin_rintf(a * 65536.0f);   // 0..4 (4 is the smallest normal)
  } else {
    int e = (int)((__float_as_uint(a) >> 23) & 0xFF) - 127;
    uint32_t m = (uint32_t)__builtin_rintf(ldexpf(a, 2 - e));   // 4..8
    if (m == 8) { m = 4; e += 1; }
    code = ((uint32_t)(e + 15) << 2) | (m - 4);
  }
  return code | sign;
}

// E4M3FN encode with saturation: nearest representable, ties to even.
__device__ __forceinline__ uint32_t e4m3_encode(float y) {
  const uint32_t sign = (__float_as_uint(y) >> 24) & 0x80u;
  const float a = fminf(fabsf(y), kE4M3Max);
  uint32_t code;
  if (a < 0.015625f) {                       // below 2^-6: quantum 2^-9
    code = (uint32_t)__builtin_rintf(a * 512.0f);   // 0..8 (8 is the smallest normal)
  } else {
    int e = (int)((__float_as_uint(a) >> 23) & 0xFF) - 127;
    uint32_t m = (uint32_t)__builtin_rintf(ldexpf(a, 3 - e));   // 8..16
    if (m == 16) { m = 8; e += 1; }
    code = ((uint32_t)(e + 7) << 3) | (m - 8);
  }
  return code | sign;
}

// Dequantized value of (t, c) as stored: window tokens from the fp16 ring.

template <int SIDE>
__device__ __forceinline__ float dequant_elem(const Plan& p, const uint8_t* arena, int b, int h,
                                              int64_t t, int c, int64_t Tq) {
  const SideFmt& f = SIDE == SIDE_K ? p.k : p.v;
  const int64_t bh = (int64_t)b * p.Hkv + h;
  if (t >= Tq) {
    const int64_t slot = t % p.Rs;
    if (SIDE == SIDE_K) return (float)((const _Float16*)(arena + p.ring_k))[(bh * p.Rs + slot) * p.D + c];
    return ring_v_elem(p, arena, bh, slot, c);
  }
  uint32_t code;
  if (SIDE == SIDE_K) {
    const uint8_t* row = arena + f.codes + (bh * p.Tc + t) * p.k_row_bytes;
    const int bit = c * f.bits;
    if (f.bits == 32) code = ((const uint32_t*)row)[c];
    else if (f.bits == 16) code = ((const uint16_t*)row)[c];
    else code = (row[bit >> 3] >> (bit & 7)) & ((1u << f.bits) - 1);
  } else {
    const uint8_t* wp = arena + f.codes + bh * p.v_nblk * p.v_block_bytes +
                        vblock_word_byte(t, c, p.D, f.bits, p.v_block_bytes);
    const int k = (int)(t & 7), bit = k * f.bits;
    if (f.bits == 32) code = ((const uint32_t*)wp)[k];
    else if (f.bits == 16) code = ((const uint16_t*)wp)[k];
    else code = (wp[bit >> 3] >> (bit & 7)) & ((1u << f.bits) - 1);
  }
  if (f.scheme == KVQ_NONE) {
    if (f.bits == 16) return (float)__builtin_bit_cast(_Float16, (uint16_t)code);
    return __uint_as_float(code);
  }
  const int64_t mi = meta_index(p, f, b, h, t, c);
  const float s = load_meta(arena + f.scale, mi, f.meta16);
  if (f.scheme == KVQ_FP8_E4M3) return e4m3_decode(code) * s;
  if (f.scheme == KVQ_FP8_E5M2) return e5m2_decode(code) * s;
  if (f.scheme == KVQ_INT_SYM) return (float)(int8_t)(uint8_t)code * s;
  const float z = load_meta(arena + f.zero, mi, f.meta16);
  const float prod = (float)code * s;
  return prod + z;
}

}  // namespace kvq
