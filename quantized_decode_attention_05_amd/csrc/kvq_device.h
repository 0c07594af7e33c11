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

// Index of the scale / zero-point of channel c of the token in token row tr
// (row_of) of sequence-head bh = b * Hkv + h.  Per-tensor and whole-axis
// groups exist only in contiguous caches: one entry / row per (b, h).
__device__ __forceinline__ int64_t meta_index_row(const Plan& p, const SideFmt& f, int64_t bh, int h,
                                                  int64_t tr, int c) {
  if (is_fp8(f.scheme)) return h;
  if (f.axis == KVQ_PER_TENSOR) return bh;
  if (f.axis == KVQ_PER_CHANNEL) {
    if (f.group) return (tr / f.group) * p.D + c;
    return bh * p.D + c;
  }
  return tr * f.meta_cols + c / f.group;
}

// The same for token t of a contiguous cache (token row bh * Tc + t).
__device__ __forceinline__ int64_t meta_index(const Plan& p, const SideFmt& f, int b, int h,
                                              int64_t t, int c) {
  const int64_t bh = (int64_t)b * p.Hkv + h;
  return meta_index_row(p, f, bh, h, bh * p.Tc + t, c);
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

// FP8 encodes with saturation: the magnitude is clamped to the largest finite
// value (so NaN and infinity give the largest code, and the sign, also of
// zero, is kept), then gfx950's conversion instruction rounds to the nearest
// representable value, ties to even, subnormals included.  For inputs within
// the range this is the same rounding as encoding by exponent and mantissa
// (checked over every fp32 bit pattern from 0 to a little past the maximum
// of each format); the instruction converts two values, the low byte of the
// result is the first.
__device__ __forceinline__ uint32_t e5m2_encode(float y) {
  const float c = __builtin_copysignf(fminf(fabsf(y), kE5M2Max), y);
  return (uint32_t)__builtin_amdgcn_cvt_pk_bf8_f32(c, c, 0, false) & 0xFFu;
}

__device__ __forceinline__ uint32_t e4m3_encode(float y) {
  const float c = __builtin_copysignf(fminf(fabsf(y), kE4M3Max), y);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(c, c, 0, false) & 0xFFu;
}

// Scale and zero-point a group with minimum mn and maximum mx (for symmetric
// groups mx holds the absmax) is stored with, as the fp32 values that codes
// and dequantization use: fp32 metadata keeps them as computed; fp16 metadata
// rounds the zero-point down and the scale up (and the symmetric scale up) so
// the stored grid still spans the group.
__device__ __forceinline__ void meta_values(const SideFmt& f, float mn, float mx, float* s, float* z) {
  if (f.scheme == KVQ_INT_ASYM) {
    if (f.meta16) {
      const _Float16 zh = f16_directed(mn, false);
      float sc;
      asym_params((float)zh, mx, f.bits, &sc);
      *s = (float)f16_directed(sc, true);
      *z = (float)zh;
    } else {
      asym_params(mn, mx, f.bits, s);
      *z = mn;
    }
  } else {
    const float sc = fmaxf(mx, 1e-8f) / 127.0f;
    *s = f.meta16 ? (float)f16_directed(sc, true) : sc;
    *z = 0.0f;
  }
}

// Store the values meta_values gives (exact in the storage type) at index mi.
__device__ __forceinline__ void store_meta_values(const SideFmt& f, uint8_t* arena, int64_t mi, float s,
                                                  float z) {
  if (f.meta16) {
    ((_Float16*)(arena + f.scale))[mi] = (_Float16)s;
    if (f.scheme == KVQ_INT_ASYM) ((_Float16*)(arena + f.zero))[mi] = (_Float16)z;
  } else {
    ((float*)(arena + f.scale))[mi] = s;
    if (f.scheme == KVQ_INT_ASYM) ((float*)(arena + f.zero))[mi] = z;
  }
}

__device__ __forceinline__ void store_meta(const Plan& p, const SideFmt& f, uint8_t* arena,
                                           int64_t mi, float mn, float mx) {
  (void)p;
  float s, z;
  meta_values(f, mn, mx, &s, &z);
  store_meta_values(f, arena, mi, s, z);
}

// Dequantized value of (t, c) as stored: window tokens from the fp16 ring.

template <int SIDE>
__device__ __forceinline__ float dequant_elem(const Plan& p, const uint8_t* arena, int b, int h,
                                              int64_t t, int c, int64_t Tq, const PageMap& pm = PageMap{nullptr, 0}) {
  const SideFmt& f = SIDE == SIDE_K ? p.k : p.v;
  const int64_t bh = (int64_t)b * p.Hkv + h;
  if (t >= Tq) {
    const int64_t slot = t % p.Rs;
    if (SIDE == SIDE_K) return (float)((const _Float16*)(arena + p.ring_k))[(bh * p.Rs + slot) * p.D + c];
    return ring_v_elem(p, arena, bh, slot, c);
  }
  const int64_t tr = read_row(p, pm, b, h, t);
  uint32_t code;
  if (SIDE == SIDE_K) {
    const uint8_t* row = arena + f.codes + tr * p.k_row_bytes;
    const int bit = c * f.bits;
    if (f.bits == 32) code = ((const uint32_t*)row)[c];
    else if (f.bits == 16) code = ((const uint16_t*)row)[c];
    else code = (row[bit >> 3] >> (bit & 7)) & ((1u << f.bits) - 1);
  } else {
    const uint8_t* wp = arena + f.codes + vblock_word_byte(tr, c, p.D, f.bits, p.v_block_bytes);
    const int k = (int)(t & 7), bit = k * f.bits;
    if (f.bits == 32) code = ((const uint32_t*)wp)[k];
    else if (f.bits == 16) code = ((const uint16_t*)wp)[k];
    else code = (wp[bit >> 3] >> (bit & 7)) & ((1u << f.bits) - 1);
  }
  if (f.scheme == KVQ_NONE) {
    if (f.bits == 16) return (float)__builtin_bit_cast(_Float16, (uint16_t)code);
    return __uint_as_float(code);
  }
  const int64_t mi = meta_index_row(p, f, bh, h, tr, c);
  const float s = load_meta(arena + f.scale, mi, f.meta16);
  if (f.scheme == KVQ_FP8_E4M3) return e4m3_decode(code) * s;
  if (f.scheme == KVQ_FP8_E5M2) return e5m2_decode(code) * s;
  if (f.scheme == KVQ_INT_SYM) return (float)(int8_t)(uint8_t)code * s;
  const float z = load_meta(arena + f.zero, mi, f.meta16);
  const float prod = (float)code * s;
  return prod + z;
}

// Largest |x| of the values staged from 16 bytes of input (8 values of a
// 16-bit type, 4 of fp32), as the quantizers stage them (through fp16 when the
// cache keeps a window).
template <int DT, bool WIN>
__device__ __forceinline__ float absmax16(const uint4& w) {
  float m = 0.0f;
  const uint32_t q[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    float a, b;
    if constexpr (DT == KVQ_F32) {
      a = __uint_as_float(q[j]);
      b = 0.0f;
    } else if constexpr (DT == KVQ_F16) {
      a = (float)__builtin_bit_cast(_Float16, (uint16_t)(q[j] & 0xFFFFu));
      b = (float)__builtin_bit_cast(_Float16, (uint16_t)(q[j] >> 16));
    } else {
      a = bf16_to_f32((uint16_t)(q[j] & 0xFFFFu));
      b = bf16_to_f32((uint16_t)(q[j] >> 16));
    }
    if constexpr (WIN) { a = stage_f16(a); b = stage_f16(b); }
    m = fmaxf(m, fmaxf(fabsf(a), fabsf(b)));
  }
  return m;
}

// absmax over the values of kv head h of every sequence b < B (run b holds
// lens(b) values from base + (b * Hkv + h) * per_seq elements; per_seq and
// every lens(b) a multiple of the values per 16 bytes, runs 16-byte
// aligned), by the threads of a grid-stride (gid, stride), for input dtype DT
// (staged through fp16 when WIN).  Each round issues sixteen 16-byte loads
// (four sequences, four strides) before using any; a load past its run's end
// reads the run's first granule (every run of a launch with a nonempty run
// holds per_seq >= lens values) and its result is dropped, so no load sits
// behind a branch.
template <int DT, bool WIN, typename Lens>
__device__ __forceinline__ float absmax_runs(const void* base, int B, int Hkv, int h, int64_t per_seq,
                                             int64_t gid, int64_t stride, Lens lens) {
  constexpr int per = DT == KVQ_F32 ? 4 : 8;
  constexpr int esz = DT == KVQ_F32 ? 4 : 2;
  float m = 0.0f;
  for (int b0 = 0; b0 < B; b0 += 4) {
    const uint4* v[4];
    int64_t nv[4], nmax = 0;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int b = b0 + u < B ? b0 + u : b0;
      v[u] = (const uint4*)((const uint8_t*)base + ((int64_t)b * Hkv + h) * per_seq * esz);
      nv[u] = b0 + u < B ? lens(b) / per : 0;
      nmax = nv[u] > nmax ? nv[u] : nmax;
    }
    for (int64_t i = gid; i < nmax; i += 4 * stride) {
      uint4 w[4][4];
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const int64_t e = i + k * stride;
          w[u][k] = v[u][e < nv[u] ? e : 0];
        }
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const float a = absmax16<DT, WIN>(w[u][k]);
          m = i + k * stride < nv[u] ? fmaxf(m, a) : m;
        }
    }
  }
  return m;
}

}  // namespace kvq
