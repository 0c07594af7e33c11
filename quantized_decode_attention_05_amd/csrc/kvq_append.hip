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
// Work split.  One work-group of 256 threads per (unit, kv head, sequence):
// a quantize unit is one key group (U = Gt tokens; 32 when keys have no token
// groups), a ring unit is up to 32 window tokens.  Each sequence's range comes
// from device data (the lengths of a ragged batch) or from the call's uniform
// t0, so units a sequence does not need exit at once.  A thread owns 16-byte
// granules of 8 consecutive channels of one token, loaded with 128-bit loads.
//  - per-channel key groups: min / max over the granules a thread holds, then
//    over the lanes holding the same channels (cross-lane shuffles), then over
//    the four wavefronts (LDS); the group's scale / zero-point rows are
//    written and every thread encodes its elements against them and writes
//    its part of each packed key row (D * b / 8 bytes per token);
//  - per-token value groups: min / max over the lanes holding one group's
//    channels (shuffles); codes go through LDS so that each thread assembles
//    whole words of the 32-token value block layout (8 tokens of one channel
//    per word) and no two threads write one byte.
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

// Code field (masked to the format's bits) of value x under scale s (rs =
// recip_or_nan(s)) and zero z; S >= 0 fixes the scheme at compile time.
template <int S>
__device__ __forceinline__ uint32_t code_t(const SideFmt& f, float x, float s, float rs, float z) {
  switch (S >= 0 ? S : f.scheme) {
    case KVQ_NONE:
      if (f.bits == 16) { const _Float16 hv = (_Float16)x; return (uint32_t)__builtin_bit_cast(uint16_t, hv); }
      return __float_as_uint(x);
    case KVQ_FP8_E4M3: return e4m3_encode(x / s);
    case KVQ_FP8_E5M2: return e5m2_encode(x / s);
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
  if (bits == 2) {
    uint32_t v = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) v |= (c[j] & 3u) << (2 * j);
    ((uint16_t*)row)[cb] = (uint16_t)v;
  } else if (bits == 4) {
    uint32_t v = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) v |= (c[j] & 15u) << (4 * j);
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

  // ---- keys --------------------------------------------------------------------
  {
    constexpr int NG = U / TPP;            // granules per thread
    float x[NG][8];
#pragma unroll
    for (int i = 0; i < NG; ++i) {
      const int64_t t = u0 + tq + TPP * i;
      if (t >= v_lo && t < v_hi) load_granule<SIDE_K, D>(p, a, b, h, t, t0, 8 * cb, x[i]);
      else {
#pragma unroll
        for (int j = 0; j < 8; ++j) x[i][j] = 0.0f;
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
        for (int j = 0; j < 8; ++j) { s[j] = fp8s; z[j] = 0.0f; rs[j] = 1.0f; }
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
      if (ok) load_granule<SIDE_V, D>(p, a, b, h, t, t0, 8 * cb, x);
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
      const float rv = v_int ? recip_or_nan(sv) : 1.0f;
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
  const int64_t x = blockIdx.x;
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

// KS / VS >= 0 fix the key / value scheme and KAX >= 0 the key axis at
// compile time, so that an instance holds only its own encoder (the whole
// unrolled body then stays in the instruction cache).
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
  const int64_t x = (int64_t)blockIdx.x * 4 + wave;
  const int64_t bh = (int64_t)b * p.Hkv + h;

  if (x >= a.units_q) {
    // window tokens of one 32-token block into their ring slots
    if (!(a.phases & 2)) return;
    const int64_t w_lo = q_hi > t0 ? q_hi : t0, w_hi = t0 + nb;
    const int64_t blk = (w_lo & ~(int64_t)31) + 32 * (x - a.units_q);
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
    return;
  }
  if (!(a.phases & 1) || x >= n_qu) return;
  const int64_t u0 = u_first + 32 * x;
  const int64_t v_lo = u0 > q_lo ? u0 : q_lo, v_hi = u0 + 32 < q_hi ? u0 + 32 : q_hi;
  const int32_t pg = page_of(p, a.pm, b, u0);     // the unit's page (units never straddle pages)
  bool ok[8];
  float xk[8][8], xv[8][8];
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
#pragma unroll
      for (int i = 0; i < 8; ++i) { st[i] = s8; zt[i] = 0.0f; rt[i] = 1.0f; }
    }
    if (pg >= 0) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        if (!ok[i]) continue;
        if (k_int && (cb % (fk.group / 8)) == 0)
          store_meta_values(fk, a.arena, meta_index_row(p, fk, bh, h, row_of(p, pg, h, u0 + 8 * r + i), 8 * cb),
                            st[i], zt[i]);
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
#pragma unroll
    for (int i = 0; i < 8; ++i)
      if (ok[i] && pg >= 0 && (cb % (fv.group / 8)) == 0)
        store_meta_values(fv, a.arena, meta_index_row(p, fv, bh, h, row_of(p, pg, h, u0 + 8 * r + i), 8 * cb),
                          vs[i], vz[i]);
  } else {
    const float s8 = is_fp8(vsch) ? ((const float*)(a.arena + fv.scale))[h] : 1.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) { vs[i] = s8; vz[i] = 0.0f; vr[i] = 1.0f; }
  }
  if (pg < 0) return;
  uint32_t valid = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) valid |= (ok[i] ? 1u : 0u) << i;
  if (!valid) return;
  const int bits = fv.bits;
  const uint32_t mask = (1u << bits) - 1;
  uint8_t* blk = a.arena + fv.codes + (row_of(p, pg, h, u0) >> 5) * p.v_block_bytes;
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
}

// FP8 calibration over the valid tokens of every sequence (new_lens), for
// paged calls: absmax per (kv head, side) into amax (u32 bit patterns).
__global__ void __launch_bounds__(256) fp8_absmax_lens(Plan p, const void* kin, const void* vin, int n,
                                                        const int32_t* new_lens, uint32_t* amax) {
  const int h = blockIdx.y, side = blockIdx.z;
  const void* in = side ? vin : kin;
  const int64_t per_seq = (int64_t)n * p.D;
  const int64_t nel = per_seq * p.B;
  float m = 0.0f;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < nel;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t b = i / per_seq, r = i % per_seq;
    const int32_t nl = new_lens ? new_lens[b] : n;
    if (r / p.D >= nl) continue;
    float x = load_in(in, (b * p.Hkv + h) * per_seq + r, p.in_dtype);
    if (p.window) x = stage_f16(x);
    m = fmaxf(m, fabsf(x));
  }
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
  // quantize units a sequence can need: the call's tokens plus the window it
  // already held (< Rs), from a group-aligned start; ring units: one per
  // 32-token block of window tokens
  const int64_t U = p.unit;
  const int64_t w = p.Rs > 0 ? p.Rs : 0;
  a.units_q = (int32_t)((n + w + U - 1) / U + 2);
  const int64_t units_r = p.window ? ((n < w ? n : w) + 31) / 32 + 1 : 0;
  const dim3 grid((unsigned)(a.units_q + units_r), p.Hkv, p.B);
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
  const dim3 grid_w((unsigned)((a.units_q + units_r + 3) / 4), p.Hkv, p.B);
  // keys per channel and values per token, both asymmetric integers (the
  // recipe of the "Different Axes" page)
  const bool kivi = p.k.scheme == KVQ_INT_ASYM && p.k.axis == KVQ_PER_CHANNEL && p.v.scheme == KVQ_INT_ASYM;
  auto go = [&](int phases) {
    a.phases = phases;
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
  const int64_t nel = (int64_t)p.B * n * p.D;
  int64_t chunks = (nel + 255) / 256;
  if (chunks > 512) chunks = 512;
  if (chunks < 1) chunks = 1;
  hipLaunchKernelGGL(fp8_absmax_lens, dim3((unsigned)chunks, p.Hkv, 2), dim3(256), 0, s, p, k_new, v_new, n,
                     new_lens, amax);
  return hipGetLastError();
}

}  // namespace kvq
