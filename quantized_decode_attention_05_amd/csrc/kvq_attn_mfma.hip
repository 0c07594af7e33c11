// MFMA split-K decode attention for the hot cache formats on gfx950.
//
// Same computation as the generic kernel (per query head: logits q . k_hat /
// sqrt(d) in log2 units, online softmax, p . v_hat; "FP8 KV Cache
// Quantization: Why Keys Break Before Values", section "Why does the K cache
// break before the V cache?"), organised for 64-wide wavefronts and the
// 16x16x32 fp16 matrix instruction:
//
//  * QK^T as S^T = K_tile . Q^T: A = 16 tokens x 32 channels of codes, B = the
//    query heads of one kv head as columns (hi and lo fp16 halves of the fp32
//    query in separate columns, so fp16 operands lose nothing).  Codes are
//    exact in fp16; with per-channel keys the per-channel scale folds into the
//    query columns and the zero-point into a per-head bias:
//      logit = sum_c (q_c s_c) x_c + sum_c q_c z_c.
//    2- and 4-bit codes become fp16 through the fp4 / fp8 conversion
//    instructions (exact, two codes each); 8-bit codes by ORing their bits
//    into the mantissa of 1024 and subtracting 1024 (exact).
//  * With pre-RoPE keys ("KV Cache Quantization: Why Keys and Values Need
//    Different Axes", section "Where does RoPE break this?") each lane
//    dequantizes its 32 channels to fp32, rotates the channel pairs by
//    position * theta_i and packs fp16 operands (dequantize -> rotate -> dot).
//  * PV as O = P . V_tile: A = probabilities of 8 tokens per lane times the
//    per-token value scale, B = value codes read straight from the 32-token
//    block layout, whose lane order is exactly this instruction's B-operand
//    order.  The 16 A rows are (value channel group, query head) pairs, row
//    R = group * n_rep + head, so one A operand serves every channel group;
//    tile i keeps the rows of its own group.  Zero-points enter through
//    per-row bias sums.  For this the query columns repeat the heads
//    (column n is head n mod n_rep), which costs nothing: the columns beyond
//    n_rep would otherwise be padding.
//  * The S^T accumulator of two 16-token tiles (token rows permuted so that
//    lane (n, g) holds tokens 8g..8g+7) is already the PV A operand of head n:
//    no data moves between QK^T and PV.
//
// Each work-group (4 wavefronts) takes one (sequence, kv head, token split);
// wavefronts walk disjoint runs of 32-token steps and their softmax states
// are combined through LDS before one partial per split is written.
#include <type_traits>

#include "kvq_internal.h"
#include "kvq_launch.h"
#include "kvq_device.h"

namespace kvq {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float float2v __attribute__((ext_vector_type(2)));
typedef uint32_t u32;

// Tuning knobs: the wavefronts per SIMD the register allocation must allow
// (0: compiler's choice) and the LDS stages per wavefront (0: by stage size).
#ifndef KVQ_MFMA_STAGES
#define KVQ_MFMA_STAGES 0
#endif
#ifndef KVQ_MFMA_WAVES_PER_EU
#define KVQ_MFMA_WAVES_PER_EU 2
#endif

namespace mf {

constexpr float kNegBig = -1.0e30f;
constexpr float kLog2e = 1.4426950408889634f;
constexpr int kWaves = 4;
constexpr u32 kMagic = 0x64006400u;    // fp16 1024 in both halves

enum Fmt { INT2 = 2, INT4 = 4, INT8 = 8, FP8 = 9, BF8 = 10 };   // FP8: E4M3, BF8: E5M2
__host__ __device__ constexpr bool is_f8(int f) { return f == FP8 || f == BF8; }

struct Args {
  const uint8_t* arena;
  const void* q;
  float* ws_o;
  float* ws_ml;
  int64_t T, Tq, chunk;
  int32_t S;
  float qscale;
  float neg1;   // -1.0f, passed in so that r - (float)h stays one mixed fp16/fp32 FMA
  // decode step: the new token of every sequence, appended by the work-group
  // whose range holds position t_new (mode 1: fp16 window, 2: FP8 codes)
  const void* k_new;
  const void* v_new;
  int64_t t_new;
  int32_t app_mode;
  uint8_t* arena_w;   // the arena, writable (decode-step appends only)
  // ragged / paged calls: sequence b holds seq_lens[b] + lens_add tokens
  // (clamped to [0, T]), read through the block table
  PageMap pm;
  const int32_t* seq_lens;
  int32_t lens_add;
  // query heads in groups of hg per work-group, ngroups groups per kv head
  // (grid y = kv head * ngroups + group)
  int32_t hg, ngroups;
};

__device__ __forceinline__ half8 pack8(u32 a, u32 b, u32 c, u32 d) {
  union { u32 u[4]; half8 h; } x;
  x.u[0] = a; x.u[1] = b; x.u[2] = c; x.u[3] = d;
  return x.h;
}
__device__ __forceinline__ u32 h2u(half2v h) { return __builtin_bit_cast(u32, h); }
__device__ __forceinline__ u32 pk_f16(float a, float b) {
  float2v v = {a, b};
  return h2u(__builtin_convertvector(v, half2v));
}
// (1024 + x) as fp16 -> x, exactly (both are fp16 integers)
__device__ __forceinline__ u32 unmagic(u32 v) {
  const half2v m = {(_Float16)1024.0f, (_Float16)1024.0f};
  return h2u(__builtin_bit_cast(half2v, v) - m);
}
// (x & mask) | 1024-pattern, then minus 1024: two fp16 codes in one instruction
// pair plus the subtraction.  The AND-OR is written out because the compiler
// splits it into two instructions when both constants are literals.  Its
// result always passes through the compiler-generated subtraction before a
// matrix instruction reads it: the compiler's hazard checks do not look inside
// inline assembly, and a matrix instruction needs wait states after a vector
// instruction writes one of its source registers.
__device__ __forceinline__ u32 code_pair(u32 x, u32 mask) {
  u32 r;
  asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(x), "v"(mask), "v"(kMagic));
  return unmagic(r);
}
// ---- direct global -> LDS streaming ------------------------------------------------
// Each lane moves 16 bytes from its own global address to LDS byte
// lds_base + 16 * lane (lds_base wave-uniform, in M0).  Issued as inline
// assembly so that the compiler's wait-count bookkeeping, which would make
// every later LDS read wait for all outstanding loads, does not see them; the
// kernel waits for each stage itself with s_waitcnt vmcnt.  Nothing else in
// the streaming loop issues vector-memory loads, so the counts are exact.
__device__ __forceinline__ void dma16(u32 lds_base, const void* gptr) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off" :: "s"(lds_base), "v"(gptr) : "memory", "m0");
}
template <int N> __device__ __forceinline__ void wait_vmem() {
  asm volatile("s_waitcnt vmcnt(%0)" :: "n"(N) : "memory");
}

__device__ __forceinline__ floatx4 mfma(half8 a, half8 b, floatx4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ float lo_f(u32 x) { return (float)__builtin_bit_cast(half2v, x)[0]; }
__device__ __forceinline__ float hi_f(u32 x) { return (float)__builtin_bit_cast(half2v, x)[1]; }

// fp16 residuals (r0 - h.lo, r1 - h.hi) of two fp32 values whose fp16
// roundings are packed in h (neg1 = -1.0f, opaque to the compiler so the
// subtraction stays a mixed-precision FMA with an fp16 source).
__device__ __forceinline__ u32 f16_residual2(u32 h, float r0, float r1, float neg1) {
  const _Float16 a = (_Float16)__builtin_fmaf(lo_f(h), neg1, r0);
  const _Float16 b = (_Float16)__builtin_fmaf(hi_f(h), neg1, r1);
  const half2v v = {a, b};
  return h2u(v);
}

// ---- 2- and 4-bit codes through the conversion instructions ----------------------
// A 2-bit code c in the low bits of a 4-bit field is the E2M1 value c / 2, and
// a 4-bit code in the low bits of a byte is the E4M3 value c / 512 (the
// subnormals and the first binade are evenly spaced), so the scaled fp4 -> fp16
// and fp8 -> fp16 conversions return codes exactly, two per instruction.  A
// dword masked with 0x33333333 (INT2) or 0x0F0F0F0F (INT4) keeps codes 0 and 2
// of every run of four; shifted right by one code width first, codes 1 and 3.
// So register r of a lane's 32 codes holds codes (4 (r >> 1) + (r & 1), + 2),
// and fp16 number f of the registers in order is code nib_pos(f).
__device__ constexpr int nib_pos(int f) { return 4 * (f >> 2) + ((f >> 1) & 1) + 2 * (f & 1); }

__device__ __forceinline__ u32 fp4_pair(u32 x, int byte) {   // byte: compile-time after unrolling
  switch (byte & 3) {
    case 0: return h2u(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(x, 2.0f, 0));
    case 1: return h2u(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(x, 2.0f, 1));
    case 2: return h2u(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(x, 2.0f, 2));
    default: return h2u(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(x, 2.0f, 3));
  }
}
__device__ __forceinline__ u32 fp8_pair(u32 x, int word) {
  return h2u(word & 1 ? __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(x, 512.0f, true)
                      : __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(x, 512.0f, false));
}

// Position of the e-th fp16 of k-step j inside a lane's 32 key channels, for
// the register order each code width unpacks into.
template <int KF, bool ROPE>
__device__ __forceinline__ int kslot(int j, int e) {
  if (ROPE && KF == INT2) return 16 * (j >> 1) + 4 * (j & 1) + (e >> 1) + 8 * (e & 1);   // (c, c+8)
  if (ROPE || KF == INT8 || KF == FP8) return 8 * j + e;                  // natural
  return 8 * j + nib_pos(e);                                              // INT2 / INT4
}

// Pre-RoPE INT2 keys only feed fp32 FMAs, so a code need not become an exact
// integer: register i (0..7) of a code dword holds codes i and i + 8 as the fp16
// values 1 + c 2^(p_i - 10), the code ORed into the mantissa of 1.0 at bit p_i
// after at most one shift of the dword (two shifts per dword in all).  The
// per-pair coefficients absorb the factor 2^(10 - p_i) and the offset; with
// p_i >= 4 the offset is at most 64 code steps, so the fp32 FMAs lose nothing
// that matters against the fp16 rounding of the rotated key.
__device__ constexpr int int2_pos(int i) { return i < 2 ? 4 + 2 * i : (i < 5 ? 2 * i : 2 * i - 6); }
__device__ __forceinline__ u32 int2_pos_reg(u32 x, int i) {
  const u32 y = i < 2 ? x << 4 : (i < 5 ? x : x >> 6);
  u32 r;
  asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(y), "v"(0x00030003u << int2_pos(i)), "v"(0x3C003C00u));
  return r;
}

template <int F> struct Bits { static constexpr int v = is_f8(F) ? 8 : F; };

// LDS position of 16-byte granule q (channels 4q..4q+3) of a key scale or
// zero-point row.  The four lane groups g read granules 8g + i at the same
// time (broadcast over the 16 lanes of a group); XOR-ing bits 1-2 with g puts
// the four in different bank groups.  An involution, so the loads that fill
// the row use it too.
__device__ __forceinline__ int km_pos(int q) { return q ^ (((q >> 3) & 3) << 1); }


// LDS position of the 16-byte granule of token t (its four group scales, or
// zero-points) when values have four channel groups: lane group g reads tokens
// 8g + k at the same time; rotating each run of 8 by t/8 spreads the four over
// bank groups.  vm_src is the inverse (which token's granule a filling lane
// fetches).
__device__ __forceinline__ int vm_pos(int t) { return (t & ~7) | ((t + (t >> 3)) & 7); }
__device__ __forceinline__ int vm_src(int l) { return (l & ~7) | ((l - (l >> 3)) & 7); }

// fp16 scale / zero-point rows staged at reg (scales in bytes [0, 8H), zero-
// points in [8H, 16H), natural order; H = N / 2) -> the fp32 layout of the
// same region: granule G < N holds the four values of granule perm(G mod H)
// of the scale row (G < H) or the zero-point row.  PERM: 0 identity, 1 km_pos,
// 2 vm_src.  The whole wavefront reads the staged rows before it writes over
// them (one wavefront's LDS operations complete in order).
template <int N, int PERM>
__device__ __forceinline__ void widen_meta(uint8_t* reg, int lane) {
  constexpr int H = N / 2, PER = (N + 63) / 64;
  uint2 v[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int G = lane + 64 * i;
    const int q = G % H;
    const int src = PERM == 1 ? km_pos(q) : (PERM == 2 ? vm_src(q) : q);
    if (G < N) v[i] = *(const uint2*)(reg + (G < H ? 0 : 8 * H) + 8 * src);
  }
  asm volatile("" ::: "memory");
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int G = lane + 64 * i;
    if (G < N) {
      const half2v a = __builtin_bit_cast(half2v, v[i].x), b = __builtin_bit_cast(half2v, v[i].y);
      *(float4*)(reg + 16 * G) = make_float4((float)a[0], (float)a[1], (float)b[0], (float)b[1]);
    }
  }
}

// ---- key operand unpacking -------------------------------------------------------

// Exact fp16 codes of one lane's 32 key channels in kslot order, from KB dwords.
template <int KF>
__device__ __forceinline__ u32 key_code_reg(const u32* w, int r);
template <int KF>
__device__ __forceinline__ void unpack_k_codes(const u32* w, half8* A) {
  if constexpr (KF == INT2 || KF == INT4) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
      A[j] = pack8(key_code_reg<KF>(w, 4 * j), key_code_reg<KF>(w, 4 * j + 1),
                   key_code_reg<KF>(w, 4 * j + 2), key_code_reg<KF>(w, 4 * j + 3));
  } else {  // INT8: natural pairs (c, c+1)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      u32 r[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const u32 src = w[2 * j + (i >> 1)];
        const int sh = 16 * (i & 1);
        r[i] = unmagic((((src >> sh) & 0xFFu) | (((src >> (sh + 8)) & 0xFFu) << 16)) | kMagic);
      }
      A[j] = pack8(r[0], r[1], r[2], r[3]);
    }
  }
}

// Exact fp16 values of the two 8-bit codes in bytes (0, 1) (hi: (2, 3)) of x.
// E4M3 through the conversion instruction; an E5M2 byte is the high byte of
// the fp16 with the same value, so one byte permute places two of them.
template <int F>
__device__ __forceinline__ u32 f8_pair(u32 x, bool hi) {
  if constexpr (F == BF8) return __builtin_amdgcn_perm(x, x, hi ? 0x030C020Cu : 0x010C000Cu);
  else return h2u(hi ? __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(x, 1.0f, true)
                     : __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(x, 1.0f, false));
}

// Exact fp16 values of 32 E4M3 / E5M2 codes (natural order).
template <int F>
__device__ __forceinline__ void unpack_k_f8(const u32* w, half8* A) {
#pragma unroll
  for (int j = 0; j < 4; ++j)
    A[j] = pack8(f8_pair<F>(w[2 * j], false), f8_pair<F>(w[2 * j], true),
                 f8_pair<F>(w[2 * j + 1], false), f8_pair<F>(w[2 * j + 1], true));
}

// Exact fp16 codes of a lane's 32 key channels come as 16 half2 registers;
// channel e sits in register code_reg<KF>(e), half code_half<KF>(e).  This
// decodes register r alone, where it is first used.
template <int KF>
__device__ __forceinline__ u32 key_code_reg(const u32* w, int r) {
  if constexpr (KF == INT2) {
    const u32 x = w[r >> 3];
    return fp4_pair(r & 1 ? (x >> 2) & 0x33333333u : x & 0x33333333u, r >> 1);
  } else if constexpr (KF == INT4) {
    const u32 x = w[r >> 2];
    return fp8_pair(r & 1 ? (x >> 4) & 0x0F0F0F0Fu : x & 0x0F0F0F0Fu, r >> 1);
  } else if constexpr (is_f8(KF)) {
    return f8_pair<KF>(w[r >> 1], r & 1);   // channels 2r, 2r + 1: bytes (0, 1) or (2, 3)
  } else {
    const u32 src = w[r >> 1];
    const int sh = 16 * (r & 1);
    return unmagic((((src >> sh) & 0xFFu) | (((src >> (sh + 8)) & 0xFFu) << 16)) | kMagic);
  }
}
template <int KF> __device__ constexpr int code_reg(int e) {
  return (KF == INT2 || KF == INT4) ? 2 * (e >> 2) + (e & 1) : e >> 1;
}
template <int KF> __device__ constexpr int code_half(int e) {
  return (KF == INT2 || KF == INT4) ? (e >> 1) & 1 : e & 1;
}

// ---- value operand unpacking -----------------------------------------------------

// Tile i of a lane's value chunk as the B operand.  INT2 / INT4: fp16 number f
// is token nib_pos(f); INT8 / FP8: token pairs (r, r+4) (vtok gives the order).
template <int VF>
__device__ __forceinline__ half8 unpack_v(const u32* w, int i) {
  if constexpr (VF == INT4) {
    const u32 x = w[i];                                                      // token k at bits 4k
    const u32 ev = x & 0x0F0F0F0Fu, od = (x >> 4) & 0x0F0F0F0Fu;
    return pack8(fp8_pair(ev, 0), fp8_pair(od, 0), fp8_pair(ev, 1), fp8_pair(od, 1));
  } else if constexpr (VF == INT2) {
    // word i = 16 bits at half (i & 1) of dword i/2; token k at bit 2k
    const u32 x = w[i >> 1];
    const u32 ev = x & 0x33333333u, od = (x >> 2) & 0x33333333u;
    const int b = 2 * (i & 1);
    return pack8(fp4_pair(ev, b), fp4_pair(od, b), fp4_pair(ev, b + 1), fp4_pair(od, b + 1));
  } else if constexpr (VF == INT8) {
    const u32 d0 = w[2 * i], d1 = w[2 * i + 1];
    u32 r[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) r[k] = unmagic((((d0 >> (8 * k)) & 0xFFu) | (((d1 >> (8 * k)) & 0xFFu) << 16)) | kMagic);
    return pack8(r[0], r[1], r[2], r[3]);
  } else {  // FP8 (E4M3 or E5M2)
    const u32 d0 = w[2 * i], d1 = w[2 * i + 1];
    const u32 y0 = (d0 & 0xFFu) | ((d1 & 0xFFu) << 8) | ((d0 & 0xFF00u) << 8) | ((d1 & 0xFF00u) << 16);
    const u32 y1 = ((d0 >> 16) & 0xFFu) | ((d1 >> 8) & 0xFF00u) | ((d0 >> 8) & 0xFF0000u) | (d1 & 0xFF000000u);
    return pack8(f8_pair<VF>(y0, false), f8_pair<VF>(y0, true), f8_pair<VF>(y1, false), f8_pair<VF>(y1, true));
  }
}

// Token of fp16 number f of a value tile's B operand.
template <int VF> __device__ constexpr int vtok(int f) {
  return (VF == INT2 || VF == INT4) ? nib_pos(f) : (f >> 1) + 4 * (f & 1);
}

// fp16 window values: word i = 8 fp16 (tokens 0..7) in dwords 4i..4i+3.
__device__ __forceinline__ half8 unpack_v_f16(const u32* w, int i) {
  const u32 a = w[4 * i], b = w[4 * i + 1], c = w[4 * i + 2], d = w[4 * i + 3];
  return pack8((a & 0xFFFFu) | (c << 16), (a >> 16) | (c & 0xFFFF0000u),
               (b & 0xFFFFu) | (d << 16), (b >> 16) | (d & 0xFFFF0000u));
}

// keep only fp16 halves whose token is valid (bit k of `valid` = token k of 8)
__device__ __forceinline__ half8 mask_tokens(half8 h, u32 valid) {
  union { half8 h; u32 u[4]; } x;
  x.h = h;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const u32 m = ((valid >> r) & 1u ? 0x0000FFFFu : 0u) | ((valid >> (r + 4)) & 1u ? 0xFFFF0000u : 0u);
    x.u[r] &= m;
  }
  return x.h;
}

template <int N>
__device__ __forceinline__ void load_dw(const uint8_t* p, u32* w) {
  if constexpr (N == 2) {
    const uint2 v = *(const uint2*)p;
    w[0] = v.x; w[1] = v.y;
  } else {
#pragma unroll
    for (int i = 0; i < N / 4; ++i) {
      const uint4 v = ((const uint4*)p)[i];
      w[4 * i] = v.x; w[4 * i + 1] = v.y; w[4 * i + 2] = v.z; w[4 * i + 3] = v.w;
    }
  }
}

// Lane pairs (l, l ^ 16) and (l, l ^ 32) through gfx950's permlane swaps (VALU
// operations, no LDS round trip).  Swapping a value with itself leaves each lane
// holding its own value in one result and its partner's in the other, so a
// symmetric combination of the two equals x op partner in every lane (and fp32
// addition and max are commutative, so the results match a shuffle exactly).
// Called with the whole wavefront active.
__device__ __forceinline__ float wave_max16(float x) {   // max over lanes n, n+16, n+32, n+48
  const u32 b = __float_as_uint(x);
  const auto r = __builtin_amdgcn_permlane16_swap(b, b, false, false);
  x = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
  const u32 c = __float_as_uint(x);
  const auto t = __builtin_amdgcn_permlane32_swap(c, c, false, false);
  return fmaxf(__uint_as_float(t[0]), __uint_as_float(t[1]));
}
__device__ __forceinline__ float wave_sum16(float x) {
  const u32 b = __float_as_uint(x);
  const auto r = __builtin_amdgcn_permlane16_swap(b, b, false, false);
  x = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  const u32 c = __float_as_uint(x);
  const auto t = __builtin_amdgcn_permlane32_swap(c, c, false, false);
  return __uint_as_float(t[0]) + __uint_as_float(t[1]);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Per-lane data of one 32-token step (codes and per-token value scale / zero).
template <int KW, int VW, int NVM>
struct StepData {
  u32 k0[KW], k1[KW], v[VW];
  float vs[NVM], vz[NVM];
  __device__ void zero_meta() {
#pragma unroll
    for (int i = 0; i < NVM; ++i) { vs[i] = 0.0f; vz[i] = 0.0f; }
  }
};

}  // namespace mf

using namespace mf;

// One decode-attention pass-1 work-group.  KF/VF: key/value code format;
// ROPE: keys cached before RoPE; VG: value channel groups (INT values);
// PV2: 32 PV rows (8 heads x 4 value groups) in two A operands of 16 rows;
// KSPLIT: rotated keys enter the matrix unit as hi + lo fp16 halves.
// D = 128, n_rep <= 8 (<= 16 with one value group).
template <int KF, int VF, bool ROPE, int VG, bool KSPLIT, bool PV2>
__global__ void __launch_bounds__(256)
#if KVQ_MFMA_WAVES_PER_EU > 0
__attribute__((amdgpu_waves_per_eu(KVQ_MFMA_WAVES_PER_EU, KVQ_MFMA_WAVES_PER_EU)))
#endif
attn_mfma(Plan p, Args a) {
  constexpr int D = 128;
  constexpr int KB = Bits<KF>::v, VB = Bits<VF>::v;
  constexpr int KDW = KB;                 // dwords of key data per lane (32 channels)
  constexpr int VDW = 2 * VB;             // dwords of value data per lane per 32-token block
  constexpr bool KINT = !is_f8(KF), VINT = !is_f8(VF);
  constexpr int VGC = D / VG;             // value channels per group

  // Per-wavefront LDS ring of NB stages; a stage holds one 32-token step:
  // key rows, the value block, value scale/zero, the key group's scale/zero
  // rows and (pre-RoPE keys) the step's coarse cos/sin row.
  constexpr int KROW = D * KB / 8;
  constexpr int SZ_K = 32 * KROW, SZ_V = 32 * D * VB / 8;
  // (pre-RoPE FP8 keys: no key metadata, but the region holds the step's pair coefficients)
  constexpr int SZ_VM = VINT ? 2 * 32 * VG * 4 : 0, SZ_KM = (KINT || ROPE) ? 2 * D * 4 : 0, SZ_KT = ROPE ? 64 * 8 : 0;
  constexpr int OFF_V = SZ_K, OFF_VM = OFF_V + SZ_V, OFF_KM = OFF_VM + SZ_VM, OFF_KT = OFF_KM + SZ_KM;
  constexpr int SLOT = OFF_KT + SZ_KT;
  // query rows: up to 16 heads per kv head with one value group (the PV rows
  // are then the heads), 8 otherwise
  constexpr int QROWS = VG == 1 ? 16 : 8;
  // Stages per wavefront: 3 (2 for slots over 6 KB), but no more than keep
  // two work-groups on a CU (80 KB of LDS each, with the query rows, the RoPE
  // table and the reduction scratch), at least 2, and enough to hold the
  // wavefront's O rows after the loop.
  constexpr int LDS_FIXED = QROWS * D * 4 + (ROPE ? 64 * 32 * 8 : 8) + kWaves * QROWS * 2 * 4;
  // (1.5 KB kept free: the page table of paged calls is dynamic LDS)
  constexpr int NB_FIT = (80 * 1024 - 1536 - LDS_FIXED) / (kWaves * SLOT);
  constexpr int NB_DEF = SLOT <= 6144 ? 3 : 2;
  constexpr int NB_LDS = NB_FIT < NB_DEF ? (NB_FIT > 2 ? NB_FIT : 2) : NB_DEF;
  constexpr int NB_O = (QROWS * D * 4 + SLOT - 1) / SLOT;
  constexpr int NB = KVQ_MFMA_STAGES > 0 ? KVQ_MFMA_STAGES : (NB_LDS > NB_O ? NB_LDS : NB_O);
  constexpr int N_DMA = SZ_K / 1024 + SZ_V / 1024 + (SZ_VM + 1023) / 1024 + (KINT ? 1 : 0) + (ROPE ? 1 : 0);
  static_assert(SZ_K % 1024 == 0 && SZ_V % 1024 == 0 && NB * SLOT >= (VG == 1 ? 16 : 8) * D * 4,
                "stage layout (a wavefront's ring holds its O rows after the loop)");

  __shared__ float q_s[QROWS][D];
  // fine RoPE table, pair-major with the token offset XOR-swizzled by the
  // lane row so that one row's 16 lanes (16 offsets, one pair) hit distinct banks
  __shared__ float2 fine_s[ROPE ? 64 : 1][ROPE ? 32 : 1];
  // the rings; after the streaming loop a wavefront's ring holds its O rows
  __shared__ __attribute__((aligned(16))) uint8_t ring_s[kWaves][NB * SLOT];
  __shared__ float red_ml[kWaves][QROWS][2];
  // page ids of this split's token blocks (paged caches; dynamic LDS)
  extern __shared__ int32_t page_s[];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = tid >> 6;
  const int n = lane & 15, g = lane >> 4;
  const int split = blockIdx.x, kvh = blockIdx.y / a.ngroups, b = blockIdx.z;
  // this work-group's query heads: hb .. hb + n_rep - 1 of the kv head's p.n_rep
  const int hb = (blockIdx.y - kvh * a.ngroups) * a.hg;
  const int n_rep = a.hg < p.n_rep - hb ? a.hg : p.n_rep - hb;
  const int64_t hq0 = (int64_t)b * p.Hq + (int64_t)kvh * p.n_rep + hb;   // first query head
  const int64_t bh = (int64_t)b * p.Hkv + kvh;
  const uint8_t* arena = a.arena;
  // tokens of this sequence (ragged batches: from its length)
  int64_t T = a.T, Tq = a.Tq;
  if (a.seq_lens) {
    int64_t tl = (int64_t)a.seq_lens[b] + a.lens_add;
    tl = tl < 0 ? 0 : (tl > a.T ? a.T : tl);
    T = tl;
    Tq = quantized_tokens(p, tl);
  }
  const bool paged = a.pm.bt != nullptr;
  const int64_t lo = (int64_t)split * a.chunk;
  const int64_t hi = lo + a.chunk < T ? lo + a.chunk : T;
  const int64_t blk0 = lo / p.P;          // first page-table block of this split

  // decode step: append the new token of this (sequence, kv head) first when
  // it falls in this split (threads 0..D-1 write its key, D..2D-1 its value),
  // exactly as the append kernels do; the stores complete before the barrier
  // below, ahead of every read of the cache by this work-group.
  if (a.app_mode != 0 && a.t_new >= (int64_t)split * a.chunk && a.t_new < (int64_t)split * a.chunk + a.chunk &&
      tid < 2 * D) {
    const bool is_v = tid >= D;
    const int c = is_v ? tid - D : tid;
    const int64_t t = a.t_new;
    const float x = load_in(is_v ? a.v_new : a.k_new, bh * D + c, p.in_dtype);
    if (a.app_mode == 1) {
      const int64_t slot = t % p.Rs;
      if (!is_v) {
        ((_Float16*)(a.arena_w + p.ring_k))[(bh * p.Rs + slot) * D + c] = (_Float16)x;
      } else {
        const int rblock = kVBlock * D * 2;
        uint8_t* base = a.arena_w + p.ring_v + (uint64_t)bh * (p.Rs / kVBlock) * rblock;
        ((_Float16*)(base + vblock_word_byte(slot, c, D, 16, rblock)))[slot & 7] = (_Float16)x;
      }
    } else {
      const SideFmt& f = is_v ? p.v : p.k;
      const float s = ((const float*)(a.arena_w + f.scale))[kvh];
      const uint8_t code = (uint8_t)(f.scheme == KVQ_FP8_E4M3 ? e4m3_encode(x / s) : e5m2_encode(x / s));
      if (!is_v) a.arena_w[p.k.codes + (bh * p.Tc + t) * p.k_row_bytes + c] = code;
      else a.arena_w[p.v.codes + bh * p.v_nblk * p.v_block_bytes + vblock_word_byte(t, c, D, 8, p.v_block_bytes) + (t & 7)] = code;
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  }
  for (int e = tid; e < n_rep * D; e += 256) {
    const int r = e / D, c = e % D;
    q_s[r][c] = load_in(a.q, (hq0 + r) * D + c, p.in_dtype) * a.qscale;
  }
  if (paged && hi > lo) {
    const int64_t nblk = (hi - 1) / p.P - blk0 + 1;   // <= kMaxSplitPages (split count)
    for (int64_t j = tid; j < nblk && j < kMaxSplitPages; j += 256) {
      const int32_t pg = page_of(p, a.pm, b, (blk0 + j) * p.P);
      page_s[j] = pg < 0 ? 0 : pg;
    }
  }
  if constexpr (ROPE) {
    const float2* tab = (const float2*)(arena + p.rope);
    for (int e = tid; e < 32 * 64; e += 256) {
      const int dlt = e >> 6, pr = e & 63;
      fine_s[pr][dlt ^ (4 * ((pr >> 4) & 3))] = tab[e];
    }
  }
  __syncthreads();

  // token range of this split and of this wavefront
  const int64_t q_end = hi < Tq ? hi : Tq;                     // quantized part [lo, q_end)
  const int64_t w_beg = lo > Tq ? lo : Tq;                     // window part [w_beg, hi)
  const int64_t nq = q_end > lo ? (q_end - lo + 31) / 32 : 0;  // quantized steps
  const int64_t s_w0 = w_beg & ~(int64_t)31;
  const int64_t nw = hi > w_beg ? (hi - s_w0 + 31) / 32 : 0;   // window steps
  const int64_t nsteps = nq + nw;
  // Steps of this wavefront: FP8 caches (nothing per key group) take every
  // kWaves-th step, so that the work-group streams one contiguous run of the
  // cache; other formats take a contiguous block of steps (key groups span
  // consecutive steps).
  constexpr bool IL = !KINT && !VINT;
  constexpr int64_t STRIDE = IL ? kWaves : 1;
  const int64_t per_wave = (nsteps + kWaves - 1) / kWaves;
  const int64_t st_beg = IL ? wave : wave * per_wave;
  const int64_t st_end = IL ? nsteps : (st_beg + per_wave < nsteps ? st_beg + per_wave : nsteps);

  // query columns: column n is head n mod n_rep (hi and lo fp16 halves of the
  // fp32 query in two operands).  Lane (n, g) is A row n of PV: value group
  // n / n_rep (rows past the last group are computed and never read).
  const int head = n % n_rep;
  const int vgrp = (n / n_rep) < VG ? n / n_rep : VG - 1;
  // PV2 (n_rep = 8, VG = 4): the second A operand's row n is value group vgrp + 2
  static_assert(!PV2 || VG == 4, "two PV row halves need four value groups");

  half8 Bq[4], Bl[4];   // query operand (hi, lo) of the current key group / window
  float kbias = 0.0f;   // per-column logit bias from the key zero-points
  bool new_kgrp = true;  // the step being computed starts a key group (or is the first)
  int b_mode = -1;      // 0: quantized keys, 1: window keys

  // Bq/Bl for per-channel factors sc (or a uniform factor); returns this
  // lane's part of sum_c q_c z_c
  auto build_b = [&](const float* sc, const float* zc, float uniform, bool natural) __attribute__((always_inline)) {
    float qz = 0.0f;
    // this lane's 32 channel scales / zero-points, fetched with wide loads up front
    float sv[32], zv[32];
    if (sc) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float4 a4 = ((const float4*)sc)[km_pos(8 * g + i)], b4 = ((const float4*)zc)[km_pos(8 * g + i)];
        sv[4 * i] = a4.x; sv[4 * i + 1] = a4.y; sv[4 * i + 2] = a4.z; sv[4 * i + 3] = a4.w;
        zv[4 * i] = b4.x; zv[4 * i + 1] = b4.y; zv[4 * i + 2] = b4.z; zv[4 * i + 3] = b4.w;
      }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      u32 rh[4], rl[4];
#pragma unroll
      for (int e2 = 0; e2 < 4; ++e2) {
        float full[2];
#pragma unroll
        for (int hlf = 0; hlf < 2; ++hlf) {
          const int e = 2 * e2 + hlf;
          const int cl = natural ? 8 * j + e : kslot<KF, ROPE>(j, e);
          const float qv = q_s[head][32 * g + cl];   // already times the logit scale
          full[hlf] = qv * (sc ? sv[cl] : uniform);
          if (sc) qz = __builtin_fmaf(qv, zv[cl], qz);
        }
        rh[e2] = pk_f16(full[0], full[1]);
        rl[e2] = f16_residual2(rh[e2], full[0], full[1], a.neg1);
      }
      Bq[j] = pack8(rh[0], rh[1], rh[2], rh[3]);
      Bl[j] = pack8(rl[0], rl[1], rl[2], rl[3]);
    }
    return qz;
  };

  // softmax / output state (lane (n, g): head n for n < n_rep)
  float m_run = kNegBig, l_run = 0.0f;
  float vbias = 0.0f;   // sum_t p_t z_t of this lane's PV row
  float vbias1 = 0.0f;  // the same for the lane's row of the second half (PV2)
  floatx4 O[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) O[i] = floatx4{0.f, 0.f, 0.f, 0.f};

  const float k_fp8 = is_f8(KF) ? ((const float*)(arena + p.k.scale))[kvh] : 1.0f;
  const float v_fp8 = is_f8(VF) ? ((const float*)(arena + p.v.scale))[kvh] : 1.0f;
  uint8_t* const ring = ring_s[wave];
  const u32 ring_lds = (u32)(size_t)(__attribute__((address_space(3))) uint8_t*)&ring_s[0][0] + wave * (NB * SLOT);

  const int tok_in0 = 8 * (n >> 2) + (n & 3);   // A row n -> token of tile 0 (+4 for tile 1)

  // Stage of a quantized step: issue its loads straight into LDS slot sl.
  // Each lane keeps one global pointer per stream, set at the wavefront's
  // first quantized step and advanced by constant strides (the key-metadata
  // pointer by one row when a key group ends).
  const uint8_t *pk = nullptr, *pv = nullptr, *pvm0 = nullptr, *pvm1 = nullptr, *pkm = nullptr, *prp = nullptr;
  // fp16 scale / zero-point metadata: the stage brings the two fp16 rows
  // (scales, then zero-points, natural order) into the first half of the
  // slot's metadata region and widen_meta rebuilds the fp32 granule layout
  // below from them once the stage has landed
  const bool vm16 = VINT && p.v.meta16, km16 = KINT && p.k.meta16;
  const int vesz = vm16 ? 2 : 4, kesz = km16 ? 2 : 4;
  // page the issue side is in and the first token past it (paged caches): the
  // step loop compares against page_end instead of dividing by P every step
  int64_t page_end = 0, page_j = 0;
  // stream pointers of the step whose first token sits in token row tr, with
  // its key group's metadata in row krow
  auto set_ptrs = [&](int64_t tr, int64_t krow) __attribute__((always_inline)) {
    pk = arena + p.k.codes + tr * KROW + 16 * lane;
    pv = arena + p.v.codes + (tr >> 5) * SZ_V + 16 * lane;
    if constexpr (VINT) {
      // 16-byte granules: 8*VG of scales, then 8*VG of zero-points
      const uint8_t* vs = arena + p.v.scale + tr * VG * vesz;
      const uint8_t* vz = arena + p.v.zero + tr * VG * vesz;
      if (vm16) {
        // 4*VG granules of each fp16 row
        if constexpr (VG == 8) {
          pvm0 = vs + 16 * lane;
          pvm1 = vz + 16 * lane;
        } else {
          pvm0 = lane < 4 * VG ? vs + 16 * lane : vz + 16 * (lane - 4 * VG);
        }
      } else if constexpr (VG == 8) {
        pvm0 = vs + 16 * lane;
        pvm1 = vz + 16 * lane;
      } else {
        if constexpr (VG == 4) pvm0 = lane < 32 ? vs + 16 * vm_src(lane) : vz + 16 * vm_src(lane - 32);
        else pvm0 = lane < 8 * VG ? vs + 16 * lane : vz + 16 * (lane - 8 * VG);
      }
    }
    if constexpr (KINT) {
      // scale row (lanes 0-31) and zero-point row (lanes 32-63) of the key
      // group; fp16 rows: lanes 0-15 and 16-31
      const int64_t mrow = krow * D * kesz;
      if (km16) pkm = lane < 16 ? arena + p.k.scale + mrow + 16 * lane : arena + p.k.zero + mrow + 16 * (lane - 16);
      else pkm = lane < 32 ? arena + p.k.scale + mrow + 16 * km_pos(lane)
                           : arena + p.k.zero + mrow + 16 * km_pos(lane - 32);
    }
  };
  auto init_ptrs = [&](int64_t t0) __attribute__((always_inline)) {
    // token row of t0: through this split's page table, or (b, h)'s own rows
    int64_t tr;
    if (paged) {
      // every issued step lies below the split's end, inside the table; the
      // clamp only keeps set-up lookups of unused pointers inside the array
      const int64_t j = t0 / p.P;
      page_j = j;
      page_end = (j + 1) * p.P;
      int64_t jj = j - blk0;
      jj = jj < 0 ? 0 : (jj > kMaxSplitPages - 1 ? kMaxSplitPages - 1 : jj);
      tr = ((int64_t)page_s[jj] * p.Hkv + kvh) * p.P + (t0 - j * p.P);
    } else {
      tr = bh * p.Tc + t0;
    }
    set_ptrs(tr, KINT ? tr / p.k.group : 0);
    if constexpr (ROPE) prp = arena + p.rope + ((32 + (t0 >> 5)) * 64) * 8 + 16 * lane;
  };
  // key-group rows per page (pages hold whole key groups)
  const int64_t page_groups = KINT && paged ? p.P / p.k.group : 0;
  // The issue side has passed page_end (paged caches): the pointers of the
  // page it entered, with no division.  Steps of caches with per-group key
  // metadata advance 32 tokens at a time and pages are whole multiples of 32
  // tokens, so such a step enters its page at the page's first token, where
  // a key group starts; interleaved FP8 steps may enter further in.
  auto next_page = [&](int64_t t0) __attribute__((always_inline)) {
    do {
      ++page_j;
      page_end += p.P;
    } while (t0 >= page_end);
    int64_t jj = page_j - blk0;
    jj = jj < 0 ? 0 : (jj > kMaxSplitPages - 1 ? kMaxSplitPages - 1 : jj);
    const int64_t base = (int64_t)page_s[jj] * p.Hkv + kvh;
    set_ptrs(base * p.P + (t0 - (page_end - p.P)), base * page_groups);
  };
  auto issue = [&](int sl) __attribute__((always_inline)) {
    const u32 sb = __builtin_amdgcn_readfirstlane(ring_lds + sl * SLOT);
#pragma unroll
    for (int c = 0; c < SZ_K / 1024; ++c) dma16(sb + 1024 * c, pk + 1024 * c);
#pragma unroll
    for (int c = 0; c < SZ_V / 1024; ++c) dma16(sb + OFF_V + 1024 * c, pv + 1024 * c);
    if constexpr (VINT) {
      if constexpr (VG == 8) {
        if (!vm16) {
          dma16(sb + OFF_VM, pvm0);
          dma16(sb + OFF_VM + 1024, pvm1);
        } else if (lane < 32) {
          dma16(sb + OFF_VM, pvm0);
          dma16(sb + OFF_VM + 512, pvm1);
        }
      } else if (lane < (vm16 ? 8 : 16) * VG) {
        dma16(sb + OFF_VM, pvm0);
      }
    }
    if constexpr (KINT) {
      if (!km16 || lane < 32) dma16(sb + OFF_KM, pkm);
    }
    if constexpr (ROPE) {
      if (lane < 32) dma16(sb + OFF_KT, prp);
    }
  };
  auto advance_ptrs = [&](bool group_ends) __attribute__((always_inline)) {
    pk += SZ_K * STRIDE;
    pv += SZ_V * STRIDE;
    if constexpr (VINT) {
      pvm0 += 32 * VG * vesz;
      if constexpr (VG == 8) pvm1 += 32 * VG * vesz;
    }
    if constexpr (KINT) { if (group_ends) pkm += D * kesz; }
    if constexpr (ROPE) prp += 64 * 8 * STRIDE;
  };
  // Registers of a quantized step from its LDS slot.
  auto read_slot = [&](int sl, StepData<KDW, VDW, VINT ? 8 : 1>& d) __attribute__((always_inline)) {
    const uint8_t* st_l = ring + sl * SLOT;
    const uint8_t* kr = st_l + tok_in0 * KROW + g * (4 * KDW);
    load_dw<KDW>(kr, d.k0);
    load_dw<KDW>(kr + 4 * KROW, d.k1);
    load_dw<VDW>(st_l + OFF_V + lane * (4 * VDW), d.v);
    if constexpr (VINT) {
      const float* sp = (const float*)(st_l + OFF_VM) + 8 * g * VG + vgrp;
      const float* zp = sp + 32 * VG;
      if constexpr (VG == 1) {
        const float4 s0 = ((const float4*)sp)[0], s1 = ((const float4*)sp)[1];
        const float4 z0 = ((const float4*)zp)[0], z1 = ((const float4*)zp)[1];
        d.vs[0] = s0.x; d.vs[1] = s0.y; d.vs[2] = s0.z; d.vs[3] = s0.w;
        d.vs[4] = s1.x; d.vs[5] = s1.y; d.vs[6] = s1.z; d.vs[7] = s1.w;
        d.vz[0] = z0.x; d.vz[1] = z0.y; d.vz[2] = z0.z; d.vz[3] = z0.w;
        d.vz[4] = z1.x; d.vz[5] = z1.y; d.vz[6] = z1.z; d.vz[7] = z1.w;
      } else {
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          if constexpr (VG == 4) {
            const float* vm = (const float*)(st_l + OFF_VM) + 4 * vm_pos(8 * g + k) + vgrp;
            d.vs[k] = vm[0];
            d.vz[k] = vm[128];
          } else {
            d.vs[k] = sp[k * VG];
            d.vz[k] = zp[k * VG];
          }
        }
      }
    }
  };
  int cur_slot = 0;   // slot of the quantized step being computed
  auto load_r = [&](int64_t t0, StepData<16, 32, 1>& d) __attribute__((always_inline)) {
    load_dw<16>(arena + p.ring_k + ((bh * p.Rs + ((t0 + tok_in0) % p.Rs)) * D + 32 * g) * 2, d.k0);
    load_dw<16>(arena + p.ring_k + ((bh * p.Rs + ((t0 + tok_in0 + 4) % p.Rs)) * D + 32 * g) * 2, d.k1);
    load_dw<32>(arena + p.ring_v + (bh * (p.Rs / 32) + ((t0 % p.Rs) >> 5)) * (32 * D * 2) + lane * 128, d.v);
  };

  // One 32-token step: tokens [t0, t0 + 32), valid within [v_lo, v_hi).
  // RING: tokens from the fp16 window; FULL: every token of the step is valid.
  auto step = [&](auto ring_tag, auto full_tag, int64_t t0, int64_t v_lo, int64_t v_hi, const auto& d) __attribute__((always_inline)) {
    constexpr bool RING = decltype(ring_tag)::value;
    constexpr bool FULL = decltype(full_tag)::value;

    // ---- query operand of this step ---------------------------------------------
    if constexpr (!RING) {
      if constexpr (KINT && !ROPE) {
        if (b_mode != 0 || new_kgrp) {
          const float* sc = (const float*)(ring + cur_slot * SLOT + OFF_KM);   // granules at km_pos
          const float* zc = sc + D;
          kbias = wave_sum16(build_b(sc, zc, 1.0f, false));
          b_mode = 0;
        }
      } else if (b_mode != 0) {
        build_b(nullptr, nullptr, k_fp8, !(ROPE && KF == INT2));
        kbias = 0.0f;
        b_mode = 0;
      }
    } else if (b_mode != 1) {
      build_b(nullptr, nullptr, 1.0f, true);
      kbias = 0.0f;
      b_mode = 1;
    }

    // ---- S^T = K . Q^T for the two 16-token tiles ----------------------------
    floatx4 S[2];
    if constexpr (ROPE) {
      const float2* crow = (const float2*)(arena + p.rope) + (32 + (t0 >> 5)) * 64 + 16 * g;
      // the coefficients of this lane group's 16 pairs in the step's slot, in
      // pair order: one base per step, each pair's read an immediate offset
      // from it (lane group g reads pairs 16g..16g+15; the 16 lanes of a group
      // read one address, a broadcast)
      const float4* uvb = (const float4*)(ring + cur_slot * SLOT + OFF_KM) + 16 * g;
      const float2* wvb = (const float2*)(ring + cur_slot * SLOT + OFF_KT) + 16 * g;
      floatx4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        // Pairs of this k-step (first channel cp[pr], lane-local): natural
        // (8j + 2pr), or for INT2 codes the channels b, b+2, b+8, b+10 with
        // b = 16 (j >> 1) + 4 (j & 1), whose rotated values pack as (c, c+8).
        constexpr bool C8 = KF == INT2 && !RING;
        int cp[4];
#pragma unroll
        for (int pr = 0; pr < 4; ++pr)
          cp[pr] = C8 ? 16 * (j >> 1) + 4 * (j & 1) + 2 * (pr & 1) + 8 * (pr >> 1) : 8 * j + 2 * pr;
        // quantized steps: the pairs' coefficients; window steps: their coarse angles
        float4 uv[4];
        float2 wv[4], cc[4];
#pragma unroll
        for (int pr = 0; pr < 4; ++pr) {
          if constexpr (!RING) {
            uv[pr] = uvb[cp[pr] >> 1];
            wv[pr] = wvb[cp[pr] >> 1];
          } else {
            cc[pr] = crow[cp[pr] >> 1];
          }
        }
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const u32* w = u ? d.k1 : d.k0;
          const int dt = tok_in0 + 4 * u;               // token offset in the step (t0 is 32-aligned)
          float rx[4], ry[4];
#pragma unroll
          for (int pr = 0; pr < 4; ++pr) {
            const int e = cp[pr];
            const float2 ff = fine_s[16 * g + (e >> 1)][dt ^ (4 * g)];
            float r0, r1;
            if constexpr (!RING) {
              // coarse-rotated pair from its codes, then the fine rotation
              float cx, cy;
              if constexpr (C8) {
                const u32 h0 = int2_pos_reg(w[e >> 4], e & 7), h1 = int2_pos_reg(w[e >> 4], (e & 7) + 1);
                cx = (e >> 3) & 1 ? hi_f(h0) : lo_f(h0);
                cy = (e >> 3) & 1 ? hi_f(h1) : lo_f(h1);
              } else {
                const u32 c0 = key_code_reg<KF>(w, code_reg<KF>(e)), c1 = key_code_reg<KF>(w, code_reg<KF>(e + 1));
                cx = code_half<KF>(e) ? hi_f(c0) : lo_f(c0);
                cy = code_half<KF>(e + 1) ? hi_f(c1) : lo_f(c1);
              }
              const float px = __builtin_fmaf(cx, uv[pr].x, __builtin_fmaf(cy, uv[pr].z, wv[pr].x));
              const float py = __builtin_fmaf(cx, uv[pr].y, __builtin_fmaf(cy, uv[pr].w, wv[pr].y));
              r0 = px * ff.x - py * ff.y;
              r1 = px * ff.y + py * ff.x;
            } else {
              const float k0 = lo_f(w[e >> 1]), k1 = hi_f(w[e >> 1]);
              const float cs = cc[pr].x * ff.x - cc[pr].y * ff.y;
              const float sn = cc[pr].y * ff.x + cc[pr].x * ff.y;
              r0 = k0 * cs - k1 * sn;
              r1 = k0 * sn + k1 * cs;
            }
            rx[pr] = r0;
            ry[pr] = r1;
          }
          // operand registers: natural (pair pr in register pr) or (c, c+8)
          float lo_v[4], hi_v[4];
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            if constexpr (C8) {
              const int pa = q >> 1;                     // pairs pa (low halves) and pa + 2 (high halves)
              lo_v[q] = q & 1 ? ry[pa] : rx[pa];
              hi_v[q] = q & 1 ? ry[pa + 2] : rx[pa + 2];
            } else {
              lo_v[q] = rx[q];
              hi_v[q] = ry[q];
            }
          }
          u32 r[4], rl[4];
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            r[q] = pk_f16(lo_v[q], hi_v[q]);
            if constexpr (KSPLIT) rl[q] = f16_residual2(r[q], lo_v[q], hi_v[q], a.neg1);
          }
          floatx4& acc = u ? acc1 : acc0;
          const half8 ah = pack8(r[0], r[1], r[2], r[3]);
          acc = mfma(ah, Bq[j], acc);
          acc = mfma(ah, Bl[j], acc);
          if constexpr (KSPLIT) acc = mfma(pack8(rl[0], rl[1], rl[2], rl[3]), Bq[j], acc);
        }
        // keep the scheduler from hoisting every k-step's LDS reads at once
        // (register pressure): one k-step's operands are live at a time
        __builtin_amdgcn_sched_barrier(0);
      }
      S[0] = acc0;
      S[1] = acc1;
    } else {
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const u32* w = u ? d.k1 : d.k0;
        half8 A[4];
        if constexpr (RING) {
#pragma unroll
          for (int j = 0; j < 4; ++j) A[j] = pack8(w[4 * j], w[4 * j + 1], w[4 * j + 2], w[4 * j + 3]);
        } else if constexpr (is_f8(KF)) {
          unpack_k_f8<KF>(w, A);
        } else {
          unpack_k_codes<KF>(w, A);
        }
        floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          acc = mfma(A[j], Bq[j], acc);
          acc = mfma(A[j], Bl[j], acc);
        }
        S[u] = acc;
      }
    }

    // ---- logits of lane (n, g): head n, tokens 8g + k -------------------------
    // Lanes n >= n_rep compute rows that are never read; they are left unmasked.
    float x[8];
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int i = 0; i < 4; ++i) x[4 * u + i] = ROPE ? S[u][i] : S[u][i] + kbias;   // pre-RoPE: zero-points sit in the pair coefficients
    u32 valid = 0xFFu;
    if constexpr (!FULL) {
      valid = 0;
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int64_t t = t0 + 8 * g + k;
        const bool ok = t >= v_lo && t < v_hi;
        valid |= (ok ? 1u : 0u) << k;
        if (!ok) x[k] = kNegBig;
      }
    }

    // ---- online softmax (accumulators rescaled only when a running max rises) ----
    float mx = x[0];
#pragma unroll
    for (int k = 1; k < 8; ++k) mx = fmaxf(mx, x[k]);
    mx = wave_max16(mx);
    if (__any(mx > m_run)) {
      const float m_new = fmaxf(m_run, mx);
      const float alpha = fast_exp2(m_run - m_new);
      m_run = m_new;
      l_run *= alpha;
      vbias *= alpha;
      if constexpr (PV2) vbias1 *= alpha;
      float al[4];    // lane (c, g') holds rows (heads) 4g'+i
#pragma unroll
      for (int i = 0; i < 4; ++i) al[i] = __shfl(alpha, (4 * g + i) & 15, 64);
#pragma unroll
      for (int t8 = 0; t8 < 8; ++t8)
#pragma unroll
        for (int i = 0; i < 4; ++i) O[t8][i] *= al[i];
    }
    float pk[8], psum = 0.0f;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      pk[k] = fast_exp2(x[k] - m_run);
      if constexpr (!FULL) pk[k] = ((valid >> k) & 1u) ? pk[k] : 0.0f;
      psum += pk[k];
    }
    l_run += psum;

    // ---- PV -------------------------------------------------------------------------
    if constexpr (!RING && VINT) {
      // A = p * s as hi + lo fp16 halves (lo = exact residual by FMA); z enters
      // through the row's bias
      auto build_a = [&](const float* vs, const float* vz, half8& Ah, half8& Al) __attribute__((always_inline)) {
        u32 rh[4], rl[4];
        float zsum = 0.0f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float sv[2], pv[2];
#pragma unroll
          for (int hlf = 0; hlf < 2; ++hlf) {
            const int k = vtok<VF>(2 * i + hlf);
            sv[hlf] = vs[k];
            pv[hlf] = pk[k];
            float zt = vz[k];
            if constexpr (!FULL) {
              const bool ok = (valid >> k) & 1u;
              sv[hlf] = ok ? sv[hlf] : 0.0f;
              zt = ok ? zt : 0.0f;
            }
            zsum = __builtin_fmaf(pv[hlf], zt, zsum);
          }
          rh[i] = pk_f16(pv[0] * sv[0], pv[1] * sv[1]);
          rl[i] = pk_f16(__builtin_fmaf(pv[0], sv[0], -lo_f(rh[i])), __builtin_fmaf(pv[1], sv[1], -hi_f(rh[i])));
        }
        Ah = pack8(rh[0], rh[1], rh[2], rh[3]);
        Al = pack8(rl[0], rl[1], rl[2], rl[3]);
        return zsum;
      };
      half8 Ah, Al;
      vbias += build_a(d.vs, d.vz, Ah, Al);
#pragma unroll
      for (int i = 0; i < (PV2 ? 4 : 8); ++i) {
        const half8 bv = unpack_v<VF>(d.v, i);
        O[i] = mfma(Ah, bv, O[i]);
        O[i] = mfma(Al, bv, O[i]);
      }
      if constexpr (PV2) {
        // second half: value groups 2, 3 (tiles 4-7), metadata read from the slot
        float vs1[8], vz1[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          const float* vm = (const float*)(ring + cur_slot * SLOT + OFF_VM) + 4 * vm_pos(8 * g + k) + vgrp + 2;
          vs1[k] = vm[0];
          vz1[k] = vm[128];
        }
        vbias1 += build_a(vs1, vz1, Ah, Al);
#pragma unroll
        for (int i = 4; i < 8; ++i) {
          const half8 bv = unpack_v<VF>(d.v, i);
          O[i] = mfma(Ah, bv, O[i]);
          O[i] = mfma(Al, bv, O[i]);
        }
      }
    } else {
      // FP8 values: A = p * v_scale; window values: A = p
      const float vsc = (!RING && is_f8(VF)) ? v_fp8 : 1.0f;
      u32 r[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) r[i] = pk_f16(pk[i] * vsc, pk[i + 4] * vsc);
      const half8 Ap = pack8(r[0], r[1], r[2], r[3]);
      u32 vv = 0xFFu;
      if constexpr (!FULL) vv = __shfl(valid, 16 * g, 64);   // validity of the B lane's tokens
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        half8 bv;
        if constexpr (RING) bv = unpack_v_f16(d.v, i);
        else bv = unpack_v<VF>(d.v, i);
        // bytes of invalid tokens may not be finite values: zero them
        if constexpr (!FULL) bv = mask_tokens(bv, vv);
        O[i] = mfma(Ap, bv, O[i]);
      }
    }
  };

  auto qstep = [&](int64_t st, const StepData<KDW, VDW, VINT ? 8 : 1>& d) __attribute__((always_inline)) {
    const int64_t t0 = lo + st * 32;
    if (t0 + 32 <= q_end) step(std::false_type{}, std::true_type{}, t0, lo, q_end, d);
    else step(std::false_type{}, std::false_type{}, t0, lo, q_end, d);
  };

  const int64_t qs_end = st_end < nq ? st_end : nq;
  // pre-RoPE INT2 keys: position factors 2^(10 - p) of channel pair `lane` (channels 2 lane, 2 lane + 1)
  const float2 pf = make_float2((float)(1 << (10 - int2_pos(2 * (lane & 3)))), (float)(1 << (10 - int2_pos(2 * (lane & 3) + 1))));
  {
    // Streaming loop: NB - 1 stages in flight; a stage is consumed (waited
    // for, read into registers), the next stage is issued into the slot freed
    // by the previous step, then the step is computed.
    // Key groups are tracked incrementally (one division up front): the
    // issue side (position i_pos, offset i_rem in its key group) and the
    // compute side (c_rem) each advance by one 32-token step per iteration.
    const int64_t qs_beg = st_beg < qs_end ? st_beg : qs_end;
    const int kG = KINT ? p.k.group : 32;
    int64_t i_pos = lo + qs_beg * 32;
    int i_rem = (int)(i_pos % kG);
    int c_rem = i_rem;
    const int64_t iss_end = lo + qs_end * 32;   // this wavefront's quantized steps only
    init_ptrs(i_pos);
    auto next_issue = [&](int sl_) __attribute__((always_inline)) {
      if (i_pos < iss_end) issue(sl_);
      if constexpr (IL) {
        i_pos += 32 * STRIDE;      // kG = 32: one step per group, i_rem stays 0
        advance_ptrs(true);
      } else {
        i_pos += 32;
        i_rem += 32;
        const bool ends = i_rem == kG;
        if (ends) i_rem = 0;
        advance_ptrs(ends);
      }
      // a paged cache continues on another page: pointers from the page table
      // (steps only move forward, so leaving the page means passing its end)
      if (paged) {
        if (i_pos < iss_end && i_pos >= page_end) next_page(i_pos);
      }
    };
#pragma unroll
    for (int i = 0; i < NB - 1; ++i) next_issue(i);
    int sl = 0;
    for (int64_t st = qs_beg; st < qs_end; st += STRIDE) {
      // stages of steps st, st + STRIDE, ... (those below qs_end) are in flight
      if (st + (NB - 2) * STRIDE < qs_end) wait_vmem<N_DMA * (NB - 2)>();
      else wait_vmem<0>();
      if constexpr (VINT) {
        if (vm16) widen_meta<VG == 8 ? 128 : 16 * VG, VG == 4 ? 2 : 0>(ring + sl * SLOT + OFF_VM, lane);
      }
      if constexpr (KINT) {
        if (km16) widen_meta<64, 1>(ring + sl * SLOT + OFF_KM, lane);
      }
      StepData<KDW, VDW, VINT ? 8 : 1> d;
      read_slot(sl, d);
      cur_slot = sl;
      if constexpr (ROPE) {
        // Lane i: channel pair i.  A pre-RoPE key pair of this step is
        // (x, y) = (sx cx + zx, sy cy + zy); rotating it by the step's coarse
        // angle (C, S) gives cx u + cy v + w with u = sx (C, S),
        // v = sy (-S, C), w = (C zx - S zy, S zx + C zy).  Each (token, pair)
        // then needs four FMAs and the fine rotation by its offset in the step.
        // The coefficients replace the key-metadata and coarse rows in the
        // slot: (u, v) over the 1 KB scale/zero rows, w over the coarse row.
        uint8_t* st_l = ring + sl * SLOT;
        const float2 cs2 = ((const float2*)(st_l + OFF_KT))[lane];
        const int mo = 16 * km_pos(lane >> 1) + 8 * (lane & 1);
        // FP8 keys: codes are the values (s = 1, z = 0); the per-head scale
        // sits in the query operand
        float2 s2 = make_float2(1.0f, 1.0f), z2 = make_float2(0.0f, 0.0f);
        if constexpr (KINT) {
          s2 = *(const float2*)(st_l + OFF_KM + mo);
          z2 = *(const float2*)(st_l + OFF_KM + 4 * D + mo);
        }
        asm volatile("" ::: "memory");   // every lane's reads before any lane's writes
        if constexpr (KF == INT2) {
          // codes arrive as 1 + c 2^(p - 10): x = s c + z = (s f) h + (z - s f), f = 2^(10 - p)
          s2.x *= pf.x;
          s2.y *= pf.y;
          z2.x -= s2.x;
          z2.y -= s2.y;
        }
        ((float4*)(st_l + OFF_KM))[lane] = make_float4(s2.x * cs2.x, s2.x * cs2.y, -s2.y * cs2.y, s2.y * cs2.x);
        ((float2*)(st_l + OFF_KT))[lane] =
            make_float2(cs2.x * z2.x - cs2.y * z2.y, cs2.y * z2.x + cs2.x * z2.y);
      }
      next_issue(sl == 0 ? NB - 1 : sl - 1);
      new_kgrp = new_kgrp || c_rem == 0;
      qstep(st, d);
      new_kgrp = false;
      c_rem += 32;
      if (c_rem == kG) c_rem = 0;
      sl = sl == NB - 1 ? 0 : sl + 1;
    }
  }
  // window steps: st_beg .. st_end (stride STRIDE) from nq on
  const int64_t w_first = st_beg >= nq ? st_beg : (IL ? nq + ((st_beg - nq) % STRIDE + STRIDE) % STRIDE : nq);
  for (int64_t st = w_first; st < st_end; st += STRIDE) {
    StepData<16, 32, 1> d;
    const int64_t t0 = s_w0 + (st - nq) * 32;
    load_r(t0, d);
    step(std::true_type{}, std::false_type{}, t0, w_beg, hi, d);
  }

  // ---- combine the wavefronts of the work-group ------------------------------------
  l_run = wave_sum16(l_run);
  vbias = wave_sum16(vbias);
  if constexpr (PV2) vbias1 = wave_sum16(vbias1);
  if (g == 0 && n < n_rep) {
    red_ml[wave][n][0] = m_run;
    red_ml[wave][n][1] = l_run;
  }
  float (*const red_o_w)[D] = (float (*)[D])ring;   // this wavefront's O rows
  // O rows -> LDS with the row's value bias added.  Accumulator row r of this
  // lane is A row R = 4g + r (value group R / n_rep, head R mod n_rep); tile i
  // keeps the rows of its own group.  Row R's bias lives in lane R.
  float rbias[4], rbias1[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    rbias[r] = __shfl(vbias, (4 * g + r) & 15, 64);
    rbias1[r] = PV2 ? __shfl(vbias1, (4 * g + r) & 15, 64) : 0.0f;
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int c = 16 * i + n;
    // tile i's value group, relative to its half's first group (PV2: tiles
    // 4-7 are the second half, groups 2 and 3)
    const bool h1 = PV2 && i >= 4;
    const int gi = (VINT ? (16 * i) / VGC : 0) - (h1 ? 2 : 0);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int R = 4 * g + r;
      if (R / n_rep == gi) red_o_w[R - gi * n_rep][c] = O[i][r] + (VINT ? (h1 ? rbias1[r] : rbias[r]) : 0.0f);
    }
  }
  __syncthreads();
  for (int e = tid; e < n_rep * D; e += 256) {
    const int r = e / D, c = e % D;
    float M = kNegBig;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, red_ml[w][r][0]);
    float L = 0.0f, acc = 0.0f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float f = fast_exp2(red_ml[w][r][0] - M);
      L += f * red_ml[w][r][1];
      acc += f * ((const float (*)[D])ring_s[w])[r][c];
    }
    const int64_t hq = hq0 + r;
    a.ws_o[(hq * a.S + split) * D + c] = acc;
    if (c == 0) {
      a.ws_ml[(hq * a.S + split) * 2 + 0] = M;
      a.ws_ml[(hq * a.S + split) * 2 + 1] = L;
    }
  }
}

// ---- dispatch ---------------------------------------------------------------------------

static int kfmt(const Plan& p) {
  if (p.k.scheme == KVQ_FP8_E4M3) return FP8;
  if (p.k.scheme == KVQ_FP8_E5M2) return BF8;
  if (p.k.scheme == KVQ_INT_ASYM && p.k.axis == KVQ_PER_CHANNEL && p.k.group > 0 && p.k.group % 32 == 0)
    return p.k.bits;
  return -1;
}
static int vfmt(const Plan& p) {
  if (p.v.scheme == KVQ_FP8_E4M3) return FP8;
  if (p.v.scheme == KVQ_FP8_E5M2) return BF8;
  if (p.v.scheme == KVQ_INT_ASYM && p.v.axis == KVQ_PER_TOKEN && p.v.group >= 16) return p.v.bits;
  return -1;
}

static int vgroups(const Plan& p) { return is_fp8(p.v.scheme) ? 1 : 128 / p.v.group; }

bool mfma_supported(const Plan& p) {
  // any number of query heads per kv head: they are split into groups that
  // fit the PV rows (mfma_head_group), one work-group per group
  return p.D == 128 && kfmt(p) >= 0 && vfmt(p) >= 0;
}

// PV rows are (value group, head) pairs: 16 in one A operand, or 32 in two
// (8 heads x 4 value groups with INT2 / INT4 codes on both sides).  The heads
// of a kv head are split into the fewest groups that fit, of near-equal size.
static bool pv2_formats(const Plan& p) {
  const int kf = kfmt(p), vf = vfmt(p);
  return vgroups(p) == 4 && (kf == INT2 || kf == INT4) && (vf == INT2 || vf == INT4);
}
int mfma_head_group(const Plan& p) {
  if (pv2_formats(p) && p.n_rep % 8 == 0) return 8;
  const int cap = 16 / vgroups(p);
  const int ng = (p.n_rep + cap - 1) / cap;
  return (p.n_rep + ng - 1) / ng;
}

// dynamic LDS of a launch: the split's page table for paged calls
static size_t page_lds(const Args& a) { return a.pm.bt ? kMaxSplitPages * sizeof(int32_t) : 0; }

template <int KF, int VF, int VG>
static void launch_kvg(const Plan& p, dim3 grid, hipStream_t s, const Args& a) {
  constexpr bool kPV2 = VG == 4 && (KF == INT2 || KF == INT4) && (VF == INT2 || VF == INT4);
  if constexpr (kPV2) {
    if (a.hg * VG > 16) {
      if (p.pre_rope) hipLaunchKernelGGL((attn_mfma<KF, VF, true, VG, true, true>), grid, dim3(256), page_lds(a), s, p, a);
      else hipLaunchKernelGGL((attn_mfma<KF, VF, false, VG, false, true>), grid, dim3(256), page_lds(a), s, p, a);
      return;
    }
  }
  if (p.pre_rope) {
    hipLaunchKernelGGL((attn_mfma<KF, VF, true, VG, true, false>), grid, dim3(256), page_lds(a), s, p, a);
  } else {
    hipLaunchKernelGGL((attn_mfma<KF, VF, false, VG, false, false>), grid, dim3(256), page_lds(a), s, p, a);
  }
}

template <int KF, int VF>
static void launch_kv(const Plan& p, dim3 grid, hipStream_t s, const Args& a) {
  if constexpr (is_f8(VF)) {
    launch_kvg<KF, VF, 1>(p, grid, s, a);
  } else {
    switch (vgroups(p)) {
      case 1: launch_kvg<KF, VF, 1>(p, grid, s, a); break;
      case 2: launch_kvg<KF, VF, 2>(p, grid, s, a); break;
      case 4: launch_kvg<KF, VF, 4>(p, grid, s, a); break;
      default: launch_kvg<KF, VF, 8>(p, grid, s, a); break;   // n_rep <= 2
    }
  }
}

template <int KF>
static void launch_k(const Plan& p, dim3 grid, hipStream_t s, const Args& a) {
  switch (vfmt(p)) {
    case INT2: launch_kv<KF, INT2>(p, grid, s, a); break;
    case INT4: launch_kv<KF, INT4>(p, grid, s, a); break;
    case INT8: launch_kv<KF, INT8>(p, grid, s, a); break;
    case BF8: launch_kv<KF, BF8>(p, grid, s, a); break;
    default: launch_kv<KF, FP8>(p, grid, s, a); break;
  }
}

hipError_t launch_attention_mfma(const Plan& p, const AttnPlan& ap, const void* arena, const void* q,
                                 float sm_scale, void* ws, hipStream_t s, const StepAppend* app,
                                 const Ragged* rg) {
  Args a{(const uint8_t*)arena, q, (float*)((uint8_t*)ws + ap.ws_o), (float*)((uint8_t*)ws + ap.ws_ml),
         ap.T, ap.Tq, ap.chunk, ap.splits, sm_scale * kLog2e, -1.0f,
         app ? app->k : nullptr, app ? app->v : nullptr, app ? app->t : 0, app ? app->mode : 0,
         (uint8_t*)arena, rg ? rg->pm : PageMap{nullptr, 0}, rg ? rg->seq_lens : nullptr,
         rg ? rg->lens_add : 0, ap.hg, ap.ngroups};
  dim3 grid(ap.splits, p.Hkv * ap.ngroups, p.B);
  switch (kfmt(p)) {
    case INT2: launch_k<INT2>(p, grid, s, a); break;
    case INT4: launch_k<INT4>(p, grid, s, a); break;
    case INT8: launch_k<INT8>(p, grid, s, a); break;
    case BF8: launch_k<BF8>(p, grid, s, a); break;
    default: launch_k<FP8>(p, grid, s, a); break;
  }
  return hipGetLastError();
}

}  // namespace kvq
