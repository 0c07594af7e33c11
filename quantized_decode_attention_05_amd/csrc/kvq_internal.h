// Internal plan of a cache config: resolved groups, section offsets and the
// residual split, computed once on the host and passed to kernels by value.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/kvq.h"

namespace kvq {

constexpr int kVBlock = 32;      // tokens per V code block
constexpr int kRingAlign = 32;   // ring slots are a multiple of this
constexpr int kMaxHeadsPerKv = 256;   // query heads per kv head (Hq / Hkv)
constexpr float kE4M3Max = 448.0f;
constexpr float kE5M2Max = 57344.0f;

// FP8 schemes: bytes with one fp32 scale per kv head (1.0 for E5M2)
__host__ __device__ inline bool is_fp8(int scheme) {
  return scheme == KVQ_FP8_E4M3 || scheme == KVQ_FP8_E5M2;
}

// One side (K or V) of the cache.
struct SideFmt {
  int32_t scheme;     // enum kvq_scheme
  int32_t bits;       // code bits (2, 4, 8, 16, 32)
  int32_t axis;       // enum kvq_axis (INT schemes)
  int32_t group;      // resolved: PER_CHANNEL tokens per group (0 = whole axis), PER_TOKEN channels
  int32_t meta_cols;  // innermost extent of scale/zero
  int32_t meta16;     // INT scale / zero stored as fp16 (else fp32)
  int64_t meta_rows;  // rows of scale/zero per (b, h)
  uint64_t codes, scale, zero;  // byte offsets in the arena (UINT64_MAX = absent)
};

struct Plan {
  int32_t B, Hq, Hkv, D, n_rep;
  int32_t in_dtype, out_dtype;
  int32_t R, Gt, Rs;      // residual, token group, ring slots
  int32_t window;         // every token staged through fp16
  int32_t one_shot;       // whole-axis / per-tensor groups
  int32_t pre_rope;
  float rope_base;
  int64_t Tc;             // token capacity (rounded)
  int64_t max_tokens;
  int32_t k_row_bytes, v_block_bytes;
  int64_t v_nblk;         // V code blocks per (b, h)
  SideFmt k, v;
  uint64_t ring_k, ring_v, rope, fp8_calib, total;
  int64_t rope_rows;      // coarse rope rows (Tc/32 + 1)
  // token sections: `pages` pages of P tokens per kv head ([pages][H][P] token
  // rows); a contiguous cache is one page of Tc tokens per sequence
  int32_t paged;          // block tables (page_tokens > 0)
  int64_t P;              // tokens per page (Tc when contiguous)
  int32_t pages;          // pages of the token sections (B when contiguous)
  int32_t unit;           // tokens per work-group of the one-pass append kernel
                          // (max(Gt, 32)); 0 when that kernel does not serve the format
};

// Block table of a paged call (bt == nullptr: contiguous cache).
struct PageMap {
  const int32_t* bt;      // [B][max_blocks]
  int32_t max_blocks;
};

// Builds the plan; returns KVQ_OK or an error status.
int make_plan(const kvq_config* cfg, Plan* p);

__host__ __device__ inline int64_t quantized_tokens(const Plan& p, int64_t T) {
  if (p.one_shot) return T;
  int64_t r = T - p.R;
  if (r < 0) r = 0;
  return (int64_t)p.Gt * (r / p.Gt);
}

// Page holding token t of sequence b (b itself for a contiguous cache); -1
// when the block-table entry is past the row or outside the pool.
__device__ __forceinline__ int32_t page_of(const Plan& p, const PageMap& m, int b, int64_t t) {
  if (!m.bt) return b;
  const int64_t j = t / p.P;
  if (j >= m.max_blocks) return -1;
  const int32_t pg = m.bt[(int64_t)b * m.max_blocks + j];
  return (pg >= 0 && pg < p.pages) ? pg : -1;
}

// Token row of token t of kv head h in page `page`: the index of its row in
// the [pages][H][P] token sections.
__device__ __forceinline__ int64_t row_of(const Plan& p, int32_t page, int h, int64_t t) {
  const int64_t tt = p.paged ? t - (t / p.P) * p.P : t;
  return ((int64_t)page * p.Hkv + h) * p.P + tt;
}

// Token row of (b, h, t) for reads: an entry outside the pool reads page 0.
__device__ __forceinline__ int64_t read_row(const Plan& p, const PageMap& m, int b, int h, int64_t t) {
  const int32_t pg = page_of(p, m, b, t);
  return row_of(p, pg < 0 ? 0 : pg, h, t);
}

// ---- device helpers shared by the kernels ----------------------------------

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(((uint32_t)b) << 16);
}

__device__ __forceinline__ float load_in(const void* p, int64_t i, int dtype) {
  if (dtype == KVQ_F32) return ((const float*)p)[i];
  if (dtype == KVQ_F16) return (float)((const _Float16*)p)[i];
  return bf16_to_f32(((const uint16_t*)p)[i]);
}

// fp32 -> fp16 (round to nearest even) -> fp32
__device__ __forceinline__ float stage_f16(float x) { return (float)(_Float16)x; }

// Value of an E5M2 code byte (finite codes; infinities and NaNs never produced).
__device__ __forceinline__ float e5m2_decode(uint32_t c) {
  uint32_t e = (c >> 2) & 0x1F, m = c & 3;
  float mag = (e == 0) ? (float)m * 1.52587890625e-05f                  // m * 2^-16
                       : __uint_as_float(((e + 112u) << 23) | (m << 21)); // (1+m/4) 2^(e-15)
  return (c & 0x80) ? -mag : mag;
}

// Value of an E4M3FN code byte (finite codes; NaN codes never produced).
__device__ __forceinline__ float e4m3_decode(uint32_t c) {
  uint32_t e = (c >> 3) & 0xF, m = c & 7;
  float mag = (e == 0) ? (float)m * 0.001953125f                      // m * 2^-9
                       : __uint_as_float(((e + 120u) << 23) | (m << 20)); // (1+m/8) 2^(e-7)
  return (c & 0x80) ? -mag : mag;
}

// V block layout: byte offset of the word holding (t, c), and bit offset of
// code k inside that word.  Word = 8 codes of `bits` bits.
__device__ __forceinline__ int64_t vblock_word_byte(int64_t t, int c, int D, int bits,
                                                    int block_bytes) {
  int64_t blk = t >> 5;
  int tau = (int)(t & 31);
  int g = tau >> 3, n = c & 15, i = c >> 4;
  int lane = 16 * g + n;
  int64_t word = (int64_t)lane * (D >> 4) + i;
  return blk * block_bytes + word * bits;   // a word is 8*bits bits = bits bytes
}

}  // namespace kvq
