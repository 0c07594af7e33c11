// Quantize-append, FP8 calibration, fp16 window and dequantize kernels.
//
// Built with -ffp-contract=off and IEEE division: every arithmetic step of
// the encodings is one fp32 rounding, in the order the pages' listings give:
//  - asymmetric min-max ("KV Cache Quantization: Why Keys and Values Need
//    Different Axes", section "Why does per-token key quantization destroy
//    accuracy?"): scale = max(max-min, 1e-8)/(2^b-1), code = clamp(rint(
//    (x-min)/scale), 0, 2^b-1), x_hat = code*scale + min;
//  - symmetric absmax INT8 ("FP8 KV Cache Quantization: Why Keys Break Before
//    Values", section "Why does the K cache break before the V cache?"):
//    scale = absmax/127, code = clamp(rint(x/scale), -127, 127);
//  - FP8 E4M3 with per-kv-head scales (same page, "Why do per-tensor scales
//    waste bits on the K cache?"): code = E4M3(x/scale), saturating at 448.
//
// Work split: a reduction kernel writes (scale, zero) per group, then an
// encode kernel computes and packs the codes of whole output words (a K row
// dword or a V block word), so no two threads ever write the same byte.
#include "kvq_internal.h"
#include "kvq_launch.h"
#include "kvq_device.h"

namespace kvq {

// Code field of value x for side format f (meta already stored for INT).
__device__ __forceinline__ uint32_t encode_elem(const Plan& p, const SideFmt& f, const uint8_t* arena,
                                                int b, int h, int64_t t, int c, float x) {
  if (f.scheme == KVQ_NONE) {
    if (f.bits == 16) { _Float16 hv = (_Float16)x; return (uint32_t)__builtin_bit_cast(uint16_t, hv); }
    return __float_as_uint(x);
  }
  const int64_t mi = meta_index(p, f, b, h, t, c);
  const float s = load_meta(arena + f.scale, mi, f.meta16);
  if (f.scheme == KVQ_FP8_E4M3) return e4m3_encode(x / s);
  if (f.scheme == KVQ_FP8_E5M2) return e5m2_encode(x / s);   // s = 1
  if (f.scheme == KVQ_INT_SYM) return sym_code(x, s);
  const float z = load_meta(arena + f.zero, mi, f.meta16);
  return asym_code(x, s, z, f.bits);
}

// ---- reductions (scale / zero per group) -------------------------------------

// Per-channel groups: one block per (group, head, sequence), one thread per
// channel looping over the group's tokens (loads coalesce across channels).
template <int SIDE>
__global__ void reduce_channel_groups(Plan p, Src s, int64_t g_lo, int64_t t_lo, int64_t t_len) {
  const SideFmt& f = SIDE == SIDE_K ? p.k : p.v;
  const int c = threadIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int64_t tb = f.group ? (g_lo + blockIdx.x) * f.group : t_lo;
  const int64_t te = f.group ? tb + f.group : t_lo + t_len;
  const bool sym = f.scheme == KVQ_INT_SYM;
  float mn = INFINITY, mx = -INFINITY;
  for (int64_t t = tb; t < te; ++t) {
    float x = src_val<SIDE>(p, s, b, h, t, c);
    if (sym) { mx = fmaxf(mx, fabsf(x)); }
    else { mn = fminf(mn, x); mx = fmaxf(mx, x); }
  }
  store_meta(p, f, (uint8_t*)s.arena, meta_index(p, f, b, h, tb, c), mn, mx);
}

// Per-token groups: one wavefront per token; lane l holds channels l and l+64;
// min/max over Gc consecutive channels by butterfly shuffles.
template <int SIDE>
__global__ void __launch_bounds__(256) reduce_token_groups(Plan p, Src s, int64_t t_lo, int64_t t_len) {
  const SideFmt& f = SIDE == SIDE_K ? p.k : p.v;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int h = blockIdx.y, b = blockIdx.z;
  const int64_t ti = (int64_t)blockIdx.x * 4 + wave;
  if (ti >= t_len) return;
  const int64_t t = t_lo + ti;
  const bool sym = f.scheme == KVQ_INT_SYM;
  const int Gc = f.group;
  const int halves = p.D / 64;
  float mn[2], mx[2];
  for (int j = 0; j < halves; ++j) {
    float x = src_val<SIDE>(p, s, b, h, t, lane + 64 * j);
    mn[j] = sym ? -fabsf(x) : x;
    mx[j] = sym ? fabsf(x) : x;
  }
  if (Gc == 128) {  // D == 128: one group over both halves
    mn[0] = fminf(mn[0], mn[1]);
    mx[0] = fmaxf(mx[0], mx[1]);
  }
  const int width = Gc >= 64 ? 64 : Gc;
  const int nj = (Gc == 128) ? 1 : halves;
  for (int j = 0; j < nj; ++j) {
    for (int off = width >> 1; off > 0; off >>= 1) {
      mn[j] = fminf(mn[j], __shfl_xor(mn[j], off, 64));
      mx[j] = fmaxf(mx[j], __shfl_xor(mx[j], off, 64));
    }
    const int c = lane + 64 * j;
    if ((c % Gc) == 0) store_meta(p, f, (uint8_t*)s.arena, meta_index(p, f, b, h, t, c), mn[j], mx[j]);
  }
}

// Per-tensor: one block per (head, sequence) over all tokens and channels.
template <int SIDE>
__global__ void __launch_bounds__(256) reduce_tensor(Plan p, Src s, int64_t t_len) {
  const SideFmt& f = SIDE == SIDE_K ? p.k : p.v;
  const int h = blockIdx.y, b = blockIdx.z;
  const bool sym = f.scheme == KVQ_INT_SYM;
  float mn = INFINITY, mx = -INFINITY;
  const int64_t nel = t_len * p.D;
  for (int64_t i = threadIdx.x; i < nel; i += blockDim.x) {
    float x = src_val<SIDE>(p, s, b, h, i / p.D, (int)(i % p.D));
    if (sym) { mx = fmaxf(mx, fabsf(x)); } else { mn = fminf(mn, x); mx = fmaxf(mx, x); }
  }
  for (int off = 32; off > 0; off >>= 1) {
    mn = fminf(mn, __shfl_xor(mn, off, 64));
    mx = fmaxf(mx, __shfl_xor(mx, off, 64));
  }
  __shared__ float smn[4], smx[4];
  if ((threadIdx.x & 63) == 0) { smn[threadIdx.x >> 6] = mn; smx[threadIdx.x >> 6] = mx; }
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int w = 1; w < 4; ++w) { mn = fminf(mn, smn[w]); mx = fmaxf(mx, smx[w]); }
    store_meta(p, f, (uint8_t*)s.arena, meta_index(p, f, b, h, 0, 0), mn, mx);
  }
}

// ---- encode kernels ------------------------------------------------------------

// K rows: one work item per (token, dword of the row).
__device__ __forceinline__ void encode_k_item(const Plan& p, const Src& s, int64_t t_lo, int64_t t_len,
                                              int64_t i) {
  const int dw_per_row = p.k_row_bytes / 4;
  const int per = 32 / p.k.bits;                 // channels per dword
  const int j = (int)(i % dw_per_row);
  int64_t r = i / dw_per_row;
  const int64_t t = t_lo + r % t_len;
  r /= t_len;
  const int h = (int)(r % p.Hkv), b = (int)(r / p.Hkv);
  uint32_t word = 0;
  for (int u = 0; u < per; ++u) {
    const int c = j * per + u;
    const float x = src_val<SIDE_K>(p, s, b, h, t, c);
    const uint32_t code = encode_elem(p, p.k, s.arena, b, h, t, c, x);
    word |= (p.k.bits == 32 ? code : (code & ((1u << p.k.bits) - 1))) << (u * p.k.bits);
  }
  const int64_t bh = (int64_t)b * p.Hkv + h;
  uint32_t* row = (uint32_t*)((uint8_t*)s.arena + p.k.codes + (bh * p.Tc + t) * p.k_row_bytes);
  row[j] = word;
}

// V blocks: one work item per word (8 tokens x 1 channel).  Words only partly
// inside [t_lo, t_lo + t_len) keep their other codes (read-modify-write).
__device__ __forceinline__ void encode_v_item(const Plan& p, const Src& s, int64_t t_lo, int64_t t_len,
                                              int64_t i) {
  const int bits = p.v.bits;
  const int words_per_block = 64 * (p.D / 16);
  const int64_t blk_lo = t_lo / kVBlock, blk_hi = (t_lo + t_len - 1) / kVBlock + 1;
  const int64_t nblk = blk_hi - blk_lo;
  {
    const int w = (int)(i % words_per_block);
    int64_t r = i / words_per_block;
    const int64_t blk = blk_lo + r % nblk;
    r /= nblk;
    const int h = (int)(r % p.Hkv), b = (int)(r / p.Hkv);
    const int lane = w / (p.D / 16), tile = w % (p.D / 16);
    const int g = lane >> 4, n = lane & 15;
    const int c = tile * 16 + n;
    const int64_t bh = (int64_t)b * p.Hkv + h;
    uint8_t* wp = (uint8_t*)s.arena + p.v.codes + (bh * p.v_nblk + blk) * p.v_block_bytes +
                  (int64_t)w * bits;
    uint32_t buf[8];
    const int nbytes = bits;                       // word = 8 codes * bits bits = bits bytes
    const int ndw = (nbytes + 3) / 4;
    bool full = true;
    for (int k = 0; k < 8; ++k) {
      const int64_t t = blk * kVBlock + 8 * g + k;
      if (t < t_lo || t >= t_lo + t_len) full = false;
    }
    if (bits == 2) buf[0] = full ? 0u : (uint32_t)*(uint16_t*)wp;
    else for (int d = 0; d < ndw; ++d) buf[d] = full ? 0u : ((uint32_t*)wp)[d];
    for (int k = 0; k < 8; ++k) {
      const int64_t t = blk * kVBlock + 8 * g + k;
      if (t < t_lo || t >= t_lo + t_len) continue;
      const float x = src_val<SIDE_V>(p, s, b, h, t, c);
      uint32_t code = encode_elem(p, p.v, s.arena, b, h, t, c, x);
      const int bit = k * bits;
      if (bits == 32) { buf[k] = code; continue; }
      const uint32_t mask = (1u << bits) - 1;
      code &= mask;
      buf[bit >> 5] = (buf[bit >> 5] & ~(mask << (bit & 31))) | (code << (bit & 31));
    }
    if (bits == 2) *(uint16_t*)wp = (uint16_t)buf[0];
    else for (int d = 0; d < ndw; ++d) ((uint32_t*)wp)[d] = buf[d];
  }
}

// K rows and V blocks of tokens [t_lo, t_lo + t_len) in one launch: items
// [0, nk) are K-row dwords, [nk, nk + nv) V-block words (disjoint bytes).
__global__ void encode_kv(Plan p, Src sk, Src sv, int64_t t_lo, int64_t t_len, int64_t nk, int64_t nv) {
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < nk + nv;
       i += (int64_t)gridDim.x * blockDim.x) {
    if (i < nk) encode_k_item(p, sk, t_lo, t_len, i);
    else encode_v_item(p, sv, t_lo, t_len, i - nk);
  }
}

// fp16 window: token t -> slot t mod Rs of ring K (rows) and ring V (blocks),
// both in one launch: items [0, n) write keys, [n, 2n) values.
__global__ void write_ring_kv(Plan p, Src sk, const void* vin, int64_t w_lo, int64_t w_len) {
  uint8_t* arena = (uint8_t*)sk.arena;
  const int64_t n = (int64_t)p.B * p.Hkv * w_len * p.D;
  const int rblock = kVBlock * p.D * 2;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < 2 * n;
       i += (int64_t)gridDim.x * blockDim.x) {
    const bool is_v = i >= n;
    const int64_t e = is_v ? i - n : i;
    const int c = (int)(e % p.D);
    int64_t r = e / p.D;
    const int64_t t = w_lo + r % w_len;
    r /= w_len;
    const int h = (int)(r % p.Hkv), b = (int)(r / p.Hkv);
    const int64_t bh = (int64_t)b * p.Hkv + h;
    const int64_t slot = t % p.Rs;
    const int64_t src = (bh * sk.n + (t - sk.t0)) * p.D + c;
    if (!is_v) {
      const _Float16 kx = (_Float16)load_in(sk.in, src, p.in_dtype);
      ((_Float16*)(arena + p.ring_k))[(bh * p.Rs + slot) * p.D + c] = kx;
    } else {
      const _Float16 vx = (_Float16)load_in(vin, src, p.in_dtype);
      uint8_t* base = arena + p.ring_v + (uint64_t)bh * (p.Rs / kVBlock) * rblock;
      ((_Float16*)(base + vblock_word_byte(slot, c, p.D, 16, rblock)))[slot & 7] = vx;
    }
  }
}

// ---- FP8 scale setup -----------------------------------------------------------

__global__ void fp8_zero(uint32_t* amax, int n) {
  int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) amax[i] = 0u;
}

// absmax over (sequence, token, channel) of kv head h: grid (chunks, Hkv, 2 sides).
template <int DT, bool WIN>
__global__ void __launch_bounds__(256) fp8_absmax(Plan p, const void* kin, const void* vin, int n,
                                                   uint32_t* amax) {
  const int h = blockIdx.y, side = blockIdx.z;
  const void* in = side ? vin : kin;
  // each sequence's run of n * D values (a multiple of 8, 16-byte aligned)
  const int64_t per_seq = (int64_t)n * p.D;
  const int64_t gid = blockIdx.x * (int64_t)blockDim.x + threadIdx.x, stride = (int64_t)gridDim.x * blockDim.x;
  float m = absmax_runs<DT, WIN>(in, p.B, p.Hkv, h, per_seq, gid, stride, [=](int) { return per_seq; });
  for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, 64));
  __shared__ float sm[4];
  if ((threadIdx.x & 63) == 0) sm[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int w = 1; w < 4; ++w) m = fmaxf(m, sm[w]);
    atomicMax(&amax[side * p.Hkv + h], __float_as_uint(m));   // non-negative floats order as uints
  }
}

// scale = absmax/448 (1.0 when absmax is 0), or the caller's scale, or 1.0.
__global__ void fp8_finalize(Plan p, uint8_t* arena, const uint32_t* amax, const float* ks,
                             const float* vs, int mode) {
  const int h = threadIdx.x;
  if (h >= p.Hkv) return;
  for (int side = 0; side < 2; ++side) {
    const SideFmt& f = side ? p.v : p.k;
    if (!is_fp8(f.scheme)) continue;
    const float* given = side ? vs : ks;
    float s = 1.0f;                       // E5M2 takes no scale
    if (f.scheme != KVQ_FP8_E4M3) {
      s = 1.0f;
    } else if (mode == 1) {
      const float a = __uint_as_float(amax[side * p.Hkv + h]);
      s = (a == 0.0f) ? 1.0f : a / kE4M3Max;
    } else if (given) {
      s = given[h];
    }
    ((float*)(arena + f.scale))[h] = s;
  }
}

// ---- RoPE tables (fp64 angles, rounded to fp32) ---------------------------------

__global__ void rope_tables(Plan p, uint8_t* arena) {
  const int half = p.D / 2;
  const int64_t rows = kVBlock + p.rope_rows;
  const int64_t total = rows * half;
  float2* tab = (float2*)(arena + p.rope);
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int pair = (int)(i % half);
    const int64_t row = i / half;
    const double theta = pow((double)p.rope_base, -2.0 * pair / (double)p.D);
    const double pos = row < kVBlock ? (double)row : (double)(row - kVBlock) * kVBlock;
    double sn, cs;
    sincos(pos * theta, &sn, &cs);
    tab[i] = make_float2((float)cs, (float)sn);
  }
}

__global__ void dequantize_kernel(Plan p, const uint8_t* arena, int64_t T, int64_t Tq, float* kout,
                                  float* vout) {
  const int64_t total = (int64_t)p.B * p.Hkv * T * p.D;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int c = (int)(i % p.D);
    int64_t r = i / p.D;
    const int64_t t = r % T;
    r /= T;
    const int h = (int)(r % p.Hkv), b = (int)(r / p.Hkv);
    if (kout) kout[i] = dequant_elem<SIDE_K>(p, arena, b, h, t, c, Tq);
    if (vout) vout[i] = dequant_elem<SIDE_V>(p, arena, b, h, t, c, Tq);
  }
}

// ---- launchers -----------------------------------------------------------------

static unsigned grid_for(int64_t total, int block) {
  int64_t g = (total + block - 1) / block;
  if (g > 65536) g = 65536;
  if (g < 1) g = 1;
  return (unsigned)g;
}

hipError_t launch_rope_tables(const Plan& p, void* arena, hipStream_t s) {
  const int64_t total = (int64_t)(kVBlock + p.rope_rows) * (p.D / 2);
  hipLaunchKernelGGL(rope_tables, dim3(grid_for(total, 256)), dim3(256), 0, s, p, (uint8_t*)arena);
  return hipGetLastError();
}

hipError_t launch_fp8_finalize(const Plan& p, void* arena, const float* k_scale, const float* v_scale,
                               bool calibrate, hipStream_t s) {
  uint32_t* amax = (uint32_t*)((uint8_t*)arena + p.fp8_calib);
  hipLaunchKernelGGL(fp8_finalize, dim3(1), dim3(64 * ((p.Hkv + 63) / 64)), 0, s, p, (uint8_t*)arena,
                     (const uint32_t*)amax, k_scale, v_scale, calibrate ? 1 : 0);
  return hipGetLastError();
}

hipError_t launch_fp8_setup(const Plan& p, void* arena, const void* k_new, const void* v_new,
                            int n_new, const float* k_scale, const float* v_scale, bool calibrate,
                            hipStream_t s, const int32_t* new_lens) {
  uint32_t* amax = (uint32_t*)((uint8_t*)arena + p.fp8_calib);
  if (calibrate) {
    hipLaunchKernelGGL(fp8_zero, dim3(1), dim3(64 * ((2 * p.Hkv + 63) / 64)), 0, s, amax, 2 * p.Hkv);
    if (new_lens) {
      const hipError_t e = launch_fp8_absmax_lens(p, k_new, v_new, n_new, new_lens, amax, s);
      if (e != hipSuccess) return e;
    } else {
      const dim3 grid(fp8_absmax_blocks(p, n_new), p.Hkv, 2);
      const bool win = p.window != 0;
      if (p.in_dtype == KVQ_F32) {
        if (win) hipLaunchKernelGGL((fp8_absmax<KVQ_F32, true>), grid, dim3(256), 0, s, p, k_new, v_new, n_new, amax);
        else hipLaunchKernelGGL((fp8_absmax<KVQ_F32, false>), grid, dim3(256), 0, s, p, k_new, v_new, n_new, amax);
      } else if (p.in_dtype == KVQ_F16) {
        if (win) hipLaunchKernelGGL((fp8_absmax<KVQ_F16, true>), grid, dim3(256), 0, s, p, k_new, v_new, n_new, amax);
        else hipLaunchKernelGGL((fp8_absmax<KVQ_F16, false>), grid, dim3(256), 0, s, p, k_new, v_new, n_new, amax);
      } else {
        if (win) hipLaunchKernelGGL((fp8_absmax<KVQ_BF16, true>), grid, dim3(256), 0, s, p, k_new, v_new, n_new, amax);
        else hipLaunchKernelGGL((fp8_absmax<KVQ_BF16, false>), grid, dim3(256), 0, s, p, k_new, v_new, n_new, amax);
      }
    }
  }
  return launch_fp8_finalize(p, arena, k_scale, v_scale, calibrate, s);
}

template <int SIDE>
static void launch_reduce(const Plan& p, const Src& src, int64_t q_lo, int64_t q_hi, hipStream_t s) {
  const SideFmt& f = SIDE == SIDE_K ? p.k : p.v;
  if (f.scheme != KVQ_INT_ASYM && f.scheme != KVQ_INT_SYM) return;
  const int64_t len = q_hi - q_lo;
  if (f.axis == KVQ_PER_CHANNEL) {
    const int64_t ng = f.group ? len / f.group : 1;
    const int64_t g_lo = f.group ? q_lo / f.group : 0;
    hipLaunchKernelGGL(reduce_channel_groups<SIDE>, dim3((unsigned)ng, p.Hkv, p.B), dim3(p.D), 0, s,
                       p, src, g_lo, q_lo, len);
  } else if (f.axis == KVQ_PER_TOKEN) {
    hipLaunchKernelGGL(reduce_token_groups<SIDE>, dim3((unsigned)((len + 3) / 4), p.Hkv, p.B),
                       dim3(256), 0, s, p, src, q_lo, len);
  } else {
    hipLaunchKernelGGL(reduce_tensor<SIDE>, dim3(1, p.Hkv, p.B), dim3(256), 0, s, p, src, len);
  }
}

hipError_t launch_quantize_range(const Plan& p, void* arena, int64_t t0, int n_new, int64_t q_lo,
                                 int64_t q_hi, const void* k_new, const void* v_new, hipStream_t s) {
  Src sk{(const uint8_t*)arena, k_new, t0, n_new};
  Src sv{(const uint8_t*)arena, v_new, t0, n_new};
  const int64_t len = q_hi - q_lo;
  hipError_t e;
  launch_reduce<SIDE_K>(p, sk, q_lo, q_hi, s);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  launch_reduce<SIDE_V>(p, sv, q_lo, q_hi, s);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const int64_t kw = (int64_t)p.B * p.Hkv * len * (p.k_row_bytes / 4);
  const int64_t nblk = (q_hi - 1) / kVBlock - q_lo / kVBlock + 1;
  const int64_t vw = (int64_t)p.B * p.Hkv * nblk * 64 * (p.D / 16);
  hipLaunchKernelGGL(encode_kv, dim3(grid_for(kw + vw, 256)), dim3(256), 0, s, p, sk, sv, q_lo, len, kw, vw);
  return hipGetLastError();
}

hipError_t launch_ring_write(const Plan& p, void* arena, int64_t t0, int n_new, int64_t w_lo,
                             const void* k_new, const void* v_new, hipStream_t s) {
  Src sk{(const uint8_t*)arena, k_new, t0, n_new};
  const int64_t w_len = t0 + n_new - w_lo;
  const int64_t total = (int64_t)p.B * p.Hkv * w_len * p.D;
  hipLaunchKernelGGL(write_ring_kv, dim3(grid_for(2 * total, 256)), dim3(256), 0, s, p, sk, v_new, w_lo, w_len);
  return hipGetLastError();
}

// Paged / ragged: sequence b's first seq_lens[b] tokens (clamped to max_T)
// into rows [0, seq_lens[b]) of [B][Hkv][max_T][D]; later rows untouched.
__global__ void dequantize_paged(Plan p, const uint8_t* arena, PageMap pm, const int32_t* seq_lens,
                                 int64_t max_T, float* kout, float* vout) {
  const int64_t total = (int64_t)p.B * p.Hkv * max_T * p.D;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int c = (int)(i % p.D);
    int64_t r = i / p.D;
    const int64_t t = r % max_T;
    r /= max_T;
    const int h = (int)(r % p.Hkv), b = (int)(r / p.Hkv);
    int64_t Tb = seq_lens[b];
    if (Tb > max_T) Tb = max_T;
    if (t >= Tb) continue;
    const int64_t Tq = quantized_tokens(p, Tb);
    if (kout) kout[i] = dequant_elem<SIDE_K>(p, arena, b, h, t, c, Tq, pm);
    if (vout) vout[i] = dequant_elem<SIDE_V>(p, arena, b, h, t, c, Tq, pm);
  }
}

hipError_t launch_dequantize_paged(const Plan& p, const void* arena, const PageMap& pm,
                                   const int32_t* seq_lens, int64_t max_T, float* k_out, float* v_out,
                                   hipStream_t s) {
  const int64_t total = (int64_t)p.B * p.Hkv * max_T * p.D;
  hipLaunchKernelGGL(dequantize_paged, dim3(grid_for(total, 256)), dim3(256), 0, s, p, (const uint8_t*)arena,
                     pm, seq_lens, max_T, k_out, v_out);
  return hipGetLastError();
}

hipError_t launch_dequantize(const Plan& p, const void* arena, int64_t T, float* k_out, float* v_out,
                             hipStream_t s) {
  const int64_t total = (int64_t)p.B * p.Hkv * T * p.D;
  hipLaunchKernelGGL(dequantize_kernel, dim3(grid_for(total, 256)), dim3(256), 0, s, p,
                     (const uint8_t*)arena, T, quantized_tokens(p, T), k_out, v_out);
  return hipGetLastError();
}

}  // namespace kvq
