/*
 * kvq.h -- quantized KV cache and single-query decode attention for MI355X
 * (gfx950).  C ABI: plain pointers and sizes; the caller owns every buffer.
 *
 * What is computed (citations are page titles and sections):
 *
 *  - Attention of one new query per sequence against the cached keys and
 *    values: logits_j = q . k_j / sqrt(d), p = softmax(logits), out =
 *    sum_j p_j v_j  ("FP8 KV Cache Quantization: Why Keys Break Before Values",
 *    section "Why does the K cache break before the V cache?"; "Why Keys Are
 *    More Sensitive Than Values in INT8 KV Cache Quantization", section
 *    "Computational Paths for Key and Value").  With grouped-query attention
 *    query head h reads kv head h / (Hq / Hkv) ("KV Cache Quantization: Why
 *    Keys and Values Need Different Axes", section "Why does this get worse
 *    with GQA and MLA?").
 *  - Keys and values are configured independently ("FP8 KV Cache
 *    Quantization...", section "How do you configure asymmetric KV cache
 *    quantization?"): per-channel keys and per-token values ("...Need
 *    Different Axes", section "Why does per-token key quantization destroy
 *    accuracy?"), asymmetric min-max INT2/4/8 with scale and zero-point (the
 *    quant_dequant listing there), symmetric absmax INT8 (the qint8 listing of
 *    the FP8 page), or FP8 E4M3 with per-kv-head k_scale / v_scale (FP8 page,
 *    TL;DR and "Why do per-tensor scales waste bits on the K cache?"; unit
 *    scale when uncalibrated).
 *  - A full-precision (fp16) window of the most recent tokens, folded into
 *    the quantized cache in blocks ("...Need Different Axes", section "What
 *    should I actually turn on in production?"), and optional pre-RoPE keys
 *    rotated after dequantization inside attention (same page, "Where does
 *    RoPE break this?").
 *
 * Conventions
 *  - Every call returns an int status (KVQ_OK = 0, errors < 0).  Arguments are
 *    validated on the host before any HIP call; on error nothing is launched
 *    and no buffer is touched.  No call aborts or throws across the ABI.
 *  - Device work is enqueued asynchronously on the caller's stream; no call
 *    synchronizes the host.  The library never allocates or frees memory.
 *    A launching call first clears the thread's sticky HIP error (left by
 *    earlier, unrelated calls) so that KVQ_ERR_HIP reports its own launches;
 *    set KVQ_LOG=1 to print the HIP error name.
 *  - The library is stateless: the caller tracks T, the number of tokens in
 *    the cache.  Distinct caches on distinct streams may be used from
 *    different host threads.  Calls on one cache must be stream-ordered.
 *  - Device pointers must be 16-byte aligned (arena and workspace 256-byte).
 *  - head_dim must be 64 or 128 (a multiple of 32 for INT2 values).
 */
#ifndef KVQ_H
#define KVQ_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes ------------------------------------------------------ */
#define KVQ_OK                 0
#define KVQ_ERR_INVALID_ARG   -1  /* bad config or argument value                 */
#define KVQ_ERR_UNSUPPORTED   -2  /* valid but not supported (e.g. append to a     */
                                  /* whole-axis group, which would rescale history) */
#define KVQ_ERR_CAPACITY      -3  /* t0 + n_new > max_tokens, or T > max_tokens     */
#define KVQ_ERR_ALIGN         -4  /* a pointer is not aligned as required           */
#define KVQ_ERR_NULL          -5  /* a required pointer is NULL                     */
#define KVQ_ERR_WORKSPACE     -6  /* workspace smaller than kvq_workspace_bytes     */
#define KVQ_ERR_HIP           -7  /* a HIP launch failed (hipGetLastError)          */

/* ---- enums ----------------------------------------------------------- */
enum kvq_scheme {
  KVQ_NONE     = 0,  /* unquantized: bits 16 -> fp16 storage, 32 -> fp32          */
  KVQ_INT_ASYM = 1,  /* asymmetric min-max: bits 2, 4 or 8, codes in [0, 2^b-1]    */
  KVQ_INT_SYM  = 2,  /* symmetric absmax INT8: bits 8, codes in [-127, 127]        */
  KVQ_FP8_E4M3 = 3,  /* OCP E4M3FN bytes with one fp32 scale per kv head           */
  KVQ_FP8_E5M2 = 4   /* OCP E5M2 bytes, no scales (stored scale fixed at 1.0);      */
                     /* saturates at +-57344 ("FP8 KV Cache Quantization: Why Keys */
                     /* Break Before Values", section "Why do per-tensor scales   */
                     /* waste bits on the K cache?"; that it needs no scales:     */
                     /* section "How do you configure asymmetric KV cache         */
                     /* quantization?")                                           */
};
enum kvq_axis {      /* grouping axis of INT schemes (ignored for NONE / FP8)      */
  KVQ_PER_TENSOR  = 0, /* one (scale, zero) per (sequence, kv head)                */
  KVQ_PER_CHANNEL = 1, /* one per channel per group of `group` tokens; 0 = all     */
  KVQ_PER_TOKEN   = 2  /* one per token per group of `group` channels; 0 = all     */
};
enum kvq_dtype { KVQ_F32 = 0, KVQ_F16 = 1, KVQ_BF16 = 2 };

#define KVQ_CALIBRATE 1u     /* quantize_append flag: FP8 scales = absmax / 448   */
#define KVQ_INIT      2u     /* paged append flag: this call starts the cache      */
                             /* (writes the RoPE tables and the FP8 scales)        */

typedef struct kvq_tensor_spec {
  int32_t scheme;  /* enum kvq_scheme                                            */
  int32_t bits;    /* see enum kvq_scheme                                        */
  int32_t axis;    /* enum kvq_axis                                              */
  int32_t group;   /* tokens (PER_CHANNEL) or channels (PER_TOKEN); 0 = whole axis */
} kvq_tensor_spec;

typedef struct kvq_config {
  int32_t batch;          /* B: sequences                                        */
  int32_t num_q_heads;    /* Hq                                                  */
  int32_t num_kv_heads;   /* Hkv, Hq % Hkv == 0, Hq / Hkv <= 256                 */
  int32_t head_dim;       /* D: 64 or 128                                        */
  int64_t max_tokens;     /* capacity per sequence                               */
  int32_t in_dtype;       /* dtype of k_new, v_new and q (enum kvq_dtype)       */
  int32_t out_dtype;      /* dtype of the attention output (enum kvq_dtype)     */
  kvq_tensor_spec k;      /* key cache format                                    */
  kvq_tensor_spec v;      /* value cache format                                  */
  int32_t residual;       /* R: most recent tokens kept in fp16 (0 = none)       */
  int32_t pre_rope_k;     /* 1: keys are cached before RoPE and rotated in attention */
  float   rope_base;      /* RoPE base (theta_i = base^(-2i/D)) when pre_rope_k  */
  int32_t meta_dtype;     /* storage of the scale / zero-point of INT sides:     */
                          /* KVQ_F32 (0) or KVQ_F16 (1), see below               */
  int32_t page_tokens;    /* P > 0: paged cache of num_pages pages of P tokens,  */
                          /* addressed through block tables (see "Paged        */
                          /* caches" below); 0: contiguous per sequence         */
  int32_t num_pages;      /* pages in the pool (paged caches; 0 otherwise)       */
} kvq_config;

/*
 * fp16 scale / zero-point metadata (meta_dtype = KVQ_F16; FP8 scales stay
 * fp32).  Halves the metadata bytes, which for small groups are as large as
 * the codes (INT2 with groups of 32: 8 bytes of fp32 scale and zero per 32
 * two-bit codes).  The stored values are chosen so that the group still spans
 * its range: asymmetric groups store z = the largest fp16 <= the group
 * minimum and s = the smallest fp16 >= fl(max(fl(max - z), 1e-8) / (2^b - 1));
 * symmetric groups s = the smallest fp16 >= fl(max(absmax, 1e-8) / 127).
 * Codes and dequantization then use these fp16 values (exactly, in fp32) in
 * the formulas of the fp32 case, so |x - x_hat| <= s / 2 still holds, with s
 * the stored fp16 scale.  Values outside the fp16 range saturate the stored
 * z or s at +-65504 (their codes then clip); the bound needs every group
 * within +-65504 and ranges up to 65504 * (2^b - 1).
 */

/*
 * Arena layout.  One caller-allocated device buffer holds the whole cache; its
 * sections are listed below in order, each starting at a 256-byte aligned
 * offset (SIZE_MAX when absent).  Shapes use Tc = token_capacity (max_tokens
 * rounded up to a multiple of 32 and of the per-channel group), H = Hkv.
 * The token sections (codes and INT metadata) of a contiguous cache hold one
 * page of Tc tokens per sequence; a paged cache (page_tokens = P > 0) holds
 * num_pages pages of P tokens, so below [B][H][Tc] reads [num_pages][H][P]
 * and token t of sequence b sits in page block_table[b][t / P] at t mod P.
 *
 *  k_codes  [B][H][Tc][D*bK/8]   token rows: channel c at bit bK*(c mod 8/bK)
 *                                of byte c*bK/8, low bits first; INT_SYM is
 *                                two's complement; NONE stores fp16/fp32 LE.
 *  k_scale  fp32 (fp16 for INT sides when meta_dtype = KVQ_F16)
 *                PER_TENSOR [B][H]; PER_CHANNEL [B][H][Tc/G or 1][D];
 *                PER_TOKEN [B][H][Tc][D/Gc]; FP8 [H] fp32 (1.0 for E5M2).
 *  k_zero   same type and shape as k_scale (INT_ASYM only; the group
 *                minimum, or its fp16 rounding toward -inf).
 *  v_codes  [B][H][Tc/32][32*D*bV/8]  32-token blocks: token t = 32*blk +
 *                8*g + k and channel c = 16*i + n go to word i of lane
 *                l = 16*g + n; each lane owns D/16 consecutive words of 8*bV
 *                bits; code k sits at bit k*bV of its word (little-endian).
 *  v_scale, v_zero   as for K, for the value spec.
 *  ring_k   fp16 [B][H][Rs][D]   window tokens, token t in slot t mod Rs.
 *  ring_v   fp16 [B][H][Rs/32][32*D*2]  window values in the 32-token block
 *                layout above (bV = 16).
 *  rope     fp32 tables of cos/sin written when t0 == 0 (pre_rope_k only).
 *  fp8_calib  u32 [2][H] scratch of FP8 calibration.
 *
 * Tokens [0, Tq(T)) are quantized and [Tq(T), T) sit in the ring, with
 * Tq(T) = Gt * floor(max(T - R, 0) / Gt), Gt = group of a finite PER_CHANNEL
 * INT spec (1 otherwise); whole-axis and per-tensor groups quantize all tokens
 * at once (Tq = T, R must be 0).  Rs = roundup(R + Gt, 32) when R > 0 or
 * Gt > 1 (then every token is staged through fp16 round-to-nearest-even),
 * else 0.
 */
typedef struct kvq_layout {
  size_t k_codes, k_scale, k_zero;
  size_t v_codes, v_scale, v_zero;
  size_t ring_k, ring_v;
  size_t rope, fp8_calib;
  size_t total_bytes;        /* == kvq_arena_bytes                                */
  int64_t token_capacity;    /* Tc                                                */
  int32_t k_row_bytes;       /* D*bK/8                                            */
  int32_t v_block_bytes;     /* 32*D*bV/8                                         */
  int32_t ring_slots;        /* Rs                                                */
  int32_t token_group;       /* Gt                                                */
  int32_t k_meta_cols, v_meta_cols;  /* innermost extent of the scale arrays     */
  int64_t page_tokens;       /* tokens per page: P, or Tc for a contiguous cache  */
  int32_t pages;             /* pages of the token sections: num_pages, or B      */
  int32_t reserved;
} kvq_layout;

/* Validate a config (host only).  Returns KVQ_OK or KVQ_ERR_INVALID_ARG. */
int kvq_validate_config(const kvq_config* cfg);

/* Fill *out with the arena layout above (host only). */
int kvq_arena_layout(const kvq_config* cfg, kvq_layout* out);

/* Bytes of the arena for cfg (host only). */
int kvq_arena_bytes(const kvq_config* cfg, size_t* bytes);

/* Tq(T): tokens quantized when the cache holds T tokens (host only); < 0 on error. */
int64_t kvq_quantized_tokens(const kvq_config* cfg, int64_t T);

/*
 * Append n_new tokens at positions [t0, t0 + n_new) of every sequence: keys
 * per channel over groups of tokens, values per token over groups of channels
 * ("KV Cache Quantization: Why Keys and Values Need Different Axes", section
 * "Why does per-token key quantization destroy accuracy?", whose
 * quant_dequant listing gives the min-max encoding), symmetric INT8 as the
 * qint8 listing of "FP8 KV Cache Quantization: Why Keys Break Before Values"
 * (section "Why does the K cache break before the V cache?"), FP8 E4M3 with
 * per-head scales and their failure modes as that page's section "Why do
 * per-tensor scales waste bits on the K cache?" describes them, and the most
 * recent tokens kept in fp16 and folded in blocks ("...Need Different Axes",
 * section "What should I actually turn on in production?").
 *   k_new, v_new: device [B][Hkv][n_new][D] in cfg->in_dtype (values as
 *                 computed by the model: pre-RoPE keys when cfg->pre_rope_k).
 *   k_scale, v_scale: FP8 E4M3 only; device fp32 [Hkv] scales to store at
 *                 t0 == 0, or NULL.  With KVQ_CALIBRATE (t0 == 0 only) the
 *                 scales are absmax/448 per kv head over this call's tokens of
 *                 all sequences; with neither, 1.0.  Later calls reuse the
 *                 stored scales and saturate values beyond +-448*scale.  An
 *                 E5M2 side takes no scale (KVQ_ERR_INVALID_ARG if one is
 *                 passed for it), ignores KVQ_CALIBRATE, stores 1.0 and
 *                 saturates beyond +-57344.
 * A cache is started by a call with t0 == 0, which also writes the RoPE tables.
 * Tokens that leave the fp16 window are quantized in blocks of Gt ("folds");
 * the result equals quantizing the same tokens in one call.
 */
int kvq_quantize_append(const kvq_config* cfg, void* arena, int64_t t0, int32_t n_new,
                        const void* k_new, const void* v_new,
                        const float* k_scale, const float* v_scale,
                        uint32_t flags, hipStream_t stream);

/* Attention kernel choice and split count (NULL = defaults). */
typedef struct kvq_attn_options {
  int32_t kernel;       /* 0 auto, 1 generic VALU kernel, 2 MFMA kernel (error if unsupported) */
  int32_t num_splits;   /* token splits per (sequence, kv head); 0 = automatic   */
  int32_t reserved[6];  /* must be 0                                             */
} kvq_attn_options;

/* Workspace bytes needed by kvq_decode_attention for T tokens (host only).  The
 * size never decreases with T, so the size for the largest T a caller will use
 * (e.g. max_tokens) serves every smaller T with the same options. */
int kvq_workspace_bytes(const kvq_config* cfg, int64_t T, const kvq_attn_options* opt,
                        size_t* bytes);

/*
 * Decode attention of one query per (sequence, query head) over the T cached
 * tokens, dequantizing inside QK^T, softmax and PV (keys rotated by RoPE at
 * their positions after dequantization when cfg->pre_rope_k).
 *   q:   device [B][Hq][D] in cfg->in_dtype (already rotated to position T-1
 *        when keys are pre-RoPE).
 *   out: device [B][Hq][D] in cfg->out_dtype (fp32 recommended).
 *   sm_scale: logit scale, normally 1/sqrt(D).
 *   workspace: device scratch of kvq_workspace_bytes (split partials).
 * T must satisfy 1 <= T <= max_tokens.  The query heads of a kv head are
 * served together by each work-group when they fit its rows (16 (value
 * group, head) rows, 32 for eight heads over four INT2/INT4 value groups);
 * more heads are split into groups of near-equal size, each group streaming
 * the kv head's cache itself.
 */
int kvq_decode_attention(const kvq_config* cfg, const void* arena, int64_t T,
                         const void* q, void* out, float sm_scale,
                         void* workspace, size_t workspace_bytes,
                         const kvq_attn_options* opt, hipStream_t stream);

/*
 * Decode attention without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  Same computation, kernels and result,
 * bit for bit, as kvq_decode_attention with the same options; the split
 * partials go to a device array of KVQ_STATIC_WORKSPACE_BYTES owned by the
 * library (one per GPU, held until the process ends) instead of a caller
 * workspace.  Nothing is allocated: a call whose kvq_workspace_bytes(cfg, T,
 * opt) exceeds the array returns KVQ_ERR_WORKSPACE before any HIP call (use
 * fewer splits or kvq_decode_attention).  The array belongs to the current
 * device; `stream` must be a stream of that device.  Every call on one GPU
 * shares the array: calls that may overlap on one GPU (different streams, or
 * host threads) race and give wrong results; serialize them.  The first call
 * on a device looks up the array's address (KVQ_ERR_HIP if that fails).
 */
#define KVQ_STATIC_WORKSPACE_BYTES (16u << 20)
int kvq_decode_attention_static(const kvq_config* cfg, const void* arena, int64_t T,
                                const void* q, void* out, float sm_scale,
                                const kvq_attn_options* opt, hipStream_t stream);

/*
 * One decode step: append one token per sequence at position t0 (t0 >= 1, a
 * cache started by kvq_quantize_append) and attend over T = t0 + 1 tokens.
 * The result, cache bytes and output, equals kvq_quantize_append(t0, 1)
 * followed by kvq_decode_attention(T) (the append order of the decode step:
 * "...Need Different Axes", section "What should I actually turn on in
 * production?", and the decode loop of the configs).  When the MFMA kernel
 * serves the shape with one work-group per (sequence, kv head, split) (at
 * most 16 query heads per kv head, fewer with several value groups) and the
 * new token needs no fold (it enters the fp16 window, or both sides are FP8
 * with no window), the append runs inside the attention launch: the
 * work-group whose token range holds t0 writes the token before it reads
 * the cache, so one launch does both; otherwise the two calls run in turn.  Arguments as in the two calls (k_new, v_new:
 * [B][Hkv][1][D] in cfg->in_dtype; no FP8 scales or calibration here).
 */
int kvq_decode_step(const kvq_config* cfg, void* arena, int64_t t0, const void* k_new,
                    const void* v_new, const void* q, void* out, float sm_scale,
                    void* workspace, size_t workspace_bytes, const kvq_attn_options* opt,
                    hipStream_t stream);

/* Host only: 1 if kvq_decode_step at t0 appends inside the attention launch,
 * 0 if it runs a separate append first; < 0 on an invalid argument. */
int kvq_decode_step_fused(const kvq_config* cfg, int64_t t0, const kvq_attn_options* opt);

/*
 * Dequantize the cache as stored (pre-RoPE keys stay unrotated) to fp32
 * [B][Hkv][T][D], the dequantize halves of the listings cited at
 * kvq_quantize_append: x_hat = code*scale + zero with two roundings (INT_ASYM),
 * code*scale (INT_SYM), E4M3(code)*scale (FP8), window tokens widened from
 * fp16.  Either output may be NULL.
 */
int kvq_dequantize(const kvq_config* cfg, const void* arena, int64_t T,
                   float* k_out, float* v_out, hipStream_t stream);

/*
 * Paged caches (page_tokens = P > 0).  The pages describe the paged,
 * append-only caches of serving stacks, where per-channel key groups are
 * formed within fixed-size blocks and the most recent tokens stay in full
 * precision ("FP8 KV Cache Quantization: Why Keys Break Before Values",
 * section "Should you quantize keys pre-RoPE or post-RoPE?"; "KV Cache
 * Quantization: Why Keys and Values Need Different Axes", section "What
 * should I actually turn on in production?": the window is folded in
 * blocks).  A page holds P consecutive tokens of one sequence for all kv
 * heads; P is a multiple of 32 and of the key group Gt, so a page holds whole
 * key groups and whole 32-token value blocks and no group straddles pages.
 * The fp16 window stays per sequence (ring_k / ring_v).  Whole-axis and
 * per-tensor groups (which would rescale history on append) are refused.
 *
 * Common arguments:
 *   block_table: device int32 [B][max_blocks]: page of tokens
 *                [j*P, (j+1)*P) of sequence b at block_table[b*max_blocks + j].
 *                Pages are owned by the caller, who hands each sequence the
 *                pages its length needs (distinct sequences use distinct
 *                pages).  An entry outside [0, num_pages) is never written
 *                through (its tokens are skipped by appends) and reads as page
 *                0 (that sequence's attention is then unspecified).
 *   seq_lens:    device int32 [B]: tokens each sequence holds (before the call
 *                for appends and decode steps; at the call for attention and
 *                dequantize).  Sequences differ in length (ragged batches).
 * Lengths are device data: a sequence whose range does not fit max_tokens
 * or its block-table row is skipped by appends (its cache is left unchanged),
 * and attention clamps lengths to [0, max_seq_len]; a sequence of length 0
 * gets a zero output.
 */

/*
 * Paged append: append new_lens[b] tokens (n_max if new_lens is NULL) at
 * positions [seq_lens[b], seq_lens[b] + new_lens[b]) of each sequence b.
 *   k_new, v_new: device [B][Hkv][n_max][D] in cfg->in_dtype; sequence b uses
 *                 its first new_lens[b] tokens.
 *   flags: KVQ_INIT on the call that starts the cache (every sequence empty):
 *          it writes the RoPE tables and the FP8 scales (k_scale / v_scale if
 *          given, absmax / 448 over the call's tokens of all sequences with
 *          KVQ_CALIBRATE, else 1.0; E5M2 as in kvq_quantize_append).
 * Per-channel key groups and per-token value groups are formed and packed in
 * one pass (staged through fp16 when the cache has a window); tokens leaving
 * the window are folded in blocks of Gt.  Bytes written equal those of
 * kvq_quantize_append on a contiguous cache with the same tokens.
 */
int kvq_paged_quantize_append(const kvq_config* cfg, void* arena, const int32_t* block_table,
                              int32_t max_blocks, const int32_t* seq_lens,
                              const int32_t* new_lens, int32_t n_max, const void* k_new,
                              const void* v_new, const float* k_scale, const float* v_scale,
                              uint32_t flags, hipStream_t stream);

/*
 * Paged decode attention of one query per (sequence, query head) over the
 * seq_lens[b] cached tokens of each sequence (as kvq_decode_attention).
 * max_seq_len (host) bounds every seq_lens[b]; it sizes the split grid and
 * the workspace (kvq_workspace_bytes(cfg, max_seq_len, opt)) and must satisfy
 * max_seq_len <= max_tokens and max_seq_len <= max_blocks * P.
 */
int kvq_paged_decode_attention(const kvq_config* cfg, const void* arena,
                               const int32_t* block_table, int32_t max_blocks,
                               const int32_t* seq_lens, int64_t max_seq_len, const void* q,
                               void* out, float sm_scale, void* workspace,
                               size_t workspace_bytes, const kvq_attn_options* opt,
                               hipStream_t stream);

/*
 * Paged decode step: append one token per sequence at seq_lens[b] (k_new,
 * v_new: [B][Hkv][1][D]) and attend over seq_lens[b] + 1 tokens; max_seq_len
 * bounds seq_lens[b] + 1.  Equals kvq_paged_quantize_append followed by
 * kvq_paged_decode_attention with the lengths plus one.  The caller advances
 * its seq_lens afterwards.
 */
int kvq_paged_decode_step(const kvq_config* cfg, void* arena, const int32_t* block_table,
                          int32_t max_blocks, const int32_t* seq_lens, int64_t max_seq_len,
                          const void* k_new, const void* v_new, const void* q, void* out,
                          float sm_scale, void* workspace, size_t workspace_bytes,
                          const kvq_attn_options* opt, hipStream_t stream);

/*
 * Paged dequantize: sequence b's first seq_lens[b] tokens to fp32
 * [B][Hkv][max_seq_len][D] (later rows are left as they are).
 */
int kvq_paged_dequantize(const kvq_config* cfg, const void* arena, const int32_t* block_table,
                         int32_t max_blocks, const int32_t* seq_lens, int64_t max_seq_len,
                         float* k_out, float* v_out, hipStream_t stream);

/* Static description of a status code. */
const char* kvq_status_string(int status);

/* ABI version: bumped when the arena layout or a signature changes, or an
 * entry point is added (2: kvq_decode_step; 3: kvq_config.meta_dtype;
 * 4: kvq_decode_attention_static; 5: paged caches, kvq_config.page_tokens /
 * num_pages, kvq_layout.page_tokens / pages). */
int kvq_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif /* KVQ_H */
