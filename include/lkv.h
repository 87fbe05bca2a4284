/*
 * lkv.h -- C ABI of liblkv: decode attention over a compressed (latent) KV
 * cache on AMD Instinct MI355X (gfx950).
 *
 * What the library computes is stated by the pages it is built from:
 *   [GQLA] "GQLA: Group-Query Latent Attention for Hardware-Adaptive Large
 *          Language Model Decoding" (gist.science explainer), technical
 *          summary section 2 "Methodology": the MQA-absorbed path (all h_q
 *          query heads, W_UK folded into the query, attend over one shared
 *          per-token latent c_KV of width r_kv = d_c plus one shared RoPE key
 *          of width d^R_h = d_rope; the latent is also the value, and the
 *          output P.c_KV goes on to the folded W_UV), and the GQA path (the
 *          latent expanded once into g key/value groups of width d_h, stored
 *          beside the shared RoPE key; decode then runs plain grouped-query
 *          attention with no per-step expansion); W_UK and W_UV indexed by
 *          group.
 *   [GLA]  article on Grouped-Tied / Grouped Latent Attention (Zadouri,
 *          Strauss, Dao), section on GLA: a few latent heads, each shared by
 *          a group of query heads.
 *   [X]    X post by @classiclarryd on MLA vs GQA: GQA "copies" one KV head
 *          per group of query heads.
 * Paging, per-sequence lengths, the LSE output and split-KV are the
 * serving-side statement of the same problem; the pages do not fix them, and
 * this header does.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Every pointer named "device" is a HIP device pointer on the current
 *    device; "host" pointers are ordinary host memory.  The caller allocates
 *    and owns every buffer, workspace included.  The library keeps no pointer
 *    after a call returns and never allocates device memory.
 *  - Calls are asynchronous on `stream` (a hipStream_t; NULL = the null
 *    stream).  Buffers must stay alive until that stream work completes.
 *  - Every argument struct begins with `struct_size`, which must equal
 *    sizeof(the struct) as compiled against this header.
 *  - Strides are in elements.  Query, output and LSE arrays are dense,
 *    row-major, in the shapes given.
 *  - Cache tokens: the block table (device, int32 [batch, max_pages]) maps
 *    logical token j of sequence b to physical page block_table[b][j /
 *    page_size], slot j % page_size.  Entries past a sequence's last page are
 *    never read (padding such as -1 is fine).  Slots past the sequence length
 *    are never read either: they may hold any bits, NaN included.
 *  - seqlens (device, int32 [batch]) is the total cache length L_b,
 *    including the s_q tokens of this step, which already sit at positions
 *    L_b - s_q .. L_b - 1.  With causal != 0, query token t sees cache
 *    positions [0, L_b - s_q + t]; with causal == 0 it sees [0, L_b).  A row
 *    that sees no token (L_b == 0, or L_b < s_q when causal) yields O = 0 and
 *    LSE = -inf.  Device-resident values (lengths, table entries) are a
 *    caller contract: 0 <= L_b <= max_pages * page_size and every table entry
 *    of a used page names a page inside the cache.
 *  - Host-side checks of that contract.  The entry points that read a block
 *    table take optional host copies: seqlens_host (int32 [batch]),
 *    block_table_host (int32 [batch, max_pages]) and num_pages (the number
 *    of pages in the cache pool, 0 = unknown).  Given seqlens_host, every
 *    L_b must lie in [0, max_pages * page_size]; given block_table_host too,
 *    every entry of a used page (the first ceil(L_b / page_size) of row b)
 *    must be >= 0 and, when num_pages > 0, below num_pages.  A violation
 *    returns LKV_ERR_SHAPE naming the first bad entry, before any launch.
 *    The host copies must equal the device values.  With the environment
 *    variable LKV_DEBUG_CHECKS set to 1 when the library first checks it,
 *    copies the caller did not give are read back from the device (the
 *    call then synchronises `stream`) and the same checks run on every call.
 *  - Scores are softmax_scale * <q, k>, with softmax_scale positive and
 *    finite (else LKV_ERR_SHAPE); LSE is the natural log of the sum of
 *    exp(score) over the visible tokens, in float32.
 *  - Outputs have the input dtype; bf16 paths round to nearest even.  bf16
 *    inputs are multiplied on the MFMA units with float32 accumulation; the
 *    softmax probabilities are rounded to bf16 before the P.V product.
 *  - Errors: every host-checkable precondition is checked before any launch;
 *    a failure returns a status other than LKV_OK, launches nothing and
 *    leaves a message readable through lkv_last_error() on the calling
 *    thread.  No exception and no abort crosses this boundary.
 */
#ifndef LKV_H
#define LKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define LKV_ABI_VERSION 5

typedef enum {
  LKV_OK = 0,
  LKV_ERR_NULL = 1,        /* a required pointer is NULL */
  LKV_ERR_SHAPE = 2,       /* a size is out of range or inconsistent */
  LKV_ERR_UNSUPPORTED = 3, /* no kernel for this dtype / width / page size */
  LKV_ERR_ALIGN = 4,       /* a pointer or stride breaks the 16-byte rule */
  LKV_ERR_WORKSPACE = 5,   /* workspace missing or smaller than required */
  LKV_ERR_HIP = 6,         /* a HIP runtime call failed (message has details) */
  LKV_ERR_STRUCT = 7       /* struct_size does not match this header */
} lkv_status;

typedef enum { LKV_F32 = 0, LKV_BF16 = 1 } lkv_dtype;

/* LKV_ABI_VERSION of the built library. */
int lkv_abi_version(void);

/* Text of the last non-OK status returned on the calling thread ("" if
 * none).  The pointer stays valid until the next call on that thread. */
const char *lkv_last_error(void);

/* ------------------------------------------------------------------------
 * lkv_mla_decode -- MLA absorbed decode [GQLA section 2, MQA-absorbed path;
 * GLA section for n_latent > 1].
 *
 * For row (b, t, h), latent head l = h / (h_q / n_latent):
 *   score_j = softmax_scale * ( <q_nope[b,t,h,:], c_kv(j, l)>
 *                             + <q_rope[b,t,h,:], k_rope(j)> )
 *   out[b,t,h,:] = sum_j softmax(score)_j * c_kv(j, l)      (latent = value)
 *   lse[b,t,h]   = ln sum_j exp(score_j)
 *
 *   q_nope  device [batch, s_q, h_q, d_c]      absorbed query (W_UK folded in)
 *   q_rope  device [batch, s_q, h_q, d_rope]
 *   c_kv    device, element (page p, slot s, latent l, d) at
 *           (p*page_size + s)*kv_tok_stride + l*d_c + d
 *   k_rope  device, element (p, s, e) at (p*page_size + s)*rope_tok_stride + e
 *           (one RoPE key shared by every latent head).  c_kv and k_rope may
 *           alias one packed [.., n_latent*d_c + d_rope] buffer.
 *   out     device [batch, s_q, h_q, d_c], dtype of the inputs
 *   lse     device float32 [batch, s_q, h_q], or NULL
 *   workspace  device, at least lkv_mla_decode_workspace_size() bytes, 256-byte
 *           aligned.  Its contents need no initialisation and are scratch.
 *   num_splits  0 = automatic.  Otherwise the number of equal shares the
 *           concatenated cache tiles of the batch are cut into per query-row
 *           group (split-KV; a share may span several sequences and a
 *           sequence several shares; partial results are merged with the
 *           LSE-weighted combine of lkv_split_combine).
 *   seqlens_host  host int32 [batch] copy of seqlens, or NULL.  Used to skip
 *           the combine pass when no sequence is split, and for the
 *           host-side checks (with block_table_host, num_pages); it must
 *           equal the device values.
 *   kv_fp8, kv_scale  8-bit cache: with kv_fp8 nonzero, c_kv and k_rope hold
 *           OCP 8-bit float E4M3 codes x8 (one byte per element, strides in
 *           bytes) of the values kv_scale * x8, one scale for every cache of
 *           the call; queries and output stay bf16.  Each code converts
 *           exactly to bf16, so the arithmetic is that of the bf16 path on
 *           the dequantised values.  Needs dtype LKV_BF16, kv_scale positive
 *           and finite, cache strides multiples of 16 and 16-byte aligned
 *           cache pointers, and the widths (d_c, d_rope) in {(512, 64),
 *           (256, 64), (128, 64)}, plus (512, 0) and (256, 0) when a latent
 *           head has more than 32 query rows (s_q * h_q / n_latent).
 *           kv_fp8 = 0: the caches hold the dtype of the inputs and kv_scale
 *           is ignored.
 *   kernel_events  optional pair of hipEvent_t (either may be NULL), for
 *           timing the attention kernel alone (not the combine pass): they
 *           are attached to that kernel's launch (hipExtLaunchKernel) and
 *           take its start and end times, with no marker packet added to
 *           the stream.  Not recorded when the batch is empty.
 * Supported: bf16 with (d_c, d_rope) in {(512, 64), (256, 64), (128, 64),
 *   (512, 0)}, and also (256, 0) when a latent head has more than 32 query
 *   rows ((h_q / n_latent) * s_q > 32); f32 with d_c + d_rope <= 1024.  Any
 *   page_size >= 1.  Pointers 16-byte aligned, strides multiples of 8
 *   elements (bf16) or 4 (f32).
 * ---------------------------------------------------------------------- */
typedef struct {
  uint32_t struct_size;
  int32_t dtype; /* lkv_dtype */
  int32_t batch, s_q, h_q, n_latent, d_c, d_rope, page_size, max_pages;
  float softmax_scale;
  int32_t causal;
  int32_t num_splits;
  const void *q_nope;
  const void *q_rope;
  const void *c_kv;
  int64_t kv_tok_stride;
  const void *k_rope;
  int64_t rope_tok_stride;
  const int32_t *block_table;
  const int32_t *seqlens;
  const int32_t *seqlens_host;
  void *out;
  float *lse;
  void *workspace;
  size_t workspace_bytes;
  void *stream; /* hipStream_t */
  void *kernel_events[2]; /* hipEvent_t or NULL each */
  int32_t kv_fp8;  /* nonzero: 8-bit cache, see above */
  float kv_scale;  /* its dequantisation scale */
  /* host-side contract checks (see the conventions above); NULL / 0 = none */
  const int32_t *block_table_host;
  int64_t num_pages;
} lkv_mla_args;

lkv_status lkv_mla_decode(const lkv_mla_args *args);

/* Workspace bytes lkv_mla_decode needs for these arguments (pointers may be
 * NULL; only sizes, dtype and num_splits are read). */
lkv_status lkv_mla_decode_workspace_size(const lkv_mla_args *args, size_t *bytes);

/* ------------------------------------------------------------------------
 * lkv_mla_decode_noalloc -- lkv_mla_decode for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, hosts
 * that forbid allocation): the same computation and kernels, with the split
 * partials and per-sequence plan kept in a static device array of the
 * library (LKV_NOALLOC_SCRATCH_BYTES per GPU, reserved on each GPU the
 * library runs on until the process ends) instead of a caller workspace.
 * args->workspace and args->workspace_bytes are ignored; the caller still
 * passes every input and output.  Arguments whose workspace size
 * (lkv_mla_decode_workspace_size) exceeds LKV_NOALLOC_SCRATCH_BYTES are
 * rejected with LKV_ERR_WORKSPACE before any launch.  No device or host
 * memory is allocated (LKV_DEBUG_CHECKS read-backs are not done here; the
 * host-copy checks are).  Every call on one GPU shares that GPU's array:
 * calls that overlap on one GPU (on different streams, or from different
 * threads) race and must be serialised by the caller.  The array's contents
 * need no initialisation and are not meaningful after a call.
 * ---------------------------------------------------------------------- */
#define LKV_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
lkv_status lkv_mla_decode_noalloc(const lkv_mla_args *args);

/* ------------------------------------------------------------------------
 * lkv_gqa_decode -- grouped-query decode over an expanded cache [GQLA
 * section 2, GQA path: g groups of K/V width d_h plus the shared RoPE key;
 * with d_rope == 0 it is plain GQA, the X post's "copying"].
 *
 * For row (b, t, h), KV head g = h / (h_q / n_kv):
 *   score_j = softmax_scale * ( <q[b,t,h,:], K(j, g)> + <q_rope[b,t,h,:], k_rope(j)> )
 *   out[b,t,h,:] = sum_j softmax(score)_j * V(j, g)
 *
 *   q        device [batch, s_q, h_q, d_h]
 *   q_rope   device [batch, s_q, h_q, d_rope], NULL iff d_rope == 0
 *   k_cache  device, element (p, s, g, d) at (p*page_size + s)*k_tok_stride + g*d_h + d
 *   v_cache  device, element (p, s, g, d) at (p*page_size + s)*v_tok_stride + g*d_h + d
 *   k_rope   device, as in lkv_mla_args; NULL iff d_rope == 0
 *   out      device [batch, s_q, h_q, d_h];  lse device float32 [batch, s_q, h_q] or NULL
 *   workspace / num_splits / seqlens_host / kernel_events / kv_fp8 /
 *   kv_scale as in lkv_mla_args (8-bit caches: k_cache, v_cache and k_rope
 *   all hold codes; (d_h, d_rope) in {(128, 64), (128, 0)}).
 * Supported: bf16 with (d_h, d_rope) in {(128, 64), (128, 0), (64, 0),
 *   (256, 0)}; f32 with d_h + d_rope <= 1024.
 * ---------------------------------------------------------------------- */
typedef struct {
  uint32_t struct_size;
  int32_t dtype;
  int32_t batch, s_q, h_q, n_kv, d_h, d_rope, page_size, max_pages;
  float softmax_scale;
  int32_t causal;
  int32_t num_splits;
  const void *q;
  const void *q_rope;
  const void *k_cache;
  int64_t k_tok_stride;
  const void *v_cache;
  int64_t v_tok_stride;
  const void *k_rope;
  int64_t rope_tok_stride;
  const int32_t *block_table;
  const int32_t *seqlens;
  const int32_t *seqlens_host;
  void *out;
  float *lse;
  void *workspace;
  size_t workspace_bytes;
  void *stream;
  void *kernel_events[2]; /* hipEvent_t or NULL each */
  int32_t kv_fp8;  /* as in lkv_mla_args */
  float kv_scale;
  const int32_t *block_table_host; /* as in lkv_mla_args */
  int64_t num_pages;
} lkv_gqa_args;

lkv_status lkv_gqa_decode(const lkv_gqa_args *args);
lkv_status lkv_gqa_decode_workspace_size(const lkv_gqa_args *args, size_t *bytes);

/* ------------------------------------------------------------------------
 * lkv_gqla_expand_latent -- cache-write-time expansion of the latent into g
 * key/value groups [GQLA section 2, GQA path: expanded once, then no
 * per-step latent expansion].
 *
 * For every sequence b and token j in [start_pos[b], seqlens[b]), with
 * row = block_table[b][j / page_size]*page_size + j % page_size:
 *   k_out(row, g, :) = c_kv(row, :) . W_UK[g]      (d_c -> d_h)
 *   v_out(row, g, :) = c_kv(row, :) . W_UV[g]
 * computed with float32 accumulation and rounded to bf16 (nearest even).
 * The expanded caches use the same page ids as the latent cache.
 *
 *   c_kv    device bf16, element (row, d) at row*kv_tok_stride + d
 *   w_uk, w_uv  device bf16 [g, d_c, d_h] (row-major: d_c rows of d_h)
 *   start_pos   device int32 [batch] or NULL (= 0): append-only expansion
 *   k_out, v_out  device bf16, element (row, g, e) at row*k_tok_stride + g*d_h + e
 *                 (v_tok_stride for v_out)
 *   out_fp8, out_scale  8-bit expanded caches: with out_fp8 nonzero, k_out
 *           and v_out receive OCP 8-bit float E4M3 codes (one byte per
 *           element, strides in bytes, multiples of 16) of y = fl32(r * s),
 *           where r is the float32 result and s = fl32(1 / out_scale): y is
 *           rounded to the nearest code (ties to the even code), magnitudes
 *           past 448 (infinities included) saturate to +-448, and a NaN
 *           gives the NaN code S.1111.111.  When out_scale is a power of two
 *           the product is exact and r is rounded once; otherwise the
 *           float32 product adds one rounding of relative size 2^-24 before
 *           the encoding.  This is the cache that lkv_gqa_decode reads with
 *           kv_fp8 = 1, kv_scale = out_scale.  out_scale must be positive,
 *           finite and with a finite float32 reciprocal.
 * Supported: bf16, d_c a multiple of 64 up to 512, d_h in {64, 128, 256}.
 * Rows outside [start_pos, seqlens) are not written.
 * ---------------------------------------------------------------------- */
typedef struct {
  uint32_t struct_size;
  int32_t dtype;
  int32_t batch, g, d_c, d_h, page_size, max_pages;
  const void *c_kv;
  int64_t kv_tok_stride;
  const void *w_uk;
  const void *w_uv;
  const int32_t *block_table;
  const int32_t *seqlens;
  const int32_t *start_pos;
  void *k_out;
  int64_t k_tok_stride;
  void *v_out;
  int64_t v_tok_stride;
  void *stream;
  int32_t out_fp8;  /* nonzero: 8-bit expanded caches, see above */
  float out_scale;  /* their scale */
  /* host-side contract checks (see the conventions above); NULL / 0 = none */
  const int32_t *seqlens_host;
  const int32_t *block_table_host;
  int64_t num_pages;
} lkv_expand_args;

lkv_status lkv_gqla_expand_latent(const lkv_expand_args *args);

/* ------------------------------------------------------------------------
 * lkv_absorb_query / lkv_up_project -- the per-head projections on either
 * side of absorbed decode [GQLA section 2, MQA-absorbed path: W_UK folds
 * into the query, W_UV into the output].  For query row (b, t, h), with
 * weight block wb = h / (h_q / n_w) of w [n_w, d_c, d_h] (n_w = h_q for
 * per-head weights, n_w = g for GQLA's group-indexed weights):
 *   lkv_absorb_query   y[b,t,h,k] = sum_d w[wb][k][d] * x[b,t,h,d]
 *                      (x: the per-head query [batch, s_q, h_q, d_h];
 *                       y: the absorbed query [batch, s_q, h_q, d_c])
 *   lkv_up_project     y[b,t,h,d] = sum_k x[b,t,h,k] * w[wb][k][d]
 *                      (x: the latent output [batch, s_q, h_q, d_c];
 *                       y: [batch, s_q, h_q, d_h])
 * float32 accumulation, bf16 output (round to nearest even).
 *   x, w, y  device bf16, dense row-major as shown, 16-byte aligned
 * Supported: bf16, d_c and d_h multiples of 64; h_q a multiple of n_w.
 * ---------------------------------------------------------------------- */
typedef struct {
  uint32_t struct_size;
  int32_t dtype;
  int32_t batch, s_q, h_q, n_w, d_c, d_h;
  const void *x;
  const void *w;
  void *y;
  void *stream;
} lkv_proj_args;

lkv_status lkv_absorb_query(const lkv_proj_args *args);
lkv_status lkv_up_project(const lkv_proj_args *args);

/* ------------------------------------------------------------------------
 * lkv_append_tokens -- cache write of a step's new tokens [GQLA section 2:
 * every token's latent (plus the shared RoPE key) is cached once].  Row t of
 * sequence b's new rows is copied to logical position j = seqlens[b] - s_q
 * + t (skipped when j < 0), i.e. cache row
 * block_table[b][j / page_size]*page_size + j % page_size.
 *   src      device [batch, s_q, width] elements (dtype), dense
 *   cache    device, row r at r*tok_stride elements (of the cache's type)
 *   seqlens  device int32 [batch]: lengths including the new tokens
 *   out_fp8, out_scale  8-bit cache (the caches lkv_mla_decode and
 *           lkv_gqa_decode read with kv_fp8 = 1, kv_scale = out_scale, e.g.
 *           the RoPE key beside 8-bit expanded caches): with out_fp8 nonzero
 *           each bf16 value x becomes the OCP E4M3 code of fl32(x * s), s =
 *           fl32(1 / out_scale), rounded to the nearest code (ties to even),
 *           saturating at +-448, NaN to S.1111.111 -- one byte per element.
 *           Needs dtype LKV_BF16 and out_scale positive, finite, with a
 *           finite float32 reciprocal.
 * Supported: bf16 or f32 (8-bit output from bf16); width and tok_stride
 * multiples of 16 bytes of the cache's element; src and cache 16-byte
 * aligned; tok_stride >= width.
 * ---------------------------------------------------------------------- */
typedef struct {
  uint32_t struct_size;
  int32_t dtype;
  int32_t batch, s_q, width, page_size, max_pages;
  const void *src;
  void *cache;
  int64_t tok_stride;
  const int32_t *block_table;
  const int32_t *seqlens;
  void *stream;
  /* host-side contract checks (see the conventions above); NULL / 0 = none */
  const int32_t *seqlens_host;
  const int32_t *block_table_host;
  int64_t num_pages;
  int32_t out_fp8;  /* nonzero: 8-bit (E4M3) cache, see above */
  float out_scale;
} lkv_append_args;

lkv_status lkv_append_tokens(const lkv_append_args *args);

/* ------------------------------------------------------------------------
 * lkv_split_combine -- merge split-KV partial results with their LSEs.
 * For sequence b, works w in [work_offsets[b], work_offsets[b+1]):
 *   lse = ln sum_w exp(lse_part[w]),  out = sum_w exp(lse_part[w] - lse) o_part[w]
 * A work with lse_part = -inf contributes nothing; a sequence with no
 * contributing work gets out = 0 and lse = -inf.
 *
 *   o_part        device float32 [n_work, s_q, h_q, d_v]
 *   lse_part      device float32 [n_work, s_q, h_q]
 *   work_offsets  device int32 [batch + 1], non-decreasing, last = n_work
 *   out           device [batch, s_q, h_q, d_v] of `dtype`; lse float32 or NULL
 * Supported: d_v a multiple of 4 up to 1024.
 * ---------------------------------------------------------------------- */
typedef struct {
  uint32_t struct_size;
  int32_t dtype;
  int32_t batch, s_q, h_q, d_v, n_work;
  const float *o_part;
  const float *lse_part;
  const int32_t *work_offsets;
  void *out;
  float *lse;
  void *stream;
} lkv_combine_args;

lkv_status lkv_split_combine(const lkv_combine_args *args);

#ifdef __cplusplus
}
#endif

#endif /* LKV_H */
