// abi.cpp -- the extern "C" boundary of liblkv (declared in include/lkv.h).
//
// Host-side only: argument validation, the split-KV share count, workspace
// carving and kernel dispatch.  Every check runs before any launch; a failed
// check returns a status and leaves a message for lkv_last_error().
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "lkv.h"
#include "lkv_internal.h"

namespace {

thread_local std::string g_error;

lkv_status fail(lkv_status s, const char *fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_error = buf;
  return s;
}

lkv_status hip_fail(hipError_t e, const char *what) {
  return fail(LKV_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

// Compute units of the current device, cached per device id.
int device_cus(int *out) {
  static std::mutex mu;
  static int cache[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return -1;
  std::lock_guard<std::mutex> lock(mu);
  if (dev >= 0 && dev < 64 && cache[dev] > 0) {
    *out = cache[dev];
    return 0;
  }
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return -1;
  if (dev >= 0 && dev < 64) cache[dev] = cus;
  *out = cus;
  return 0;
}

// LKV_DEBUG_CHECKS=1 in the environment (read once): read missing host
// copies of the lengths and the block table back from the device for the
// contract checks.
bool debug_checks() {
  static const bool on = [] {
    const char *v = std::getenv("LKV_DEBUG_CHECKS");
    return v && std::strcmp(v, "1") == 0;
  }();
  return on;
}

// Host copies of the device-resident part of the contract: sequence lengths
// and block-table entries.  Null members are not checked.
struct HostView {
  const int32_t *seqlens;  // [B]
  const int32_t *table;    // [B, max_pages]
  long long num_pages;     // pool size, 0 = unknown
};

// 0 <= L_b <= max_pages * page_size; every entry of a used page names a page
// of the pool.  Runs on the host before any launch.
lkv_status check_contract(int B, int page_size, int max_pages, const HostView &h) {
  if (!h.seqlens || B <= 0) return LKV_OK;
  const long long cap = (long long)max_pages * page_size;
  for (int b = 0; b < B; ++b) {
    const long long L = h.seqlens[b];
    if (L < 0 || L > cap)
      return fail(LKV_ERR_SHAPE, "seqlens[%d] = %lld is outside [0, max_pages * page_size = %lld]", b, L, cap);
    if (!h.table) continue;
    const long long used = (L + page_size - 1) / page_size;
    const int32_t *row = h.table + (size_t)b * (size_t)max_pages;
    for (long long i = 0; i < used; ++i) {
      const long long pg = row[i];
      if (pg < 0 || (h.num_pages > 0 && pg >= h.num_pages))
        return fail(LKV_ERR_SHAPE, "block_table[%d][%lld] = %lld is not a page of the pool (%lld pages)", b, i, pg,
                    h.num_pages);
    }
  }
  return LKV_OK;
}

// The contract checks of one call: with the caller's host copies, and under
// LKV_DEBUG_CHECKS=1 with copies read back from the device for the missing
// ones (synchronising the stream).
lkv_status check_call_contract(int B, int page_size, int max_pages, const int32_t *seqlens_dev,
                               const int32_t *table_dev, HostView h, hipStream_t stream) {
  std::vector<int32_t> sl, tb;
  if (debug_checks() && B > 0 && (!h.seqlens || !h.table)) {
    hipError_t e = hipSuccess;
    if (!h.seqlens) {
      sl.resize((size_t)B);
      e = hipMemcpyAsync(sl.data(), seqlens_dev, sl.size() * sizeof(int32_t), hipMemcpyDeviceToHost, stream);
      h.seqlens = sl.data();
    }
    if (e == hipSuccess && !h.table) {
      tb.resize((size_t)B * (size_t)max_pages);
      e = hipMemcpyAsync(tb.data(), table_dev, tb.size() * sizeof(int32_t), hipMemcpyDeviceToHost, stream);
      h.table = tb.data();
    }
    if (e == hipSuccess) e = hipStreamSynchronize(stream);
    if (e != hipSuccess) return hip_fail(e, "LKV_DEBUG_CHECKS read-back of lengths and block table");
  }
  return check_contract(B, page_size, max_pages, h);
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }
bool aligned4(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 3) == 0; }
size_t round256(size_t x) { return (x + 255) & ~size_t(255); }

int log2_exact(int x) {
  if (x <= 0 || (x & (x - 1))) return -1;
  int s = 0;
  while ((1 << s) < x) ++s;
  return s;
}

int seq_tiles(int L) { return L <= 0 ? 1 : (L + lkv::kTile - 1) / lkv::kTile; }

// Problem shape common to the two decode entry points.
struct Shape {
  int dtype, B, s_q, h_q, n_kvh, dk, dr, dv, page_size, max_pages, causal, num_splits;
  bool v_alias;
  bool fp8;        // the caches hold OCP E4M3 codes
  float kv_scale;  // their dequantisation scale
};

// Kernel for many query rows over one latent head (score and value products
// on separate waves), else the row-tiled kernel.
enum { kLatentNone = 0, kLatentSplit = 1 };

struct Plan {
  int latent;      // kernel for many rows over one latent (0: the row-tiled kernel)
  int rows;        // query rows per work-group (bf16 path)
  int row_tiles;
  int n_chunks;
  size_t ws_opart, ws_lse, ws_meta, ws_total;
};

lkv_status make_plan(const Shape &s, Plan *pl) {
  const int rows_per_kvh = s.s_q * (s.h_q / s.n_kvh);
  // Many query rows over one latent: one work-group takes 64 of them and
  // reads each cache tile once for all of them.
  pl->latent = kLatentNone;
  if (s.dtype == LKV_BF16 && s.v_alias && rows_per_kvh > 32 && lkv::mla_split_supported(s.dk, s.dr))
    pl->latent = kLatentSplit;
  pl->rows = pl->latent == kLatentSplit ? lkv::mla_split_rows(s.dk, s.dr, rows_per_kvh, s.fp8)
                                        : lkv::mfma_decode_rows(rows_per_kvh);
  pl->row_tiles = (rows_per_kvh + pl->rows - 1) / pl->rows;
  int cus = 0;
  if (device_cus(&cus) != 0) return fail(LKV_ERR_HIP, "cannot query the device compute-unit count");
  const int groups = s.n_kvh * pl->row_tiles;
  // automatic plan: one share per row group for every work-group slot of the
  // chip (CUs x work-groups resident per CU)
  int per_cu = 1;
  if (s.dtype == LKV_BF16 && pl->latent == kLatentNone)
    per_cu = lkv::mfma_decode_blocks_per_cu(s.dk, s.dr, s.dv, s.v_alias, pl->rows, s.fp8);
  int chunks = s.num_splits > 0 ? s.num_splits : std::max(1, cus * per_cu / std::max(1, groups));
  chunks = std::min(chunks, 1 << 20);
  pl->n_chunks = chunks;
  const size_t slots = (size_t)s.B + (size_t)chunks;
  const size_t rows = (size_t)s.s_q * s.h_q;
  pl->ws_opart = round256(slots * rows * s.dv * sizeof(float));
  pl->ws_lse = round256(slots * rows * sizeof(float));
  pl->ws_meta = round256((size_t)s.B * 2 * sizeof(int32_t));
  pl->ws_total = s.dtype == LKV_BF16 ? pl->ws_opart + pl->ws_lse + pl->ws_meta : 0;
  return LKV_OK;
}

// With host lengths: does any sequence span more than one share?
bool any_split(const int32_t *seqlens_host, int B, int n_chunks) {
  long long total = 0;
  for (int b = 0; b < B; ++b) total += seq_tiles(seqlens_host[b]);
  const long long chunk = (total + n_chunks - 1) / n_chunks;
  long long cu = 0;
  for (int b = 0; b < B; ++b) {
    const int nb = seq_tiles(seqlens_host[b]);
    if (cu / chunk != (cu + nb - 1) / chunk) return true;
    cu += nb;
  }
  return false;
}

lkv_status check_shape(const Shape &s) {
  if (s.dtype != LKV_F32 && s.dtype != LKV_BF16) return fail(LKV_ERR_UNSUPPORTED, "dtype %d is not LKV_F32 or LKV_BF16", s.dtype);
  if (s.B < 0 || s.B > 65536) return fail(LKV_ERR_SHAPE, "batch %d outside [0, 65536]", s.B);
  if (s.s_q < 1 || s.s_q > 64) return fail(LKV_ERR_SHAPE, "s_q %d outside [1, 64]", s.s_q);
  if (s.h_q < 1 || s.n_kvh < 1 || s.h_q % s.n_kvh)
    return fail(LKV_ERR_SHAPE, "h_q %d must be a positive multiple of the %d KV/latent heads", s.h_q, s.n_kvh);
  if (s.dk < 1 || s.dr < 0 || s.dv < 1) return fail(LKV_ERR_SHAPE, "head widths must be positive");
  if (s.page_size < 1 || s.max_pages < 1) return fail(LKV_ERR_SHAPE, "page_size and max_pages must be positive");
  if ((long long)s.page_size * s.max_pages > (1LL << 30)) return fail(LKV_ERR_SHAPE, "page_size * max_pages exceeds 2^30 tokens");
  if ((long long)s.B * s.s_q * s.h_q > (1LL << 30)) return fail(LKV_ERR_SHAPE, "batch * s_q * h_q exceeds 2^30 rows");
  if (s.num_splits < 0) return fail(LKV_ERR_SHAPE, "num_splits %d is negative", s.num_splits);
  if (s.fp8) {
    if (s.dtype != LKV_BF16) return fail(LKV_ERR_UNSUPPORTED, "an 8-bit cache needs bf16 queries and output");
    if (!(s.kv_scale > 0.f) || !std::isfinite(s.kv_scale))
      return fail(LKV_ERR_SHAPE, "kv_scale %g must be positive and finite", (double)s.kv_scale);
    const int rows_per_kvh = s.s_q * (s.h_q / s.n_kvh);
    const bool many = s.v_alias && rows_per_kvh > 32 && lkv::mla_split_supported(s.dk, s.dr);
    if (!many && !lkv::mfma_decode_supported(s.dk, s.dr, s.dv, s.v_alias, true))
      return fail(LKV_ERR_UNSUPPORTED,
                  "no 8-bit-cache kernel for key width %d + RoPE %d, value width %d (%s); compiled: latent "
                  "512+64, 256+64, 128+64 (and 512+0, 256+0 above 32 rows per latent head); grouped 128+64, "
                  "128+0",
                  s.dk, s.dr, s.dv, s.v_alias ? "latent" : "grouped");
  } else if (s.dtype == LKV_BF16) {
    const int rows_per_kvh = s.s_q * (s.h_q / s.n_kvh);
    const bool many = s.v_alias && rows_per_kvh > 32 && lkv::mla_split_supported(s.dk, s.dr);
    if (!many && !lkv::mfma_decode_supported(s.dk, s.dr, s.dv, s.v_alias, false))
      return fail(LKV_ERR_UNSUPPORTED,
                  "no bf16 kernel for key width %d + RoPE %d, value width %d (%s); compiled: latent "
                  "512+64, 256+64, 128+64, 512+0; grouped 128+64, 128+0, 64+0, 256+0",
                  s.dk, s.dr, s.dv, s.v_alias ? "latent" : "grouped");
  } else if (s.dv > 1024) {
    return fail(LKV_ERR_UNSUPPORTED, "float32 path supports value width up to 1024, got %d", s.dv);
  }
  return LKV_OK;
}

struct Ptrs {
  const void *q, *q_rope, *k, *r, *v;
  long long k_stride, r_stride, v_stride;
  const int32_t *bt, *seqlens, *seqlens_host, *bt_host;
  long long num_pages;
  void *out;
  float *lse;
  void *ws;
  size_t ws_bytes;
  hipStream_t stream;
  void *const *events;  // [2], entries may be NULL
};

lkv_status check_ptrs(const Shape &s, const Ptrs &p) {
  if (!p.q || !p.k || !p.v || !p.bt || !p.seqlens || !p.out) return fail(LKV_ERR_NULL, "a required pointer is NULL");
  if (s.dr > 0 && (!p.q_rope || !p.r)) return fail(LKV_ERR_NULL, "d_rope > 0 needs q_rope and k_rope");
  if (s.dr == 0 && (p.q_rope || p.r)) return fail(LKV_ERR_SHAPE, "q_rope / k_rope given with d_rope == 0");
  const long long kv_need = s.v_alias ? (long long)s.n_kvh * s.dk : (long long)s.n_kvh * s.dk;
  if (p.k_stride < kv_need) return fail(LKV_ERR_SHAPE, "key token stride %lld < %lld", p.k_stride, kv_need);
  if (!s.v_alias && p.v_stride < (long long)s.n_kvh * s.dv)
    return fail(LKV_ERR_SHAPE, "value token stride %lld < %lld", p.v_stride, (long long)s.n_kvh * s.dv);
  if (s.dr > 0 && p.r_stride < s.dr) return fail(LKV_ERR_SHAPE, "RoPE token stride %lld < d_rope %d", p.r_stride, s.dr);
  if (s.dtype == LKV_BF16) {
    const void *all[] = {p.q, p.q_rope, p.k, p.r, p.v, p.out};
    for (const void *x : all)
      if (x && !aligned16(x)) return fail(LKV_ERR_ALIGN, "bf16 buffers must be 16-byte aligned");
    if (p.k_stride % 8 || p.v_stride % 8 || (s.dr > 0 && p.r_stride % 8))
      return fail(LKV_ERR_ALIGN, "bf16 token strides must be multiples of 8 elements");
    if (s.fp8 && (p.k_stride % 16 || p.v_stride % 16 || (s.dr > 0 && p.r_stride % 16)))
      return fail(LKV_ERR_ALIGN, "8-bit cache token strides must be multiples of 16 elements");
    // tile loads address 64 token rows from one base with 32-bit offsets
    if (p.k_stride > (1 << 24) || p.v_stride > (1 << 24) || p.r_stride > (1 << 24))
      return fail(LKV_ERR_SHAPE, "bf16 token strides above 2^24 elements are not supported");
    if (!p.ws) return fail(LKV_ERR_WORKSPACE, "workspace is NULL");
    if (reinterpret_cast<uintptr_t>(p.ws) & 255) return fail(LKV_ERR_ALIGN, "workspace must be 256-byte aligned");
  } else {
    const void *all[] = {p.q, p.q_rope, p.k, p.r, p.v, p.out};
    for (const void *x : all)
      if (x && !aligned4(x)) return fail(LKV_ERR_ALIGN, "float32 buffers must be 4-byte aligned");
  }
  if (p.lse && !aligned4(p.lse)) return fail(LKV_ERR_ALIGN, "lse must be 4-byte aligned");
  return LKV_OK;
}

lkv_status run_decode(const Shape &s, const Ptrs &p, float scale, bool readback = true) {
  lkv_status st = check_shape(s);
  if (st != LKV_OK) return st;
  if (!(scale > 0.f) || !std::isfinite(scale))
    return fail(LKV_ERR_SHAPE, "softmax_scale %g must be positive and finite", (double)scale);
  if (s.B == 0) return LKV_OK;  // nothing to compute; pointers of empty tensors may be NULL
  if ((st = check_ptrs(s, p)) != LKV_OK) return st;
  if (readback) {
    if ((st = check_call_contract(s.B, s.page_size, s.max_pages, p.seqlens, p.bt,
                                  HostView{p.seqlens_host, p.bt_host, p.num_pages}, p.stream)) != LKV_OK)
      return st;
  } else if ((st = check_contract(s.B, s.page_size, s.max_pages, HostView{p.seqlens_host, p.bt_host, p.num_pages})) !=
             LKV_OK) {
    return st;
  }
  Plan pl;
  if ((st = make_plan(s, &pl)) != LKV_OK) return st;
  if (s.dtype == LKV_BF16 && p.ws_bytes < pl.ws_total)
    return fail(LKV_ERR_WORKSPACE, "workspace has %zu bytes, need %zu", p.ws_bytes, pl.ws_total);

  lkv::DecodeParams d{};
  d.q = p.q;
  d.q_rope = p.q_rope;
  d.k = p.k;
  d.r = p.r;
  d.v = p.v;
  d.k_stride = p.k_stride;
  d.r_stride = p.r_stride;
  d.v_stride = p.v_stride;
  d.block_table = p.bt;
  d.seqlens = p.seqlens;
  d.out = p.out;
  d.lse = p.lse;
  d.B = s.B;
  d.s_q = s.s_q;
  d.h_q = s.h_q;
  d.n_kvh = s.n_kvh;
  d.hpk = s.h_q / s.n_kvh;
  d.page_size = s.page_size;
  d.page_shift = log2_exact(s.page_size);
  d.max_pages = s.max_pages;
  d.rows_per_kvh = s.s_q * d.hpk;
  d.tile_rows = pl.rows;
  d.row_tiles = pl.row_tiles;
  d.n_chunks = pl.n_chunks;
  d.causal = s.causal ? 1 : 0;
  // an 8-bit cache holds values kv_scale * code: the scores take the
  // factor through the softmax scale, the output through its normalisation
  d.scale_log2 = scale * (s.fp8 ? s.kv_scale : 1.f) * 1.4426950408889634f;
  d.out_scale = s.fp8 ? s.kv_scale : 1.f;
  d.fp8 = s.fp8 ? 1 : 0;
  d.dk = s.dk;
  d.dr = s.dr;
  d.dv = s.dv;

  lkv::LaunchEvents ev;
  ev.start = static_cast<hipEvent_t>(p.events[0]);
  ev.stop = static_cast<hipEvent_t>(p.events[1]);
  hipError_t e;
  if (s.dtype == LKV_F32) {
    e = lkv::launch_f32_decode(d, p.stream, ev);
    if (e != hipSuccess) return hip_fail(e, "float32 decode launch");
    return LKV_OK;
  }
  char *ws = static_cast<char *>(p.ws);
  d.o_part = reinterpret_cast<float *>(ws);
  d.lse_part = reinterpret_cast<float *>(ws + pl.ws_opart);
  d.meta = reinterpret_cast<int32_t *>(ws + pl.ws_opart + pl.ws_lse);
  e = pl.latent == kLatentSplit ? lkv::launch_mla_split(d, p.stream, ev)
                                : lkv::launch_mfma_decode(d, s.v_alias, pl.rows, p.stream, ev);
  if (e != hipSuccess) return hip_fail(e, "decode launch");
  if (p.seqlens_host && !any_split(p.seqlens_host, s.B, pl.n_chunks)) return LKV_OK;
  lkv::CombineParams c{};
  c.o_part = d.o_part;
  c.lse_part = d.lse_part;
  c.meta = d.meta;
  c.offsets = nullptr;
  c.out = p.out;
  c.lse = p.lse;
  c.B = s.B;
  c.s_q = s.s_q;
  c.h_q = s.h_q;
  c.dv = s.dv;
  c.skip_single = 1;
  c.out_bf16 = 1;
  e = lkv::launch_combine(c, p.stream);
  if (e != hipSuccess) return hip_fail(e, "combine launch");
  return LKV_OK;
}

Shape mla_shape(const lkv_mla_args *a) {
  return Shape{a->dtype, a->batch, a->s_q, a->h_q, a->n_latent, a->d_c, a->d_rope, a->d_c,
               a->page_size, a->max_pages, a->causal, a->num_splits, true, a->kv_fp8 != 0, a->kv_scale};
}

Shape gqa_shape(const lkv_gqa_args *a) {
  return Shape{a->dtype, a->batch, a->s_q, a->h_q, a->n_kv, a->d_h, a->d_rope, a->d_h,
               a->page_size, a->max_pages, a->causal, a->num_splits, false, a->kv_fp8 != 0, a->kv_scale};
}

}  // namespace

extern "C" {

int lkv_abi_version(void) { return LKV_ABI_VERSION; }

const char *lkv_last_error(void) { return g_error.c_str(); }

lkv_status lkv_mla_decode_workspace_size(const lkv_mla_args *a, size_t *bytes) {
  if (!a || !bytes) return fail(LKV_ERR_NULL, "args or bytes is NULL");
  if (a->struct_size != sizeof(lkv_mla_args)) return fail(LKV_ERR_STRUCT, "struct_size %u != %zu", a->struct_size, sizeof(lkv_mla_args));
  const Shape s = mla_shape(a);
  lkv_status st = check_shape(s);
  if (st != LKV_OK) return st;
  Plan pl;
  if ((st = make_plan(s, &pl)) != LKV_OK) return st;
  *bytes = pl.ws_total;
  return LKV_OK;
}

lkv_status lkv_mla_decode(const lkv_mla_args *a) {
  if (!a) return fail(LKV_ERR_NULL, "args is NULL");
  if (a->struct_size != sizeof(lkv_mla_args)) return fail(LKV_ERR_STRUCT, "struct_size %u != %zu", a->struct_size, sizeof(lkv_mla_args));
  const Shape s = mla_shape(a);
  if (a->n_latent >= 1 && a->kv_tok_stride < (long long)a->n_latent * a->d_c)
    return fail(LKV_ERR_SHAPE, "kv_tok_stride %lld < n_latent * d_c", (long long)a->kv_tok_stride);
  Ptrs p{a->q_nope, a->q_rope, a->c_kv, a->k_rope, a->c_kv, a->kv_tok_stride, a->rope_tok_stride,
         a->kv_tok_stride, a->block_table, a->seqlens, a->seqlens_host, a->block_table_host,
         (long long)a->num_pages, a->out, a->lse, a->workspace, a->workspace_bytes,
         static_cast<hipStream_t>(a->stream), a->kernel_events};
  return run_decode(s, p, a->softmax_scale);
}

lkv_status lkv_mla_decode_noalloc(const lkv_mla_args *a) {
  if (!a) return fail(LKV_ERR_NULL, "args is NULL");
  if (a->struct_size != sizeof(lkv_mla_args)) return fail(LKV_ERR_STRUCT, "struct_size %u != %zu", a->struct_size, sizeof(lkv_mla_args));
  const Shape s = mla_shape(a);
  if (a->n_latent >= 1 && a->kv_tok_stride < (long long)a->n_latent * a->d_c)
    return fail(LKV_ERR_SHAPE, "kv_tok_stride %lld < n_latent * d_c", (long long)a->kv_tok_stride);
  lkv_status st = check_shape(s);
  if (st != LKV_OK) return st;
  void *ws = nullptr;
  size_t cap = 0;
  if (s.B > 0) {
    Plan pl;
    if ((st = make_plan(s, &pl)) != LKV_OK) return st;
    if (pl.ws_total > LKV_NOALLOC_SCRATCH_BYTES)
      return fail(LKV_ERR_WORKSPACE,
                  "lkv_mla_decode_noalloc: these arguments need %zu bytes of scratch, above the library's static "
                  "%zu bytes (LKV_NOALLOC_SCRATCH_BYTES); use lkv_mla_decode with a workspace",
                  pl.ws_total, (size_t)LKV_NOALLOC_SCRATCH_BYTES);
    const hipError_t e = lkv::static_scratch(&ws, &cap);
    if (e != hipSuccess) return hip_fail(e, "static scratch address");
  }
  Ptrs p{a->q_nope, a->q_rope, a->c_kv, a->k_rope, a->c_kv, a->kv_tok_stride, a->rope_tok_stride,
         a->kv_tok_stride, a->block_table, a->seqlens, a->seqlens_host, a->block_table_host,
         (long long)a->num_pages, a->out, a->lse, ws, cap, static_cast<hipStream_t>(a->stream), a->kernel_events};
  return run_decode(s, p, a->softmax_scale, false);
}

lkv_status lkv_gqa_decode_workspace_size(const lkv_gqa_args *a, size_t *bytes) {
  if (!a || !bytes) return fail(LKV_ERR_NULL, "args or bytes is NULL");
  if (a->struct_size != sizeof(lkv_gqa_args)) return fail(LKV_ERR_STRUCT, "struct_size %u != %zu", a->struct_size, sizeof(lkv_gqa_args));
  const Shape s = gqa_shape(a);
  lkv_status st = check_shape(s);
  if (st != LKV_OK) return st;
  Plan pl;
  if ((st = make_plan(s, &pl)) != LKV_OK) return st;
  *bytes = pl.ws_total;
  return LKV_OK;
}

lkv_status lkv_gqa_decode(const lkv_gqa_args *a) {
  if (!a) return fail(LKV_ERR_NULL, "args is NULL");
  if (a->struct_size != sizeof(lkv_gqa_args)) return fail(LKV_ERR_STRUCT, "struct_size %u != %zu", a->struct_size, sizeof(lkv_gqa_args));
  const Shape s = gqa_shape(a);
  if (!a->v_cache) return fail(LKV_ERR_NULL, "v_cache is NULL");
  Ptrs p{a->q, a->q_rope, a->k_cache, a->k_rope, a->v_cache, a->k_tok_stride, a->rope_tok_stride,
         a->v_tok_stride, a->block_table, a->seqlens, a->seqlens_host, a->block_table_host,
         (long long)a->num_pages, a->out, a->lse, a->workspace, a->workspace_bytes,
         static_cast<hipStream_t>(a->stream), a->kernel_events};
  return run_decode(s, p, a->softmax_scale);
}

lkv_status lkv_gqla_expand_latent(const lkv_expand_args *a) {
  if (!a) return fail(LKV_ERR_NULL, "args is NULL");
  if (a->struct_size != sizeof(lkv_expand_args)) return fail(LKV_ERR_STRUCT, "struct_size %u != %zu", a->struct_size, sizeof(lkv_expand_args));
  if (a->dtype != LKV_BF16) return fail(LKV_ERR_UNSUPPORTED, "latent expansion is bf16 only");
  if (a->batch < 0 || a->g < 1 || a->page_size < 1 || a->max_pages < 1) return fail(LKV_ERR_SHAPE, "non-positive size");
  if ((long long)a->page_size * a->max_pages > (1LL << 30)) return fail(LKV_ERR_SHAPE, "page_size * max_pages exceeds 2^30 tokens");
  if (!lkv::expand_supported(a->d_c, a->d_h))
    return fail(LKV_ERR_UNSUPPORTED, "expansion needs d_c a multiple of 64 in [64, 512] and d_h in {64, 128, 256}; got %d, %d", a->d_c, a->d_h);
  if (!a->c_kv || !a->w_uk || !a->w_uv || !a->block_table || !a->seqlens || !a->k_out || !a->v_out)
    return fail(LKV_ERR_NULL, "a required pointer is NULL");
  const void *all[] = {a->c_kv, a->w_uk, a->w_uv, a->k_out, a->v_out};
  for (const void *x : all)
    if (!aligned16(x)) return fail(LKV_ERR_ALIGN, "bf16 buffers must be 16-byte aligned");
  if (a->kv_tok_stride < a->d_c || a->kv_tok_stride % 8) return fail(LKV_ERR_ALIGN, "kv_tok_stride must be >= d_c and a multiple of 8");
  if (a->k_tok_stride < (long long)a->g * a->d_h || a->v_tok_stride < (long long)a->g * a->d_h)
    return fail(LKV_ERR_SHAPE, "k/v token strides must be >= g * d_h");
  // the output tile leaves in 16-byte pieces: bf16 strides are multiples of
  // 8 elements
  if (!a->out_fp8 && (a->k_tok_stride % 8 || a->v_tok_stride % 8))
    return fail(LKV_ERR_ALIGN, "bf16 expanded cache token strides must be multiples of 8 elements");
  if (a->out_fp8) {
    if (!(a->out_scale > 0.f) || !std::isfinite(a->out_scale) || !std::isfinite(1.f / a->out_scale))
      return fail(LKV_ERR_SHAPE, "out_scale %g must be positive, finite and have a finite reciprocal",
                  (double)a->out_scale);
    if (a->k_tok_stride % 16 || a->v_tok_stride % 16)
      return fail(LKV_ERR_ALIGN, "8-bit expanded cache token strides must be multiples of 16 bytes");
  }
  if (a->batch == 0) return LKV_OK;
  if ((long long)a->batch * ((a->max_pages * (long long)a->page_size + 63) / 64) > 0x7fffffffLL)
    return fail(LKV_ERR_SHAPE, "too many tiles for one launch");
  {
    const lkv_status st = check_call_contract(a->batch, a->page_size, a->max_pages, a->seqlens, a->block_table,
                                              HostView{a->seqlens_host, a->block_table_host, (long long)a->num_pages},
                                              static_cast<hipStream_t>(a->stream));
    if (st != LKV_OK) return st;
  }
  lkv::ExpandParams p{};
  p.c = a->c_kv;
  p.c_stride = a->kv_tok_stride;
  p.w_uk = a->w_uk;
  p.w_uv = a->w_uv;
  p.block_table = a->block_table;
  p.seqlens = a->seqlens;
  p.start_pos = a->start_pos;
  p.k_out = a->k_out;
  p.v_out = a->v_out;
  p.k_stride = a->k_tok_stride;
  p.v_stride = a->v_tok_stride;
  p.B = a->batch;
  p.g = a->g;
  p.d_c = a->d_c;
  p.d_h = a->d_h;
  p.page_size = a->page_size;
  p.max_pages = a->max_pages;
  p.out_fp8 = a->out_fp8 != 0;
  p.out_inv_scale = a->out_fp8 ? 1.f / a->out_scale : 1.f;
  hipError_t e = lkv::launch_expand(p, static_cast<hipStream_t>(a->stream));
  if (e != hipSuccess) return hip_fail(e, "expansion launch");
  return LKV_OK;
}

static lkv_status run_proj(const lkv_proj_args *a, bool up) {
  if (!a) return fail(LKV_ERR_NULL, "args is NULL");
  if (a->struct_size != sizeof(lkv_proj_args)) return fail(LKV_ERR_STRUCT, "struct_size %u != %zu", a->struct_size, sizeof(lkv_proj_args));
  if (a->dtype != LKV_BF16) return fail(LKV_ERR_UNSUPPORTED, "projections are bf16 only");
  if (a->batch < 0 || a->s_q < 1 || a->h_q < 1 || a->n_w < 1 || a->h_q % a->n_w)
    return fail(LKV_ERR_SHAPE, "h_q %d must be a positive multiple of n_w %d (batch %d, s_q %d)", a->h_q, a->n_w, a->batch, a->s_q);
  if (!lkv::proj_supported(a->d_c, a->d_h))
    return fail(LKV_ERR_UNSUPPORTED, "projections need d_c and d_h multiples of 64; got %d, %d", a->d_c, a->d_h);
  if (!a->x || !a->w || !a->y) return fail(LKV_ERR_NULL, "a required pointer is NULL");
  if (!aligned16(a->x) || !aligned16(a->w) || !aligned16(a->y)) return fail(LKV_ERR_ALIGN, "x, w and y must be 16-byte aligned");
  if ((long long)a->batch * a->s_q * a->h_q > (1LL << 30)) return fail(LKV_ERR_SHAPE, "batch * s_q * h_q exceeds 2^30 rows");
  if (a->batch == 0) return LKV_OK;
  lkv::ProjParams p{};
  p.x = a->x;
  p.w = a->w;
  p.y = a->y;
  p.B = a->batch;
  p.s_q = a->s_q;
  p.h_q = a->h_q;
  p.n_w = a->n_w;
  p.d_c = a->d_c;
  p.d_h = a->d_h;
  hipError_t e = lkv::launch_proj(p, up, static_cast<hipStream_t>(a->stream));
  if (e == hipErrorInvalidValue) return fail(LKV_ERR_SHAPE, "too many tiles for one launch");
  if (e != hipSuccess) return hip_fail(e, up ? "up-projection launch" : "absorb launch");
  return LKV_OK;
}

lkv_status lkv_absorb_query(const lkv_proj_args *a) { return run_proj(a, false); }

lkv_status lkv_up_project(const lkv_proj_args *a) { return run_proj(a, true); }

lkv_status lkv_append_tokens(const lkv_append_args *a) {
  if (!a) return fail(LKV_ERR_NULL, "args is NULL");
  if (a->struct_size != sizeof(lkv_append_args)) return fail(LKV_ERR_STRUCT, "struct_size %u != %zu", a->struct_size, sizeof(lkv_append_args));
  if (a->dtype != LKV_F32 && a->dtype != LKV_BF16) return fail(LKV_ERR_UNSUPPORTED, "dtype %d", a->dtype);
  if (a->batch < 0 || a->s_q < 1 || a->width < 1 || a->page_size < 1 || a->max_pages < 1)
    return fail(LKV_ERR_SHAPE, "non-positive size");
  if ((long long)a->page_size * a->max_pages > (1LL << 30)) return fail(LKV_ERR_SHAPE, "page_size * max_pages exceeds 2^30 tokens");
  if (a->out_fp8) {
    if (a->dtype != LKV_BF16) return fail(LKV_ERR_UNSUPPORTED, "an 8-bit cache is written from bf16 rows");
    if (!(a->out_scale > 0.f) || !std::isfinite(a->out_scale) || !std::isfinite(1.f / a->out_scale))
      return fail(LKV_ERR_SHAPE, "out_scale %g must be positive, finite and have a finite reciprocal", (double)a->out_scale);
  }
  const int es = a->dtype == LKV_BF16 ? 2 : 4;
  const int ces = a->out_fp8 ? 1 : es;  // bytes per cache element
  if (a->tok_stride < a->width) return fail(LKV_ERR_SHAPE, "tok_stride %lld < width %d", (long long)a->tok_stride, a->width);
  if (((long long)a->width * ces) % 16 || (a->tok_stride * ces) % 16)
    return fail(LKV_ERR_ALIGN, "width and tok_stride must be multiples of 16 bytes of the cache");
  if (!a->src || !a->cache || !a->block_table || !a->seqlens) return fail(LKV_ERR_NULL, "a required pointer is NULL");
  if (!aligned16(a->src) || !aligned16(a->cache)) return fail(LKV_ERR_ALIGN, "src and cache must be 16-byte aligned");
  if ((long long)a->batch * a->s_q > (1LL << 30)) return fail(LKV_ERR_SHAPE, "batch * s_q exceeds 2^30 rows");
  if (a->batch == 0) return LKV_OK;
  {
    const lkv_status st = check_call_contract(a->batch, a->page_size, a->max_pages, a->seqlens, a->block_table,
                                              HostView{a->seqlens_host, a->block_table_host, (long long)a->num_pages},
                                              static_cast<hipStream_t>(a->stream));
    if (st != LKV_OK) return st;
  }
  lkv::AppendParams p{};
  p.src = a->src;
  p.cache = a->cache;
  p.block_table = a->block_table;
  p.seqlens = a->seqlens;
  p.B = a->batch;
  p.s_q = a->s_q;
  p.page_size = a->page_size;
  p.max_pages = a->max_pages;
  p.row_bytes = a->width * es;
  p.tok_stride_bytes = a->tok_stride * ces;
  p.out_fp8 = a->out_fp8 != 0;
  p.out_inv_scale = a->out_fp8 ? 1.f / a->out_scale : 1.f;
  hipError_t e = lkv::launch_append(p, static_cast<hipStream_t>(a->stream));
  if (e != hipSuccess) return hip_fail(e, "append launch");
  return LKV_OK;
}

lkv_status lkv_split_combine(const lkv_combine_args *a) {
  if (!a) return fail(LKV_ERR_NULL, "args is NULL");
  if (a->struct_size != sizeof(lkv_combine_args)) return fail(LKV_ERR_STRUCT, "struct_size %u != %zu", a->struct_size, sizeof(lkv_combine_args));
  if (a->dtype != LKV_F32 && a->dtype != LKV_BF16) return fail(LKV_ERR_UNSUPPORTED, "dtype %d", a->dtype);
  if (a->batch < 0 || a->s_q < 1 || a->h_q < 1 || a->n_work < 0) return fail(LKV_ERR_SHAPE, "non-positive size");
  if (a->d_v < 4 || a->d_v > 1024 || a->d_v % 4) return fail(LKV_ERR_UNSUPPORTED, "d_v must be a multiple of 4 in [4, 1024], got %d", a->d_v);
  if (!a->o_part || !a->lse_part || !a->work_offsets || !a->out) return fail(LKV_ERR_NULL, "a required pointer is NULL");
  if (!aligned16(a->o_part) || !aligned4(a->lse_part)) return fail(LKV_ERR_ALIGN, "o_part must be 16-byte aligned");
  if (a->dtype == LKV_BF16 ? (reinterpret_cast<uintptr_t>(a->out) & 7) : !aligned16(a->out))
    return fail(LKV_ERR_ALIGN, "out must be 8-byte (bf16) or 16-byte (float32) aligned");
  if (a->batch == 0) return LKV_OK;
  lkv::CombineParams c{};
  c.o_part = a->o_part;
  c.lse_part = a->lse_part;
  c.meta = nullptr;
  c.offsets = a->work_offsets;
  c.out = a->out;
  c.lse = a->lse;
  c.B = a->batch;
  c.s_q = a->s_q;
  c.h_q = a->h_q;
  c.dv = a->d_v;
  c.skip_single = 0;
  c.out_bf16 = a->dtype == LKV_BF16;
  hipError_t e = lkv::launch_combine(c, static_cast<hipStream_t>(a->stream));
  if (e != hipSuccess) return hip_fail(e, "combine launch");
  return LKV_OK;
}

}  // extern "C"
