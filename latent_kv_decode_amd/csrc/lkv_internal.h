// lkv_internal.h -- parameter blocks and launcher declarations shared by the
// C ABI (abi.cpp) and the HIP kernel files.  Not part of the public ABI.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lkv {

// Timing events attached to one kernel launch (either may be null): the
// runtime stamps them with that dispatch's own start and end times, so no
// marker packet enters the stream.
struct LaunchEvents {
  hipEvent_t start = nullptr, stop = nullptr;
};

template <typename K, typename... A>
inline hipError_t launch_timed(K kernel, dim3 grid, dim3 block, hipStream_t s, const LaunchEvents &ev, A... args) {
  if (ev.start || ev.stop)
    hipExtLaunchKernelGGL(kernel, grid, block, 0, s, ev.start, ev.stop, 0, args...);
  else
    hipLaunchKernelGGL(kernel, grid, block, 0, s, args...);
  return hipGetLastError();
}

// Cache tokens per tile: the unit of work of the decode kernels and of the
// split-KV planner.
constexpr int kTile = 64;

// One decode pass, latent (MLA) or expanded (GQA) cache.  "KV head" below is
// the latent head of the MLA path or the KV group of the GQA path; query head
// h uses KV head h / hpk.
struct DecodeParams {
  const void *q;       // [B, s_q, h_q, dk]
  const void *q_rope;  // [B, s_q, h_q, dr] (dr > 0)
  const void *k;       // key main part: token row r, KV head g at r*k_stride + g*dk
  const void *r;       // shared RoPE key: token row r at r*r_stride
  const void *v;       // value: token row r, KV head g at r*v_stride + g*dv
  long long k_stride, r_stride, v_stride;
  const int32_t *block_table;  // [B, max_pages]
  const int32_t *seqlens;      // [B]
  void *out;                   // [B, s_q, h_q, dv]
  float *lse;                  // [B, s_q, h_q] or null
  float *o_part;               // [slots, s_q, h_q, dv]
  float *lse_part;             // [slots, s_q, h_q]
  int32_t *meta;               // [B][2]: first partial slot, number of partials
  int B, s_q, h_q, n_kvh, hpk;
  int page_size, page_shift;   // page_shift = log2(page_size) or -1
  int max_pages;
  int rows_per_kvh;            // s_q * hpk
  int tile_rows;               // query rows per work-group (ROWS)
  int row_tiles;               // ceil(rows_per_kvh / ROWS)
  int n_chunks;                // split-KV shares of the concatenated tiles
  int causal;
  float scale_log2;            // softmax scale * log2(e) (times the cache scale)
  float out_scale;             // factor on the normalised output: the cache's
                               // dequantisation scale (8-bit cache), else 1
  int fp8;                     // the caches hold OCP E4M3 codes (row-tiled kernel)
  int dk, dr, dv;              // widths (used by the generic fp32 kernel)
};

struct CombineParams {
  const float *o_part;
  const float *lse_part;
  const int32_t *meta;          // [B][2] (start, count) when offsets == null
  const int32_t *offsets;       // [B+1] or null
  void *out;
  float *lse;
  int B, s_q, h_q, dv;
  int skip_single;              // 1: sequences with <= 1 partial are already final
  int out_bf16;
};

struct ProjParams {
  const void *x;                // [B, s_q, h_q, K] rows
  const void *w;                // [n_w, d_c, d_h]
  void *y;                      // [B, s_q, h_q, N] rows
  int B, s_q, h_q, n_w, d_c, d_h;
};

struct AppendParams {
  const void *src;              // [B, s_q] rows of row_bytes
  void *cache;                  // cache row r at r * tok_stride_bytes
  const int32_t *block_table, *seqlens;
  int B, s_q, page_size, max_pages;
  int row_bytes;                 // of a source row
  long long tok_stride_bytes;
  int out_fp8;                   // nonzero: bf16 source -> E4M3 codes of value * out_inv_scale
  float out_inv_scale;
};

struct ExpandParams {
  const void *c;                // latent, row r at r*c_stride
  long long c_stride;
  const void *w_uk, *w_uv;      // [g, d_c, d_h]
  const int32_t *block_table, *seqlens, *start_pos;
  void *k_out, *v_out;
  long long k_stride, v_stride;  // elements (bf16) or bytes (8-bit output)
  int B, g, d_c, d_h, page_size, max_pages;
  int out_fp8;                    // nonzero: E4M3 codes of value * out_inv_scale
  float out_inv_scale;            // 1 / out_scale in float32
};

// Launchers return hipSuccess or the launch error.  `bf16_variant` selects a
// compiled instantiation; launchers return hipErrorInvalidValue when none
// matches (the ABI checks support before calling).
bool mfma_decode_supported(int dk, int dr, int dv, bool v_alias, bool fp8);
int mfma_decode_rows(int rows_per_kvh);  // ROWS template used for this problem
// Work-groups of the instantiation for (dk, dr, dv, v_alias, rows) that fit
// on one CU at once.
int mfma_decode_blocks_per_cu(int dk, int dr, int dv, bool v_alias, int rows, bool fp8);
hipError_t launch_mfma_decode(const DecodeParams &p, bool v_alias, int rows, hipStream_t s,
                              const LaunchEvents &ev);
// Latent path with the score and value products on different waves, 64 query
// rows per work-group (decode_split.hip).
bool mla_split_supported(int dk, int dr);
// Query rows per work-group of the kernel launch_mla_split uses for these
// widths, rows per latent head and cache type.
int mla_split_rows(int dk, int dr, int rows_per_kvh, bool fp8);
hipError_t launch_mla_split(const DecodeParams &p, hipStream_t s, const LaunchEvents &ev);
hipError_t launch_f32_decode(const DecodeParams &p, hipStream_t s, const LaunchEvents &ev);
hipError_t launch_combine(const CombineParams &p, hipStream_t s);
bool proj_supported(int d_c, int d_h);
// up == false: q' = W_UK q (d_h -> d_c); up == true: o = O' W_UV (d_c -> d_h)
hipError_t launch_proj(const ProjParams &p, bool up, hipStream_t s);
hipError_t launch_append(const AppendParams &p, hipStream_t s);
bool expand_supported(int d_c, int d_h);
hipError_t launch_expand(const ExpandParams &p, hipStream_t s);
// Device address and size of the current device's static scratch array
// (noalloc.hip); the address is looked up once per device.
hipError_t static_scratch(void **ptr, size_t *bytes);

}  // namespace lkv
