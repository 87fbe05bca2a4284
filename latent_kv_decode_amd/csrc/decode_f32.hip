// decode_f32.hip -- float32 paged decode attention (MLA absorbed or GQA).
//
// The float32 path has no bf16 rounding anywhere: scores, softmax and the
// weighted sum run in fp32 on the vector ALUs.  It serves small float32
// problems (the pages' shapes scaled down for checking) at any widths.  Same
// definitions as the MFMA kernels [GQLA explainer, technical summary section
// 2: MQA-absorbed path and GQA path].
//
// One wave per query row (b, t, h).  The row's cache is swept in tiles of T
// tokens: the wave copies the tile's token rows (key, RoPE key and, for a
// separate value cache, value) from the paged caches into LDS with
// direct-to-LDS loads (consecutive lanes read consecutive elements of one
// row; a tile's loads are all in flight together), then lane j computes the
// score of token j from LDS, the tile's softmax update runs across the wave,
// and the weighted sum takes lanes over the value columns.  T follows from
// the row width so that a tile fits the work-group's LDS.
#include "lkv_internal.h"

namespace lkv {
namespace {

constexpr int kMaxDv = 1024;
constexpr int kPerLane = kMaxDv / 64;
constexpr int kLdsBytes = 60 * 1024;

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// Tokens per tile for a row layout of `width` floats (key + RoPE key +
// separate value) after the query's dq floats: the LDS holds the query and
// T padded rows of width + 1 floats.
__host__ __device__ inline int f32_tile_tokens(int width, int dq) {
  const int avail = kLdsBytes / 4 - dq;
  const int t = avail / (width + 1);
  return t < 1 ? 1 : (t > 64 ? 64 : t);
}

__global__ void __launch_bounds__(64) f32_decode_kernel(const DecodeParams p) {
  extern __shared__ float lds[];
  const int lane = threadIdx.x;
  const long long row = blockIdx.x;
  const int h = (int)(row % p.h_q);
  const int t = (int)((row / p.h_q) % p.s_q);
  const int b = (int)(row / ((long long)p.h_q * p.s_q));
  const int kvh = h / p.hpk;
  const int L = p.seqlens[b];
  const int nvis = p.causal ? L - p.s_q + t + 1 : L;
  const bool v_alias = p.v == p.k && p.v_stride == p.k_stride && p.dv == p.dk;
  const int dq = p.dk + p.dr;                  // query (and key) width
  const int width = dq + (v_alias ? 0 : p.dv);  // floats per staged token row
  const int T = f32_tile_tokens(width, dq);
  const int pitch = width + 1;
  float *q_l = lds;              // [dq]
  float *tile = lds + dq;        // [T][pitch]
  const float *q = static_cast<const float *>(p.q) + row * p.dk;
  const float *qr = p.dr ? static_cast<const float *>(p.q_rope) + row * p.dr : nullptr;
  const float *kc = static_cast<const float *>(p.k) + (long long)kvh * p.dk;
  const float *rc = static_cast<const float *>(p.r);
  const float *vc = static_cast<const float *>(p.v) + (long long)kvh * p.dv;
  const int32_t *bt = p.block_table + (long long)b * p.max_pages;
  // value column v of token row j in the tile: the latent (MLA) or the
  // staged value part (GQA)
  const int voff = v_alias ? 0 : dq;

  for (int d = lane; d < dq; d += 64) q_l[d] = d < p.dk ? q[d] : qr[d - p.dk];

  float o[kPerLane];
#pragma unroll
  for (int i = 0; i < kPerLane; ++i) o[i] = 0.f;
  float m = -__builtin_inff(), l = 0.f;

  for (int j0 = 0; j0 < nvis; j0 += T) {
    const int cnt = min(T, nvis - j0);
    // cache row of token j0 + lane (lanes < cnt)
    int crow = 0;
    if (lane < cnt) {
      const int j = j0 + lane;
      crow = bt[j / p.page_size] * p.page_size + j % p.page_size;
    }
    __syncthreads();  // previous tile's reads are done
    // direct-to-LDS loads, all in flight together: element c = 64 i + lane
    // of token row tok goes to tile[tok][c]
    for (int tok = 0; tok < cnt; ++tok) {
      const long long r = __shfl(crow, tok);
      for (int c0 = 0; c0 < width; c0 += 64) {
        const int c = c0 + lane;
        if (c < width) {
          const float *src = c < p.dk ? kc + r * p.k_stride + c
                             : c < dq ? rc + r * p.r_stride + (c - p.dk)
                                      : vc + r * p.v_stride + (c - dq);
          __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void *)(tile + tok * pitch + c0),
                                           4, 0, 0);
        }
      }
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    float s = -__builtin_inff();
    if (lane < cnt) {
      const float *kr = tile + lane * pitch;
      float dot = 0.f;
      for (int d = 0; d < dq; ++d) dot += q_l[d] * kr[d];
      s = dot * p.scale_log2;
    }
    const float mnew = fmaxf(m, wave_max(s));
    const float muse = mnew == -__builtin_inff() ? 0.f : mnew;
    const float alpha = __builtin_amdgcn_exp2f(m - muse);
    const float pj = __builtin_amdgcn_exp2f(s - muse);
    l = l * alpha + wave_sum(pj);
    m = mnew;
#pragma unroll
    for (int i = 0; i < kPerLane; ++i) o[i] *= alpha;
    for (int jj = 0; jj < cnt; ++jj) {
      const float pw = __shfl(pj, jj);
      const float *vr = tile + jj * pitch + voff;
#pragma unroll
      for (int i = 0; i < kPerLane; ++i) {
        const int d = lane + 64 * i;
        if (d < p.dv) o[i] += pw * vr[d];
      }
    }
  }
  const float inv = l > 0.f ? 1.f / l : 0.f;
  float *out = static_cast<float *>(p.out) + row * p.dv;
#pragma unroll
  for (int i = 0; i < kPerLane; ++i) {
    const int d = lane + 64 * i;
    if (d < p.dv) out[d] = o[i] * inv;
  }
  if (p.lse && lane == 0)
    p.lse[row] = l > 0.f ? (m + __log2f(l)) * 0.693147180559945309f : -__builtin_inff();
}

}  // namespace

hipError_t launch_f32_decode(const DecodeParams &p, hipStream_t s, const LaunchEvents &ev) {
  const long long rows = (long long)p.B * p.s_q * p.h_q;
  if (rows == 0) return hipSuccess;
  if (rows > 0x7fffffffLL) return hipErrorInvalidValue;
  const bool v_alias = p.v == p.k && p.v_stride == p.k_stride && p.dv == p.dk;
  const int dq = p.dk + p.dr;
  const int width = dq + (v_alias ? 0 : p.dv);
  const int T = f32_tile_tokens(width, dq);
  const size_t lds = (size_t)(dq + T * (width + 1)) * sizeof(float);
  if (lds > (size_t)kLdsBytes + 64 * sizeof(float) + 4096) return hipErrorInvalidValue;
  if (ev.start || ev.stop)
    hipExtLaunchKernelGGL(f32_decode_kernel, dim3((unsigned)rows), dim3(64), lds, s, ev.start, ev.stop, 0, p);
  else
    hipLaunchKernelGGL(f32_decode_kernel, dim3((unsigned)rows), dim3(64), lds, s, p);
  return hipGetLastError();
}

}  // namespace lkv
