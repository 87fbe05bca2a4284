// decode_f32.hip -- float32 paged decode attention (MLA absorbed or GQA).
//
// The float32 path has no bf16 rounding anywhere: scores, softmax and the
// weighted sum run in fp32 on the vector ALUs.  It serves small float32
// problems (the pages' shapes scaled down for checking) at any widths.  Same
// definitions as the MFMA kernels [GQLA explainer, technical summary section
// 2: MQA-absorbed path and GQA path].
//
// Four waves per query row (b, t, h): wave w sweeps tiles w, w + 4, ... of
// the row's visible cache in tiles of T tokens, with its own online softmax.
// A wave copies a tile's token rows (key, RoPE key and, for a separate value
// cache, value) from the paged caches into its own LDS region with
// direct-to-LDS loads (consecutive lanes read consecutive elements of one
// row; a tile's loads are all in flight together); then lane j computes the
// score of token j from LDS, the tile's softmax update runs across the wave,
// and the weighted sum takes lanes over the value columns.  At the end the
// four partial results are merged through LDS with the same rule that merges
// split-KV partials (each weighed by exp of its maximum against the largest).
// T follows from the row width so that four tiles fit the LDS.  The rows of
// one sequence run on one XCD (work-group index mod 8), so that the heads
// reading the same cache rows share that XCD's L2.
#include "lkv_internal.h"

namespace lkv {
namespace {

constexpr int kMaxDv = 1024;
constexpr int kPerLane = kMaxDv / 64;
constexpr int kWaves = 4;
constexpr int kLdsBytes = 128 * 1024;

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
// separate value) after the query's dq floats: the LDS holds the query and,
// per wave, T padded rows of width + 1 floats.
__host__ __device__ inline int f32_tile_tokens(int width, int dq) {
  const int avail = (kLdsBytes / 4 - dq) / kWaves;
  const int t = avail / (width + 1);
  return t < 1 ? 1 : (t > 64 ? 64 : t);
}

// rows_per_xcd: rows handled on one XCD, a multiple of the rows of one
// sequence; work-group i runs row (i mod 8) * rows_per_xcd + i / 8.
__global__ void __launch_bounds__(64 * kWaves) f32_decode_kernel(const DecodeParams p, long long rows_per_xcd) {
  extern __shared__ float lds[];
  __shared__ float s_ml[2 * kWaves];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const long long row = (long long)(blockIdx.x & 7) * rows_per_xcd + (blockIdx.x >> 3);
  if (row >= (long long)p.B * p.s_q * p.h_q) return;  // whole work-group
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
  float *q_l = lds;                             // [dq]
  float *tile = lds + dq + wv * T * pitch;      // this wave's [T][pitch]
  const float *q = static_cast<const float *>(p.q) + row * p.dk;
  const float *qr = p.dr ? static_cast<const float *>(p.q_rope) + row * p.dr : nullptr;
  const float *kc = static_cast<const float *>(p.k) + (long long)kvh * p.dk;
  const float *rc = static_cast<const float *>(p.r);
  const float *vc = static_cast<const float *>(p.v) + (long long)kvh * p.dv;
  const int32_t *bt = p.block_table + (long long)b * p.max_pages;
  // value column v of token row j in the tile: the latent (MLA) or the
  // staged value part (GQA)
  const int voff = v_alias ? 0 : dq;
  const int nblk = (p.dv + 63) / 64;  // 64-column blocks of the value

  for (int d = threadIdx.x; d < dq; d += 64 * kWaves) q_l[d] = d < p.dk ? q[d] : qr[d - p.dk];
  __syncthreads();

  float o[kPerLane];
#pragma unroll
  for (int i = 0; i < kPerLane; ++i) o[i] = 0.f;
  float m = -__builtin_inff(), l = 0.f;

  // this wave's tiles; the loop bounds are wave-uniform and differ between
  // waves, so only wave-level ordering is used inside
  for (int j0 = wv * T; j0 < nvis; j0 += kWaves * T) {
    const int cnt = min(T, nvis - j0);
    // cache row of token j0 + lane (lanes < cnt)
    int crow = 0;
    if (lane < cnt) {
      const int j = j0 + lane;
      crow = bt[j / p.page_size] * p.page_size + j % p.page_size;
    }
    // the previous tile's LDS reads are complete before it is overwritten
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    // direct-to-LDS loads, all in flight together, one region at a time
    // (key, RoPE key, separate value), 64 columns per instruction: element
    // c of token row tok goes to tile[tok][at + c]
    auto stage = [&](const float *base, long long stride, int cols, int at) {
      for (int tok = 0; tok < cnt; ++tok) {
        const float *src = base + (long long)__builtin_amdgcn_readlane(crow, tok) * stride + lane;
        float *dst = tile + tok * pitch + at;
        for (int c0 = 0; c0 < cols; c0 += 64)
          if (c0 + lane < cols)
            __builtin_amdgcn_global_load_lds(src + c0, (__attribute__((address_space(3))) void *)(dst + c0), 4, 0, 0);
      }
    };
    stage(kc, p.k_stride, p.dk, 0);
    if (p.dr) stage(rc, p.r_stride, p.dr, p.dk);
    if (!v_alias) stage(vc, p.v_stride, p.dv, dq);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
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
    // weighted sum: value column lane + 64 i (a wave-uniform bound on i, the
    // last partial block read clamped and weighted by zero past dv)
    const float *vt = tile + voff;
#pragma unroll
    for (int i = 0; i < kPerLane; ++i) {
      if (i < nblk) {
        const int d = lane + 64 * i;
        const int dc = min(d, p.dv - 1);
        const float keep = d < p.dv ? 1.f : 0.f;
        float acc = 0.f;
        int jj = 0;
        for (; jj + 4 <= cnt; jj += 4) {
          const float v0 = vt[(jj + 0) * pitch + dc], v1 = vt[(jj + 1) * pitch + dc];
          const float v2 = vt[(jj + 2) * pitch + dc], v3 = vt[(jj + 3) * pitch + dc];
          acc += __int_as_float(__builtin_amdgcn_readlane(__float_as_int(pj), jj + 0)) * v0;
          acc += __int_as_float(__builtin_amdgcn_readlane(__float_as_int(pj), jj + 1)) * v1;
          acc += __int_as_float(__builtin_amdgcn_readlane(__float_as_int(pj), jj + 2)) * v2;
          acc += __int_as_float(__builtin_amdgcn_readlane(__float_as_int(pj), jj + 3)) * v3;
        }
        for (; jj < cnt; ++jj) acc += __int_as_float(__builtin_amdgcn_readlane(__float_as_int(pj), jj)) * vt[jj * pitch + dc];
        o[i] += keep * acc;
      }
    }
  }

  // ---- merge the four waves' results: weights 2^(m_w - M) with M the
  // largest maximum (a wave that saw no token weighs nothing)
  __syncthreads();  // every wave is done with its tile region
  float *o_l = lds + dq;  // [kWaves][dv], over the tile regions
  if (lane == 0) {
    s_ml[wv] = m;
    s_ml[kWaves + wv] = l;
  }
#pragma unroll
  for (int i = 0; i < kPerLane; ++i) {
    const int d = lane + 64 * i;
    if (i < nblk && d < p.dv) o_l[wv * p.dv + d] = o[i];
  }
  __syncthreads();
  float mm = -__builtin_inff();
#pragma unroll
  for (int w = 0; w < kWaves; ++w) mm = fmaxf(mm, s_ml[w]);
  float wgt[kWaves], lt = 0.f;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    wgt[w] = s_ml[w] == -__builtin_inff() ? 0.f : __builtin_amdgcn_exp2f(s_ml[w] - mm);
    lt += wgt[w] * s_ml[kWaves + w];
  }
  const float inv = lt > 0.f ? 1.f / lt : 0.f;
  float *out = static_cast<float *>(p.out) + row * p.dv;
  for (int d = threadIdx.x; d < p.dv; d += 64 * kWaves) {
    float acc = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) acc += wgt[w] * o_l[w * p.dv + d];
    out[d] = acc * inv;
  }
  if (p.lse && threadIdx.x == 0)
    p.lse[row] = lt > 0.f ? (mm + __log2f(lt)) * 0.693147180559945309f : -__builtin_inff();
}

}  // namespace

hipError_t launch_f32_decode(const DecodeParams &p, hipStream_t s, const LaunchEvents &ev) {
  const long long rows = (long long)p.B * p.s_q * p.h_q;
  if (rows == 0) return hipSuccess;
  // rows per XCD: an eighth of the rows, rounded up to whole sequences
  const long long per_seq = (long long)p.s_q * p.h_q;
  const long long per_xcd = ((rows + 7) / 8 + per_seq - 1) / per_seq * per_seq;
  const long long grid = 8 * per_xcd;
  if (grid > 0x7fffffffLL) return hipErrorInvalidValue;
  const bool v_alias = p.v == p.k && p.v_stride == p.k_stride && p.dv == p.dk;
  const int dq = p.dk + p.dr;
  const int width = dq + (v_alias ? 0 : p.dv);
  const int T = f32_tile_tokens(width, dq);
  // the tiles, and after them the merge area [kWaves][dv], fit the LDS
  const size_t lds = (size_t)(dq + kWaves * T * (width + 1)) * sizeof(float);
  if (lds > (size_t)kLdsBytes || (size_t)kWaves * p.dv > (size_t)kWaves * T * (width + 1))
    return hipErrorInvalidValue;
  if (ev.start || ev.stop)
    hipExtLaunchKernelGGL(f32_decode_kernel, dim3((unsigned)grid), dim3(64 * kWaves), lds, s, ev.start, ev.stop, 0,
                          p, per_xcd);
  else
    hipLaunchKernelGGL(f32_decode_kernel, dim3((unsigned)grid), dim3(64 * kWaves), lds, s, p, per_xcd);
  return hipGetLastError();
}

}  // namespace lkv
