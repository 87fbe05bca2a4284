// decode_f32.hip -- float32 paged decode attention (MLA absorbed or GQA).
//
// The float32 path has no bf16 rounding anywhere: scores, softmax and the
// weighted sum run in fp32 on the vector ALUs.  It serves small float32
// problems (the pages' shapes scaled down for checking), so it favours
// plainness over speed: one wave per query row (b, t, h), lanes over cache
// tokens for the scores, lanes over value columns for the weighted sum, with
// an online softmax across 64-token blocks.  Same definitions as the MFMA
// kernel [GQLA explainer, technical summary section 2: MQA-absorbed path and
// GQA path].
#include "lkv_internal.h"

namespace lkv {
namespace {

constexpr int kMaxDv = 1024;
constexpr int kPerLane = kMaxDv / 64;

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

__global__ void __launch_bounds__(256) f32_decode_kernel(const DecodeParams p) {
  const int lane = threadIdx.x & 63;
  const long long row = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= (long long)p.B * p.s_q * p.h_q) return;
  const int h = (int)(row % p.h_q);
  const int t = (int)((row / p.h_q) % p.s_q);
  const int b = (int)(row / ((long long)p.h_q * p.s_q));
  const int kvh = h / p.hpk;
  const int L = p.seqlens[b];
  const int nvis = p.causal ? L - p.s_q + t + 1 : L;
  const float *q = static_cast<const float *>(p.q) + row * p.dk;
  const float *qr = p.dr ? static_cast<const float *>(p.q_rope) + row * p.dr : nullptr;
  const float *kc = static_cast<const float *>(p.k) + (long long)kvh * p.dk;
  const float *rc = static_cast<const float *>(p.r);
  const float *vc = static_cast<const float *>(p.v) + (long long)kvh * p.dv;
  const int32_t *bt = p.block_table + (long long)b * p.max_pages;

  float o[kPerLane];
#pragma unroll
  for (int i = 0; i < kPerLane; ++i) o[i] = 0.f;
  float m = -__builtin_inff(), l = 0.f;

  for (int j0 = 0; j0 < nvis; j0 += 64) {
    const int j = j0 + lane;
    int crow = -1;
    float s = -__builtin_inff();
    if (j < nvis) {
      crow = bt[j / p.page_size] * p.page_size + j % p.page_size;
      const float *kr = kc + (long long)crow * p.k_stride;
      float dot = 0.f;
      for (int d = 0; d < p.dk; ++d) dot += q[d] * kr[d];
      if (p.dr) {
        const float *rr = rc + (long long)crow * p.r_stride;
        for (int e = 0; e < p.dr; ++e) dot += qr[e] * rr[e];
      }
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
    const int cnt = min(64, nvis - j0);
    for (int jj = 0; jj < cnt; ++jj) {
      const float pw = __shfl(pj, jj);
      const int rr = __shfl(crow, jj);
      const float *vr = vc + (long long)rr * p.v_stride;
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
  return launch_timed(f32_decode_kernel, dim3((unsigned)((rows + 3) / 4)), dim3(256), s, ev, p);
}

}  // namespace lkv
