// combine.hip -- split-KV merge of partial attention results.
//
// For one sequence b with partial works s (float32 O_s, LSE_s), per row:
//   LSE = ln sum_s exp(LSE_s),   O = sum_s exp(LSE_s - LSE) O_s.
// A work with LSE_s = -inf (it saw no token) weighs nothing; a row with no
// contributing work gets O = 0 and LSE = -inf.  This is the merge that makes
// a split decode pass equal to a single pass; the pages state the decode
// computation only as one softmax over the whole cache, and the merge follows
// from writing that softmax over a partition of the cache.
//
// One wave per (b, t, h) row; lanes stride over the value columns in float4.
#include "lkv_internal.h"

namespace lkv {
namespace {

typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;
constexpr int kMaxWorks = 64;  // per-lane cache of weights; more works loop

__global__ void __launch_bounds__(256) combine_kernel(const CombineParams p) {
  const int lane = threadIdx.x & 63;
  const long long rpb = (long long)p.s_q * p.h_q;
  const long long row = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= (long long)p.B * rpb) return;
  const int b = (int)(row / rpb);
  const long long r = row % rpb;
  int start, count;
  if (p.offsets) {
    start = p.offsets[b];
    count = p.offsets[b + 1] - start;
  } else {
    start = p.meta[2 * b];
    count = p.meta[2 * b + 1];
  }
  if (p.skip_single && count <= 1) return;

  // maximum LSE over the works (lanes stride over works)
  float m = -__builtin_inff();
  for (int s = lane; s < count; s += 64) m = fmaxf(m, p.lse_part[(long long)(start + s) * rpb + r]);
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
  float total = -__builtin_inff();
  if (m != -__builtin_inff()) {
    float z = 0.f;
    for (int s = lane; s < count; s += 64) z += expf(p.lse_part[(long long)(start + s) * rpb + r] - m);
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) z += __shfl_xor(z, o);
    total = m + logf(z);
  }
  for (int d = 4 * lane; d < p.dv; d += 256) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    if (total != -__builtin_inff()) {
      for (int s = 0; s < count; ++s) {
        const long long pr = (long long)(start + s) * rpb + r;
        const float ls = p.lse_part[pr];
        if (ls == -__builtin_inff()) continue;
        const float wgt = expf(ls - total);
        acc += wgt * *reinterpret_cast<const f32x4 *>(p.o_part + pr * p.dv + d);
      }
    }
    if (p.out_bf16) {
      bf16x4 o;
#pragma unroll
      for (int i = 0; i < 4; ++i) o[i] = static_cast<__bf16>(acc[i]);
      *reinterpret_cast<bf16x4 *>(static_cast<__bf16 *>(p.out) + row * p.dv + d) = o;
    } else {
      *reinterpret_cast<f32x4 *>(static_cast<float *>(p.out) + row * p.dv + d) = acc;
    }
  }
  if (p.lse && lane == 0) p.lse[row] = total;
}

}  // namespace

hipError_t launch_combine(const CombineParams &p, hipStream_t s) {
  const long long rows = (long long)p.B * p.s_q * p.h_q;
  if (rows == 0) return hipSuccess;
  hipLaunchKernelGGL(combine_kernel, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace lkv
