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
// A row with at most 4 works loads all its partials at once; with more, the
// weights of up to 64 works sit one per lane and the loads go 4 at a time.
#include "lkv_internal.h"

namespace lkv {
namespace {

typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;

__device__ __forceinline__ void store4(const CombineParams &p, long long at, const f32x4 &v) {
  if (p.out_bf16) {
    bf16x4 o;
#pragma unroll
    for (int i = 0; i < 4; ++i) o[i] = static_cast<__bf16>(v[i]);
    *reinterpret_cast<bf16x4 *>(static_cast<__bf16 *>(p.out) + at) = o;
  } else {
    *reinterpret_cast<f32x4 *>(static_cast<float *>(p.out) + at) = v;
  }
}

// A row with N (1..4) works: every lane loads its columns of all N partials
// at once (up to 4 passes of 256 columns), then weighs and sums them.
template <int N>
__device__ __forceinline__ void combine_few(const CombineParams &p, long long row, long long r, int start,
                                            int lane) {
  const long long rpb = (long long)p.s_q * p.h_q;
  float ls[N], wgt[N];
  float m = -__builtin_inff();
#pragma unroll
  for (int s = 0; s < N; ++s) {
    ls[s] = p.lse_part[(long long)(start + s) * rpb + r];
    m = fmaxf(m, ls[s]);
  }
  float total = -__builtin_inff();
  if (m != -__builtin_inff()) {
    float z = 0.f;
#pragma unroll
    for (int s = 0; s < N; ++s) z += expf(ls[s] - m);
    total = m + logf(z);
  }
#pragma unroll
  for (int s = 0; s < N; ++s)
    wgt[s] = total == -__builtin_inff() || ls[s] == -__builtin_inff() ? 0.f : expf(ls[s] - total);
  const float *base = p.o_part + ((long long)start * rpb + r) * p.dv;
  const long long work_stride = rpb * p.dv;
  f32x4 v[4][N];
#pragma unroll
  for (int pass = 0; pass < 4; ++pass) {
    const int d = 4 * lane + 256 * pass;
    if (d < p.dv) {
#pragma unroll
      for (int s = 0; s < N; ++s) v[pass][s] = *reinterpret_cast<const f32x4 *>(base + s * work_stride + d);
    }
  }
#pragma unroll
  for (int pass = 0; pass < 4; ++pass) {
    const int d = 4 * lane + 256 * pass;
    if (d < p.dv) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      // a work of weight 0 is skipped, whatever its partial holds
#pragma unroll
      for (int s = 0; s < N; ++s)
        if (wgt[s] != 0.f) acc += wgt[s] * v[pass][s];
      store4(p, row * p.dv + d, acc);
    }
  }
  if (p.lse && lane == 0) p.lse[row] = total;
}

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
  switch (count) {
    case 1: combine_few<1>(p, row, r, start, lane); return;
    case 2: combine_few<2>(p, row, r, start, lane); return;
    case 3: combine_few<3>(p, row, r, start, lane); return;
    case 4: combine_few<4>(p, row, r, start, lane); return;
    default: break;
  }

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
  const bool live = total != -__builtin_inff();
  // output columns: lane covers 4 columns per pass of 256
  const int npass = (p.dv + 255) / 256;
  const float *orow = p.o_part + r * p.dv;
  const long long work_stride = rpb * p.dv;  // elements between the same row of consecutive works
  for (int d = 4 * lane, pass = 0; pass < npass; d += 256, ++pass) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    // every lane runs the loop (the weights move between lanes); a lane past
    // the last column reads the last four and stores nothing
    const int dd = min(d, p.dv - 4);
    if (live) {
      // works in groups of 64: lane s of the wave holds the weight of work
      // g0 + s; the loads of one group are independent and issue 4 at a time
      for (int g0 = 0; g0 < count; g0 += 64) {
        const int ng = min(64, count - g0);
        float wl = 0.f;
        if (lane < ng) {
          const float ls = p.lse_part[(long long)(start + g0 + lane) * rpb + r];
          wl = ls == -__builtin_inff() ? 0.f : expf(ls - total);
        }
        const float *base = orow + (long long)(start + g0) * work_stride + dd;
        // a work of weight 0 (LSE -inf, or negligible) is skipped, whatever
        // its partial holds
        auto add = [&](int s, const f32x4 &v) {
          const float wgt = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wl), s));
          if (wgt != 0.f) acc += wgt * v;
        };
        int s = 0;
        for (; s + 4 <= ng; s += 4) {
          const f32x4 v0 = *reinterpret_cast<const f32x4 *>(base + (long long)s * work_stride);
          const f32x4 v1 = *reinterpret_cast<const f32x4 *>(base + (long long)(s + 1) * work_stride);
          const f32x4 v2 = *reinterpret_cast<const f32x4 *>(base + (long long)(s + 2) * work_stride);
          const f32x4 v3 = *reinterpret_cast<const f32x4 *>(base + (long long)(s + 3) * work_stride);
          add(s, v0);
          add(s + 1, v1);
          add(s + 2, v2);
          add(s + 3, v3);
        }
        for (; s < ng; ++s) add(s, *reinterpret_cast<const f32x4 *>(base + (long long)s * work_stride));
      }
    }
    if (d < p.dv) store4(p, row * p.dv + d, acc);
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
