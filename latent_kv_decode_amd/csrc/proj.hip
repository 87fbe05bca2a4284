// proj.hip -- the steps on either side of absorbed decode.
//
// [GQLA explainer, technical summary section 2, MQA-absorbed path]: W_UK
// folds into the query and W_UV into the output, so the decode kernel sees
// only the latent.  Per query row (b, t, h), with weight block
// wb = h / (h_q / n_w) of W [n_w, d_c, d_h]:
//   absorb      y[k] = sum_d W[wb][k][d] x[d]      (x: d_h wide, y: d_c wide)
//   up-project  y[d] = sum_k x[k] W[wb][k][d]      (x: d_c wide, y: d_h wide)
// Both are products Y = X M with M = W[wb]^T (absorb) or W[wb] (up), taken
// over the rows that share a weight block.
//
// A work-group computes 64 rows x 64 output columns of one weight block over
// K-chunks of 64 staged in LDS.  Wave w takes output columns 16 w .. 16 w +
// 15 of all 64 rows: D^T = M^T X^T with v_mfma_f32_16x16x32_bf16, A = M^T
// (a weight row as is for the absorb; a transposing LDS read of the
// row-major weight for the up-projection), B = X^T (rows of X as is).
// float32 accumulation, bf16 output.
//
// Also the cache write of the new tokens: row t of the step's new rows of
// sequence b goes to position L_b - s_q + t of its paged cache, as is or as
// OCP E4M3 codes of the values times 1 / scale (an 8-bit cache).
#include "e4m3.h"
#include "lkv_internal.h"

namespace lkv {
namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short s16x4;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(4 * sizeof(unsigned)))) unsigned u32x4;
typedef __bf16 bf16;

constexpr int kPT = 64;  // rows, columns and K per tile

__device__ __forceinline__ s16x4 lds_read_tr(const bf16 *p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4 *)(p));
}
__device__ __forceinline__ bf16x8 join(s16x4 lo, s16x4 hi) {
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// UP == false: absorb (K = d_h, N = d_c); UP == true: up-projection (K =
// d_c, N = d_h).
template <bool UP>
__global__ void __launch_bounds__(256) proj_kernel(const ProjParams p) {
  __shared__ __attribute__((aligned(16))) bf16 s_x[kPT * kPT];  // [row][k]
  __shared__ __attribute__((aligned(16))) bf16 s_m[kPT * kPT];  // absorb [n][k]; up [k][n]
  __shared__ int s_row[kPT];

  const int K = UP ? p.d_c : p.d_h, N = UP ? p.d_h : p.d_c;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, g = lane >> 4, n = lane & 15;
  const int hpw = p.h_q / p.n_w;
  const long long rows_per_block = (long long)p.B * p.s_q * hpw;
  const int n_rt = (int)((rows_per_block + kPT - 1) / kPT), n_ct = N / kPT;
  // block -> (weight block, row tile, column tile)
  const long long bx = blockIdx.x;
  const int ct = (int)(bx % n_ct);
  const long long rest = bx / n_ct;
  const int rt = (int)(rest % n_rt), wb = (int)(rest / n_rt);
  if (tid < kPT) {
    const long long i = (long long)rt * kPT + tid;  // row within the weight block
    s_row[tid] = i < rows_per_block ? (int)((i / hpw) * p.h_q + wb * hpw + i % hpw) : -1;
  }
  __syncthreads();

  const bf16 *x = static_cast<const bf16 *>(p.x);
  const bf16 *wm = static_cast<const bf16 *>(p.w) + (long long)wb * p.d_c * p.d_h;
  f32x4 acc[4];
#pragma unroll
  for (int rb = 0; rb < 4; ++rb) acc[rb] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int k0 = 0; k0 < K; k0 += kPT) {
    // stage X [64 rows][64 k] and the weight chunk, 2 sixteen-byte pieces
    // per thread each (8 consecutive lanes cover one 128-byte row)
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int piece = tid + 256 * u, r = piece >> 3, ch = piece & 7;
      const int row = s_row[r];
      u32x4 v = {0u, 0u, 0u, 0u};
      if (row >= 0) v = *reinterpret_cast<const u32x4 *>(x + (long long)row * K + k0 + 8 * ch);
      *reinterpret_cast<u32x4 *>(s_x + r * kPT + 8 * ch) = v;
      // absorb: weight rows are output columns n (K contiguous);
      // up: weight rows are k (output columns contiguous)
      const bf16 *src = UP ? wm + (long long)(k0 + r) * p.d_h + ct * kPT + 8 * ch
                           : wm + (long long)(ct * kPT + r) * p.d_h + k0 + 8 * ch;
      *reinterpret_cast<u32x4 *>(s_m + r * kPT + 8 * ch) = *reinterpret_cast<const u32x4 *>(src);
    }
    __syncthreads();
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      bf16x8 a;
      if constexpr (UP) {
        // M^T fragment: columns 16 w + 4 (n mod 4) .. + 3 of weight rows rk
        // and rk + 4 (transposed)
        const int rk = 32 * ks + 8 * g + (n >> 2), col = 16 * w + 4 * (n & 3);
        a = join(lds_read_tr(s_m + rk * kPT + col), lds_read_tr(s_m + (rk + 4) * kPT + col));
      } else {
        // M^T row = weight row 16 w + n, K 32 ks + 8 g ..
        a = *reinterpret_cast<const bf16x8 *>(s_m + (16 * w + n) * kPT + 32 * ks + 8 * g);
      }
#pragma unroll
      for (int rb = 0; rb < 4; ++rb) {
        const bf16x8 b = *reinterpret_cast<const bf16x8 *>(s_x + (16 * rb + n) * kPT + 32 * ks + 8 * g);
        acc[rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[rb], 0, 0, 0);
      }
    }
    __syncthreads();
  }

  // D^T tile: columns 16 w + 4 g .. + 3 of row 16 rb + n
  bf16 *y = static_cast<bf16 *>(p.y);
#pragma unroll
  for (int rb = 0; rb < 4; ++rb) {
    const int row = s_row[16 * rb + n];
    if (row < 0) continue;
    bf16x4 o;
#pragma unroll
    for (int i = 0; i < 4; ++i) o[i] = static_cast<bf16>(acc[rb][i]);
    *reinterpret_cast<bf16x4 *>(y + (long long)row * N + ct * kPT + 16 * w + 4 * g) = o;
  }
}

// One wave per new token row: 16-byte pieces of the row to its cache slot.
__global__ void __launch_bounds__(256) append_kernel(const AppendParams p) {
  const long long r = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= (long long)p.B * p.s_q) return;
  const int lane = threadIdx.x & 63;
  const int b = (int)(r / p.s_q), t = (int)(r % p.s_q);
  const int j = p.seqlens[b] - p.s_q + t;  // position of this new token
  if (j < 0) return;
  const int32_t *bt = p.block_table + (long long)b * p.max_pages;
  const long long row = (long long)bt[j / p.page_size] * p.page_size + j % p.page_size;
  const char *src = static_cast<const char *>(p.src) + r * p.row_bytes;
  char *dst = static_cast<char *>(p.cache) + row * p.tok_stride_bytes;
  if (p.out_fp8) {
    // eight bf16 values (16 bytes of the source row) -> eight codes
    for (int o = 16 * lane; o < p.row_bytes; o += 16 * 64) {
      const u32x4 v = *reinterpret_cast<const u32x4 *>(src + o);
      unsigned w[2] = {0u, 0u};
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const unsigned half = (v[i >> 1] >> (16 * (i & 1))) & 0xFFFFu;
        w[i >> 2] |= e4m3_encode(__uint_as_float(half << 16) * p.out_inv_scale) << (8 * (i & 3));
      }
      *reinterpret_cast<unsigned long long *>(dst + o / 2) = ((unsigned long long)w[1] << 32) | w[0];
    }
    return;
  }
  for (int o = 16 * lane; o < p.row_bytes; o += 16 * 64)
    *reinterpret_cast<u32x4 *>(dst + o) = *reinterpret_cast<const u32x4 *>(src + o);
}

}  // namespace

bool proj_supported(int d_c, int d_h) {
  return d_c >= 64 && d_c % 64 == 0 && d_h >= 64 && d_h % 64 == 0;
}

hipError_t launch_proj(const ProjParams &p, bool up, hipStream_t s) {
  const long long rows_per_block = (long long)p.B * p.s_q * (p.h_q / p.n_w);
  const long long n_rt = (rows_per_block + kPT - 1) / kPT;
  const long long n_ct = (up ? p.d_h : p.d_c) / kPT;
  const long long grid = (long long)p.n_w * n_rt * n_ct;
  if (grid == 0) return hipSuccess;
  if (grid > 0x7fffffffLL) return hipErrorInvalidValue;
  if (up) hipLaunchKernelGGL(proj_kernel<true>, dim3((unsigned)grid), dim3(256), 0, s, p);
  else hipLaunchKernelGGL(proj_kernel<false>, dim3((unsigned)grid), dim3(256), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_append(const AppendParams &p, hipStream_t s) {
  const long long rows = (long long)p.B * p.s_q;
  if (rows == 0) return hipSuccess;
  hipLaunchKernelGGL(append_kernel, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace lkv
