// expand.hip -- latent expansion into g key/value groups at cache-write time.
//
// [GQLA explainer, technical summary section 2, GQA path]: the latent c_KV of
// every token is expanded once into g key groups K_g = c W_UK[g] and g value
// groups V_g = c W_UV[g] (width d_h each), stored beside the shared RoPE key
// under the same page ids, so that decode runs plain grouped-query attention
// with no per-step expansion.
//
// One work-group per 64-token tile of one sequence.  The tile's latents sit
// in LDS for the whole work-group; the 2g weight blocks [d_c x d_h] stream
// through LDS in 64-row chunks (register prefetch of the next chunk).  Each
// wave computes D^T = W^T C^T for a quarter of the d_h output columns and all
// 64 tokens with v_mfma_f32_16x16x32_bf16: A = W^T read from the row-major
// weight chunk with ds_read_b64_tr_b16, B = C^T read row-wise from the latent
// tile.  float32 accumulation, bf16 output (round to nearest even).
#include "lkv_internal.h"

namespace lkv {
namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short s16x4;
typedef __attribute__((__vector_size__(8 * sizeof(short)))) short s16x8;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(4 * sizeof(unsigned)))) unsigned u32x4;
typedef __bf16 bf16;

constexpr int kMaxDc = 512;

__device__ __forceinline__ int swz(int chunk, int row) {
  const int t = row & 7;
  return chunk ^ (((t & 3) << 1) | (t >> 2));
}
__device__ __forceinline__ s16x4 lds_read_tr(const bf16 *p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4 *)(p));
}
__device__ __forceinline__ bf16x8 join(s16x4 lo, s16x4 hi) {
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

template <int DH>
__global__ void __launch_bounds__(256) expand_kernel(const ExpandParams p) {
  constexpr int DHW = DH / 4;             // output columns per wave
  constexpr int MT = DHW / 16;
  constexpr int WCH = 64 * DH / 8 / 256;  // 16-byte loads per thread per weight chunk
  __shared__ __attribute__((aligned(16))) bf16 s_c[kTile * kMaxDc];
  __shared__ __attribute__((aligned(16))) bf16 s_w[2][64 * DH];
  __shared__ int s_row[kTile];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, g = lane >> 4, n = lane & 15;
  const int max_tiles = (p.max_pages * p.page_size + kTile - 1) / kTile;
  const int b = blockIdx.x / max_tiles, tile = blockIdx.x % max_tiles;
  const int L = p.seqlens[b];
  const int j0 = p.start_pos ? p.start_pos[b] : 0;
  if (tile * kTile >= L || (tile + 1) * kTile <= j0) return;
  const int32_t *bt = p.block_table + (long long)b * p.max_pages;
  if (tid < kTile) {
    const int j = tile * kTile + tid;
    s_row[tid] = (j < L && j >= j0) ? bt[j / p.page_size] * p.page_size + j % p.page_size : -1;
  }
  __syncthreads();

  // latent tile -> LDS (zeros for tokens that are not expanded)
  const bf16 *cbase = static_cast<const bf16 *>(p.c);
  const int cpr = p.d_c / 8;
  for (int idx = tid; idx < kTile * cpr; idx += 256) {
    const int tok = idx / cpr, ch = idx % cpr;
    const int row = s_row[tok];
    u32x4 v = {0u, 0u, 0u, 0u};
    if (row >= 0) v = *reinterpret_cast<const u32x4 *>(cbase + (long long)row * p.c_stride + 8 * ch);
    *reinterpret_cast<u32x4 *>(s_c + tok * p.d_c + swz(ch, tok) * 8) = v;
  }

  const int nchunk = p.d_c / 64;
  const int nblk = 2 * p.g;
  const int total = nblk * nchunk;
  u32x4 pre[WCH];
  auto wsrc = [&](int step) -> const bf16 * {
    const int blk = step / nchunk, kc = step % nchunk;
    const bf16 *wm = static_cast<const bf16 *>(blk < p.g ? p.w_uk : p.w_uv);
    return wm + ((long long)(blk % p.g) * p.d_c + 64 * kc) * DH;
  };
  auto load_w = [&](int step) {
    const bf16 *src = wsrc(step);
#pragma unroll
    for (int u = 0; u < WCH; ++u) {
      const int idx = tid + 256 * u;  // 16-byte chunk in the [64][DH] block
      pre[u] = *reinterpret_cast<const u32x4 *>(src + 8 * idx);
    }
  };
  auto store_w = [&](int buf) {
#pragma unroll
    for (int u = 0; u < WCH; ++u) {
      const int idx = tid + 256 * u;
      const int r = idx / (DH / 8), ch = idx % (DH / 8);
      *reinterpret_cast<u32x4 *>(&s_w[buf][r * DH + swz(ch, r) * 8]) = pre[u];
    }
  };

  load_w(0);
  store_w(0);
  __syncthreads();
  f32x4 acc[MT][4];
  for (int step = 0; step < total; ++step) {
    const int kc = step % nchunk, buf = step & 1;
    if (kc == 0) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) acc[mt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    if (step + 1 < total) load_w(step + 1);
    const bf16 *wt = s_w[buf];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      bf16x8 bc[4];
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        const int tok = 16 * nt + n;
        bc[nt] = *reinterpret_cast<const bf16x8 *>(s_c + tok * p.d_c + swz(8 * kc + 4 * ks + g, tok) * 8);
      }
      const int rk = 32 * ks + 8 * g + (n >> 2);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const int col = w * DHW + 16 * mt + 4 * (n & 3);
        const int ch = col >> 3, off = col & 7;
        const bf16x8 a = join(lds_read_tr(wt + rk * DH + swz(ch, rk) * 8 + off),
                              lds_read_tr(wt + (rk + 4) * DH + swz(ch, rk + 4) * 8 + off));
#pragma unroll
        for (int nt = 0; nt < 4; ++nt)
          acc[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bc[nt], acc[mt][nt], 0, 0, 0);
      }
    }
    if (kc == nchunk - 1) {
      const int blk = step / nchunk;
      bf16 *dst = static_cast<bf16 *>(blk < p.g ? p.k_out : p.v_out);
      const long long ostride = blk < p.g ? p.k_stride : p.v_stride;
      const int grp = blk % p.g;
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        const int row = s_row[16 * nt + n];
        if (row < 0) continue;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          bf16x4 o;
#pragma unroll
          for (int i = 0; i < 4; ++i) o[i] = static_cast<bf16>(acc[mt][nt][i]);
          *reinterpret_cast<bf16x4 *>(dst + (long long)row * ostride + (long long)grp * DH + w * DHW +
                                      16 * mt + 4 * g) = o;
        }
      }
    }
    if (step + 1 < total) store_w(buf ^ 1);
    __syncthreads();
  }
}

}  // namespace

bool expand_supported(int d_c, int d_h) {
  return d_c >= 64 && d_c <= kMaxDc && d_c % 64 == 0 && (d_h == 64 || d_h == 128 || d_h == 256);
}

hipError_t launch_expand(const ExpandParams &p, hipStream_t s) {
  const int max_tiles = (p.max_pages * p.page_size + kTile - 1) / kTile;
  const long long grid = (long long)p.B * max_tiles;
  if (grid == 0) return hipSuccess;
  switch (p.d_h) {
    case 64: hipLaunchKernelGGL(expand_kernel<64>, dim3((unsigned)grid), dim3(256), 0, s, p); break;
    case 128: hipLaunchKernelGGL(expand_kernel<128>, dim3((unsigned)grid), dim3(256), 0, s, p); break;
    case 256: hipLaunchKernelGGL(expand_kernel<256>, dim3((unsigned)grid), dim3(256), 0, s, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace lkv
