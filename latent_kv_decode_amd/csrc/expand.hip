// expand.hip -- latent expansion into g key/value groups at cache-write time.
//
// [GQLA explainer, technical summary section 2, GQA path]: the latent c_KV of
// every token is expanded once into g key groups K_g = c W_UK[g] and g value
// groups V_g = c W_UV[g] (width d_h each), stored beside the shared RoPE key
// under the same page ids, so that decode runs plain grouped-query attention
// with no per-step expansion.
//
// As one matrix product: D [tokens x 2 g d_h] = C [tokens x d_c] W, where
// column j of W is column j mod d_h of block j / d_h, blocks 0..g-1 being
// W_UK[0..g-1] and g..2g-1 W_UV[0..g-1]; the tokens are gathered from (and the
// outputs scattered to) cache rows through the block table.
//
// A work-group computes a 256-token x 256-column tile of D over K-chunks of
// 64 (double-buffered in LDS, the next chunk prefetched into registers while
// the current one is multiplied).  Eight waves: wave w takes tokens
// 128 (w mod 2) .. and columns 64 (w / 2) .. of the tile and computes
// D^T = W^T C^T with v_mfma_f32_16x16x32_bf16 (A = W^T from the row-major
// weight chunk through ds_read_b64_tr_b16, B = C^T read row-wise from the
// token chunk): 32 products per 32-deep k-step for 12 fragment reads.  The
// column tiles of one token tile run on one XCD, so that its latent rows are
// read from HBM once.  float32 accumulation, bf16 output (round to nearest
// even).  The finished tile goes through the (then free) staging LDS in
// row-major order, so that each token's columns leave as whole 16-byte
// pieces of contiguous runs rather than as scattered 8-byte stores.
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

constexpr int kMaxDc = 512;
constexpr int kTM = 256;        // tokens per work-group
constexpr int kTN = 256;        // output columns per work-group
constexpr int kKC = 64;         // K-chunk
constexpr int kThreadsX = 512;  // 8 waves

// Token chunk [256][64]: rows of 8 sixteen-byte chunks; chunk c of row r at
// c ^ ((r / 2) mod 8), so that sixteen rows read at one chunk column hit
// distinct banks.
__device__ __forceinline__ int swz_c(int c, int r) { return c ^ ((r >> 1) & 7); }
// Weight chunk [64][256]: rows of 32 chunks (512 bytes, one full pass over
// the banks, so every row starts on bank 0).  A transpose read covers rows
// 8g + (0..3) and + 4 for g = 0..3 at one chunk pair: the low three chunk
// bits take a bijection of r mod 8 and chunk bits 3..4 take (r / 8) mod 4,
// which puts the rows of one read on distinct banks.
__device__ __forceinline__ int swz_w(int c, int r) {
  const int t = r & 7;
  return c ^ (((t & 3) << 1) | (t >> 2) | (((r >> 3) & 3) << 3));
}
__device__ __forceinline__ s16x4 lds_read_tr(const bf16 *p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4 *)(p));
}
__device__ __forceinline__ bf16x8 join(s16x4 lo, s16x4 hi) {
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

template <int DH>
__global__ void __launch_bounds__(kThreadsX) expand_kernel(const ExpandParams p) {
  static_assert(kTN % DH == 0 || DH % kTN == 0, "column tile and group width");
  // staging buffers (token and weight chunks, double-buffered), reused at
  // the end for the bf16 output tile [kTM][kTN]
  static_assert(2 * kTM * kKC + 2 * kKC * kTN == kTM * kTN, "output tile fits the staging LDS");
  __shared__ __attribute__((aligned(16))) bf16 s_mem[2 * kTM * kKC + 2 * kKC * kTN];
  bf16(*s_c)[kTM * kKC] = reinterpret_cast<bf16(*)[kTM * kKC]>(s_mem);
  bf16(*s_w)[kKC * kTN] = reinterpret_cast<bf16(*)[kKC * kTN]>(s_mem + 2 * kTM * kKC);
  __shared__ int s_row[kTM];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, g = lane >> 4, n = lane & 15;
  // block -> (token tile, column tile); the column tiles of one token tile
  // share an XCD (block index mod 8)
  const int ncols = 2 * p.g * DH;
  const int n_ct = (ncols + kTN - 1) / kTN;  // the last tile may be partial
  const int tiles_per_seq = (p.max_pages * p.page_size + kTM - 1) / kTM;
  const int bx = blockIdx.x;
  const int rest = bx >> 3;
  const int ct = rest % n_ct;
  const int tt = (rest / n_ct) * 8 + (bx & 7);
  if (tt >= p.B * tiles_per_seq) return;
  const int b = tt / tiles_per_seq, tile = tt % tiles_per_seq;
  const int L = p.seqlens[b];
  const int j0 = p.start_pos ? p.start_pos[b] : 0;
  if (tile * kTM >= L || (tile + 1) * kTM <= j0) return;
  const int32_t *bt = p.block_table + (long long)b * p.max_pages;
  if (tid < kTM) {
    const int j = tile * kTM + tid;
    s_row[tid] = (j < L && j >= j0) ? bt[j / p.page_size] * p.page_size + j % p.page_size : -1;
  }
  __syncthreads();

  // ---- staging: thread tid moves sixteen-byte pieces tid + 512 u (u < 4)
  // of the token chunk (piece i: token i / 8, chunk i mod 8) and of the
  // weight chunk (row i / 32, column chunk i mod 32), K-chunk kc: eight
  // consecutive lanes read one token's 128 bytes, thirty-two one weight
  // row's 512.
  const bf16 *cbase = static_cast<const bf16 *>(p.c);
  const int col0 = ct * kTN;
  const int a_ch = tid & 7, w_ch = tid & 31;
  int a_row[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) a_row[u] = s_row[(tid + 512 * u) >> 3];
  // weight column chunk -> (block, offset): column 8 w_ch of the tile
  const int w_col = col0 + 8 * w_ch;
  const int w_blk = w_col / DH, w_d = w_col % DH;
  const bf16 *w_mat = static_cast<const bf16 *>(w_blk < p.g ? p.w_uk : p.w_uv) +
                      (long long)(w_blk % p.g) * p.d_c * DH + w_d;
  u32x4 pa[4], pw[4];
  auto load_chunk = [&](int kc) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      u32x4 v = {0u, 0u, 0u, 0u};
      if (a_row[u] >= 0)
        v = *reinterpret_cast<const u32x4 *>(cbase + (long long)a_row[u] * p.c_stride + kc * kKC + 8 * a_ch);
      pa[u] = v;
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int k = kc * kKC + ((tid + 512 * u) >> 5);
      u32x4 v = {0u, 0u, 0u, 0u};
      if (w_col < ncols) v = *reinterpret_cast<const u32x4 *>(w_mat + (long long)k * DH);
      pw[u] = v;
    }
  };
  auto store_chunk = [&](int buf) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int tok = (tid + 512 * u) >> 3;
      *reinterpret_cast<u32x4 *>(&s_c[buf][tok * kKC + swz_c(a_ch, tok) * 8]) = pa[u];
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int r = (tid + 512 * u) >> 5;
      *reinterpret_cast<u32x4 *>(&s_w[buf][r * kTN + swz_w(w_ch, r) * 8]) = pw[u];
    }
  };

  // ---- this wave's share: tokens 128 wt + 16 nt + n, columns 64 wc + 16 mt
  const int wt = w & 1, wc = w >> 1;
  f32x4 acc[4][8];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) acc[mt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int nkc = p.d_c / kKC;
  load_chunk(0);
  store_chunk(0);
  __syncthreads();
  for (int kc = 0; kc < nkc; ++kc) {
    const int buf = kc & 1;
    if (kc + 1 < nkc) load_chunk(kc + 1);
    const bf16 *ct_ = s_c[buf];
    const bf16 *wt_ = s_w[buf];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      // B = C^T: token 128 wt + 16 nt + n, K 32 ks + 8 g .. + 7
      bf16x8 bc[8];
#pragma unroll
      for (int nt = 0; nt < 8; ++nt) {
        const int tok = 128 * wt + 16 * nt + n;
        bc[nt] = *reinterpret_cast<const bf16x8 *>(ct_ + tok * kKC + swz_c(4 * ks + g, tok) * 8);
      }
      // A = W^T: column 64 wc + 16 mt + 4 (n mod 4) .. + 3 of weight rows
      // rk and rk + 4
      const int rk = 32 * ks + 8 * g + (n >> 2);
      bf16x8 aw[4];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        const int col = 64 * wc + 16 * mt + 4 * (n & 3);
        const int ch = col >> 3, off = col & 7;
        aw[mt] = join(lds_read_tr(wt_ + rk * kTN + swz_w(ch, rk) * 8 + off),
                      lds_read_tr(wt_ + (rk + 4) * kTN + swz_w(ch, rk + 4) * 8 + off));
      }
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int nt = 0; nt < 8; ++nt)
          acc[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aw[mt], bc[nt], acc[mt][nt], 0, 0, 0);
    }
    // the other buffer was last read in the previous chunk, before the
    // barrier that ended it
    if (kc + 1 < nkc) store_chunk(buf ^ 1);
    __syncthreads();
  }

  if (p.out_fp8) {
    // ---- 8-bit caches: codes of value * (1 / out_scale), rounded once from
    // the float32 results, into LDS as a [token][column] byte tile (16-byte chunk
    // c of token row t at c ^ (t mod 16)), then out in 16-byte pieces
    unsigned char *s8 = reinterpret_cast<unsigned char *>(s_mem);
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) {
      const int tok = 128 * wt + 16 * nt + n;
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        const int col = 64 * wc + 16 * mt + 4 * g;
        unsigned word = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) word |= e4m3_encode(acc[mt][nt][i] * p.out_inv_scale) << (8 * i);
        *reinterpret_cast<unsigned *>(s8 + tok * kTN + (((col >> 4) ^ (tok & 15)) << 4) + (col & 15)) = word;
      }
    }
    __syncthreads();
#pragma unroll 4
    for (int u = 0; u < kTM * kTN / 16 / kThreadsX; ++u) {
      const int q = tid + kThreadsX * u, tok = q >> 4, c = q & 15;
      const int row = s_row[tok];
      const int col = col0 + 16 * c;
      if (row < 0 || col >= ncols) continue;
      const u32x4 v = *reinterpret_cast<const u32x4 *>(s8 + tok * kTN + ((c ^ (tok & 15)) << 4));
      const int blk = col / DH, d = col % DH;
      unsigned char *dst = static_cast<unsigned char *>(blk < p.g ? p.k_out : p.v_out);
      const long long ostride = blk < p.g ? p.k_stride : p.v_stride;
      *reinterpret_cast<u32x4 *>(dst + (long long)row * ostride + (long long)(blk % p.g) * DH + d) = v;
    }
    return;
  }

  // ---- D^T tile (columns 4 g .. + 3 of token n per lane) into LDS as a
  // row-major [token][column] bf16 tile; 16-byte chunk c of token row t at
  // c ^ 2 (t mod 16), so that the 16 tokens x 4 column groups of one write
  // hit distinct banks.  (The loop's last barrier ended every read of the
  // staging buffers.)
#pragma unroll
  for (int nt = 0; nt < 8; ++nt) {
    const int tok = 128 * wt + 16 * nt + n;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      const int col = 64 * wc + 16 * mt + 4 * g;
      const int ch = (col >> 3) ^ ((tok & 15) << 1);
      bf16x4 o;
#pragma unroll
      for (int i = 0; i < 4; ++i) o[i] = static_cast<bf16>(acc[mt][nt][i]);
      *reinterpret_cast<bf16x4 *>(s_mem + tok * kTN + ch * 8 + (col & 7)) = o;
    }
  }
  __syncthreads();
  // ---- out: piece q = tid + 512 u is chunk q mod 32 (8 columns) of token
  // row q / 32; half a wave covers one token's 512 bytes
#pragma unroll 4
  for (int u = 0; u < kTM * kTN / 8 / kThreadsX; ++u) {
    const int q = tid + kThreadsX * u, tok = q >> 5, c = q & 31;
    const int row = s_row[tok];
    const int col = col0 + 8 * c;
    if (row < 0 || col >= ncols) continue;
    const u32x4 v = *reinterpret_cast<const u32x4 *>(s_mem + tok * kTN + ((c ^ ((tok & 15) << 1)) * 8));
    const int blk = col / DH, d = col % DH;
    bf16 *dst = static_cast<bf16 *>(blk < p.g ? p.k_out : p.v_out);
    const long long ostride = blk < p.g ? p.k_stride : p.v_stride;
    *reinterpret_cast<u32x4 *>(dst + (long long)row * ostride + (long long)(blk % p.g) * DH + d) = v;
  }
}

}  // namespace

bool expand_supported(int d_c, int d_h) {
  return d_c >= 64 && d_c <= kMaxDc && d_c % 64 == 0 && (d_h == 64 || d_h == 128 || d_h == 256);
}

hipError_t launch_expand(const ExpandParams &p, hipStream_t s) {
  const long long tiles = (long long)p.B * ((p.max_pages * (long long)p.page_size + kTM - 1) / kTM);
  const int n_ct = (2 * p.g * p.d_h + kTN - 1) / kTN;
  if (tiles == 0 || n_ct == 0) return hipSuccess;
  const long long grid = (tiles + 7) / 8 * 8 * n_ct;
  if (grid > 0x7fffffffLL) return hipErrorInvalidValue;
  switch (p.d_h) {
    case 64: hipLaunchKernelGGL(expand_kernel<64>, dim3((unsigned)grid), dim3(kThreadsX), 0, s, p); break;
    case 128: hipLaunchKernelGGL(expand_kernel<128>, dim3((unsigned)grid), dim3(kThreadsX), 0, s, p); break;
    case 256: hipLaunchKernelGGL(expand_kernel<256>, dim3((unsigned)grid), dim3(kThreadsX), 0, s, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace lkv
