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
// 32, brought into LDS by direct-to-LDS loads through a ring of four stages,
// three chunks ahead of the products (every wave issues four 1-KiB loads per
// chunk and waits only for the chunk it is about to read, then one barrier).
// Eight waves: wave w takes tokens 128 (w mod 2) .. and columns 64 (w / 2) ..
// of the tile and computes D^T = W^T C^T with v_mfma_f32_16x16x32_bf16 (A =
// W^T from the row-major weight chunk through ds_read_b64_tr_b16, B = C^T
// read row-wise from the token chunk): 32 products per chunk for 12 fragment
// reads.  The column tiles of one token tile run on one XCD, so that its
// latent rows are read from HBM once.  float32 accumulation, bf16 output
// (round to nearest even).  The finished tile goes through the (then free)
// stages in row-major order, so that each token's columns leave as whole
// 16-byte pieces of contiguous runs, with streaming stores (the output is
// not read again here, and in the cache it would push out the latent rows
// the other column tiles still read).
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
constexpr int kThreadsX = 512;  // 8 waves
constexpr int kKC = 32;         // K-chunk
constexpr int kStage = kTM * kKC + kKC * kTN;  // bf16 elements per stage (32 KiB)

// Token chunk [256][32]: rows of 4 sixteen-byte pieces; piece c of row r at
// slot c ^ ((r / 2) mod 4).  Chosen by measurement (SQ_LDS_BANK_CONFLICT):
// with this pattern the B-operand reads (16 rows, pieces g = 0..3) add no
// bank conflicts, where no swizzle, r mod 4 or (r / 4) mod 4 add 33 M
// conflict cycles per launch at the GQLA g = 8 shape.
__device__ __forceinline__ int swz_t(int c, int r) { return c ^ ((r >> 1) & 3); }
// Weight chunk [32][256]: rows of 32 pieces (512 bytes, one full pass over
// the banks, so every row starts on bank 0).  A transpose read covers rows
// 8g + (0..3) and + 4 for g = 0..3 at one piece pair: the low three piece
// bits take a bijection of r mod 8 and piece bits 3..4 take (r / 8) mod 4,
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

// Stage layout: token chunk, then weight chunk.  One wave instruction fills
// 1 KiB of a stage in lane order; lane i fetches the piece whose swizzled
// slot is i, so the swizzle costs nothing at store time.
template <int DH>
__global__ void __launch_bounds__(kThreadsX) expand_kernel(const ExpandParams p) {
  static_assert(kTN % DH == 0 || DH % kTN == 0, "column tile and group width");
  static_assert(4 * kStage == kTM * kTN, "output tile fits the four stages");
  __shared__ __attribute__((aligned(16))) bf16 s_st0[kStage];
  __shared__ __attribute__((aligned(16))) bf16 s_st1[kStage];
  __shared__ __attribute__((aligned(16))) bf16 s_st2[kStage];
  __shared__ __attribute__((aligned(16))) bf16 s_st3[kStage];
  __shared__ int s_row[kTM];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, g = lane >> 4, n = lane & 15;
  const int wu = __builtin_amdgcn_readfirstlane(w);
  const int ncols = 2 * p.g * DH;
  const int n_ct = (ncols + kTN - 1) / kTN;
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

  // ---- this wave's loads: token rows 32 wu + 16 u + lane / 4 (piece slot
  // lane mod 4) and weight rows 4 wu + 2 u + lane / 32 (slot lane mod 32),
  // u = 0, 1.  Invalid tokens read row 0 (their outputs are not written);
  // columns past the last group read the first weight row.
  const int col0 = ct * kTN;
  const char *tsrc[2];
  const char *wsrc[2];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int r = 32 * wu + 16 * u + (lane >> 2);
    const int row = max(s_row[r], 0);
    const int c = swz_t(lane & 3, r);
    tsrc[u] = reinterpret_cast<const char *>(static_cast<const bf16 *>(p.c) + (long long)row * p.c_stride + 8 * c);
    const int kr = 4 * wu + 2 * u + (lane >> 5);
    const int cw = swz_w(lane & 31, kr);
    const int col = col0 + 8 * cw;
    const bf16 *wm = static_cast<const bf16 *>(p.w_uk);
    long long off = 0;
    if (col < ncols) {
      const int blk = col / DH, d = col % DH;
      wm = static_cast<const bf16 *>(blk < p.g ? p.w_uk : p.w_uv);
      off = (long long)(blk % p.g) * p.d_c * DH + d;
    }
    wsrc[u] = reinterpret_cast<const char *>(wm + off + (long long)kr * DH);
  }
  auto issue = [&](int kc, bf16 *st) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < 2; ++u)
      __builtin_amdgcn_global_load_lds(tsrc[u] + kc * (kKC * 2),
                                       (__attribute__((address_space(3))) void *)(st + (32 * wu + 16 * u) * kKC),
                                       16, 0, 0);
#pragma unroll
    for (int u = 0; u < 2; ++u)
      __builtin_amdgcn_global_load_lds(wsrc[u] + (long long)kc * (kKC * DH * 2),
                                       (__attribute__((address_space(3))) void *)(st + kTM * kKC + (4 * wu + 2 * u) * kTN),
                                       16, 0, 0);
  };

  // ---- this wave's share: tokens 128 wt + 16 nt + n, columns 64 wc + 16 mt
  const int wt = w & 1, wc = w >> 1;
  f32x4 acc[4][8];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) acc[mt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
  auto compute = [&](const bf16 *st) __attribute__((always_inline)) {
    const bf16 *ct_ = st;
    const bf16 *wt_ = st + kTM * kKC;
    bf16x8 bc[8];
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) {
      const int tok = 128 * wt + 16 * nt + n;
      bc[nt] = *reinterpret_cast<const bf16x8 *>(ct_ + tok * kKC + swz_t(g, tok) * 8);
    }
    const int rk = 8 * g + (n >> 2);
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
  };
  // barrier without the global-memory fence of __syncthreads() (which would
  // wait for every load in flight): each wave has waited for its own loads
  auto barrier = [&]() __attribute__((always_inline)) {
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };

  // Every step issues one chunk (past the last chunk, a copy of the last
  // one into a stage that is not read again), so this wave always has the
  // same count of loads in flight: chunk kc has landed once at most 8 (the
  // next two chunks) remain.
  const int nkc = p.d_c / kKC;
  issue(0, s_st0);
  issue(min(1, nkc - 1), s_st1);
  issue(min(2, nkc - 1), s_st2);
  auto step = [&](auto r_tag, int kc) __attribute__((always_inline)) {
    constexpr int R = decltype(r_tag)::value;
    bf16 *cur = R == 0 ? s_st0 : R == 1 ? s_st1 : R == 2 ? s_st2 : s_st3;
    bf16 *nxt = R == 0 ? s_st3 : R == 1 ? s_st0 : R == 2 ? s_st1 : s_st2;  // stage of chunk kc + 3
    __builtin_amdgcn_s_waitcnt(0x0F78);  // vmcnt(8)
    barrier();
    issue(min(kc + 3, nkc - 1), nxt);
    compute(cur);
  };
  int kc = 0;
  for (; kc + 4 <= nkc; kc += 4) {
    step(std::integral_constant<int, 0>{}, kc);
    step(std::integral_constant<int, 1>{}, kc + 1);
    step(std::integral_constant<int, 2>{}, kc + 2);
    step(std::integral_constant<int, 3>{}, kc + 3);
  }
  if (kc < nkc) {
    step(std::integral_constant<int, 0>{}, kc);
    if (kc + 1 < nkc) {
      step(std::integral_constant<int, 1>{}, kc + 1);
      if (kc + 2 < nkc) step(std::integral_constant<int, 2>{}, kc + 2);
    }
  }
  __builtin_amdgcn_s_waitcnt(0x0F70);
  __syncthreads();  // every stage read; the stages take the output tile

  // output tile row-major over the four stages: token t at stage t / 64
  auto orow = [&](int tok) -> bf16 * {
    const int q = tok >> 6;
    bf16 *st = q == 0 ? s_st0 : q == 1 ? s_st1 : q == 2 ? s_st2 : s_st3;
    return st + (tok & 63) * kTN;
  };
  if (p.out_fp8) {
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) {
      const int tok = 128 * wt + 16 * nt + n;
      const int q = tok >> 7;  // 8-bit tile: token t at stage t / 128, 256 bytes per row
      unsigned char *base8 = reinterpret_cast<unsigned char *>(q == 0 ? s_st0 : s_st1) + (tok & 127) * kTN;
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        const int col = 64 * wc + 16 * mt + 4 * g;
        unsigned word = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) word |= e4m3_encode(acc[mt][nt][i] * p.out_inv_scale) << (8 * i);
        *reinterpret_cast<unsigned *>(base8 + (((col >> 4) ^ (tok & 15)) << 4) + (col & 15)) = word;
      }
    }
    __syncthreads();
#pragma unroll 4
    for (int u = 0; u < kTM * kTN / 16 / kThreadsX; ++u) {
      const int q = tid + kThreadsX * u, tok = q >> 4, c = q & 15;
      const int row = s_row[tok];
      const int col = col0 + 16 * c;
      if (row < 0 || col >= ncols) continue;
      const unsigned char *base8 = reinterpret_cast<const unsigned char *>((tok >> 7) == 0 ? s_st0 : s_st1) + (tok & 127) * kTN;
      const u32x4 v = *reinterpret_cast<const u32x4 *>(base8 + ((c ^ (tok & 15)) << 4));
      const int blk = col / DH, d = col % DH;
      unsigned char *dst = static_cast<unsigned char *>(blk < p.g ? p.k_out : p.v_out);
      const long long ostride = blk < p.g ? p.k_stride : p.v_stride;
      __builtin_nontemporal_store(v, reinterpret_cast<u32x4 *>(dst + (long long)row * ostride + (long long)(blk % p.g) * DH + d));
    }
    return;
  }
#pragma unroll
  for (int nt = 0; nt < 8; ++nt) {
    const int tok = 128 * wt + 16 * nt + n;
    bf16 *r = orow(tok);
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      const int col = 64 * wc + 16 * mt + 4 * g;
      const int ch = (col >> 3) ^ ((tok & 15) << 1);
      bf16x4 o;
#pragma unroll
      for (int i = 0; i < 4; ++i) o[i] = static_cast<bf16>(acc[mt][nt][i]);
      *reinterpret_cast<bf16x4 *>(r + ch * 8 + (col & 7)) = o;
    }
  }
  __syncthreads();
#pragma unroll 4
  for (int u = 0; u < kTM * kTN / 8 / kThreadsX; ++u) {
    const int q = tid + kThreadsX * u, tok = q >> 5, c = q & 31;
    const int row = s_row[tok];
    const int col = col0 + 8 * c;
    if (row < 0 || col >= ncols) continue;
    const u32x4 v = *reinterpret_cast<const u32x4 *>(orow(tok) + ((c ^ ((tok & 15) << 1)) * 8));
    const int blk = col / DH, d = col % DH;
    bf16 *dst = static_cast<bf16 *>(blk < p.g ? p.k_out : p.v_out);
    const long long ostride = blk < p.g ? p.k_stride : p.v_stride;
    __builtin_nontemporal_store(v, reinterpret_cast<u32x4 *>(dst + (long long)row * ostride + (long long)(blk % p.g) * DH + d));
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
