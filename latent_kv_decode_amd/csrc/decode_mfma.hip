// decode_mfma.hip -- paged decode attention on the gfx950 matrix cores.
//
// One kernel serves both cache layouts of the pages:
//   * MLA absorbed path [GQLA explainer, technical summary section 2,
//     MQA-absorbed path]: every query head of a latent head attends over the
//     latent c_KV (width DK) plus a shared RoPE key (width DR); the latent is
//     also the value (V_ALIAS), so P.c_KV is what the kernel writes.  With
//     several latent heads this is GLA [Grouped Latent Attention article,
//     GLA section].
//   * GQA path [same explainer section, GQA path]: K and V of one group are
//     separate caches of width DK == DV, optionally with the shared RoPE key;
//     with DR == 0 it is plain GQA.
//
// Work decomposition.  The query rows of one KV head, (t, h) for the s_q
// new tokens and the hpk query heads that share the head, are cut into
// row tiles of ROWS (16 or 32).  The cache tiles (64 tokens) of all
// sequences are concatenated and cut into n_chunks equal shares.  A
// work-group owns one (KV head, row tile, share).  A share that holds a
// whole sequence writes the final output; a share that holds part of one
// writes a float32 partial plus its LSE, merged afterwards by the combine
// kernel.  The shares of one row group are spread over the 8 XCDs while the
// row tiles of one share stay on one XCD, so the tiles that several row
// tiles read are fetched from HBM once and hit in that XCD's L2.
//
// Per 64-token tile, 4 waves:
//   stage:  global -> registers -> LDS (double buffered, 16-byte chunks,
//           XOR-swizzled so that both read patterns below are free of bank
//           conflicts);
//   QK^T:   wave w computes S^T = K Q^T for tokens 16w..16w+15 and all ROWS
//           rows with v_mfma_f32_16x16x32_bf16 (A = K tile from LDS, B = Q
//           kept in registers for the whole sequence);
//   softmax: online, base 2; the per-row maximum of the tile is exchanged
//           through LDS, the row sums stay per lane until the end;
//   PV:     wave w computes O^T = V^T P^T for its quarter of the value
//           width; V^T comes straight from the token-major tile through
//           ds_read_b64_tr_b16, P^T through LDS as bf16.
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

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr float kLn2 = 0.693147180559945309f;

__device__ __forceinline__ float neg_inf() { return -__builtin_inff(); }

// 16-byte chunk `chunk` of LDS row `row` lives at chunk slot chunk ^ sig(row),
// sig(t) = 2*(t mod 4) + (t mod 8) / 4.  Eight consecutive rows reading one
// chunk hit eight different bank groups, and four consecutive rows reading a
// pair of chunks (the transpose read) do too.
__device__ __forceinline__ int swz(int chunk, int row) {
  const int t = row & 7;
  return chunk ^ (((t & 3) << 1) | (t >> 2));
}

__device__ __forceinline__ s16x4 lds_read_tr(const bf16 *p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4 *)(p));
}

__device__ __forceinline__ bf16x8 join(s16x4 lo, s16x4 hi) {
  s16x8 v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, v);
}

__device__ __forceinline__ int seq_tiles(int L) { return L <= 0 ? 1 : (L + kTile - 1) / kTile; }

// Split-KV plan, computed by every work-group from the device lengths: the
// tiles of all sequences (an empty sequence counts one tile) are concatenated
// and cut into n_chunks shares of `chunk` tiles.  Returns false when share c is
// empty; otherwise the first sequence overlapping it and that sequence's first
// concatenated tile.
__device__ bool plan_share(const int32_t *seqlens, int B, int C, int c, int *sh, int &chunk, int &t0,
                           int &t1, int &b0, int &cu0) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int per = (B + kThreads - 1) / kThreads;
  const int s0 = min(B, tid * per), s1 = min(B, s0 + per);
  int local = 0;
  for (int b = s0; b < s1; ++b) local += seq_tiles(seqlens[b]);
  int v = local;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    int u = __shfl_up(v, o);
    if (lane >= o) v += u;
  }
  if (lane == 63) sh[w] = v;
  __syncthreads();
  int before = 0, total = 0;
#pragma unroll
  for (int i = 0; i < kWaves; ++i) {
    int s = sh[i];
    if (i < w) before += s;
    total += s;
  }
  const int excl = before + v - local;
  chunk = (total + C - 1) / C;
  t0 = c * chunk;
  t1 = min(total, t0 + chunk);
  __syncthreads();
  if (t0 >= total) return false;
  if (t0 >= excl && t0 < excl + local) {
    int cu = excl;
    for (int b = s0; b < s1; ++b) {
      const int nb = seq_tiles(seqlens[b]);
      if (t0 < cu + nb) {
        sh[4] = b;
        sh[5] = cu;
        break;
      }
      cu += nb;
    }
  }
  __syncthreads();
  b0 = sh[4];
  cu0 = sh[5];
  return true;
}

template <int DK, int DR, int DV, bool VA, int ROWS>
struct Cfg {
  static constexpr int KW = DK + DR;
  static_assert(KW % 64 == 0 && DV % 64 == 0, "widths must be multiples of 64");
  static_assert(!VA || DV == DK, "the latent is the value");
  static constexpr int KSTR = KW;                        // LDS row stride of the key tile
  static constexpr int VSTR = VA ? KW : DV;              // LDS row stride of the value tile
  static constexpr int KTILE = kTile * KSTR;
  static constexpr int BUF = KTILE + (VA ? 0 : kTile * DV);
  static constexpr int KS = KW / 32;                     // k-steps of QK^T
  static constexpr int KSN = DK / 32;                    // of which on the main part
  static constexpr int NT = ROWS / 16;
  static constexpr int DVW = DV / kWaves;
  static constexpr int MT = DVW / 16;
  static constexpr int KC8 = KW / 64;                    // key chunks per thread per token
  static constexpr int VC8 = VA ? 0 : DV / 64;
  static constexpr int NLD = 2 * (KC8 + VC8);
  static constexpr int PSTR = kTile + 8;                 // P row stride (elements)
  static constexpr int LDS_BYTES = 2 * BUF * 2 + ROWS * PSTR * 2 + kWaves * ROWS * 4 + 64;
  static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");
};

template <int DK, int DR, int DV, bool VA, int ROWS>
__global__ void __launch_bounds__(kThreads, 1) mfma_decode_kernel(const DecodeParams p) {
  using C = Cfg<DK, DR, DV, VA, ROWS>;
  constexpr int NT = C::NT, MT = C::MT, KS = C::KS;
  __shared__ __attribute__((aligned(16))) bf16 s_buf[2 * C::BUF];
  __shared__ __attribute__((aligned(16))) bf16 s_p[ROWS * C::PSTR];
  __shared__ float s_red[kWaves * ROWS];
  __shared__ int s_plan[8];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int g = lane >> 4, n = lane & 15;

  // block -> (share, row group); the row groups of a share sit on one XCD
  const int G = p.n_kvh * p.row_tiles;
  const int bx = blockIdx.x;
  const int q8 = bx >> 3;
  const int grp = q8 % G;
  const int c = (q8 / G) * 8 + (bx & 7);
  if (c >= p.n_chunks) return;
  const int kvh = grp / p.row_tiles, rt = grp % p.row_tiles;

  int chunk, t0, t1, b, cu;
  if (!plan_share(p.seqlens, p.B, p.n_chunks, c, s_plan, chunk, t0, t1, b, cu)) return;

  const bf16 *__restrict__ qn = static_cast<const bf16 *>(p.q);
  const bf16 *__restrict__ qr_ = static_cast<const bf16 *>(p.q_rope);
  const bf16 *__restrict__ kc = static_cast<const bf16 *>(p.k) + (long long)kvh * DK;
  const bf16 *__restrict__ rc = static_cast<const bf16 *>(p.r);
  const bf16 *__restrict__ vc = static_cast<const bf16 *>(p.v) + (long long)kvh * DV;
  const int tk0 = tid >> 3, tk1 = tk0 + 32, cl = tid & 7;

  while (cu < t1) {
    const int L = p.seqlens[b];
    const int nb = seq_tiles(L);
    const int lt0 = max(cu, t0) - cu, lt1 = min(cu + nb, t1) - cu;
    const int c_first = cu / chunk, c_last = (cu + nb - 1) / chunk;
    const bool whole = c_first == c_last;
    const int slot = b + c;
    if (c == c_first && grp == 0 && tid == 0) {
      p.meta[2 * b] = b + c_first;
      p.meta[2 * b + 1] = c_last - c_first + 1;
    }
    const int32_t *bt = p.block_table + (long long)b * p.max_pages;

    // ---- the query rows of this work-group
    int lim[NT], rowid[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const int r = rt * ROWS + 16 * nt + n;
      if (r < p.rows_per_kvh) {
        const int t = r / p.hpk, h = kvh * p.hpk + r % p.hpk;
        lim[nt] = p.causal ? L - p.s_q + t + 1 : L;
        rowid[nt] = (b * p.s_q + t) * p.h_q + h;
      } else {
        lim[nt] = 0;
        rowid[nt] = -1;
      }
    }
    bf16x8 qreg[KS][NT];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        bf16x8 v = {};
        if (rowid[nt] >= 0) {
          const bf16 *src = ks < C::KSN ? qn + (long long)rowid[nt] * DK + 32 * ks + 8 * g
                                        : qr_ + (long long)rowid[nt] * DR + 32 * (ks - C::KSN) + 8 * g;
          v = *reinterpret_cast<const bf16x8 *>(src);
        }
        qreg[ks][nt] = v;
      }

    f32x4 oacc[MT][NT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) oacc[mt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_run[NT], l_part[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      m_run[nt] = neg_inf();
      l_part[nt] = 0.f;
    }

    // cache row of token tk of tile `tile`, -1 past the sequence
    auto token_row = [&](int tile, int tk) -> int {
      const int j = tile * kTile + tk;
      if (j >= L) return -1;
      int pg, sl;
      if (p.page_shift >= 0) {
        pg = bt[j >> p.page_shift];
        sl = j & (p.page_size - 1);
      } else {
        pg = bt[j / p.page_size];
        sl = j % p.page_size;
      }
      return pg * p.page_size + sl;
    };

    u32x4 pre[C::NLD];
    auto load_tile = [&](int r0, int r1) {
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int row = u ? r1 : r0;
#pragma unroll
        for (int k = 0; k < C::KC8; ++k) {
          const int ch = cl + 8 * k;
          u32x4 v = {0u, 0u, 0u, 0u};
          if (row >= 0) {
            const bf16 *src = ch < DK / 8 ? kc + (long long)row * p.k_stride + 8 * ch
                                          : rc + (long long)row * p.r_stride + 8 * (ch - DK / 8);
            v = *reinterpret_cast<const u32x4 *>(src);
          }
          pre[u * (C::KC8 + C::VC8) + k] = v;
        }
#pragma unroll
        for (int k = 0; k < C::VC8; ++k) {
          const int ch = cl + 8 * k;
          u32x4 v = {0u, 0u, 0u, 0u};
          if (row >= 0) v = *reinterpret_cast<const u32x4 *>(vc + (long long)row * p.v_stride + 8 * ch);
          pre[u * (C::KC8 + C::VC8) + C::KC8 + k] = v;
        }
      }
    };
    auto store_tile = [&](int bi) {
      bf16 *kt = s_buf + bi * C::BUF;
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int tok = u ? tk1 : tk0;
#pragma unroll
        for (int k = 0; k < C::KC8; ++k) {
          const int ch = cl + 8 * k;
          *reinterpret_cast<u32x4 *>(kt + tok * C::KSTR + swz(ch, tok) * 8) =
              pre[u * (C::KC8 + C::VC8) + k];
        }
#pragma unroll
        for (int k = 0; k < C::VC8; ++k) {
          const int ch = cl + 8 * k;
          *reinterpret_cast<u32x4 *>(kt + C::KTILE + tok * C::VSTR + swz(ch, tok) * 8) =
              pre[u * (C::KC8 + C::VC8) + C::KC8 + k];
        }
      }
    };

    // ---- pipeline prologue
    load_tile(token_row(lt0, tk0), token_row(lt0, tk1));
    store_tile(0);
    int nx0 = -1, nx1 = -1;
    if (lt0 + 1 < lt1) {
      nx0 = token_row(lt0 + 1, tk0);
      nx1 = token_row(lt0 + 1, tk1);
    }
    __syncthreads();

    for (int it = lt0; it < lt1; ++it) {
      const int bi = (it - lt0) & 1;
      const bool has_next = it + 1 < lt1;
      if (has_next) load_tile(nx0, nx1);
      int nn0 = -1, nn1 = -1;
      if (it + 2 < lt1) {
        nn0 = token_row(it + 2, tk0);
        nn1 = token_row(it + 2, tk1);
      }
      const bf16 *kt = s_buf + bi * C::BUF;

      // ---- S^T = K Q^T for tokens 16w..16w+15
      f32x4 sacc[NT];
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) sacc[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
      {
        const int tok = 16 * w + n;
        const bf16 *krow = kt + tok * C::KSTR;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const bf16x8 a = *reinterpret_cast<const bf16x8 *>(krow + swz(4 * ks + g, tok) * 8);
#pragma unroll
          for (int nt = 0; nt < NT; ++nt)
            sacc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qreg[ks][nt], sacc[nt], 0, 0, 0);
        }
      }

      // ---- mask, tile maximum
      const int tokb = it * kTile + 16 * w + 4 * g;
      float x[NT][4];
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        float mx = neg_inf();
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          x[nt][i] = (tokb + i < lim[nt]) ? sacc[nt][i] * p.scale_log2 : neg_inf();
          mx = fmaxf(mx, x[nt][i]);
        }
        mx = fmaxf(mx, __shfl_xor(mx, 16));
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        if (g == 0) s_red[w * ROWS + 16 * nt + n] = mx;
      }
      __syncthreads();

      // ---- online softmax, P^T -> LDS (bf16)
      float alpha[NT];
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        float mt = s_red[16 * nt + n];
#pragma unroll
        for (int v = 1; v < kWaves; ++v) mt = fmaxf(mt, s_red[v * ROWS + 16 * nt + n]);
        const float mnew = fmaxf(m_run[nt], mt);
        const float muse = mnew == neg_inf() ? 0.f : mnew;
        alpha[nt] = __builtin_amdgcn_exp2f(m_run[nt] - muse);
        m_run[nt] = mnew;
        bf16x4 pv;
        float sum = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float e = __builtin_amdgcn_exp2f(x[nt][i] - muse);
          sum += e;
          pv[i] = static_cast<bf16>(e);
        }
        l_part[nt] = l_part[nt] * alpha[nt] + sum;
        *reinterpret_cast<bf16x4 *>(s_p + (16 * nt + n) * C::PSTR + 16 * w + 4 * g) = pv;
      }
      __syncthreads();

      // ---- O^T = V^T P^T on this wave's value columns
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) oacc[mt][nt] *= alpha[nt];
      const bf16 *vt = VA ? kt : kt + C::KTILE;
#pragma unroll
      for (int k2 = 0; k2 < 2; ++k2) {
        bf16x8 pb[NT];
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
          pb[nt] = *reinterpret_cast<const bf16x8 *>(s_p + (16 * nt + n) * C::PSTR + 32 * k2 + 8 * g);
        const int rv = 32 * k2 + 8 * g + (n >> 2);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          const int dim = w * C::DVW + 16 * mt + 4 * (n & 3);
          const int ch = dim >> 3, off = dim & 7;
          const s16x4 lo = lds_read_tr(vt + rv * C::VSTR + swz(ch, rv) * 8 + off);
          const s16x4 hi = lds_read_tr(vt + (rv + 4) * C::VSTR + swz(ch, rv + 4) * 8 + off);
          const bf16x8 a = join(lo, hi);
#pragma unroll
          for (int nt = 0; nt < NT; ++nt)
            oacc[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pb[nt], oacc[mt][nt], 0, 0, 0);
        }
      }
      if (has_next) store_tile(bi ^ 1);
      nx0 = nn0;
      nx1 = nn1;
      __syncthreads();
    }

    // ---- row sums over lanes and waves, finalize
    float inv[NT], lse_nat[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      float v = l_part[nt];
      v += __shfl_xor(v, 16);
      v += __shfl_xor(v, 32);
      if (g == 0) s_red[w * ROWS + 16 * nt + n] = v;
    }
    __syncthreads();
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      float lt = 0.f;
#pragma unroll
      for (int v = 0; v < kWaves; ++v) lt += s_red[v * ROWS + 16 * nt + n];
      inv[nt] = lt > 0.f ? 1.f / lt : 0.f;
      lse_nat[nt] = lt > 0.f ? (m_run[nt] + __log2f(lt)) * kLn2 : neg_inf();
    }
    __syncthreads();

#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      if (rowid[nt] < 0) continue;
      if (whole) {
        bf16 *out = static_cast<bf16 *>(p.out) + (long long)rowid[nt] * DV;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          bf16x4 o;
#pragma unroll
          for (int i = 0; i < 4; ++i) o[i] = static_cast<bf16>(oacc[mt][nt][i] * inv[nt]);
          *reinterpret_cast<bf16x4 *>(out + w * C::DVW + 16 * mt + 4 * g) = o;
        }
        if (p.lse && w == 0 && g == 0) p.lse[rowid[nt]] = lse_nat[nt];
      } else {
        const long long prow = rowid[nt] + (long long)(slot - b) * p.s_q * p.h_q;
        float *op = p.o_part + prow * DV;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
          *reinterpret_cast<f32x4 *>(op + w * C::DVW + 16 * mt + 4 * g) = oacc[mt][nt] * inv[nt];
        if (w == 0 && g == 0) p.lse_part[prow] = lse_nat[nt];
      }
    }
    cu += nb;
    ++b;
  }
}

template <int DK, int DR, int DV, bool VA, int ROWS>
hipError_t launch(const DecodeParams &p, hipStream_t s) {
  const int G = p.n_kvh * p.row_tiles;
  const int cpad = (p.n_chunks + 7) / 8 * 8;
  hipLaunchKernelGGL((mfma_decode_kernel<DK, DR, DV, VA, ROWS>), dim3(G * cpad), dim3(kThreads), 0, s, p);
  return hipGetLastError();
}

template <int DK, int DR, int DV, bool VA>
hipError_t launch_rows(const DecodeParams &p, int rows, hipStream_t s) {
  return rows == 16 ? launch<DK, DR, DV, VA, 16>(p, s) : launch<DK, DR, DV, VA, 32>(p, s);
}

}  // namespace

int mfma_decode_rows(int rows_per_kvh) { return rows_per_kvh <= 16 ? 16 : 32; }

// Compiled (dk, dr, dv, latent-is-value) instantiations.
#define LKV_MFMA_VARIANTS(X)   \
  X(512, 64, 512, true)        \
  X(256, 64, 256, true)        \
  X(128, 64, 128, true)        \
  X(512, 0, 512, true)         \
  X(128, 64, 128, false)       \
  X(128, 0, 128, false)        \
  X(64, 0, 64, false)          \
  X(256, 0, 256, false)

bool mfma_decode_supported(int dk, int dr, int dv, bool v_alias, int) {
#define LKV_SUP(DK, DR, DV, VA) \
  if (dk == DK && dr == DR && dv == DV && v_alias == VA) return true;
  LKV_MFMA_VARIANTS(LKV_SUP)
#undef LKV_SUP
  return false;
}

hipError_t launch_mfma_decode(const DecodeParams &p, bool v_alias, int rows, hipStream_t s) {
#define LKV_DISPATCH(DK, DR, DV, VA) \
  if (p.dk == DK && p.dr == DR && p.dv == DV && v_alias == VA) return launch_rows<DK, DR, DV, VA>(p, rows, s);
  LKV_MFMA_VARIANTS(LKV_DISPATCH)
#undef LKV_DISPATCH
  return hipErrorInvalidValue;
}

}  // namespace lkv
