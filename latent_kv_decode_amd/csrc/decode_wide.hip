// decode_wide.hip -- MLA absorbed decode with many query rows of one latent
// head per work-group [GQLA explainer, technical summary section 2,
// MQA-absorbed path: every query head reads the one shared latent c_KV plus
// the shared RoPE key, and the latent is also the value].
//
// Why a second kernel.  When many query rows share one latent (128 heads x
// s_q), the rate at which one CU can pull tiles in (a few tens of GB/s) makes
// re-reading the same cache tiles from several work-groups expensive: every
// copy costs the CU ingest time.  Here a work-group owns 16 * NW rows (64 or
// 128) and reads each of its cache tiles once; split-KV shares over the
// concatenated tiles of the batch, merged by the LSE combine, fill the
// machine instead.
//
// Layout of the work.  NW waves; wave w owns rows 16w..16w+15 of the
// work-group outright: its query (16 rows x (d_c + d_rope), bf16) and its
// output accumulator (16 rows x d_c, fp32, transposed) stay in registers for
// the whole share.  Per 32-token half tile each wave computes S^T = K Q^T
// (A = key rows from LDS, B = query registers), an online softmax over its
// own rows (no cross-wave exchange), and O^T += V^T P^T, where P^T is taken
// straight from the S^T registers (the token order inside an MFMA k-step is
// chosen to match the S^T output layout) and V^T from the token-major tile
// through the LDS transpose read.  Tiles (64 tokens, two halves) are staged
// by direct-to-LDS loads into one of two buffers while the other is
// consumed; one barrier per 64 tokens.
#include <type_traits>

#include "lkv_internal.h"

namespace lkv {
namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short s16x4;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(4 * sizeof(unsigned)))) unsigned u32x4;
typedef __bf16 bf16;

constexpr int kHalf = 32;  // tokens per compute step
constexpr float kLn2 = 0.693147180559945309f;
// The softmax reference maximum moves only when a step's maximum exceeds it
// by more than this (base-2 units); probabilities stay below 2^kLazy.
constexpr float kLazy = 8.0f;

__device__ __forceinline__ float neg_inf() { return -__builtin_inff(); }

// LDS swizzle (64 banks of 4 bytes).  Chunk c (16 bytes) of row r of a
// region with CPR chunks per row sits at slot swz<CPR>(c, r):
//   CPR >= 16: c ^ h(r), h(r) = 2*(r mod 8) + bit3(r): sixteen consecutive
//              rows reading one chunk hit sixteen different 16-byte bank
//              groups, and eight consecutive rows reading a chunk pair (one
//              half of a transpose read) do too;
//   CPR == 8:  c ^ ((r / 2) mod 8) for 128-byte rows (two rows per 256 bytes).
template <int CPR>
__device__ __forceinline__ int swz(int c, int r) {
  static_assert(CPR == 8 || CPR % 16 == 0, "region row length");
  if constexpr (CPR >= 16) return c ^ (((r & 7) << 1) | ((r >> 3) & 1));
  else return c ^ ((r >> 1) & 7);
}

__device__ __forceinline__ s16x4 lds_read_tr(const bf16 *p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4 *)(p));
}
__device__ __forceinline__ bf16x8 join(s16x4 lo, s16x4 hi) {
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}
// s_waitcnt vmcnt(0): every direct-to-LDS load of this wave has landed.
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Reductions over the four 16-lane groups (partners l ^ 16 and l ^ 32).
__device__ __forceinline__ float xlane_max16(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xlane_max32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xlane_sum16(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float xlane_sum32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ int seq_tiles(int L) { return L <= 0 ? 1 : (L + kTile - 1) / kTile; }

// Split-KV plan, the same definition as the row-tiled kernel's: the
// concatenated 64-token tiles of all sequences (an empty sequence counts one
// tile) cut into n_chunks shares of ceil(total / n_chunks) tiles.  Returns
// false for an empty share; else the share's tile range and its first
// sequence with that sequence's first tile index.
template <int NTH>
__device__ bool plan_share(const int32_t *seqlens, int B, int C, int c, int *sh, int &chunk, int &t0,
                           int &t1, int &b0, int &cu0) {
  constexpr int NWV = NTH / 64;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int per = (B + NTH - 1) / NTH;
  const int s0 = min(B, tid * per), s1 = min(B, s0 + per);
  int local = 0;
  for (int b = s0; b < s1; ++b) local += seq_tiles(seqlens[b]);
  int v = local;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int u = __shfl_up(v, o);
    if (lane >= o) v += u;
  }
  if (lane == 63) sh[w] = v;
  __syncthreads();
  int before = 0, total = 0;
#pragma unroll
  for (int i = 0; i < NWV; ++i) {
    const int s = sh[i];
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
        sh[NWV] = b;
        sh[NWV + 1] = cu;
        break;
      }
      cu += nb;
    }
  }
  __syncthreads();
  b0 = sh[NWV];
  cu0 = sh[NWV + 1];
  return true;
}

template <int DK, int DR, int NW>
struct WCfg {
  static_assert(DK % 64 == 0 && DK >= 128 && DK <= 512 && (DR == 0 || DR == 64), "widths");
  static_assert(NW == 4 || NW == 8, "waves");
  static constexpr int NTH = 64 * NW;
  static constexpr int ROWS = 16 * NW;            // query rows per work-group
  static constexpr int KS = (DK + DR) / 32;       // QK^T k-steps
  static constexpr int KSN = DK / 32;             // of which on the latent
  static constexpr int MT = DK / 16;              // value column tiles (all of d_c)
  static constexpr int ROFF = kHalf * DK;         // RoPE region offset in a half buffer
  static constexpr int HALF = kHalf * (DK + DR);  // elements per half-tile buffer
  static constexpr int BUF = 2 * HALF;            // one 64-token tile
  static constexpr int NE = 16 / NW;              // distinct latent-load lane offsets
  static constexpr int LDS_BYTES = 2 * BUF * 2;
  static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");
};

// A wave-uniform pointer passed through readfirstlane: the opaque copy keeps
// the compiler from re-associating uniform base + lane offset into per-lane
// 64-bit pointers held across the loop (it selects the scalar-base form).
__device__ __forceinline__ const char *uniform_ptr(const char *p) {
  const unsigned long long v = reinterpret_cast<unsigned long long>(p);
  const unsigned lo = __builtin_amdgcn_readfirstlane(static_cast<unsigned>(v));
  const unsigned hi = __builtin_amdgcn_readfirstlane(static_cast<unsigned>(v >> 32));
  return reinterpret_cast<const char *>((static_cast<unsigned long long>(hi) << 32) | lo);
}

// Direct-to-LDS staging of one 64-token tile into `buf` (two halves): the
// latent rows (one token per wave instruction) and the RoPE rows (8 tokens
// per instruction).  Token t of the tile sits at cache row row0 + t when the
// whole tile lies on one page (CONTIG), else at row_reg of lane t.  Global
// addresses are a wave-uniform row base plus a per-lane 32-bit byte offset:
// lane l of the latent instruction for token t = NW*u + w fetches chunk
// swz(l, t mod 32) of the row, an offset that depends on u mod NE only
// (loff); lane l of a RoPE instruction fetches token l / 8 of its group of 8,
// chunk swz(l mod 8, row) (rloff when CONTIG).
template <int DK, int DR, int NW, bool CONTIG>
__device__ __forceinline__ void stage_tile(const char *kc, long long kstr, const char *rc, long long rstr,
                                           long long row0, int row_reg, bf16 *buf, int wu, int lane,
                                           const int (&loff)[WCfg<DK, DR, NW>::NE], int rloff) {
  using C = WCfg<DK, DR, NW>;
  constexpr int CPT = DK / 8;
#pragma unroll
  for (int u = 0; u < kTile / NW; ++u) {
    const int t = NW * u + wu;
    const long long row = CONTIG ? row0 + t : (long long)__builtin_amdgcn_readlane(row_reg, t);
    const char *base = uniform_ptr(kc + row * kstr);
    bf16 *dst = buf + (t >> 5) * C::HALF + (t & (kHalf - 1)) * DK;
    if (CPT == 64 || lane < CPT)
      __builtin_amdgcn_global_load_lds(base + static_cast<unsigned>(loff[u % C::NE]),
                                       (__attribute__((address_space(3))) void *)dst, 16, 0, 0);
  }
  if constexpr (DR > 0) {
    // 8 instructions of 8 tokens; wave w issues instructions w, w + NW, ...
#pragma unroll
    for (int u = 0; u < 8 / NW; ++u) {
      const int t0 = 8 * (NW * u + wu);
      bf16 *dst = buf + (t0 >> 5) * C::HALF + C::ROFF + (t0 & (kHalf - 1)) * DR;
      const char *src;
      if constexpr (CONTIG) {
        src = uniform_ptr(rc + (row0 + t0) * rstr) + static_cast<unsigned>(rloff);
      } else {
        const int r = (t0 & (kHalf - 1)) + (lane >> 3);
        const long long row = __shfl(row_reg, t0 + (lane >> 3));
        src = rc + row * rstr + swz<DR / 8>(lane & 7, r) * 16;
      }
      __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void *)dst, 16, 0, 0);
    }
  }
}

template <int DK, int DR, int NW>
__global__ void __launch_bounds__(64 * NW, 1) mla_wide_kernel(const DecodeParams p) {
  using C = WCfg<DK, DR, NW>;
  constexpr int KS = C::KS, KSN = C::KSN, MT = C::MT, NE = C::NE;
  // two tile buffers as distinct LDS objects, so that loads into one are
  // provably independent of reads of the other
  __shared__ __attribute__((aligned(16))) bf16 s_t0[C::BUF];
  __shared__ __attribute__((aligned(16))) bf16 s_t1[C::BUF];
  int *const s_plan = reinterpret_cast<int *>(s_t1);  // free until the first tile load

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int g = lane >> 4, n = lane & 15;
  const int wu = __builtin_amdgcn_readfirstlane(w);
  // An (empty) statement with an AGPR operand: it tells the compiler that
  // this kernel uses the accumulation registers, so it selects the MFMA forms
  // that keep the output accumulators there instead of spilling VGPRs to them.
  asm volatile("" ::"a"(0));

  // block -> (share, row group); the row groups of one share sit on one XCD
  const int G = p.n_kvh * p.row_tiles;
  const int bx = blockIdx.x;
  const int q8 = bx >> 3;
  const int grp = q8 % G;
  const int c = (q8 / G) * 8 + (bx & 7);
  if (c >= p.n_chunks) return;
  const int kvh = grp / p.row_tiles, rt = grp % p.row_tiles;

  int chunk, t0, t1, b, cu;
  if (!plan_share<C::NTH>(p.seqlens, p.B, p.n_chunks, c, s_plan, chunk, t0, t1, b, cu)) return;

  const bf16 *__restrict__ qn = static_cast<const bf16 *>(p.q);
  const bf16 *__restrict__ qr_ = static_cast<const bf16 *>(p.q_rope);
  const char *kcb = reinterpret_cast<const char *>(static_cast<const bf16 *>(p.k) + (long long)kvh * DK);
  const char *rcb = static_cast<const char *>(p.r);
  const long long kstr = p.k_stride * 2, rstr = p.r_stride * 2;
  const bool aligned_pages = p.page_shift >= 6;

  // per-lane LDS element offsets of the fragment reads within a half tile
  //  key A operand (token tile tt): row 16tt + n, chunk 4ks + g; the slot is
  //    16*(ks/4) + ((4*(ks%4) + g) ^ h(n)) (h depends on the row mod 16 only)
  int koff[4], roff[2];
#pragma unroll
  for (int e = 0; e < 4; ++e) koff[e] = n * DK + swz<DK / 8>(4 * e + g, n) * 8;
#pragma unroll
  for (int e = 0; e < 2; ++e) roff[e] = DR > 0 ? n * DR + swz<(DR > 0 ? DR : 64) / 8>(4 * e + g, n) * 8 : 0;
  //  value transpose read of column tile mt: lane (g, n) reads row 4g + n/4
  //    (and the same 16 rows on, with the same swizzle) at columns
  //    16mt + 4(n%4)..+3, i.e. chunk 2mt + (n%4)/2, element 4(n%2); the slot
  //    depends on mt mod 8 up to a multiple of 16 chunks
  int voff[8];
  {
    const int rv = 4 * g + (n >> 2);
#pragma unroll
    for (int j = 0; j < 8; ++j) voff[j] = rv * DK + swz<DK / 8>(2 * j + ((n & 3) >> 1), rv) * 8 + 4 * (n & 1);
  }
  // per-lane byte offsets of the tile loads (see stage_tile)
  int loff[NE], rloff = 0;
#pragma unroll
  for (int e = 0; e < NE; ++e) loff[e] = swz<DK / 8>(lane % (DK / 8), NW * e + wu) * 16;
  if constexpr (DR > 0)
    rloff = (int)((lane >> 3) * rstr) + swz<(DR > 0 ? DR : 64) / 8>(lane & 7, 8 * (wu & 3) + (lane >> 3)) * 16;

  while (cu < t1) {
    const int L = p.seqlens[b];
    const int nb = seq_tiles(L);
    const int lt0 = max(cu, t0) - cu, lt1 = min(cu + nb, t1) - cu;
    const int c_first = cu / chunk, c_last = (cu + nb - 1) / chunk;
    const bool whole = c_first == c_last;
    if (c == c_first && grp == 0 && tid == 0) {
      p.meta[2 * b] = b + c_first;
      p.meta[2 * b + 1] = c_last - c_first + 1;
    }
    const int32_t *bt = p.block_table + (long long)b * p.max_pages;

    // ---- this wave's 16 query rows (rows 16w.. of row tile rt)
    const int r_first = rt * C::ROWS + 16 * wu;
    const int r = r_first + n;
    int lim, rowid;
    if (r < p.rows_per_kvh) {
      const int t = r / p.hpk, h = kvh * p.hpk + r % p.hpk;
      lim = p.causal ? L - p.s_q + t + 1 : L;
      rowid = (b * p.s_q + t) * p.h_q + h;
    } else {
      lim = L;
      rowid = -1;
    }
    // every row of this wave sees at least lim_min tokens
    const int lim_min = p.causal ? L - p.s_q + r_first / p.hpk + 1 : L;
    bf16x8 qreg[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      bf16x8 v = {};
      if (rowid >= 0) {
        const bf16 *src = ks < KSN ? qn + (long long)rowid * DK + 32 * ks + 8 * g
                                   : qr_ + (long long)rowid * DR + 32 * (ks - KSN) + 8 * g;
        v = *reinterpret_cast<const bf16x8 *>(src);
      }
      qreg[ks] = v;
    }

    f32x4 oacc[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) oacc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_run = neg_inf(), l_part = 0.f;

    // block-table window (lane i: page id of logical page win + i)
    const int npages = L > 0 ? (L + p.page_size - 1) / p.page_size : 0;
    int win = -(1 << 30), btw = -1;
    auto page_of = [&](int j) -> int { return p.page_shift >= 0 ? j >> p.page_shift : j / p.page_size; };
    auto slot_of = [&](int j) -> int {
      return p.page_shift >= 0 ? j & (p.page_size - 1) : j % p.page_size;
    };
    auto ensure_window = [&](int lo, int hi) {
      if (lo < win || hi >= win + 64) {
        win = lo;
        btw = win + lane < npages ? bt[win + lane] : -1;
      }
    };
    const int row_first = L > 0 ? bt[0] * p.page_size : 0;
    auto load_tile = [&](int tile, bf16 *buf) __attribute__((always_inline)) {
      const int jb = tile * kTile;
      if (aligned_pages && jb + kTile <= L) {
        const int pi = jb >> p.page_shift;
        ensure_window(pi, pi);
        const int pg = __builtin_amdgcn_readlane(btw, pi - win);
        const long long row0 = (long long)pg * p.page_size + (jb & (p.page_size - 1));
        stage_tile<DK, DR, NW, true>(kcb, kstr, rcb, rstr, row0, 0, buf, wu, lane, loff, rloff);
      } else {
        ensure_window(page_of(jb), page_of(max(jb, min(jb + kTile, L) - 1)));
        const int j = jb + lane;
        const int pg = __shfl(btw, (page_of(j) - win) & 63);
        const int rr = j < L ? pg * p.page_size + slot_of(j) : row_first;
        stage_tile<DK, DR, NW, false>(kcb, kstr, rcb, rstr, 0, rr, buf, wu, lane, loff, rloff);
      }
    };

    // ---- prologue: first tile, and retire the query loads here (an empty
    // asm statement reading them keeps that wait out of the tile loop)
    if (L > 0) {
      load_tile(lt0, s_t0);
    } else {
      for (int i = tid; i < C::BUF / 8; i += C::NTH)
        *reinterpret_cast<u32x4 *>(s_t0 + 8 * i) = u32x4{0u, 0u, 0u, 0u};
    }
    wait_vmem();
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) asm volatile("" : "+v"(qreg[ks]));
    __syncthreads();

    // one 32-token half tile at `ht` of the current buffer, tokens jb..jb+31
    auto half_step = [&](const bf16 *ht, int jb) __attribute__((always_inline)) {
      // ---- S^T = K Q^T for token tiles tt = 0, 1 (16 tokens each); key
      // fragments are read PD k-steps ahead of their MFMAs
      constexpr int PD = 3;
      f32x4 sacc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
      bf16x8 kf[PD + 1][2];
      auto kload = [&](int ks, bf16x8 (&dst)[2]) __attribute__((always_inline)) {
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
          const bf16 *src = ks < KSN ? ht + 16 * tt * DK + koff[ks & 3] + 128 * (ks >> 2)
                                     : ht + C::ROFF + 16 * tt * DR + roff[(ks - KSN) & 1];
          dst[tt] = *reinterpret_cast<const bf16x8 *>(src);
        }
      };
#pragma unroll
      for (int ks = 0; ks < PD; ++ks) kload(ks, kf[ks]);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        if (ks + PD < KS) kload(ks + PD, kf[(ks + PD) % (PD + 1)]);
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
          sacc[tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[ks % (PD + 1)][tt], qreg[ks], sacc[tt], 0, 0, 0);
        // keep the reads PD k-steps ahead of their MFMAs (the scheduler would
        // otherwise pull them next to their use and expose the LDS latency)
        __builtin_amdgcn_sched_barrier(0);
      }

      // ---- online softmax over this wave's rows (base 2, lazy reference)
      float x[2][4];
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int i = 0; i < 4; ++i) x[tt][i] = sacc[tt][i] * p.scale_log2;
      if (jb + kHalf > lim_min) {
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (jb + 16 * tt + 4 * g + i >= lim) x[tt][i] = neg_inf();
      }
      float mx = neg_inf();
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int i = 0; i < 4; ++i) mx = fmaxf(mx, x[tt][i]);
      mx = xlane_max16(mx);
      mx = xlane_max32(mx);
      // `moved`: the row's reference maximum moves after it has contributed,
      // so its accumulated output takes the factor alpha
      float alpha = 1.f;
      bool moved = false;
      if (mx > m_run + kLazy) {
        alpha = __builtin_amdgcn_exp2f(m_run - mx);
        moved = m_run != neg_inf();
        m_run = mx;
      }
      const float muse = m_run == neg_inf() ? 0.f : m_run;
      float sum = 0.f;
      bf16x8 pb;
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float e = __builtin_amdgcn_exp2f(x[tt][i] - muse);
          sum += e;
          pb[4 * tt + i] = static_cast<bf16>(e);
        }
      l_part = l_part * alpha + sum;
      if (__builtin_amdgcn_ballot_w64(moved)) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) oacc[mt] *= alpha;
      }

      // ---- O^T += V^T P^T over all value columns (the value is the latent);
      // transpose reads run VD column tiles ahead of their MFMAs
      constexpr int VD = 4;
      bf16x8 va[VD + 1];
      auto vload = [&](int mt) __attribute__((always_inline)) {
        const bf16 *lo = ht + voff[mt & 7] + 128 * (mt >> 3);
        return join(lds_read_tr(lo), lds_read_tr(lo + 16 * DK));
      };
#pragma unroll
      for (int mt = 0; mt < VD; ++mt) va[mt] = vload(mt);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        if (mt + VD < MT) va[(mt + VD) % (VD + 1)] = vload(mt + VD);
        oacc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va[mt % (VD + 1)], pb, oacc[mt], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
    };

    auto step = [&](auto bi_tag, int it) __attribute__((always_inline)) {
      constexpr int BI = decltype(bi_tag)::value;
      bf16 *const cur = BI == 0 ? s_t0 : s_t1;
      bf16 *const nxt = BI == 0 ? s_t1 : s_t0;
      if (it + 1 < lt1) load_tile(it + 1, nxt);
      const int jb = it * kTile;
      // both halves unconditionally (a half past the end is fully masked and
      // adds nothing): straight-line code keeps the accumulators in place
      half_step(cur, jb);
      half_step(cur + C::HALF, jb + kHalf);
      wait_vmem();
      __syncthreads();
    };
    for (int it = lt0; it < lt1; it += 2) {
      step(std::integral_constant<int, 0>{}, it);
      if (it + 1 < lt1) step(std::integral_constant<int, 1>{}, it + 1);
    }

    // ---- finalize: row sum over the four lane groups, normalize, write
    float v = xlane_sum16(l_part);
    v = xlane_sum32(v);
    const float inv = v > 0.f ? 1.f / v : 0.f;
    const float lse_nat = v > 0.f ? (m_run + __log2f(v)) * kLn2 : neg_inf();
    if (rowid >= 0) {
      if (whole) {
        bf16 *out = static_cast<bf16 *>(p.out) + (long long)rowid * DK;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          bf16x4 o;
#pragma unroll
          for (int i = 0; i < 4; ++i) o[i] = static_cast<bf16>(oacc[mt][i] * inv);
          *reinterpret_cast<bf16x4 *>(out + 16 * mt + 4 * g) = o;
        }
        if (p.lse && g == 0) p.lse[rowid] = lse_nat;
      } else {
        // partial of share c for this sequence: slot b + c
        const long long prow = rowid + (long long)c * p.s_q * p.h_q;
        float *op = p.o_part + prow * DK;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) *reinterpret_cast<f32x4 *>(op + 16 * mt + 4 * g) = oacc[mt] * inv;
        if (g == 0) p.lse_part[prow] = lse_nat;
      }
    }
    // the buffers are reused by the next sequence of this share
    __syncthreads();
    cu += nb;
    ++b;
  }
}

template <int DK, int DR, int NW>
hipError_t launch_wide(const DecodeParams &p, hipStream_t s) {
  const int G = p.n_kvh * p.row_tiles;
  const int cpad = (p.n_chunks + 7) / 8 * 8;
  hipLaunchKernelGGL((mla_wide_kernel<DK, DR, NW>), dim3(G * cpad), dim3(64 * NW), 0, s, p);
  return hipGetLastError();
}

}  // namespace

bool mla_wide_supported(int dk, int dr) { return (dk == 512 || dk == 256) && (dr == 64 || dr == 0); }

int mla_wide_rows(int waves) { return 16 * waves; }

hipError_t launch_mla_wide(const DecodeParams &p, int waves, hipStream_t s) {
  if (waves != 4 && waves != 8) return hipErrorInvalidValue;
  const bool w8 = waves == 8;
  if (p.dk == 512 && p.dr == 64) return w8 ? launch_wide<512, 64, 8>(p, s) : launch_wide<512, 64, 4>(p, s);
  if (p.dk == 512 && p.dr == 0) return w8 ? launch_wide<512, 0, 8>(p, s) : launch_wide<512, 0, 4>(p, s);
  if (p.dk == 256 && p.dr == 64) return w8 ? launch_wide<256, 64, 8>(p, s) : launch_wide<256, 64, 4>(p, s);
  if (p.dk == 256 && p.dr == 0) return w8 ? launch_wide<256, 0, 8>(p, s) : launch_wide<256, 0, 4>(p, s);
  return hipErrorInvalidValue;
}

}  // namespace lkv
