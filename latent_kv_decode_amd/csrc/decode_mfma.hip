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
// With an 8-bit cache (F8: OCP E4M3 codes with one dequantisation scale) the
// next tile goes through registers instead (coalesced 16-byte loads of the
// codes), is converted to bf16 with v_cvt_pk_f32_fp8 -- every E4M3 value is
// exact in bf16 -- and written into the same swizzled tile layout at the end
// of the step; the scale is folded into the softmax scale and the output
// normalisation.  The products are unchanged.
#include <type_traits>

#include "e4m3.h"
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

// LDS swizzle.  The LDS has 64 banks of 4 bytes: a b128 read is served 16
// lanes per cycle and a b64 transpose read 32 lanes per cycle, 256 bytes each.
// Chunk `chunk` (16 bytes) of row `row` of a region with CPR chunks per row
// lives at chunk slot swz<CPR>(chunk, row):
//   CPR >= 16: chunk ^ h(row), h a bijection of row mod 16 with
//              h = 2*(row mod 4) + 8*bit3(row) + bit2(row).  Sixteen
//              consecutive rows reading one chunk hit sixteen different
//              256-byte bank slots, and the transpose read (rows r..r+3 and
//              r+8..r+11, a pair of chunks each) does too.
//   CPR == 8:  chunk ^ ((row / 2) mod 8): two 128-byte rows share a bank
//              window, so the XOR follows the row pair index.
// Row lengths are multiples of 256 bytes (CPR >= 16) or exactly 128 bytes.
template <int CPR>
__device__ __forceinline__ int swz(int chunk, int row) {
  static_assert(CPR == 8 || CPR % 16 == 0, "region row length");
  if constexpr (CPR >= 16) return chunk ^ (((row & 3) << 1) | (row & 8) | ((row >> 2) & 1));
  else return chunk ^ ((row >> 1) & 7);
}

// Direct global -> LDS staging of one tile region (64 tokens x CPT 16-byte
// chunks).  One wave instruction fills 1 KiB of LDS (64 lanes x 16 bytes, in
// lane order) with 64 / CPT whole token rows; lane i fetches the chunk whose
// swizzled slot is i, so the XOR layout costs nothing at store time.
// row_reg: lane t holds the cache row of token t of the tile.
template <int CPT, int AUX = 0>
__device__ __forceinline__ void dma_region(const bf16 *gbase, long long stride, bf16 *region,
                                           int row_reg, int w, int lane) {
  static_assert(CPT >= 8 && CPT <= 64 && CPT % 8 == 0, "chunks per token");
  constexpr int TPI = 64 / CPT;
#pragma unroll
  for (int u = 0; u < CPT / 4; ++u) {
    const int t0 = (u * 4 + w) * TPI;
    int tok, row;
    if constexpr (CPT == 64) {
      tok = t0;
      row = __builtin_amdgcn_readlane(row_reg, t0);
    } else {
      tok = t0 + lane / CPT;
      row = __shfl(row_reg, tok);
    }
    const int ch = swz<CPT>(lane % CPT, tok);
    const bf16 *src = gbase + (long long)row * stride + ch * 8;
    __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void *)(region + t0 * CPT * 8),
                                     16, 0, AUX);
  }
}

// As dma_region, for a tile whose token t sits at row base + t (whole tile on
// one page).  Addresses are a wave-uniform 64-bit base (scalar registers)
// plus a per-lane 32-bit byte offset that depends only on the parity of the
// instruction index, so the loop issues loads with no per-load vector math.
//   wu    wave index, known uniform
//   loff  per-lane byte offsets for even / odd instruction index
template <int CPT>
struct ContigDma {
  static constexpr int TPI = 64 / CPT;
  int loff[4];  // by instruction index mod 4 (the swizzle sees row mod 16)
  __device__ __forceinline__ void init(long long stride, int wu, int lane) {
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int t0 = (4 * v + wu) * TPI;
      const int tin = lane / CPT, tok = t0 + tin;
      loff[v] = tin * (int)stride * 2 + swz<CPT>(lane % CPT, tok) * 16;
    }
  }
  template <int AUX = 0>
  __device__ __forceinline__ void issue(const bf16 *base, long long stride, bf16 *region, int wu) const {
    const char *bw = reinterpret_cast<const char *>(base) + (long long)(wu * TPI) * stride * 2;
    bf16 *rw = region + wu * TPI * CPT * 8;
#pragma unroll
    for (int u = 0; u < CPT / 4; ++u) {
      const char *src = bw + (long long)(4 * u * TPI) * stride * 2 + loff[u & 3];
      __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void *)(rw + 4 * u * TPI * CPT * 8),
                                       16, 0, AUX);
    }
  }
};

// Cross-lane partners l ^ 16 and l ^ 32 through the gfx950 permlane swaps
// (VALU, no LDS round trip).
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
  return __uint_as_float(r[0]) + __uint_as_float(r[1]) - v;
}
__device__ __forceinline__ float xlane_sum32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]) - v;
}

// The softmax reference maximum moves only when a tile's maximum exceeds it by
// more than this (base-2 units), so O and the row sums are rescaled rarely;
// probabilities stay below 2^kLazy, well inside fp32 and bf16 range.
constexpr float kLazy = 8.0f;

// s_waitcnt vmcnt(0): every direct-to-LDS load of this wave has landed.
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Work-group barrier inside a tile step.  __syncthreads() also fences global
// memory, and that fence waits for every load in flight -- here the next
// tile's prefetch, which would then be exposed at every step.  This one
// retires the wave's LDS accesses (lgkmcnt 0) and meets at s_barrier; the
// empty asm statements keep the compiler from moving LDS accesses across it.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

__device__ __forceinline__ s16x4 lds_read_tr(const bf16 *p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4 *)(p));
}

__device__ __forceinline__ bf16x8 join(s16x4 lo, s16x4 hi) {
  s16x8 v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, v);
}

typedef e4m3_u32x2 u32x2;
__device__ __forceinline__ bf16x8 e4m3x8_to_bf16x8(unsigned w0, unsigned w1) {
  return __builtin_bit_cast(bf16x8, e4m3x8_to_bf16x8_bits(w0, w1));
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
  static_assert(DK % 64 == 0 && DR % 64 == 0 && DV % 64 == 0, "widths must be multiples of 64");
  static_assert(!VA || DV == DK, "the latent is the value");
  // LDS tile buffer: key main part [64][DK] and, for separate values,
  // [64][DV]; every region row is a multiple of 128 bytes.  The RoPE key
  // fragments go from memory straight to registers (each lane's share of
  // them is one contiguous 16-byte piece per k-step), which keeps the
  // buffers small enough for two work-groups per CU where that matters.
  static constexpr int VOFF = kTile * DK;                // value region offset
  static constexpr int VSTR = DV;
  static constexpr int BUF = VOFF + (VA ? 0 : kTile * DV);
  static constexpr int KS = KW / 32;                     // k-steps of QK^T
  static constexpr int KSN = DK / 32;                    // of which on the main part
  static constexpr int KSR = DR / 32;                    // and on the RoPE key
  static constexpr int NT = ROWS / 16;
  static constexpr int DVW = DV / kWaves;
  static constexpr int MT = DVW / 16;
  static constexpr int PSTR = kTile + 8;                 // P row stride (elements)
  static constexpr int LDS_BYTES = 2 * BUF * 2 + ROWS * PSTR * 2 + kWaves * ROWS * 4 + 64;
  static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");
};

template <int DK, int DR, int DV, bool VA, int ROWS, bool F8>
__global__ void __launch_bounds__(kThreads, 1) mfma_decode_kernel(const DecodeParams p) {
  using C = Cfg<DK, DR, DV, VA, ROWS>;
  constexpr int NT = C::NT, MT = C::MT, KS = C::KS;
  // two tile buffers as distinct LDS objects: the compiler can then prove
  // that direct-to-LDS loads into one never alias reads of the other and
  // keeps the prefetch in flight across the whole tile
  __shared__ __attribute__((aligned(16))) bf16 s_buf0[C::BUF];
  __shared__ __attribute__((aligned(16))) bf16 s_buf1[C::BUF];
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
  // 8-bit cache: one byte per element
  const char *__restrict__ kc8 = static_cast<const char *>(p.k) + (long long)kvh * DK;
  const char *__restrict__ rc8 = static_cast<const char *>(p.r);
  const char *__restrict__ vc8 = static_cast<const char *>(p.v) + (long long)kvh * DV;
  // a 64-token tile never straddles a page when pages are a power of two >= 64
  const bool aligned_pages = p.page_shift >= 6;
  // a row group with one row tile reads each key/value tile once: those
  // loads stream (non-temporal), leaving the cache to what several
  // work-groups read (the shared RoPE key)
  const bool stream_kv = p.row_tiles == 1;
  const int wu = __builtin_amdgcn_readfirstlane(w);
  ContigDma<DK / 8> dk_;
  ContigDma<DV / 8> dv_;
  dk_.init(p.k_stride, wu, lane);
  if constexpr (!VA) dv_.init(p.v_stride, wu, lane);

  // Per-lane LDS element offsets of the fragment reads; the rest of each
  // address is a compile-time immediate.
  //  key (QK^T A operand): row tok = 16w + n, chunk 4ks + g.  The swizzle
  //    changes the low four chunk bits only, so the slot is
  //    16*(ks/4) + ((4*(ks%4) + g) ^ h(tok)).
  int koff[4];
  {
    const int tok = 16 * w + n;
#pragma unroll
    for (int e = 0; e < 4; ++e) koff[e] = tok * DK + swz<DK / 8>(4 * e + g, tok) * 8;
  }
  //  value (transpose read): rows rv = 8g + n/4 (+4), value column block mt of
  //    this wave -> chunk w*DVW/8 + 2mt + (n%4)/2, element (n%2)*4
  int voff[2][MT];
  {
#pragma unroll
    for (int hlf = 0; hlf < 2; ++hlf) {
      const int rv = 8 * g + (n >> 2) + 4 * hlf;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const int ch = w * C::DVW / 8 + 2 * mt + ((n & 3) >> 1);
        voff[hlf][mt] = rv * C::VSTR + swz<DV / 8>(ch, rv) * 8 + 4 * (n & 1);
      }
    }
  }

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

    // ---- the query rows of this work-group.  Padded rows (past the last
    // query row) compute on a zero query and are never written.
    int lim[NT], rowid[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const int r = rt * ROWS + 16 * nt + n;
      if (r < p.rows_per_kvh) {
        const int t = r / p.hpk, h = kvh * p.hpk + r % p.hpk;
        lim[nt] = p.causal ? L - p.s_q + t + 1 : L;
        rowid[nt] = (b * p.s_q + t) * p.h_q + h;
      } else {
        lim[nt] = L;
        rowid[nt] = -1;
      }
    }
    // every row of the work-group sees at least lim_min tokens: tiles below
    // it need no mask
    const int lim_min = p.causal ? L - p.s_q + (rt * ROWS) / p.hpk + 1 : L;
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
    // m_run: the reference maximum (base 2) of each row; probabilities are
    // exp2(x - m_run) and may exceed 1 by up to 2^kLazy before O and the
    // sums are rescaled to a new reference.
    float m_run[NT], l_part[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      m_run[nt] = neg_inf();
      l_part[nt] = 0.f;
    }

    // Block-table window: lane i of every wave holds the page id of logical
    // page win + i of this sequence (-1 past its last page).  It is refilled
    // only at the top of an iteration, when no tile load is in flight.
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
        // wait here, on the refill path only: the compiler would otherwise
        // wait at the join after this branch, on every tile
        wait_vmem();
      }
    };
    const int row_first = L > 0 ? bt[0] * p.page_size : 0;

    // RoPE key fragments (QK^T A operand, k-steps KSN..KS-1) of this lane's
    // token 16w + n: the current tile's and the next one's (8-bit cache: the
    // next one's codes, converted when they become current)
    bf16x8 rcur[C::KSR > 0 ? C::KSR : 1], rnxt[C::KSR > 0 ? C::KSR : 1];
    u32x2 rraw[C::KSR > 0 ? C::KSR : 1];
    auto load_rope = [&](long long row, bf16x8 *dst) {
#pragma unroll
      for (int e = 0; e < C::KSR; ++e) {
        if constexpr (F8)
          rraw[e] = *reinterpret_cast<const u32x2 *>(rc8 + row * p.r_stride + 32 * e + 8 * g);
        else
          dst[e] = *reinterpret_cast<const bf16x8 *>(rc + row * p.r_stride + 32 * e + 8 * g);
      }
    };
    auto rope_current = [&]() {
#pragma unroll
      for (int e = 0; e < C::KSR; ++e) {
        if constexpr (F8) rcur[e] = e4m3x8_to_bf16x8(rraw[e][0], rraw[e][1]);
        else rcur[e] = rnxt[e];
      }
    };

    // 8-bit cache: the next tile's codes, 16 per thread-piece; piece q (q =
    // tid + kThreads u) is chunk q mod (D/16) of token q / (D/16) of the key
    // region, then of the value region
    constexpr int NPK = kTile * DK / 16, NPV = VA ? 0 : kTile * DV / 16;
    constexpr int NPF = F8 ? (NPK + NPV) / kThreads : 1;
    static_assert(!F8 || (NPK % kThreads == 0 && NPV % kThreads == 0), "8-bit staging");
    u32x4 stg[NPF];
    auto piece = [&](int u, int &tok, int &c16) -> bool {  // true: key region
      const int q = tid + kThreads * u;
      const bool key = q < NPK;
      const int qq = key ? q : q - NPK, per = (key ? DK : DV) / 16;
      tok = qq / per;
      c16 = qq % per;
      return key;
    };
    auto load_tile8 = [&](long long row0, int rr) {
#pragma unroll
      for (int u = 0; u < NPF; ++u) {
        int tok, c16;
        const bool key = piece(u, tok, c16);
        const long long row = row0 >= 0 ? row0 + tok : (long long)__shfl(rr, tok);
        const char *src = key ? kc8 + row * p.k_stride : vc8 + row * p.v_stride;
        stg[u] = *reinterpret_cast<const u32x4 *>(src + 16 * c16);
      }
    };
    auto store_tile8 = [&](bf16 *buf) {
#pragma unroll
      for (int u = 0; u < NPF; ++u) {
        int tok, c16;
        const bool key = piece(u, tok, c16);
        const u32x4 lo = e4m3x8_to_bf16x8_bits(stg[u][0], stg[u][1]);
        const u32x4 hi = e4m3x8_to_bf16x8_bits(stg[u][2], stg[u][3]);
        bf16 *reg = key ? buf + tok * DK : buf + C::VOFF + tok * DV;
        if (key) {
          *reinterpret_cast<u32x4 *>(reg + swz<DK / 8>(2 * c16, tok) * 8) = lo;
          *reinterpret_cast<u32x4 *>(reg + swz<DK / 8>(2 * c16 + 1, tok) * 8) = hi;
        } else {
          *reinterpret_cast<u32x4 *>(reg + swz<DV / 8>(2 * c16, tok) * 8) = lo;
          *reinterpret_cast<u32x4 *>(reg + swz<DV / 8>(2 * c16 + 1, tok) * 8) = hi;
        }
      }
    };

    auto load_tile = [&](int tile, bf16 *buf, bf16x8 *rdst) {
      const int jb = tile * kTile;
      if (aligned_pages && jb + kTile <= L) {
        // whole tile valid and inside one page: token t sits at row row0 + t
        const int pi = jb >> p.page_shift;
        ensure_window(pi, pi);
        const int pg = __builtin_amdgcn_readlane(btw, pi - win);
        const long long row0 = (long long)pg * p.page_size + (jb & (p.page_size - 1));
        if constexpr (F8) {
          load_tile8(row0, 0);
        } else if (stream_kv) {
          dk_.template issue<2>(kc + row0 * p.k_stride, p.k_stride, buf, wu);
          if constexpr (!VA) dv_.template issue<2>(vc + row0 * p.v_stride, p.v_stride, buf + C::VOFF, wu);
        } else {
          dk_.issue(kc + row0 * p.k_stride, p.k_stride, buf, wu);
          if constexpr (!VA) dv_.issue(vc + row0 * p.v_stride, p.v_stride, buf + C::VOFF, wu);
        }
        if constexpr (DR > 0) load_rope(row0 + 16 * w + n, rdst);
      } else {
        // general path: lane t computes the row of token t; tokens past the
        // sequence read token 0's row (valid, finite; their weight is 0)
        ensure_window(page_of(jb), page_of(max(jb, min(jb + kTile, L) - 1)));
        const int j = jb + lane;
        const int pg = __shfl(btw, (page_of(j) - win) & 63);
        const int rr = j < L ? pg * p.page_size + slot_of(j) : row_first;
        if constexpr (F8) {
          load_tile8(-1, rr);
        } else if (stream_kv) {
          dma_region<DK / 8, 2>(kc, p.k_stride, buf, rr, w, lane);
          if constexpr (!VA) dma_region<DV / 8, 2>(vc, p.v_stride, buf + C::VOFF, rr, w, lane);
        } else {
          dma_region<DK / 8>(kc, p.k_stride, buf, rr, w, lane);
          if constexpr (!VA) dma_region<DV / 8>(vc, p.v_stride, buf + C::VOFF, rr, w, lane);
        }
        if constexpr (DR > 0) load_rope(__shfl(rr, 16 * w + n), rdst);
      }
    };

    // ---- pipeline prologue.  The wait also retires the query loads, so no
    // wait for them is left inside the tile loop (where it would drain the
    // prefetch of the next tile as well).
    if (L > 0) {
      load_tile(lt0, s_buf0, rnxt);
      wait_vmem();
      if constexpr (F8) store_tile8(s_buf0);
      rope_current();
    } else {
#pragma unroll
      for (int e = 0; e < C::KSR; ++e) rcur[e] = bf16x8{};
      wait_vmem();
      // empty sequence: one all-masked tile of zeros
      for (int i = tid; i < C::BUF / 8; i += kThreads)
        *reinterpret_cast<u32x4 *>(s_buf0 + 8 * i) = u32x4{0u, 0u, 0u, 0u};
    }
    // Make the compiler's wait for the query loads happen here, once per
    // sequence: an empty asm statement that reads every query register
    // forces it.  Otherwise the wait lands at the first MFMA inside the tile
    // loop, every tile, where it would also drain the prefetch of the next
    // tile.
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) asm volatile("" : "+v"(qreg[ks][nt]));
    __syncthreads();

    // one tile; BI (compile time) names the buffer it reads, the other one
    // receives the next tile
    auto step = [&](auto bi_tag, int it) {
      constexpr int BI = decltype(bi_tag)::value;
      bf16 *const kt = BI == 0 ? s_buf0 : s_buf1;
      bf16 *const nxt = BI == 0 ? s_buf1 : s_buf0;
      const bool has_next = it + 1 < lt1;
      if (has_next) load_tile(it + 1, nxt, rnxt);

      // ---- S^T = K Q^T for tokens 16w..16w+15; every key fragment is read
      // before the first MFMA so the LDS latency is paid once per tile
      f32x4 sacc[NT];
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) sacc[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
      {
        bf16x8 kf[KS];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          // chunk 4ks + g of row tok: slot 8(ks/2) + ((4(ks%2) + g) ^ sig)
          if (ks < C::KSN)
            kf[ks] = *reinterpret_cast<const bf16x8 *>(kt + koff[ks & 3] + 128 * (ks >> 2));
          else
            kf[ks] = rcur[ks - C::KSN];
        }
        __builtin_amdgcn_sched_group_barrier(0x100, KS, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, KS * NT, 0);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
#pragma unroll
          for (int nt = 0; nt < NT; ++nt)
            sacc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[ks], qreg[ks][nt], sacc[nt], 0, 0, 0);
      }

      // ---- scale, mask (only on tiles that cross a row's visible length),
      // tile maximum per row over this wave's 16 tokens
      float x[NT][4];
      const bool need_mask = (it + 1) * kTile > lim_min;
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int i = 0; i < 4; ++i) x[nt][i] = sacc[nt][i] * p.scale_log2;
      if (need_mask) {
        const int tokb = it * kTile + 16 * w + 4 * g;
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (tokb + i >= lim[nt]) x[nt][i] = neg_inf();
      }
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        float mx = fmaxf(fmaxf(x[nt][0], x[nt][1]), fmaxf(x[nt][2], x[nt][3]));
        mx = fmaxf(mx, xlane_max16(mx));
        mx = fmaxf(mx, xlane_max32(mx));
        if (g == 0) s_red[w * ROWS + 16 * nt + n] = mx;
      }
      lds_barrier();

      // ---- online softmax with a lazily moved reference maximum
      bool moved = false;
      float alpha[NT];
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        float mt = s_red[16 * nt + n];
#pragma unroll
        for (int v = 1; v < kWaves; ++v) mt = fmaxf(mt, s_red[v * ROWS + 16 * nt + n]);
        // move the reference only when this tile's maximum exceeds it by more
        // than kLazy (or it is still -inf); all waves decide alike per row
        alpha[nt] = 1.f;
        if (mt > m_run[nt] + kLazy) {
          alpha[nt] = __builtin_amdgcn_exp2f(m_run[nt] - mt);
          m_run[nt] = mt;
          moved = true;
        }
        const float muse = m_run[nt] == neg_inf() ? 0.f : m_run[nt];
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
      // rescale O only when some row of this wave moved its reference
      if (__builtin_amdgcn_ballot_w64(moved)) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) oacc[mt][nt] *= alpha[nt];
      }
      lds_barrier();

      // ---- O^T = V^T P^T on this wave's value columns
      const bf16 *vt = VA ? kt : kt + C::VOFF;
#pragma unroll
      for (int k2 = 0; k2 < 2; ++k2) {
        bf16x8 pb[NT];
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
          pb[nt] = *reinterpret_cast<const bf16x8 *>(s_p + (16 * nt + n) * C::PSTR + 32 * k2 + 8 * g);
        s16x4 vlo[MT], vhi[MT];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          // rows rv and rv + 4 (+32 per k2), chunk pair of value column block mt
          const int imm = 32 * k2 * C::VSTR;
          vlo[mt] = lds_read_tr(vt + voff[0][mt] + imm);
          vhi[mt] = lds_read_tr(vt + voff[1][mt] + imm);
        }
        __builtin_amdgcn_sched_group_barrier(0x100, NT + 2 * MT, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, MT * NT, 0);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          const bf16x8 a = join(vlo[mt], vhi[mt]);
#pragma unroll
          for (int nt = 0; nt < NT; ++nt)
            oacc[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pb[nt], oacc[mt][nt], 0, 0, 0);
        }
      }
      // unconditional: a wait that only some paths take would leave the
      // compiler assuming a load may still be in flight into the next step
      wait_vmem();
      if constexpr (F8) {
        if (has_next) store_tile8(nxt);
      }
      __syncthreads();
      rope_current();
    };
    for (int it = lt0; it < lt1; it += 2) {
      step(std::integral_constant<int, 0>{}, it);
      if (it + 1 < lt1) step(std::integral_constant<int, 1>{}, it + 1);
    }

    // ---- row sums over lanes and waves, finalize
    float inv[NT], lse_nat[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      float v = l_part[nt];
      v += xlane_sum16(v);
      v += xlane_sum32(v);
      if (g == 0) s_red[w * ROWS + 16 * nt + n] = v;
    }
    __syncthreads();
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      float lt = 0.f;
#pragma unroll
      for (int v = 0; v < kWaves; ++v) lt += s_red[v * ROWS + 16 * nt + n];
      inv[nt] = lt > 0.f ? p.out_scale / lt : 0.f;
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

template <int DK, int DR, int DV, bool VA, int ROWS, bool F8>
hipError_t launch(const DecodeParams &p, hipStream_t s, const LaunchEvents &ev) {
  const int G = p.n_kvh * p.row_tiles;
  const int cpad = (p.n_chunks + 7) / 8 * 8;
  return launch_timed(mfma_decode_kernel<DK, DR, DV, VA, ROWS, F8>, dim3(G * cpad), dim3(kThreads), s, ev, p);
}

template <int DK, int DR, int DV, bool VA, bool F8>
hipError_t launch_rows(const DecodeParams &p, int rows, hipStream_t s, const LaunchEvents &ev) {
  return rows == 16 ? launch<DK, DR, DV, VA, 16, F8>(p, s, ev) : launch<DK, DR, DV, VA, 32, F8>(p, s, ev);
}

// Work-groups of one instantiation resident on a CU at once (registers and
// LDS), queried once per instantiation; 1 if the query fails.
template <int DK, int DR, int DV, bool VA, int ROWS, bool F8>
int blocks_per_cu() {
  static int cached = 0;  // the same for every gfx950 device
  if (cached == 0) {
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, mfma_decode_kernel<DK, DR, DV, VA, ROWS, F8>, kThreads,
                                                     0) != hipSuccess ||
        n < 1)
      n = 1;
    cached = n;
  }
  return cached;
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
// ... and those with an 8-bit (E4M3) cache
#define LKV_MFMA_F8_VARIANTS(X) \
  X(512, 64, 512, true)         \
  X(256, 64, 256, true)         \
  X(128, 64, 128, true)         \
  X(128, 64, 128, false)        \
  X(128, 0, 128, false)

bool mfma_decode_supported(int dk, int dr, int dv, bool v_alias, bool fp8) {
#define LKV_SUP(DK, DR, DV, VA) \
  if (dk == DK && dr == DR && dv == DV && v_alias == VA) return true;
  if (fp8) {
    LKV_MFMA_F8_VARIANTS(LKV_SUP)
  } else {
    LKV_MFMA_VARIANTS(LKV_SUP)
  }
#undef LKV_SUP
  return false;
}

int mfma_decode_blocks_per_cu(int dk, int dr, int dv, bool v_alias, int rows, bool fp8) {
#define LKV_OCC(DK, DR, DV, VA, F8)                               \
  if (dk == DK && dr == DR && dv == DV && v_alias == VA)          \
    return rows == 16 ? blocks_per_cu<DK, DR, DV, VA, 16, F8>() : blocks_per_cu<DK, DR, DV, VA, 32, F8>();
#define LKV_OCC16(DK, DR, DV, VA) LKV_OCC(DK, DR, DV, VA, false)
#define LKV_OCC8(DK, DR, DV, VA) LKV_OCC(DK, DR, DV, VA, true)
  if (fp8) {
    LKV_MFMA_F8_VARIANTS(LKV_OCC8)
  } else {
    LKV_MFMA_VARIANTS(LKV_OCC16)
  }
#undef LKV_OCC8
#undef LKV_OCC16
#undef LKV_OCC
  return 1;
}

hipError_t launch_mfma_decode(const DecodeParams &p, bool v_alias, int rows, hipStream_t s,
                              const LaunchEvents &ev) {
#define LKV_DISPATCH(DK, DR, DV, VA, F8) \
  if (p.dk == DK && p.dr == DR && p.dv == DV && v_alias == VA) return launch_rows<DK, DR, DV, VA, F8>(p, rows, s, ev);
#define LKV_DISPATCH16(DK, DR, DV, VA) LKV_DISPATCH(DK, DR, DV, VA, false)
#define LKV_DISPATCH8(DK, DR, DV, VA) LKV_DISPATCH(DK, DR, DV, VA, true)
  if (p.fp8) {
    LKV_MFMA_F8_VARIANTS(LKV_DISPATCH8)
  } else {
    LKV_MFMA_VARIANTS(LKV_DISPATCH16)
  }
#undef LKV_DISPATCH8
#undef LKV_DISPATCH16
#undef LKV_DISPATCH
  return hipErrorInvalidValue;
}

}  // namespace lkv
