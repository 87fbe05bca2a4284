// decode_wide.hip -- MLA absorbed decode with many query rows of one latent
// head per work-group [GQLA explainer, technical summary section 2,
// MQA-absorbed path: every query head reads the one shared latent c_KV plus
// the shared RoPE key, and the latent is also the value].
//
// Why a second kernel.  When many query rows share one latent (128 heads x
// s_q), a work-group that takes only a few of them makes every cache tile be
// fetched by several work-groups.  Here a work-group takes 64 * NT rows (64 or
// 128) and reads each of its cache tiles once; split-KV shares over the
// concatenated tiles of the batch, merged by the LSE combine, fill the
// machine instead.
//
// Layout of the work.  Four waves; wave w owns rows 16 NT w .. 16 NT w +
// 16 NT - 1 of the work-group outright: its query (bf16) and its output
// accumulator (fp32, transposed) stay in registers for the whole share (with
// NT = 2 the query's RoPE part sits in LDS).  Per 32-token half tile each
// wave computes S^T = K Q^T (A = key rows from LDS, B = query), an online
// softmax over its own rows (no cross-wave exchange), and O^T += V^T P^T,
// where P^T is taken straight from the S^T registers (the token order inside
// an MFMA k-step is chosen to match the S^T output layout) and V^T from the
// token-major tile through the LDS transpose read.  Each key or value
// fragment read from LDS feeds NT MFMAs, one per 16-row block.  Tiles (64
// tokens, two halves) are staged by direct-to-LDS buffer loads into one of
// two buffers while the other is consumed; one barrier per 64 tokens.
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

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kHalf = 32;  // tokens per compute step
constexpr float kLn2 = 0.693147180559945309f;
// The softmax reference maximum moves only when a step's maximum exceeds it
// by more than this (base-2 units); probabilities stay below 2^kLazy.
constexpr float kLazy = 8.0f;

__device__ __forceinline__ float neg_inf() { return -__builtin_inff(); }

// LDS swizzle.  The LDS serves 512 bytes per clock (128 banks of 4 bytes): a
// 16-byte read is served 32 lanes at a time, a transposing 8-byte read 64
// lanes at a time, so each such group must touch 32 different 16-byte slots
// of a 512-byte window.  Chunk c (16 bytes) of row r of a region with CPR
// chunks per row sits at slot swz<CPR>(c, r):
//   CPR >= 32 (rows of 512 or 1024 bytes, all rows on the same banks):
//     c ^ 2*(r mod 16).  A key read (lanes: 16 rows x 2 adjacent chunks) and
//     a value transpose read (16 rows x one chunk pair) then both cover 32
//     distinct slots;
//   CPR == 8 (128-byte RoPE rows, four rows per window): c ^ ((r / 2) mod 8).
template <int CPR>
__device__ __forceinline__ int swz(int c, int r) {
  static_assert(CPR == 8 || CPR == 32 || CPR == 64, "region row length");
  if constexpr (CPR >= 32) return c ^ ((r & 15) << 1);
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

// Multiply an MFMA accumulator tile by s in place, in the accumulation
// registers (AGPRs): the output accumulators stay there for the whole share,
// and this rare rescale must not bounce them through VGPRs.  The leading
// no-ops cover the wait states the hardware requires between an MFMA writing
// these registers and a VALU access to them (at most 19), the trailing ones
// those between a VALU write and an MFMA reading its accumulator input.
__device__ __forceinline__ void rescale_acc(f32x4 &acc, float s) {
  float a0 = acc[0], a1 = acc[1], a2 = acc[2], a3 = acc[3], t;
  asm volatile(
      "s_nop 15\n\ts_nop 15\n\t"
      "v_accvgpr_read_b32 %4, %0\n\tv_mul_f32 %4, %4, %5\n\tv_accvgpr_write_b32 %0, %4\n\t"
      "v_accvgpr_read_b32 %4, %1\n\tv_mul_f32 %4, %4, %5\n\tv_accvgpr_write_b32 %1, %4\n\t"
      "v_accvgpr_read_b32 %4, %2\n\tv_mul_f32 %4, %4, %5\n\tv_accvgpr_write_b32 %2, %4\n\t"
      "v_accvgpr_read_b32 %4, %3\n\tv_mul_f32 %4, %4, %5\n\tv_accvgpr_write_b32 %3, %4\n\t"
      "s_nop 7"
      : "+a"(a0), "+a"(a1), "+a"(a2), "+a"(a3), "=&v"(t)
      : "v"(s));
  acc = f32x4{a0, a1, a2, a3};
}

__device__ __forceinline__ int seq_tiles(int L) { return L <= 0 ? 1 : (L + kTile - 1) / kTile; }

// Split-KV plan, the same definition as the row-tiled kernel's: the
// concatenated 64-token tiles of all sequences (an empty sequence counts one
// tile) cut into n_chunks shares of ceil(total / n_chunks) tiles.  Returns
// false for an empty share; else the share's tile range and its first
// sequence with that sequence's first tile index.
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
    const int u = __shfl_up(v, o);
    if (lane >= o) v += u;
  }
  if (lane == 63) sh[w] = v;
  __syncthreads();
  int before = 0, total = 0;
#pragma unroll
  for (int i = 0; i < kWaves; ++i) {
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
        sh[kWaves] = b;
        sh[kWaves + 1] = cu;
        break;
      }
      cu += nb;
    }
  }
  __syncthreads();
  b0 = sh[kWaves];
  cu0 = sh[kWaves + 1];
  return true;
}

template <int DK, int DR, int NT>
struct WCfg {
  static_assert((DK == 512 || DK == 256) && (DR == 0 || DR == 64), "widths");
  static_assert(NT == 1 || NT == 2, "row blocks per wave");
  static constexpr int ROWS = 16 * NT * kWaves;   // query rows per work-group
  static constexpr int KS = (DK + DR) / 32;       // QK^T k-steps
  static constexpr int KSN = DK / 32;             // of which on the latent
  static constexpr int MT = DK / 16;              // value column tiles
  static constexpr int ROFF = kHalf * DK;         // RoPE region offset in a half buffer
  static constexpr int HALF = kHalf * (DK + DR);  // elements per half-tile buffer
  static constexpr int BUF = 2 * HALF;            // one 64-token tile
  static constexpr int NE = 16 / kWaves;          // distinct latent-load lane offsets
  // with two row blocks per wave the query's RoPE part lives in LDS
  static constexpr bool QRL = NT == 2 && DR > 0;
  static constexpr int QR = QRL ? ROWS * DR : 8;
  static constexpr int KQ = QRL ? KSN : KS;       // k-steps with the query in registers
  static constexpr int LDS_BYTES = (2 * BUF + (QRL ? QR : 0)) * 2;
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

// Direct-to-LDS loads go through raw buffer resources (buffer_load ... lds):
// with this MUBUF form the compiler keeps its waits on LDS reads exact while
// such loads are in flight (the FLAT-encoded global form makes it wait for
// every outstanding LDS read instead).  Dword 3 of the resource: 32-bit data
// format, no swizzle, no thread-id offset.
constexpr int kRsrcWord3 = 0x00020000;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const char *base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<char *>(uniform_ptr(base)), (short)0, 0x7fffffff,
                                           kRsrcWord3);
}
// 16 bytes per lane from base + voff + soff into dst + 16 * lane.
__device__ __forceinline__ void lds_dma16(__amdgpu_buffer_rsrc_t r, bf16 *dst, unsigned voff, unsigned soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void *)dst, 16, voff, soff, 0, 0);
}

template <int DK, int DR, int NT>
__global__ void __launch_bounds__(kThreads, 1) mla_wide_kernel(const DecodeParams p) {
  using C = WCfg<DK, DR, NT>;
  constexpr int KS = C::KS, KSN = C::KSN, MT = C::MT, NE = C::NE, KQ = C::KQ;
  constexpr int CPT = DK / 8;                  // 16-byte chunks per latent row
  constexpr int NL = kTile / kWaves, NR = DR > 0 ? 8 / kWaves : 0;
  constexpr int NI = NL + NR;                  // tile-load instructions per wave and tile
  // two tile buffers as distinct LDS objects, so that loads into one are
  // provably independent of reads of the other
  __shared__ __attribute__((aligned(16))) bf16 s_t0[C::BUF];
  __shared__ __attribute__((aligned(16))) bf16 s_t1[C::BUF];
  __shared__ __attribute__((aligned(16))) bf16 s_qr[C::QR];
  int *const s_plan = reinterpret_cast<int *>(s_t1);  // free until the first tile load

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int g = lane >> 4, n = lane & 15;
  const int wu = __builtin_amdgcn_readfirstlane(w);
  // An (empty) statement with an AGPR operand tells the compiler that this
  // kernel uses the accumulation registers, so it selects the MFMA forms
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
  if (!plan_share(p.seqlens, p.B, p.n_chunks, c, s_plan, chunk, t0, t1, b, cu)) return;

  const bf16 *__restrict__ qn = static_cast<const bf16 *>(p.q);
  const bf16 *__restrict__ qr_ = static_cast<const bf16 *>(p.q_rope);
  const char *kcb = reinterpret_cast<const char *>(static_cast<const bf16 *>(p.k) + (long long)kvh * DK);
  const char *rcb = static_cast<const char *>(p.r);
  const long long kstr = p.k_stride * 2, rstr = p.r_stride * 2;
  const bool aligned_pages = p.page_shift >= 6;

  // per-lane LDS element offsets of the fragment reads within a half tile
  //  key A operand (token tile tt): row 16tt + n, chunk 4ks + g; the slot is
  //    32*(ks/8) + ((4*(ks%8) + g) ^ 2n)
  int koff[8], roff[2], qoff[2];
#pragma unroll
  for (int e = 0; e < 8; ++e) koff[e] = n * DK + swz<CPT>(4 * e + g, n) * 8;
#pragma unroll
  for (int e = 0; e < 2; ++e) roff[e] = DR > 0 ? n * DR + swz<8>(4 * e + g, n) * 8 : 0;
  //  query RoPE B operand from LDS (row block nt: row 16 NT w + 16 nt + n,
  //    chunk 4e + g; the swizzle depends on the row mod 16 only)
#pragma unroll
  for (int e = 0; e < 2; ++e) qoff[e] = C::QRL ? n * DR + swz<8>(4 * e + g, n) * 8 : 0;
  //  value transpose read of column tile mt: lane (g, n) reads row 4g + n/4
  //    (and the same 16 rows on, same swizzle) at columns 16mt + 4(n%4)..+3,
  //    i.e. chunk 2mt + (n%4)/2, element 4(n%2); the slot is
  //    2(mt ^ row) + (n%4)/2 for mt mod 16, plus 32 chunks per 16 tiles
  int voff[16];
  {
    const int rv = 4 * g + (n >> 2);
#pragma unroll
    for (int j = 0; j < 16; ++j) voff[j] = rv * DK + swz<CPT>(2 * j + ((n & 3) >> 1), rv) * 8 + 4 * (n & 1);
  }
  // per-lane byte offsets of the tile loads: lane l of the latent instruction
  // for token t = 4u + w fetches chunk swz(l, t mod 32) of its row, an offset
  // that depends on u mod 4 only (loff); lane l of a RoPE instruction
  // fetches token l / 8 of its group of 8, chunk swz(l mod 8, row) (rloff)
  int loff[NE], rloff = 0;
#pragma unroll
  for (int e = 0; e < NE; ++e) loff[e] = swz<CPT>(lane % CPT, kWaves * e + wu) * 16;
  if constexpr (DR > 0) rloff = (int)((lane >> 3) * rstr) + swz<8>(lane & 7, 8 * wu + (lane >> 3)) * 16;

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

    // ---- this wave's 16 NT query rows
    const int r_first = rt * C::ROWS + 16 * NT * wu;
    int lim[NT], rowid[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const int r = r_first + 16 * nt + n;
      if (r < p.rows_per_kvh) {
        const int t = r / p.hpk, h = kvh * p.hpk + r % p.hpk;
        lim[nt] = p.causal ? L - p.s_q + t + 1 : L;
        rowid[nt] = (b * p.s_q + t) * p.h_q + h;
      } else {
        lim[nt] = L;
        rowid[nt] = -1;
      }
    }
    // every row of this wave sees at least lim_min tokens
    const int lim_min = p.causal ? L - p.s_q + r_first / p.hpk + 1 : L;
    bf16x8 qreg[KQ][NT];
#pragma unroll
    for (int ks = 0; ks < KQ; ++ks)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        bf16x8 v = {};
        if (rowid[nt] >= 0) {
          const bf16 *src = ks < KSN ? qn + (long long)rowid[nt] * DK + 32 * ks + 8 * g
                                     : qr_ + (long long)rowid[nt] * DR + 32 * (ks - KSN) + 8 * g;
          v = *reinterpret_cast<const bf16x8 *>(src);
        }
        qreg[ks][nt] = v;
      }
    if constexpr (C::QRL) {
      // the RoPE parts of the work-group's rows: row i at s_qr + i * DR,
      // chunk c at slot swz<8>(c, i); 8 lanes per row
      for (int i = tid; i < C::ROWS * (DR / 8); i += kThreads) {
        const int row = i / (DR / 8), ch = i % (DR / 8);
        const int r = rt * C::ROWS + row;
        u32x4 v = {0u, 0u, 0u, 0u};
        if (r < p.rows_per_kvh) {
          const int t = r / p.hpk, h = kvh * p.hpk + r % p.hpk;
          v = *reinterpret_cast<const u32x4 *>(qr_ + ((long long)(b * p.s_q + t) * p.h_q + h) * DR + 8 * ch);
        }
        *reinterpret_cast<u32x4 *>(s_qr + row * DR + swz<8>(ch, row) * 8) = v;
      }
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
    // Tile loads.  Wave w stages tokens w, w + 4, ... of a 64-token tile (one
    // latent row per instruction) and RoPE instructions w, w + 4 of 8 tokens
    // each.  When the whole tile lies on one page (mode 1) the loads use one
    // buffer resource per region at the tile's first row and are spread over
    // the compute of the previous tile (dma_issue(j), j < NI); otherwise
    // (mode 2) every token row gets its own resource and all loads are issued
    // at once.
    int dma_mode = 0;
    __amdgpu_buffer_rsrc_t rk = make_rsrc(kcb), rr = make_rsrc(rcb);
    int row_reg = 0;
    bf16 *dma_buf = s_t0;
    auto dma_prepare = [&](int tile, bf16 *buf) __attribute__((always_inline)) {
      const int jb = tile * kTile;
      dma_buf = buf;
      if (aligned_pages && jb + kTile <= L) {
        const int pi = jb >> p.page_shift;
        ensure_window(pi, pi);
        const int pg = __builtin_amdgcn_readlane(btw, pi - win);
        const long long row0 = (long long)pg * p.page_size + (jb & (p.page_size - 1));
        rk = make_rsrc(kcb + row0 * kstr);
        if constexpr (DR > 0) rr = make_rsrc(rcb + row0 * rstr);
        dma_mode = 1;
      } else {
        ensure_window(page_of(jb), page_of(max(jb, min(jb + kTile, L) - 1)));
        const int j = jb + lane;
        const int pg = __shfl(btw, (page_of(j) - win) & 63);
        row_reg = j < L ? pg * p.page_size + slot_of(j) : row_first;
        dma_mode = 2;
      }
    };
    auto dma_issue = [&](int j) __attribute__((always_inline)) {  // mode 1
      if (j < NL) {
        const int t = kWaves * j + wu;
        bf16 *dst = dma_buf + (t >> 5) * C::HALF + (t & (kHalf - 1)) * DK;
        if (CPT == 64 || lane < CPT)
          lds_dma16(rk, dst, static_cast<unsigned>(loff[j % NE]), static_cast<unsigned>(t * kstr));
      } else if constexpr (DR > 0) {
        const int t0r = 8 * (kWaves * (j - NL) + wu);
        bf16 *dst = dma_buf + (t0r >> 5) * C::HALF + C::ROFF + (t0r & (kHalf - 1)) * DR;
        lds_dma16(rr, dst, static_cast<unsigned>(rloff), static_cast<unsigned>(t0r * rstr));
      }
    };
    auto dma_all = [&]() __attribute__((always_inline)) {
      if (dma_mode == 1) {
#pragma unroll
        for (int j = 0; j < NI; ++j) dma_issue(j);
      } else {
#pragma unroll
        for (int u = 0; u < NL; ++u) {
          const int t = kWaves * u + wu;
          const long long row = __builtin_amdgcn_readlane(row_reg, t);
          bf16 *dst = dma_buf + (t >> 5) * C::HALF + (t & (kHalf - 1)) * DK;
          if (CPT == 64 || lane < CPT)
            lds_dma16(make_rsrc(kcb + row * kstr), dst, static_cast<unsigned>(loff[u % NE]), 0u);
          if constexpr (DR > 0) {
            bf16 *dr = dma_buf + (t >> 5) * C::HALF + C::ROFF + (t & (kHalf - 1)) * DR;
            if (lane < DR / 8)
              lds_dma16(make_rsrc(rcb + row * rstr), dr, static_cast<unsigned>(swz<8>(lane, t & (kHalf - 1)) * 16), 0u);
          }
        }
      }
    };

    // ---- prologue: first tile, and retire the query loads here (an empty
    // asm statement reading them keeps that wait out of the tile loop)
    if (L > 0) {
      dma_prepare(lt0, s_t0);
      dma_all();
    } else {
      for (int i = tid; i < C::BUF / 8; i += kThreads)
        *reinterpret_cast<u32x4 *>(s_t0 + 8 * i) = u32x4{0u, 0u, 0u, 0u};
    }
    wait_vmem();
#pragma unroll
    for (int ks = 0; ks < KQ; ++ks)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) asm volatile("" : "+v"(qreg[ks][nt]));
    __syncthreads();

    // issue slot s (one per k-step and per value column tile of each half)
    // spreads the next tile's mode-1 loads evenly over the tile's compute
    constexpr int NSLOT = 2 * (KS + MT);
    auto dma_slot = [&](int slot) __attribute__((always_inline)) {
      const int j0 = (slot * NI) / NSLOT, j1 = ((slot + 1) * NI) / NSLOT;
      if (j1 > j0 && dma_mode == 1) dma_issue(j0);
    };
    // the query fragment (B operand) of k-step ks, row block nt
    auto qfrag = [&](int ks, int nt) __attribute__((always_inline)) {
      if (!C::QRL || ks < KSN) return qreg[ks < KQ ? ks : 0][nt];
      return *reinterpret_cast<const bf16x8 *>(s_qr + (16 * NT * wu + 16 * nt) * DR + qoff[(ks - KSN) & 1]);
    };

    // one 32-token half tile at `ht` of the current buffer, tokens jb..jb+31
    auto half_step = [&](const bf16 *ht, int jb, int slot0) __attribute__((always_inline)) {
      // ---- S^T = K Q^T for token tiles tt = 0, 1 (16 tokens each); key
      // fragments are read PD k-steps ahead of their MFMAs, and the schedule
      // barriers keep every step in place (the scheduler would otherwise pull
      // the reads next to their use and expose the LDS latency)
      constexpr int PD = 2;
      f32x4 sacc[2][NT];
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) sacc[tt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
      bf16x8 kf[PD + 1][2];
      auto kload = [&](int ks, bf16x8 (&dst)[2]) __attribute__((always_inline)) {
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
          const bf16 *src = ks < KSN ? ht + 16 * tt * DK + koff[ks & 7] + 256 * (ks >> 3)
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
        for (int nt = 0; nt < NT; ++nt) {
          const bf16x8 q = qfrag(ks, nt);
#pragma unroll
          for (int tt = 0; tt < 2; ++tt)
            sacc[tt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[ks % (PD + 1)][tt], q, sacc[tt][nt], 0, 0, 0);
        }
        dma_slot(slot0 + ks);
        __builtin_amdgcn_sched_barrier(0);
      }

      // ---- online softmax per row block (base 2, lazy reference maximum)
      bool moved = false;
      float alpha[NT];
      bf16x8 pb[NT];
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        float x[2][4];
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
#pragma unroll
          for (int i = 0; i < 4; ++i) x[tt][i] = sacc[tt][nt][i] * p.scale_log2;
        if (jb + kHalf > lim_min) {
#pragma unroll
          for (int tt = 0; tt < 2; ++tt)
#pragma unroll
            for (int i = 0; i < 4; ++i)
              if (jb + 16 * tt + 4 * g + i >= lim[nt]) x[tt][i] = neg_inf();
        }
        float mx = neg_inf();
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
#pragma unroll
          for (int i = 0; i < 4; ++i) mx = fmaxf(mx, x[tt][i]);
        mx = xlane_max16(mx);
        mx = xlane_max32(mx);
        // `moved`: the row's reference maximum moves after it has
        // contributed, so its accumulated output takes the factor alpha
        alpha[nt] = 1.f;
        if (mx > m_run[nt] + kLazy) {
          alpha[nt] = __builtin_amdgcn_exp2f(m_run[nt] - mx);
          moved |= m_run[nt] != neg_inf();
          m_run[nt] = mx;
        }
        const float muse = m_run[nt] == neg_inf() ? 0.f : m_run[nt];
        float sum = 0.f;
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float e = __builtin_amdgcn_exp2f(x[tt][i] - muse);
            sum += e;
            pb[nt][4 * tt + i] = static_cast<bf16>(e);
          }
        l_part[nt] = l_part[nt] * alpha[nt] + sum;
      }
      if (__builtin_amdgcn_ballot_w64(moved)) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) {
            if constexpr (NT == 2) rescale_acc(oacc[mt][nt], alpha[nt]);
            else oacc[mt][nt] *= alpha[nt];
          }
      }

      // ---- O^T += V^T P^T over all value columns (the value is the latent);
      // transpose reads run VD column tiles ahead of their MFMAs
      constexpr int VD = 3;
      bf16x8 va[VD + 1];
      auto vload = [&](int mt) __attribute__((always_inline)) {
        const bf16 *lo = ht + voff[mt % 16] + 256 * (mt / 16);
        return join(lds_read_tr(lo), lds_read_tr(lo + 16 * DK));
      };
#pragma unroll
      for (int mt = 0; mt < VD; ++mt) va[mt] = vload(mt);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        if (mt + VD < MT) va[(mt + VD) % (VD + 1)] = vload(mt + VD);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
          oacc[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va[mt % (VD + 1)], pb[nt], oacc[mt][nt], 0, 0, 0);
        dma_slot(slot0 + KS + mt);
        __builtin_amdgcn_sched_barrier(0);
      }
    };

    auto step = [&](auto bi_tag, int it) __attribute__((always_inline)) {
      constexpr int BI = decltype(bi_tag)::value;
      bf16 *const cur = BI == 0 ? s_t0 : s_t1;
      bf16 *const nxt = BI == 0 ? s_t1 : s_t0;
      dma_mode = 0;
      if (it + 1 < lt1) {
        dma_prepare(it + 1, nxt);
        if (dma_mode == 2) dma_all();
      }
      const int jb = it * kTile;
      // both halves unconditionally (a half past the end is fully masked and
      // adds nothing): straight-line code keeps the accumulators in place
      half_step(cur, jb, 0);
      half_step(cur + C::HALF, jb + kHalf, KS + MT);
      wait_vmem();
      __syncthreads();
    };
    for (int it = lt0; it < lt1; it += 2) {
      step(std::integral_constant<int, 0>{}, it);
      if (it + 1 < lt1) step(std::integral_constant<int, 1>{}, it + 1);
    }

    // ---- finalize: row sums over the four lane groups, normalize, write
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      float v = xlane_sum16(l_part[nt]);
      v = xlane_sum32(v);
      const float inv = v > 0.f ? 1.f / v : 0.f;
      const float lse_nat = v > 0.f ? (m_run[nt] + __log2f(v)) * kLn2 : neg_inf();
      if (rowid[nt] < 0) continue;
      if (whole) {
        bf16 *out = static_cast<bf16 *>(p.out) + (long long)rowid[nt] * DK;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          bf16x4 o;
#pragma unroll
          for (int i = 0; i < 4; ++i) o[i] = static_cast<bf16>(oacc[mt][nt][i] * inv);
          *reinterpret_cast<bf16x4 *>(out + 16 * mt + 4 * g) = o;
        }
        if (p.lse && g == 0) p.lse[rowid[nt]] = lse_nat;
      } else {
        // partial of share c for this sequence: slot b + c
        const long long prow = rowid[nt] + (long long)c * p.s_q * p.h_q;
        float *op = p.o_part + prow * DK;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) *reinterpret_cast<f32x4 *>(op + 16 * mt + 4 * g) = oacc[mt][nt] * inv;
        if (g == 0) p.lse_part[prow] = lse_nat;
      }
    }
    // the buffers (and the query RoPE rows) are reused by the next sequence
    __syncthreads();
    cu += nb;
    ++b;
  }
}

template <int DK, int DR, int NT>
hipError_t launch_wide(const DecodeParams &p, hipStream_t s) {
  const int G = p.n_kvh * p.row_tiles;
  const int cpad = (p.n_chunks + 7) / 8 * 8;
  hipLaunchKernelGGL((mla_wide_kernel<DK, DR, NT>), dim3(G * cpad), dim3(kThreads), 0, s, p);
  return hipGetLastError();
}

template <int DK, int DR>
hipError_t launch_wide_dk(const DecodeParams &p, int nt, hipStream_t s) {
  if (nt == 1) return launch_wide<DK, DR, 1>(p, s);
  return hipErrorInvalidValue;
}

}  // namespace

bool mla_wide_supported(int dk, int dr) { return (dk == 512 || dk == 256) && (dr == 64 || dr == 0); }

int mla_wide_rows(int nt) { return 16 * kWaves * nt; }

hipError_t launch_mla_wide(const DecodeParams &p, int nt, hipStream_t s) {
  if (p.dk == 512 && p.dr == 64) return launch_wide_dk<512, 64>(p, nt, s);
  if (p.dk == 512 && p.dr == 0) return launch_wide_dk<512, 0>(p, nt, s);
  if (p.dk == 256 && p.dr == 64) return launch_wide_dk<256, 64>(p, nt, s);
  if (p.dk == 256 && p.dr == 0) return launch_wide_dk<256, 0>(p, nt, s);
  return hipErrorInvalidValue;
}

}  // namespace lkv
