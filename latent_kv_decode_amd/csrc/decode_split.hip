// decode_split.hip -- MLA absorbed decode with the score and value products
// on different waves [GQLA explainer, technical summary section 2,
// MQA-absorbed path: every query head reads the one shared latent c_KV plus
// the shared RoPE key, and the latent is also the value].
//
// A work-group takes 64 query rows of one latent head and a share of the
// batch's cache tiles.  Its eight waves split the work by stage; wave w runs
// on SIMD w mod 4, so every SIMD hosts one wave of each role:
//   waves 0..3  (score) hold the query of 16 rows each in registers and
//               compute S^T = K Q^T per 32-token tile, the online softmax
//               (running maximum, row sums) and P = exp(S - m) in bf16;
//   waves 4..7  (value) hold the output accumulator (fp32, transposed) of all
//               64 rows for a quarter of the value columns and compute
//               O^T += V^T P^T -- every value fragment read from LDS feeds
//               four row blocks.
// P (already in the MFMA operand layout) and the per-row rescale factors go
// from score to value waves through LDS, one tile behind: in iteration k the
// score waves work on tile k while the value waves work on tile k - 1, and
// one barrier per tile hands P over.  The softmax of one role overlaps the
// matrix products of the other on each SIMD.  Tiles (32 tokens) are staged
// by direct-to-LDS buffer loads into a ring of four buffers, two tiles ahead;
// the value waves issue their share of a tile before their products, the
// score waves after theirs.
//
// 8-bit (E4M3) cache: the score waves load the next tile's codes into
// registers before their products, then convert them to bf16 and write them
// in the same ring slot layout, so the products read bf16 as above.  Each
// code is converted once per work-group; the cache bytes read are halved.
// The value waves, whose accumulators fill their registers, do no staging.
#include <type_traits>

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

constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kT = 32;     // tokens per tile
constexpr int kRing = 4;   // tile buffers
constexpr int kRows = 64;  // query rows per work-group
constexpr float kLn2 = 0.693147180559945309f;
// The softmax reference maximum moves only when a tile's maximum exceeds it
// by more than this (base-2 units); probabilities stay below 2^kLazy.
constexpr float kLazy = 8.0f;


__device__ __forceinline__ float neg_inf() { return -__builtin_inff(); }

// LDS layout of a tile (128 banks of 4 bytes; a 16-byte read is served 32
// lanes at a time, a transposing 8-byte read 64 lanes at a time).
//   Latent rows: a row stride of DK + 16 elements (32 bytes of padding), so
//   row r starts 8 r banks on.  A key read (16 rows x 2 adjacent chunks) and
//   a value transpose read (16 rows x 32 bytes) both cover 128 distinct
//   banks, and the offsets of one lane's reads differ by constants that the
//   instruction's offset field holds.
//   RoPE rows (128 bytes, unpadded): chunk c of row r at slot c ^ ((r / 2)
//   mod 8).
__device__ __forceinline__ int swz_rope(int c, int r) { return c ^ ((r >> 1) & 7); }

__device__ __forceinline__ s16x4 lds_read_tr(const bf16 *p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4 *)(p));
}
__device__ __forceinline__ bf16x8 join(s16x4 lo, s16x4 hi) {
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}
// s_waitcnt vmcnt(N): at most N vector memory loads of this wave in flight.
template <int N>
__device__ __forceinline__ void wait_vmem() {
  static_assert(N >= 0 && N < 64, "vmcnt");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}

// Work-group barrier for the tile loop.  __syncthreads() also fences global
// memory, and that fence waits for every direct-to-LDS load in flight, which
// would drain the prefetch at each tile; here each wave retires its own LDS
// reads and writes (lgkmcnt 0) and the load waves have already waited (vmcnt)
// for the tile the next step needs.  The empty asm statements keep the
// compiler from moving LDS accesses across the barrier.
__device__ __forceinline__ void tile_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

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

// Share plan over 64-token units (the row-tiled kernel's definition): the
// concatenated units of all sequences (an empty sequence counts one) cut into
// n_chunks shares of ceil(total / n_chunks) units.
__device__ __forceinline__ int seq_units(int L) { return L <= 0 ? 1 : (L + kTile - 1) / kTile; }

__device__ bool plan_share(const int32_t *seqlens, int B, int C, int c, int *sh, int &chunk, int &t0,
                           int &t1, int &b0, int &cu0) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int per = (B + kThreads - 1) / kThreads;
  const int s0 = min(B, tid * per), s1 = min(B, s0 + per);
  int local = 0;
  for (int b = s0; b < s1; ++b) local += seq_units(seqlens[b]);
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
      const int nb = seq_units(seqlens[b]);
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

__device__ __forceinline__ const char *uniform_ptr(const char *p) {
  const unsigned long long v = reinterpret_cast<unsigned long long>(p);
  const unsigned lo = __builtin_amdgcn_readfirstlane(static_cast<unsigned>(v));
  const unsigned hi = __builtin_amdgcn_readfirstlane(static_cast<unsigned>(v >> 32));
  return reinterpret_cast<const char *>((static_cast<unsigned long long>(hi) << 32) | lo);
}

// Direct-to-LDS loads through raw buffer resources (buffer_load ... lds): with
// this MUBUF form the compiler keeps its waits on LDS reads exact while such
// loads are in flight.  Dword 3: 32-bit data format, no swizzle, no tid add.
// A range of 0 makes every lane out of range: nothing is read from memory
// and the LDS destination receives zeros.
constexpr int kRsrcWord3 = 0x00020000;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const char *base, int range = 0x7fffffff) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<char *>(uniform_ptr(base)), (short)0,
                                           __builtin_amdgcn_readfirstlane(range), kRsrcWord3);
}
__device__ __forceinline__ void lds_dma16(__amdgpu_buffer_rsrc_t r, bf16 *dst, unsigned voff, unsigned soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void *)dst, 16, voff, soff, 0, 0);
}

template <int DK, int DR>
struct SCfg {
  static_assert((DK == 512 || DK == 256) && (DR == 0 || DR == 64), "widths");
  static constexpr int KS = (DK + DR) / 32;   // QK^T k-steps
  static constexpr int KSN = DK / 32;         // of which on the latent
  static constexpr int MTV = DK / 64;         // value column tiles per value wave
  static constexpr int CPT = DK / 8;          // 16-byte chunks per latent row
  static constexpr int RS = DK + 16;          // latent row stride in LDS (elements)
  static constexpr int ROFF = kT * RS;        // RoPE region of a tile buffer
  static constexpr int BUF = kT * (RS + DR);  // elements per tile buffer
  // tile loads: every wave stages 4 latent rows (one instruction each); with
  // a RoPE key each score wave also stages 8 RoPE rows (one instruction when
  // the tile is on one page, eight otherwise; waiting for the count then
  // waits for more)
  static constexpr int NLL = kT / kWaves;
  static constexpr int PX = 2 * 4 * 64 * 8;  // P^T exchange [parity][row block][lane] 16 B
  static constexpr int LDS_BYTES = (kRing * BUF + PX) * 2 + 2 * 64 * 4 + 2 * 4 * 4 + 64 * 4 + 64;
  static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");
};

template <int DK, int DR, bool F8>
__global__ void __launch_bounds__(kThreads, 1) mla_split_kernel(const DecodeParams p) {
  using C = SCfg<DK, DR>;
  constexpr int KS = C::KS, KSN = C::KSN, MTV = C::MTV, CPT = C::CPT, NLL = C::NLL, RS = C::RS;
  // tile ring as distinct LDS objects (loads into one are provably
  // independent of reads of the others)
  __shared__ __attribute__((aligned(16))) bf16 s_b0[C::BUF];
  __shared__ __attribute__((aligned(16))) bf16 s_b1[C::BUF];
  __shared__ __attribute__((aligned(16))) bf16 s_b2[C::BUF];
  __shared__ __attribute__((aligned(16))) bf16 s_b3[C::BUF];
  __shared__ __attribute__((aligned(16))) bf16 s_px[C::PX];  // P^T fragments
  __shared__ float s_alpha[2][64];                           // [parity][row]
  __shared__ int s_moved[2][4];                              // [parity][16-row block]
  __shared__ float s_fin[64];                                // row sums
  __shared__ int s_plan[kWaves + 2];                         // share plan

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int g = lane >> 4, n = lane & 15;
  const int wu = __builtin_amdgcn_readfirstlane(w);

  // block -> (share, row tile); the row tiles of one share sit on one XCD
  const int G = p.n_kvh * p.row_tiles;
  const int bx = blockIdx.x;
  const int q8 = bx >> 3;
  const int grp = q8 % G;
  const int c = (q8 / G) * 8 + (bx & 7);
  if (c >= p.n_chunks) return;
  const int kvh = grp / p.row_tiles, rt = grp % p.row_tiles;

  int chunk, u0, u1, b0, cu0;
  if (!plan_share(p.seqlens, p.B, p.n_chunks, c, s_plan, chunk, u0, u1, b0, cu0)) return;

  const bf16 *__restrict__ qn = static_cast<const bf16 *>(p.q);
  const bf16 *__restrict__ qr_ = static_cast<const bf16 *>(p.q_rope);
  // cache element size: 1 byte (E4M3 code) or 2 (bf16)
  constexpr int ES = F8 ? 1 : 2;
  const char *kcb = static_cast<const char *>(p.k) + (long long)kvh * DK * ES;
  const char *rcb = static_cast<const char *>(p.r);
  const long long kstr = p.k_stride * ES, rstr = p.r_stride * ES;
  const bool aligned_pages = p.page_shift >= 5;

  // The two roles run the same loop (same tiles, same barriers); each is
  // compiled on its own so that only its own state is live.
  auto run = [&](auto role_tag) __attribute__((always_inline)) {
    constexpr bool kScore = decltype(role_tag)::value, kValue = !kScore;
    constexpr int NI = NLL + (kScore && DR > 0 ? 1 : 0);  // this wave's loads per tile
    // score wave sw: rows 16 sw .. (row block sw); value wave vw: value
    // columns 16 MTV vw ..
    const int sw = wu, vw = wu - 4;

    // ---- per-lane LDS offsets (elements) of this role's fragment reads:
    //  score: key A operand (token block tt): latent row 16tt + n, chunk
    //         4ks + g at koff0 + 16 tt RS + 32 ks; RoPE chunk 4(ks - KSN) + g
    //         at roff[(ks - KSN) mod 2] (swizzled);
    //  value: transpose read of column tile MTV vw + mt: lane (g, n) reads
    //         row 4g + n/4 (and the same 16 rows on) at columns 16 (MTV vw +
    //         mt) + 4(n%4)..+3: voff0 + 16 mt.
    int koff0 = 0, roff[2] = {0, 0}, voff0 = 0;
    if constexpr (kScore) {
      koff0 = n * RS + 8 * g;
#pragma unroll
      for (int e = 0; e < 2; ++e) roff[e] = DR > 0 ? n * DR + swz_rope(4 * e + g, n) * 8 : 0;
    } else if constexpr (kValue) {
      const int rv = 4 * g + (n >> 2);
      voff0 = rv * RS + 16 * MTV * vw + 4 * (n & 3);
    }

    // tile loads: a latent row lands as it is (lane L: bytes 16 L .. of the
    // row); a score wave's RoPE rows 8 sw .. 8 sw + 7: rofs, relative to the
    // tile's first row
    int rofs = 0;
    if constexpr (kScore && DR > 0) rofs = (int)((lane >> 3) * rstr) + swz_rope(lane & 7, 8 * sw + (lane >> 3)) * 16;

    if constexpr (!F8) {
      // One empty-range load (no memory access) into each ring buffer in
      // ring order, ahead of every path: the compiler's wait placement tracks
      // direct-to-LDS loads per buffer in order of first use, and a common
      // order on all paths keeps its waits on LDS reads exact.
      const __amdgpu_buffer_rsrc_t none = make_rsrc(kcb, 0);
      lds_dma16(none, s_b0, 0u, 0u);
      lds_dma16(none, s_b1, 0u, 0u);
      lds_dma16(none, s_b2, 0u, 0u);
      lds_dma16(none, s_b3, 0u, 0u);
      wait_vmem<0>();
    }

    int b = b0, cu = cu0;
    while (cu < u1) {
      const int L = p.seqlens[b];
      const int nb = seq_units(L);
      const int k0 = 2 * (max(cu, u0) - cu), k1 = 2 * (min(cu + nb, u1) - cu);  // 32-token tiles
      const int c_first = cu / chunk, c_last = (cu + nb - 1) / chunk;
      const bool whole = c_first == c_last;
      if (c == c_first && grp == 0 && tid == 0) {
        p.meta[2 * b] = b + c_first;
        p.meta[2 * b + 1] = c_last - c_first + 1;
      }

      // ---- rows: a score wave owns one row block, a value wave all 4
      constexpr int NB = kScore ? 1 : 4;
      const int rb0 = kScore ? sw : 0;  // first row block
      int lim[NB], rowid[NB];
#pragma unroll
      for (int nt = 0; nt < NB; ++nt) {
        const int r = rt * kRows + 16 * (rb0 + nt) + n;
        if (r < p.rows_per_kvh) {
          const int t = r / p.hpk, h = kvh * p.hpk + r % p.hpk;
          lim[nt] = p.causal ? L - p.s_q + t + 1 : L;
          rowid[nt] = (b * p.s_q + t) * p.h_q + h;
        } else {
          lim[nt] = L;
          rowid[nt] = -1;
        }
      }
      const int lim_min = p.causal ? L - p.s_q + (rt * kRows + 16 * rb0) / p.hpk + 1 : L;

      // score state: the query of the rows, running maxima, row sums;
      // value state: the output accumulator
      bf16x8 qreg[kScore ? KS : 1];
      float m_run = neg_inf(), l_part = 0.f;
      f32x4 oacc[kValue ? MTV : 1][kValue ? 4 : 1];
      if constexpr (kScore) {
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          bf16x8 v = {};
          if (rowid[0] >= 0) {
            const bf16 *src = ks < KSN ? qn + (long long)rowid[0] * DK + 32 * ks + 8 * g
                                       : qr_ + (long long)rowid[0] * DR + 32 * (ks - KSN) + 8 * g;
            v = *reinterpret_cast<const bf16x8 *>(src);
          }
          qreg[ks] = v;
        }
      } else {
#pragma unroll
        for (int mt = 0; mt < MTV; ++mt)
#pragma unroll
          for (int rb = 0; rb < 4; ++rb) oacc[mt][rb] = f32x4{0.f, 0.f, 0.f, 0.f};
      }

      // ---- block-table window and tile loads
      const int32_t *bt = p.block_table + (long long)b * p.max_pages;
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
          // retire this load here: a wait placed at its first use would sit
          // on every tile's path and drain the tile loads in flight
          wait_vmem<0>();
        }
      };
      const int row_first = L > 0 ? bt[0] * p.page_size : 0;
      // Tile k: this wave stages latent rows 8e + wu and, for a score wave,
      // RoPE rows 8 sw .. +7.  dma_rows holds the cache row of token jb +
      // (lane mod 32); tokens at or past L read row_first (valid data, masked
      // later).  A tile past the share (more == false) is issued with an empty
      // buffer range: no memory is read and the free slot takes zeros.
      bool dma_al = false;
      int dma_rows = 0, dma_range = 0;
      auto dma_prepare = [&](int k, bool more) __attribute__((always_inline)) {
        const int jb = k * kT;
        dma_range = more ? 0x7fffffff : 0;
        dma_al = aligned_pages && jb + kT <= L;
        if (dma_al) {
          const int pi = jb >> p.page_shift;
          ensure_window(pi, pi);
          const int pg = __builtin_amdgcn_readlane(btw, pi - win);
          dma_rows = pg * p.page_size + (jb & (p.page_size - 1)) + (lane & (kT - 1));
        } else {
          ensure_window(page_of(jb), page_of(max(jb, min(jb + kT, L) - 1)));
          const int j = jb + (lane & (kT - 1));
          const int pg = __shfl(btw, (page_of(j) - win) & 63);
          dma_rows = j < L ? pg * p.page_size + slot_of(j) : row_first;
        }
      };
      auto issue_tile = [&](bf16 *buf) __attribute__((always_inline)) {
        if (dma_al) {
          // whole tile on one page, rows row0 .. row0 + 31: one resource per
          // region and the row offset as the scalar offset, so a load costs
          // no vector instruction
          const long long row0 = __builtin_amdgcn_readlane(dma_rows, 0);
          const __amdgpu_buffer_rsrc_t rk = make_rsrc(kcb + row0 * kstr, dma_range);
#pragma unroll
          for (int e = 0; e < NLL; ++e) {
            const int t = kWaves * e + wu;
            if (CPT == 64 || lane < CPT)
              lds_dma16(rk, buf + t * RS, static_cast<unsigned>(16 * lane), static_cast<unsigned>(t * kstr));
          }
          if constexpr (kScore && DR > 0)
            lds_dma16(make_rsrc(rcb + row0 * rstr, dma_range), buf + C::ROFF + 8 * sw * DR,
                      static_cast<unsigned>(rofs), static_cast<unsigned>(8 * sw * rstr));
          return;
        }
#pragma unroll
        for (int e = 0; e < NLL; ++e) {
          const int t = kWaves * e + wu;
          const long long row = __builtin_amdgcn_readlane(dma_rows, t);
          if (CPT == 64 || lane < CPT)
            lds_dma16(make_rsrc(kcb + row * kstr, dma_range), buf + t * RS, static_cast<unsigned>(16 * lane), 0u);
        }
        if constexpr (kScore && DR > 0) {
          // one instruction (8 lanes) per row
#pragma unroll
          for (int q = 0; q < 8; ++q) {
            const int t = 8 * sw + q;
            const long long row = __builtin_amdgcn_readlane(dma_rows, t);
            if (lane < 8)
              lds_dma16(make_rsrc(rcb + row * rstr, dma_range), buf + C::ROFF + t * DR,
                        static_cast<unsigned>(swz_rope(lane, t) * 16), 0u);
          }
        }
      };
      auto zero_tile = [&](bf16 *buf) {
        for (int i = tid; i < C::BUF / 8; i += kThreads) *reinterpret_cast<u32x4 *>(buf + 8 * i) = u32x4{0u, 0u, 0u, 0u};
      };

      // 8-bit cache staging (score waves).  Piece q = lane + 64 i of score
      // wave sw (16 codes) is chunk q mod PPR of latent row 4 (q / PPR) + sw
      // of the tile; lanes 0..31 also stage RoPE row 8 sw + lane / 4, chunk
      // lane mod 4.  Tiles past the share (dma_range == 0) read nothing and
      // stage zeros.
      constexpr int PPR = DK / 16;
      constexpr int NPL = F8 && kScore ? 8 * PPR / 64 : 0;
      constexpr bool kRopeStage = F8 && kScore && DR > 0;
      static_assert(!F8 || 8 * PPR % 64 == 0, "8-bit staging");
      u32x4 stg[1][NPL + 1];  // one register set
      auto row_of = [&](int t) -> long long {
        return dma_al ? (long long)__builtin_amdgcn_readlane(dma_rows, 0) + t : (long long)__shfl(dma_rows, t);
      };
      // S: register set (compile time, so that the sets stay in registers)
      auto stage_load = [&](auto s_tag) __attribute__((always_inline)) {
        constexpr int S = decltype(s_tag)::value;
        if (dma_range != 0) {
#pragma unroll
          for (int i = 0; i < NPL; ++i) {
            const int q = lane + 64 * i, t = 4 * (q / PPR) + sw;
            stg[S][i] = *reinterpret_cast<const u32x4 *>(kcb + row_of(t) * kstr + 16 * (q % PPR));
          }
          if constexpr (kRopeStage) {
            stg[S][NPL] = u32x4{0u, 0u, 0u, 0u};
            if (lane < 32)
              stg[S][NPL] = *reinterpret_cast<const u32x4 *>(rcb + row_of(8 * sw + (lane >> 2)) * rstr + 16 * (lane & 3));
          }
        } else {
#pragma unroll
          for (int i = 0; i <= NPL; ++i) stg[S][i] = u32x4{0u, 0u, 0u, 0u};
        }
      };
      auto stage_store = [&](auto s_tag, bf16 *buf) __attribute__((always_inline)) {
        constexpr int S = decltype(s_tag)::value;
#pragma unroll
        for (int i = 0; i < NPL; ++i) {
          const int q = lane + 64 * i, t = 4 * (q / PPR) + sw, c16 = q % PPR;
          bf16 *row = buf + t * RS + 16 * c16;
          *reinterpret_cast<u32x4 *>(row) = e4m3x8_to_bf16x8_bits(stg[S][i][0], stg[S][i][1]);
          *reinterpret_cast<u32x4 *>(row + 8) = e4m3x8_to_bf16x8_bits(stg[S][i][2], stg[S][i][3]);
        }
        if constexpr (kRopeStage) {
          if (lane < 32) {
            const int t = 8 * sw + (lane >> 2), c16 = lane & 3;
            bf16 *row = buf + C::ROFF + t * DR;
            *reinterpret_cast<u32x4 *>(row + swz_rope(2 * c16, t) * 8) = e4m3x8_to_bf16x8_bits(stg[S][NPL][0], stg[S][NPL][1]);
            *reinterpret_cast<u32x4 *>(row + swz_rope(2 * c16 + 1, t) * 8) = e4m3x8_to_bf16x8_bits(stg[S][NPL][2], stg[S][NPL][3]);
          }
        }
      };

      // ---- score stage for tile k in buffer ht: S^T for the wave's 16 rows,
      // softmax, hand P over
      auto score_tile = [&](const bf16 *ht, int k) __attribute__((always_inline)) {
        const int jb = k * kT;
        constexpr int PD = 3;
        f32x4 sacc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
        bf16x8 kf[PD + 1][2];
        // per-stage copies of the offsets: base + offset sums formed here
        // (hoisted out of the tile loop they would stay live in registers)
        int ko0 = koff0, ro[2] = {roff[0], roff[1]};
        asm volatile("" : "+v"(ko0));
#pragma unroll
        for (int e = 0; e < 2; ++e) asm volatile("" : "+v"(ro[e]));
        auto kload = [&](int ks, bf16x8 (&dst)[2]) __attribute__((always_inline)) {
#pragma unroll
          for (int tt = 0; tt < 2; ++tt) {
            const bf16 *src = ks < KSN ? ht + 16 * tt * RS + ko0 + 32 * ks
                                       : ht + C::ROFF + 16 * tt * DR + ro[(ks - KSN) & 1];
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
          __builtin_amdgcn_sched_barrier(0);
        }
        // online softmax (base 2, lazy reference maximum).  The scale
        // (positive) is applied to the row maximum and inside the exponent's
        // fused multiply-add, not to every score.
        const int par = k & 1;
        const float sc = p.scale_log2;
        float y[2][4];
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
#pragma unroll
          for (int i = 0; i < 4; ++i) y[tt][i] = sacc[tt][i];
        if (__builtin_expect(jb + kT > lim_min, 0)) {  // the tile crosses a row's visible length
#pragma unroll
          for (int tt = 0; tt < 2; ++tt)
#pragma unroll
            for (int i = 0; i < 4; ++i)
              if (jb + 16 * tt + 4 * g + i >= lim[0]) y[tt][i] = neg_inf();
        }
        float ym = fmaxf(fmaxf(fmaxf(y[0][0], y[0][1]), fmaxf(y[0][2], y[0][3])),
                         fmaxf(fmaxf(y[1][0], y[1][1]), fmaxf(y[1][2], y[1][3])));
        ym = xlane_max16(ym);
        ym = xlane_max32(ym);
        const float mx = ym * sc;
        // the row's reference maximum moves after it has contributed: its
        // accumulated output takes the factor alpha (applied by the value
        // waves)
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
            const float e = __builtin_amdgcn_exp2f(__builtin_fmaf(y[tt][i], sc, -muse));
            sum += e;
            pb[4 * tt + i] = static_cast<bf16>(e);
          }
        l_part = l_part * alpha + sum;
        *reinterpret_cast<bf16x8 *>(s_px + ((par * 4 + sw) * 64 + lane) * 8) = pb;
        if (g == 0) s_alpha[par][16 * sw + n] = alpha;
        const bool any = __builtin_amdgcn_ballot_w64(moved) != 0;
        if (lane == 0) s_moved[par][sw] = any ? 1 : 0;
      };

      // ---- value stage for tile k in buffer ht: rescale, O^T += V^T P^T
      auto value_tile = [&](const bf16 *ht, int k) __attribute__((always_inline)) {
        const int par = k & 1;
#pragma unroll
        for (int rb = 0; rb < 4; ++rb) {
          if (s_moved[par][rb]) {
            const float a = s_alpha[par][16 * rb + n];
#pragma unroll
            for (int mt = 0; mt < MTV; ++mt) oacc[mt][rb] *= a;
          }
        }
        bf16x8 pb[4];
#pragma unroll
        for (int rb = 0; rb < 4; ++rb)
          pb[rb] = *reinterpret_cast<const bf16x8 *>(s_px + ((par * 4 + rb) * 64 + lane) * 8);
        int vo0 = voff0;
        asm volatile("" : "+v"(vo0));
        constexpr int VD = 3;
        bf16x8 va[VD + 1];
        auto vload = [&](int mt) __attribute__((always_inline)) {
          const bf16 *lo = ht + vo0 + 16 * mt;
          return join(lds_read_tr(lo), lds_read_tr(lo + 16 * RS));
        };
#pragma unroll
        for (int mt = 0; mt < VD && mt < MTV; ++mt) va[mt] = vload(mt);
#pragma unroll
        for (int mt = 0; mt < MTV; ++mt) {
          if (mt + VD < MTV) va[(mt + VD) % (VD + 1)] = vload(mt + VD);
#pragma unroll
          for (int rb = 0; rb < 4; ++rb)
            oacc[mt][rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va[mt % (VD + 1)], pb[rb], oacc[mt][rb], 0, 0, 0);
          __builtin_amdgcn_sched_barrier(0);
        }
      };

      // ---- the pipeline.  Iteration k: score waves on tile k (ring slot
      // (k - k0) mod 4), value waves on tile k - 1; every wave stages its part
      // of tile k + 2 (into the slot the value waves read in iteration k - 1)
      // and, before the barrier, waits for its part of tile k + 1.
      auto buf_of = [&](auto idx_tag) -> bf16 * {
        constexpr int I = decltype(idx_tag)::value;
        return I == 0 ? s_b0 : I == 1 ? s_b1 : I == 2 ? s_b2 : s_b3;
      };
      // prologue: tiles k0 and k0 + 1 (a sequence with no token zero-fills).
      // 8-bit cache: tile k0 goes to slot 0 now; tile k0 + 1 is loaded and
      // stored by the first iteration.
      if constexpr (F8) {
        if (L > 0) {
          if constexpr (kScore) {
            dma_prepare(k0, true);
            stage_load(std::integral_constant<int, 0>{});
            stage_store(std::integral_constant<int, 0>{}, s_b0);
          }
        } else {
          zero_tile(s_b0);
        }
      } else {
        if (L > 0) {
          dma_prepare(k0, true);
          issue_tile(s_b0);
          dma_prepare(k0 + 1, true);
          issue_tile(s_b1);
        } else {
          zero_tile(s_b0);
          zero_tile(s_b1);
        }
      }
      if constexpr (kScore) {
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) asm volatile("" : "+v"(qreg[ks]));
      }
      if constexpr (!F8) wait_vmem<NI>();  // tile k0 landed (k0 + 1 may be in flight)
      tile_barrier();

      auto iteration = [&](auto r_tag, int k, auto first_tag) __attribute__((always_inline)) {
        constexpr int R = decltype(r_tag)::value;  // (k - k0) mod 4
        constexpr bool kFirst = decltype(first_tag)::value;
        if constexpr (F8) {
          // score waves: tile k + 1 into registers (issued before the
          // products, which give the loads their time to land), then into
          // ring slot R + 1, whose last tile (k - 3) was read two iterations
          // ago.  One register set: a second set (loads two tiles ahead)
          // measured the same and spilled in the ring loop.
          if constexpr (kScore) {
            dma_prepare(k + 1, k + 1 < k1 && L > 0);
            stage_load(std::integral_constant<int, 0>{});
            if (k < k1) score_tile(buf_of(std::integral_constant<int, R>{}), k);
            stage_store(std::integral_constant<int, 0>{}, buf_of(std::integral_constant<int, (R + 1) % kRing>{}));
          } else {
            if constexpr (!kFirst) value_tile(buf_of(std::integral_constant<int, (R + kRing - 1) % kRing>{}), k - 1);
          }
          tile_barrier();
          return;
        }
        // The value waves stage their part first and the score waves theirs
        // last: the loads of one role are issued while the other role's
        // products run on the same SIMD (a load stalls its wave while the
        // address unit is busy).
        if constexpr (kScore) {
          if (k < k1) score_tile(buf_of(std::integral_constant<int, R>{}), k);
          dma_prepare(k + 2, k + 2 < k1 && L > 0);
          issue_tile(buf_of(std::integral_constant<int, (R + 2) % kRing>{}));
        } else {
          dma_prepare(k + 2, k + 2 < k1 && L > 0);
          issue_tile(buf_of(std::integral_constant<int, (R + 2) % kRing>{}));
          if constexpr (!kFirst) value_tile(buf_of(std::integral_constant<int, (R + kRing - 1) % kRing>{}), k - 1);
        }
        wait_vmem<NI>();
        tile_barrier();
      };
      // k runs k0 .. k1 (the first iteration has no value stage, the last
      // only the value stage), unrolled by the ring size so that every buffer
      // is static.  The loop body has no conditional iteration: a path that
      // skipped one would reach the loop head with another buffer's loads
      // pending, and the compiler would then wait for those before reading.
      using std::false_type;
      using std::integral_constant;
      iteration(integral_constant<int, 0>{}, k0, std::true_type{});
      int k = k0 + 1;
      for (; k + 3 <= k1; k += kRing) {
        iteration(integral_constant<int, 1>{}, k, false_type{});
        iteration(integral_constant<int, 2>{}, k + 1, false_type{});
        iteration(integral_constant<int, 3>{}, k + 2, false_type{});
        iteration(integral_constant<int, 0>{}, k + 3, false_type{});
      }
      if (k <= k1) {
        iteration(integral_constant<int, 1>{}, k, false_type{});
        if (k + 1 <= k1) {
          iteration(integral_constant<int, 2>{}, k + 1, false_type{});
          if (k + 2 <= k1) iteration(integral_constant<int, 3>{}, k + 2, false_type{});
        }
      }
      wait_vmem<0>();  // the empty-range loads of the last tiles

      // ---- finalize: score waves publish the row sums and write the LSE,
      // value waves normalize and write their columns
      if constexpr (kScore) {
        float v = xlane_sum16(l_part);
        v = xlane_sum32(v);
        const float lse_nat = v > 0.f ? (m_run + __log2f(v)) * kLn2 : neg_inf();
        if (g == 0) s_fin[16 * sw + n] = v;
        if (rowid[0] >= 0 && g == 0) {
          if (whole) {
            if (p.lse) p.lse[rowid[0]] = lse_nat;
          } else {
            p.lse_part[rowid[0] + (long long)c * p.s_q * p.h_q] = lse_nat;
          }
        }
      }
      __syncthreads();
      if constexpr (kValue) {
        const int col0 = 16 * MTV * vw;
#pragma unroll
        for (int rb = 0; rb < 4; ++rb) {
          if (rowid[rb] < 0) continue;
          const float v = s_fin[16 * rb + n];
          // out_scale: an 8-bit cache's scale (the products ran on codes)
          const float inv = v > 0.f ? p.out_scale / v : 0.f;
          if (whole) {
            bf16 *out = static_cast<bf16 *>(p.out) + (long long)rowid[rb] * DK + col0;
#pragma unroll
            for (int mt = 0; mt < MTV; ++mt) {
              bf16x4 o;
#pragma unroll
              for (int i = 0; i < 4; ++i) o[i] = static_cast<bf16>(oacc[mt][rb][i] * inv);
              *reinterpret_cast<bf16x4 *>(out + 16 * mt + 4 * g) = o;
            }
          } else {
            // partial of share c for this sequence: slot b + c
            float *op = p.o_part + (rowid[rb] + (long long)c * p.s_q * p.h_q) * DK + col0;
#pragma unroll
            for (int mt = 0; mt < MTV; ++mt) *reinterpret_cast<f32x4 *>(op + 16 * mt + 4 * g) = oacc[mt][rb] * inv;
          }
        }
      }
      // LDS (tiles, exchange, row sums) is reused by the next sequence
      __syncthreads();
      cu += nb;
      ++b;
    }
  };
  if (wu < 4) run(std::integral_constant<bool, true>{});
  else run(std::integral_constant<bool, false>{});
}

template <int DK, int DR>
hipError_t launch_split(const DecodeParams &p, hipStream_t s, const LaunchEvents &ev) {
  const int G = p.n_kvh * p.row_tiles;
  const int cpad = (p.n_chunks + 7) / 8 * 8;
  if (p.fp8) return launch_timed(mla_split_kernel<DK, DR, true>, dim3(G * cpad), dim3(kThreads), s, ev, p);
  return launch_timed(mla_split_kernel<DK, DR, false>, dim3(G * cpad), dim3(kThreads), s, ev, p);
}

}  // namespace

bool mla_split_supported(int dk, int dr) { return (dk == 512 || dk == 256) && (dr == 64 || dr == 0); }

int mla_split_rows(int, int, int, bool) { return kRows; }

hipError_t launch_mla_split(const DecodeParams &p, hipStream_t s, const LaunchEvents &ev) {
  if (p.dk == 512 && p.dr == 64) return launch_split<512, 64>(p, s, ev);
  if (p.dk == 512 && p.dr == 0) return launch_split<512, 0>(p, s, ev);
  if (p.dk == 256 && p.dr == 64) return launch_split<256, 64>(p, s, ev);
  if (p.dk == 256 && p.dr == 0) return launch_split<256, 0>(p, s, ev);
  return hipErrorInvalidValue;
}

}  // namespace lkv
