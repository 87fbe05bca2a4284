// decode_f32.hip -- float32 paged decode attention (MLA absorbed or GQA).
//
// The float32 path has no bf16 rounding anywhere: scores, softmax and the
// weighted sum run in fp32 on the vector ALUs.  It serves small float32
// problems (the pages' shapes scaled down for checking) at any widths.  Same
// definitions as the MFMA kernels [GQLA explainer, technical summary section
// 2: MQA-absorbed path and GQA path].
//
// Four waves per query row (b, t, h): wave w sweeps tiles w, w + 4, ... of
// the row's visible cache in tiles of T tokens, with its own online softmax.
// A wave copies a tile's token rows (key, RoPE key and, for a separate value
// cache, value) from the paged caches into its own LDS region with
// direct-to-LDS loads (consecutive lanes read consecutive elements of one
// row; a tile's loads are all in flight together); then lane j computes the
// score of token j from LDS, the tile's softmax update runs across the wave,
// and the weighted sum takes lanes over the value columns.  At the end the
// four partial results are merged through LDS with the same rule that merges
// split-KV partials (each weighed by exp of its maximum against the largest).
// T follows from the row width so that four tiles fit the LDS.  The rows of
// one sequence run on one XCD (work-group index mod 8), so that the heads
// reading the same cache rows share that XCD's L2.
#include "lkv_internal.h"

namespace lkv {
namespace {

constexpr int kMaxDv = 1024;
constexpr int kPerLane = kMaxDv / 64;
constexpr int kWaves = 4;
constexpr int kLdsBytes = 128 * 1024;

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// Tile geometry for a row layout of `width` floats (key + RoPE key +
// separate value) after the query's dq floats: the LDS holds the query and,
// per wave, a region of T token rows of `pitch` floats.
//   4-byte staging: pitch = width + 1 (odd: a lane-per-token read of one
//   column hits 64 different banks).
//   16-byte staging (every row segment a whole number of 16-byte chunks):
//   pitch = 4 CPR floats with CPR, the chunks per row, made odd, so that the
//   16-byte reads of 16 consecutive token rows cover distinct banks; the
//   region is rounded up to whole 64-chunk load instructions.
struct F32Tile {
  int T, pitch, region;  // tokens, floats per row, floats per wave region
};
__host__ __device__ inline F32Tile f32_tile(int width, int dq, bool v16) {
  const int avail = (kLdsBytes / 4 - dq) / kWaves;
  F32Tile t;
  if (!v16) {
    t.pitch = width + 1;
    t.T = avail / t.pitch;
    t.T = t.T < 1 ? 1 : (t.T > 64 ? 64 : t.T);
    t.region = t.T * t.pitch;
    return t;
  }
  const int cpr = (width / 4) | 1;
  t.pitch = 4 * cpr;
  t.T = 64;
  while (t.T > 1 && 4 * ((t.T * cpr + 63) / 64 * 64) > avail) --t.T;
  t.region = 4 * ((t.T * cpr + 63) / 64 * 64);
  return t;
}

// rows_per_xcd: rows handled on one XCD, a multiple of the rows of one
// sequence; work-group i runs row (i mod 8) * rows_per_xcd + i / 8.
// V16: every row segment starts 16-byte aligned and is a whole number of
// 16-byte chunks (the host checks pointers, strides and widths), so a tile is
// gathered with 16-byte direct-to-LDS loads, 64 chunks per instruction.
template <bool V16>
__global__ void __launch_bounds__(64 * kWaves) f32_decode_kernel(const DecodeParams p, long long rows_per_xcd) {
  extern __shared__ float lds[];
  __shared__ float s_ml[2 * kWaves];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const long long row = (long long)(blockIdx.x & 7) * rows_per_xcd + (blockIdx.x >> 3);
  if (row >= (long long)p.B * p.s_q * p.h_q) return;  // whole work-group
  const int h = (int)(row % p.h_q);
  const int t = (int)((row / p.h_q) % p.s_q);
  const int b = (int)(row / ((long long)p.h_q * p.s_q));
  const int kvh = h / p.hpk;
  const int L = p.seqlens[b];
  const int nvis = p.causal ? L - p.s_q + t + 1 : L;
  const bool v_alias = p.v == p.k && p.v_stride == p.k_stride && p.dv == p.dk;
  const int dq = p.dk + p.dr;                  // query (and key) width
  const int width = dq + (v_alias ? 0 : p.dv);  // floats per staged token row
  const F32Tile geo = f32_tile(width, dq, V16);
  const int T = geo.T, pitch = geo.pitch;
  float *q_l = lds;                             // [dq]
  float *tile = lds + dq + wv * geo.region;     // this wave's [T][pitch]
  const float *q = static_cast<const float *>(p.q) + row * p.dk;
  const float *qr = p.dr ? static_cast<const float *>(p.q_rope) + row * p.dr : nullptr;
  const float *kc = static_cast<const float *>(p.k) + (long long)kvh * p.dk;
  const float *rc = static_cast<const float *>(p.r);
  const float *vc = static_cast<const float *>(p.v) + (long long)kvh * p.dv;
  const int32_t *bt = p.block_table + (long long)b * p.max_pages;
  // value column v of token row j in the tile: the latent (MLA) or the
  // staged value part (GQA)
  const int voff = v_alias ? 0 : dq;
  const int nblk = (p.dv + 63) / 64;  // 64-column blocks of the value

  for (int d = threadIdx.x; d < dq; d += 64 * kWaves) q_l[d] = d < p.dk ? q[d] : qr[d - p.dk];
  __syncthreads();

  float o[kPerLane];
#pragma unroll
  for (int i = 0; i < kPerLane; ++i) o[i] = 0.f;
  float m = -__builtin_inff(), l = 0.f;

  // this wave's tiles; the loop bounds are wave-uniform and differ between
  // waves, so only wave-level ordering is used inside
  for (int j0 = wv * T; j0 < nvis; j0 += kWaves * T) {
    const int cnt = min(T, nvis - j0);
    // cache row of token j0 + lane (lanes < cnt)
    int crow = 0;
    if (lane < cnt) {
      const int j = j0 + lane;
      crow = bt[j / p.page_size] * p.page_size + j % p.page_size;
    }
    // the previous tile's LDS reads are complete before it is overwritten
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    // direct-to-LDS loads, all in flight together, one region at a time
    // (key, RoPE key, separate value), 64 columns per instruction: element
    // c of token row tok goes to tile[tok][at + c]
    auto stage = [&](const float *base, long long stride, int cols, int at) {
      for (int tok = 0; tok < cnt; ++tok) {
        const float *src = base + (long long)__builtin_amdgcn_readlane(crow, tok) * stride + lane;
        float *dst = tile + tok * pitch + at;
        for (int c0 = 0; c0 < cols; c0 += 64)
          if (c0 + lane < cols)
            __builtin_amdgcn_global_load_lds(src + c0, (__attribute__((address_space(3))) void *)(dst + c0), 4, 0, 0);
      }
    };
    if constexpr (V16) {
      // chunk q = 64 u + lane: 16 bytes of token q / CPR's row, chunk q mod
      // CPR (key, then RoPE key, then separate value; the odd padding chunk
      // and the chunks past the tile's tokens read a valid chunk that is
      // never used)
      const int cpr = pitch / 4, ck = p.dk / 4, cq = dq / 4, cw = width / 4;
      const int nq = cnt * cpr;
      for (int u = 0; 64 * u < nq; ++u) {
        const int q = 64 * u + lane;
        const int tok = min(q / cpr, cnt - 1), c = q % cpr;
        const long long r = __shfl(crow, tok);
        const float *src = kc + r * p.k_stride;
        if (q < nq) {
          if (c < ck) src += 4 * c;
          else if (c < cq) src = rc + r * p.r_stride + 4 * (c - ck);
          else if (c < cw) src = vc + r * p.v_stride + 4 * (c - cq);
        }
        __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void *)(tile + 256 * u), 16, 0, 0);
      }
    } else {
      stage(kc, p.k_stride, p.dk, 0);
      if (p.dr) stage(rc, p.r_stride, p.dr, p.dk);
      if (!v_alias) stage(vc, p.v_stride, p.dv, dq);
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    float s = -__builtin_inff();
    if (lane < cnt) {
      const float *kr = tile + lane * pitch;
      float dot = 0.f;
      if constexpr (V16) {
        // four independent partial sums over 16-byte reads
        typedef float f4 __attribute__((ext_vector_type(4)));
        f4 acc4 = {0.f, 0.f, 0.f, 0.f};
        for (int c = 0; c < dq / 4; ++c)
          acc4 += *reinterpret_cast<const f4 *>(q_l + 4 * c) * *reinterpret_cast<const f4 *>(kr + 4 * c);
        dot = (acc4[0] + acc4[1]) + (acc4[2] + acc4[3]);
      } else {
        for (int d = 0; d < dq; ++d) dot += q_l[d] * kr[d];
      }
      s = dot * p.scale_log2;
    }
    const float mnew = fmaxf(m, wave_max(s));
    const float muse = mnew == -__builtin_inff() ? 0.f : mnew;
    const float alpha = __builtin_amdgcn_exp2f(m - muse);
    const float pj = __builtin_amdgcn_exp2f(s - muse);
    l = l * alpha + wave_sum(pj);
    m = mnew;
#pragma unroll
    for (int i = 0; i < kPerLane; ++i) o[i] *= alpha;
    // weighted sum: value column lane + 64 i (a wave-uniform bound on i, the
    // last partial block read clamped and weighted by zero past dv)
    const float *vt = tile + voff;
#pragma unroll
    for (int i = 0; i < kPerLane; ++i) {
      if (i < nblk) {
        const int d = lane + 64 * i;
        const int dc = min(d, p.dv - 1);
        const float keep = d < p.dv ? 1.f : 0.f;
        float acc = 0.f;
        int jj = 0;
        if constexpr (V16) {
          // four independent partial sums
          float a1 = 0.f, a2 = 0.f, a3 = 0.f;
          for (; jj + 4 <= cnt; jj += 4) {
            acc += __int_as_float(__builtin_amdgcn_readlane(__float_as_int(pj), jj + 0)) * vt[(jj + 0) * pitch + dc];
            a1 += __int_as_float(__builtin_amdgcn_readlane(__float_as_int(pj), jj + 1)) * vt[(jj + 1) * pitch + dc];
            a2 += __int_as_float(__builtin_amdgcn_readlane(__float_as_int(pj), jj + 2)) * vt[(jj + 2) * pitch + dc];
            a3 += __int_as_float(__builtin_amdgcn_readlane(__float_as_int(pj), jj + 3)) * vt[(jj + 3) * pitch + dc];
          }
          acc = (acc + a1) + (a2 + a3);
        }
        for (; jj + 4 <= cnt; jj += 4) {
          const float v0 = vt[(jj + 0) * pitch + dc], v1 = vt[(jj + 1) * pitch + dc];
          const float v2 = vt[(jj + 2) * pitch + dc], v3 = vt[(jj + 3) * pitch + dc];
          acc += __int_as_float(__builtin_amdgcn_readlane(__float_as_int(pj), jj + 0)) * v0;
          acc += __int_as_float(__builtin_amdgcn_readlane(__float_as_int(pj), jj + 1)) * v1;
          acc += __int_as_float(__builtin_amdgcn_readlane(__float_as_int(pj), jj + 2)) * v2;
          acc += __int_as_float(__builtin_amdgcn_readlane(__float_as_int(pj), jj + 3)) * v3;
        }
        for (; jj < cnt; ++jj) acc += __int_as_float(__builtin_amdgcn_readlane(__float_as_int(pj), jj)) * vt[jj * pitch + dc];
        o[i] += keep * acc;
      }
    }
  }

  // ---- merge the four waves' results: weights 2^(m_w - M) with M the
  // largest maximum (a wave that saw no token weighs nothing)
  __syncthreads();  // every wave is done with its tile region
  float *o_l = lds + dq;  // [kWaves][dv], over the tile regions
  if (lane == 0) {
    s_ml[wv] = m;
    s_ml[kWaves + wv] = l;
  }
#pragma unroll
  for (int i = 0; i < kPerLane; ++i) {
    const int d = lane + 64 * i;
    if (i < nblk && d < p.dv) o_l[wv * p.dv + d] = o[i];
  }
  __syncthreads();
  float mm = -__builtin_inff();
#pragma unroll
  for (int w = 0; w < kWaves; ++w) mm = fmaxf(mm, s_ml[w]);
  float wgt[kWaves], lt = 0.f;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    wgt[w] = s_ml[w] == -__builtin_inff() ? 0.f : __builtin_amdgcn_exp2f(s_ml[w] - mm);
    lt += wgt[w] * s_ml[kWaves + w];
  }
  const float inv = lt > 0.f ? 1.f / lt : 0.f;
  float *out = static_cast<float *>(p.out) + row * p.dv;
  for (int d = threadIdx.x; d < p.dv; d += 64 * kWaves) {
    float acc = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) acc += wgt[w] * o_l[w * p.dv + d];
    out[d] = acc * inv;
  }
  if (p.lse && threadIdx.x == 0)
    p.lse[row] = lt > 0.f ? (mm + __log2f(lt)) * 0.693147180559945309f : -__builtin_inff();
}

}  // namespace

hipError_t launch_f32_decode(const DecodeParams &p, hipStream_t s, const LaunchEvents &ev) {
  const long long rows = (long long)p.B * p.s_q * p.h_q;
  if (rows == 0) return hipSuccess;
  // rows per XCD: an eighth of the rows, rounded up to whole sequences
  const long long per_seq = (long long)p.s_q * p.h_q;
  const long long per_xcd = ((rows + 7) / 8 + per_seq - 1) / per_seq * per_seq;
  const long long grid = 8 * per_xcd;
  if (grid > 0x7fffffffLL) return hipErrorInvalidValue;
  const bool v_alias = p.v == p.k && p.v_stride == p.k_stride && p.dv == p.dk;
  const int dq = p.dk + p.dr;
  const int width = dq + (v_alias ? 0 : p.dv);
  // 16-byte staging when every row segment starts 16-byte aligned and is a
  // whole number of 16-byte chunks
  auto al16 = [](const void *x) { return x == nullptr || (reinterpret_cast<uintptr_t>(x) & 15) == 0; };
  // the tiles, and after them the merge area [kWaves][dv], fit the LDS
  auto fits = [&](const F32Tile &g) {
    return (size_t)(dq + kWaves * g.region) * sizeof(float) <= (size_t)kLdsBytes && p.dv <= g.region &&
           g.T * g.pitch <= g.region;
  };
  bool v16 = al16(p.k) && p.dk % 4 == 0 && p.k_stride % 4 == 0 &&
             (p.dr == 0 || (al16(p.r) && p.dr % 4 == 0 && p.r_stride % 4 == 0)) &&
             (v_alias || (al16(p.v) && p.dv % 4 == 0 && p.v_stride % 4 == 0));
  // rows so wide that the 16-byte layout's padding overflows the LDS take
  // the 4-byte path
  if (v16 && !fits(f32_tile(width, dq, true))) v16 = false;
  const F32Tile geo = f32_tile(width, dq, v16);
  if (!fits(geo)) return hipErrorInvalidValue;
  const size_t lds = (size_t)(dq + kWaves * geo.region) * sizeof(float);
  auto go = [&](auto kern) {
    if (ev.start || ev.stop)
      hipExtLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(64 * kWaves), lds, s, ev.start, ev.stop, 0, p, per_xcd);
    else
      hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(64 * kWaves), lds, s, p, per_xcd);
  };
  if (v16)
    go(f32_decode_kernel<true>);
  else
    go(f32_decode_kernel<false>);
  return hipGetLastError();
}

}  // namespace lkv
