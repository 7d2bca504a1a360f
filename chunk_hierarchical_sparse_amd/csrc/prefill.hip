// prefill.hip - HSA prefill ([HSA] Methodology: per-chunk landmarks, top-K
// chunk retrieval; [HiLS] abstract: attention inside each retrieved chunk,
// fusion by the retrieval scores).
//
// Pipeline (all on one stream):
//  1. select : group-summed scores u_t . lmk_c for the chunks fully before t,
//              per-query top-K (score desc, index asc) -> idx; per-chunk
//              selection counts.
//  2. invert : scan the counts into per-chunk lists of (token, slot) entries
//              and per-chunk tile offsets (chunk-major work list).
//  3. attend : one block per (chunk, tile of entries): the chunk's K/V are
//              staged once in LDS and serve every (token, head) row that
//              selected the chunk (bf16 MFMA; fp32 inputs use a VALU kernel).
//              Each row writes its normalised chunk output and its per-head
//              retrieval score s_h(t,c) into slot `slot` of the row.
//  4. fuse   : per (token, head): w = softmax over the kept slots of s_h,
//              out = sum_k w_k o_k (the fusion epilogue), optional weights.
#include <math.h>

#include "attn_core.h"
#include "hsa_common.h"
#include "kernels.h"
#include "chunk_attend.h"
#include "prefill_common.h"

namespace hsa {

HSA_DCHECK_SOURCE()
namespace {

constexpr int kThreads = 256;
// (token, head) rows per block of the S <= 64 chunk attention: 32 tiles of
// 32 rows, 8 per wave, enough to amortise staging the chunk's K/V.
constexpr int kChunkUnitRows = 1024;

// ---------------------------------------------------------------- select --

// The invert's per-chunk counters (counts, cursor) must start at zero.  The
// select launch, which always runs right before the invert, clears them on
// the way: one launch fewer than a separate fill.
__device__ __forceinline__ void clear_invert_counters(const PrefillArgs& a) {
  const int64_t m = (int64_t)a.B * a.Hkv * a.n;
  const int64_t step = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < m; i += step) {
    a.counts[i] = 0;
    a.cursor[i] = 0;
  }
}

// Keep a descending top-KM list in registers.  Candidates of one lane
// arrive in increasing index order, so a strict '>' places a later
// equal-score candidate after the earlier one (lower index first).  The
// list is sorted, so slot j becomes max(min(s, ls[j-1]), ls[j]), which for
// ls[j-1] >= ls[j] is the median of the three (one v_med3_f32), and its
// index follows the same choice through bit masks: straight-line code.
template <int KM>
__device__ __forceinline__ void topk_insert_ordered(float (&ls)[KM], int (&li)[KM], float s,
                                                    int c) {
  int m[KM];
#pragma unroll
  for (int j = 0; j < KM; ++j) m[j] = -(int)(s > ls[j]);  // all ones where s beats slot j
#pragma unroll
  for (int j = KM - 1; j > 0; --j) {
    ls[j] = __builtin_amdgcn_fmed3f(s, ls[j - 1], ls[j]);
    const int t = (c & m[j]) | (li[j] & ~m[j]);
    li[j] = (li[j - 1] & m[j - 1]) | (t & ~m[j - 1]);
  }
  ls[0] = fmaxf(s, ls[0]);
  li[0] = (c & m[0]) | (li[0] & ~m[0]);
}

// Full (score desc, index asc) comparison for merging lists of different
// lanes/waves (bitwise, so no short-circuit branches).
__device__ __forceinline__ bool better(float s, int c, float t, int d) {
  return (s > t) | ((s == t) & (c < d));
}

template <int KM>
__device__ __forceinline__ void topk_insert_any(float (&ls)[KM], int (&li)[KM], float s, int c) {
  int m[KM];
#pragma unroll
  for (int j = 0; j < KM; ++j) m[j] = -(int)((c >= 0) & better(s, c, ls[j], li[j]));
  const int sb = __float_as_int(s);
#pragma unroll
  for (int j = KM - 1; j > 0; --j) {
    const int ts = (sb & m[j]) | (__float_as_int(ls[j]) & ~m[j]);
    const int ti = (c & m[j]) | (li[j] & ~m[j]);
    ls[j] = __int_as_float((__float_as_int(ls[j - 1]) & m[j - 1]) | (ts & ~m[j - 1]));
    li[j] = (li[j - 1] & m[j - 1]) | (ti & ~m[j - 1]);
  }
  ls[0] = __int_as_float((sb & m[0]) | (__float_as_int(ls[0]) & ~m[0]));
  li[0] = (c & m[0]) | (li[0] & ~m[0]);
}

// One block = 64 consecutive queries of one (b, group); lane = query.  The
// four waves take interleaved quarters of each 32-landmark tile and merge
// their lists at the end.  Scores are ranked unscaled (u . lmk): the
// positive factor 1/sqrt(d) does not change the order.
template <int D, int KM, int DT>
__global__ void __launch_bounds__(kThreads) select_valu_kernel(PrefillArgs a, int64_t nqt) {
  clear_invert_counters(a);
  constexpr int TILE = 32;
  constexpr int LT_BYTES = TILE * D * 4;
  constexpr int MERGE_BYTES = 3 * 64 * KM * 8;
  __shared__ __attribute__((aligned(16))) char smem[LT_BYTES > MERGE_BYTES ? LT_BYTES : MERGE_BYTES];
  float* lt = (float*)smem;                  // landmark tile, then reused for merging
  float* ms = (float*)smem;                  // [3][64][KM] scores of waves 1..3
  int* mi = (int*)(smem + 3 * 64 * KM * 4);  // [3][64][KM] indices
  const int64_t bg = blockIdx.x / nqt;
  const int64_t qt = blockIdx.x % nqt;
  const int b = (int)(bg / a.Hkv), g = (int)(bg % a.Hkv);
  const int G = a.Hq / a.Hkv;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  // selection rows are the tokens t = row * interval (every token at 1)
  const int64_t tq = qt * 64 + lane;
  const int64_t t = tq * a.interval;
  const bool tvalid = tq < a.nq;
  const int64_t navail = tvalid ? min(t / a.S, a.n) : 0;
  const int64_t tlast = min(qt * 64 + 63, a.nq - 1) * a.interval;
  const int64_t bavail = min(tlast / a.S, a.n);

  float u[D];
#pragma unroll
  for (int x = 0; x < D; ++x) u[x] = 0.f;
  if (tvalid) {
    for (int hh = 0; hh < G; ++hh) {
      const int64_t base = (((int64_t)b * a.Hq + g * G + hh) * a.L + t) * D;
#pragma unroll
      for (int x = 0; x < D; ++x) u[x] += load_elem<DT>(a.Q, base + x);
    }
  }
  float ls[KM];
  int li[KM];
#pragma unroll
  for (int j = 0; j < KM; ++j) {
    ls[j] = -INFINITY;
    li[j] = -1;
  }
  const float* lmk = a.lmk + bg * a.n * D;
  for (int64_t c0 = 0; c0 < bavail; c0 += TILE) {
    __syncthreads();
    for (int e = threadIdx.x; e < TILE * D / 4; e += kThreads) {
      const int64_t c = c0 + (e * 4) / D;
      f32x4 v = {0.f, 0.f, 0.f, 0.f};
      if (c < bavail) v = *(const f32x4*)(lmk + c0 * D + e * 4);
      *(f32x4*)(&lt[e * 4]) = v;
    }
    __syncthreads();
    for (int cc = w * (TILE / 4); cc < (w + 1) * (TILE / 4); ++cc) {
      const int64_t c = c0 + cc;
      if (c >= bavail) break;
      float dot = 0.f;
#pragma unroll
      for (int x = 0; x < D; x += 4) {
        const f32x4 l4 = *(const f32x4*)(&lt[cc * D + x]);
        dot += u[x] * l4[0];
        dot += u[x + 1] * l4[1];
        dot += u[x + 2] * l4[2];
        dot += u[x + 3] * l4[3];
      }
      topk_insert_ordered<KM>(ls, li, c < navail ? dot : -INFINITY, (int)c);
    }
  }
  __syncthreads();  // the landmark tile is dead; its LDS now holds the lists
  if (w > 0) {
#pragma unroll
    for (int j = 0; j < KM; ++j) {
      ms[((w - 1) * 64 + lane) * KM + j] = ls[j];
      mi[((w - 1) * 64 + lane) * KM + j] = li[j];
    }
  }
  __syncthreads();
  if (w != 0 || !tvalid) return;
  for (int ww = 0; ww < 3; ++ww)
    for (int j = 0; j < KM; ++j)
      topk_insert_any<KM>(ls, li, ms[(ww * 64 + lane) * KM + j], mi[(ww * 64 + lane) * KM + j]);
  int32_t* out = a.idx + (bg * a.nq + tq) * a.topk;
#pragma unroll
  for (int j = 0; j < KM; ++j)
    if (j < a.topk) out[j] = li[j];
}

// bf16 inputs: scores on MFMA.  Each wave owns 32 consecutive queries; a
// block owns 128 queries of one (b, group).  Landmark tiles of 32 chunks are
// staged in LDS split into three bf16 parts (hi + lo + lo2 == the fp32 value
// exactly), the group-summed query u likewise in registers, and
// u.lmk = sum of the six part products whose order is at most 2^-16 of the
// leading one, accumulated in fp32 by v_mfma_f32_32x32x16_bf16: the result
// is as accurate as an fp32 dot product.  S^T = LMK U^T puts one query per
// lane (lanes l and l^32 hold disjoint halves of each chunk tile), so each
// lane keeps its own sorted top-KM list; the two halves merge at the end.

template <int D, int KM>
__global__ void __launch_bounds__(kThreads, 2) select_mfma_kernel(PrefillArgs a, int64_t nqt) {
  clear_invert_counters(a);
  constexpr int QPB = 128;  // selection rows per block: 4 waves x 32
  constexpr int TILE = 32;
  constexpr int RS = D + 8;  // padded LDS row (bf16 elements)
  __shared__ __attribute__((aligned(16))) uint16_t lt[3][TILE * RS];
  // late query tiles see the most chunks: dispatch them first
  const int64_t BG = (int64_t)a.B * a.Hkv;
  const int64_t bg = blockIdx.x % BG;
  const int64_t qt = nqt - 1 - blockIdx.x / BG;
  const int b = (int)(bg / a.Hkv), g = (int)(bg % a.Hkv);
  const int G = a.Hq / a.Hkv;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int i32 = lane & 31, hf = lane >> 5;
  // selection rows are the tokens t = row * interval (every token at 1)
  const int64_t tq = qt * QPB + w * 32 + i32;
  const int64_t t = tq * a.interval;
  const bool tvalid = tq < a.nq;
  const int64_t navail = tvalid ? min(t / a.S, a.n) : 0;
  const int navail_i = (int)navail;  // n < 2^26: 32-bit compares in the top-K upkeep
  const int64_t tlast_b = min(qt * QPB + QPB - 1, a.nq - 1) * a.interval;
  const int64_t bavail = min(tlast_b / a.S, a.n);
  const int64_t tlast_w = min(qt * QPB + w * 32 + 31, a.nq - 1) * a.interval;
  const int64_t wavail = qt * QPB + w * 32 < a.nq ? min(tlast_w / a.S, a.n) : 0;

  // u = sum over the group's heads, dims 16s + 8hf + e, split in 3 parts;
  // one head's row pieces are all in flight at once (heads in order, so
  // the sum is the same as adding one head at a time)
  bf16x8 u0[D / 16], u1[D / 16], u2[D / 16];
  {
    const uint16_t* Q = (const uint16_t*)a.Q;
    float acc[D / 16][8];
#pragma unroll
    for (int s2 = 0; s2 < D / 16; ++s2)
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[s2][e] = 0.f;
    if (tvalid) {
      for (int hh = 0; hh < G; ++hh) {
        const uint16_t* qrow = Q + (((int64_t)b * a.Hq + g * G + hh) * a.L + t) * D + 8 * hf;
        u32x4 x[D / 16];
#pragma unroll
        for (int s2 = 0; s2 < D / 16; ++s2) x[s2] = *(const u32x4*)(qrow + 16 * s2);
#pragma unroll
        for (int s2 = 0; s2 < D / 16; ++s2)
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            acc[s2][2 * v] += bf16_bits_to_f32(x[s2][v] & 0xffffu);
            acc[s2][2 * v + 1] += bf16_bits_to_f32(x[s2][v] >> 16);
          }
      }
    }
#pragma unroll
    for (int s2 = 0; s2 < D / 16; ++s2) {
      u32x4 p0, p1, p2;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        uint16_t h0, l0, m0, h1, l1, m1;
        split3_bf16(acc[s2][2 * v], h0, l0, m0);
        split3_bf16(acc[s2][2 * v + 1], h1, l1, m1);
        p0[v] = (uint32_t)h0 | ((uint32_t)h1 << 16);
        p1[v] = (uint32_t)l0 | ((uint32_t)l1 << 16);
        p2[v] = (uint32_t)m0 | ((uint32_t)m1 << 16);
      }
      u0[s2] = __builtin_bit_cast(bf16x8, p0);
      u1[s2] = __builtin_bit_cast(bf16x8, p1);
      u2[s2] = __builtin_bit_cast(bf16x8, p2);
    }
  }
  float ls[KM];
  int li[KM];
#pragma unroll
  for (int j = 0; j < KM; ++j) {
    ls[j] = -INFINITY;
    li[j] = -1;
  }
  const float* lmk = a.lmk + bg * a.n * D;
  // the next landmark tile is loaded into registers while the current one is
  // scored: thread e takes float4 pieces e, e + 256, ... of the 32 x D tile
  constexpr int NPT = TILE * D / 4 / kThreads;
  f32x4 nxt[NPT];
  auto fetch = [&](int64_t cb) {
#pragma unroll
    for (int i = 0; i < NPT; ++i) {
      const int e = threadIdx.x + i * kThreads;
      const int row = (e * 4) / D, col = (e * 4) % D;
      nxt[i] = cb + row < bavail ? *(const f32x4*)(lmk + (cb + row) * D + col)
                                 : f32x4{0.f, 0.f, 0.f, 0.f};
    }
  };
  if (bavail > 0) fetch(0);
  for (int64_t c0 = 0; c0 < bavail; c0 += TILE) {
    __syncthreads();
    // stage the 32 landmark rows as three bf16 planes
#pragma unroll
    for (int i = 0; i < NPT; ++i) {
      const int e = threadIdx.x + i * kThreads;
      const int row = (e * 4) / D, col = (e * 4) % D;
      const f32x4 v = nxt[i];
      uint16_t h[4], l[4], m[4];
#pragma unroll
      for (int x = 0; x < 4; ++x) split3_bf16(v[x], h[x], l[x], m[x]);
      *(u32x2*)(&lt[0][row * RS + col]) = u32x2{(uint32_t)h[0] | ((uint32_t)h[1] << 16),
                                                (uint32_t)h[2] | ((uint32_t)h[3] << 16)};
      *(u32x2*)(&lt[1][row * RS + col]) = u32x2{(uint32_t)l[0] | ((uint32_t)l[1] << 16),
                                                (uint32_t)l[2] | ((uint32_t)l[3] << 16)};
      *(u32x2*)(&lt[2][row * RS + col]) = u32x2{(uint32_t)m[0] | ((uint32_t)m[1] << 16),
                                                (uint32_t)m[2] | ((uint32_t)m[3] << 16)};
    }
    __syncthreads();
    if (c0 + TILE < bavail) fetch(c0 + TILE);
    if (c0 >= wavail) continue;  // wave-uniform: no query of this wave sees these chunks
    f32x16 acc;
#pragma unroll
    for (int s2 = 0; s2 < D / 16; ++s2) {
      const int off = i32 * RS + 16 * s2 + 8 * hf;
      const bf16x8 l0 = *(const bf16x8*)(&lt[0][off]);
      const bf16x8 l1 = *(const bf16x8*)(&lt[1][off]);
      const bf16x8 l2 = *(const bf16x8*)(&lt[2][off]);
      const f32x16 zero = {};
      // smallest terms first; the first takes a zero accumulator operand
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(l2, u0[s2], s2 == 0 ? zero : acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(l1, u1[s2], acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(l0, u2[s2], acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(l1, u0[s2], acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(l0, u1[s2], acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(l0, u0[s2], acc, 0, 0, 0);
    }
    // lane's candidates come in increasing chunk order: r -> 8(r/4)+4hf+r%4
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int c = (int)c0 + 8 * (r >> 2) + 4 * hf + (r & 3);
      topk_insert_ordered<KM>(ls, li, c < navail_i ? acc[r] : -INFINITY, c);
    }
  }
  // merge the two halves of each query (lane l and l ^ 32)
  float os[KM];
  int oi[KM];
#pragma unroll
  for (int j = 0; j < KM; ++j) {
    os[j] = __shfl_xor(ls[j], 32, kWave);
    oi[j] = __shfl_xor(li[j], 32, kWave);
  }
  if (hf != 0 || !tvalid) return;
#pragma unroll
  for (int j = 0; j < KM; ++j) topk_insert_any<KM>(ls, li, os[j], oi[j]);
  int32_t* out = a.idx + (bg * a.nq + tq) * a.topk;
#pragma unroll
  for (int j = 0; j < KM; ++j)
    if (j < a.topk) out[j] = li[j];
}

// ---------------------------------------------------------------- invert --

// One block per (b, group): exclusive scans of the selection counts
// (entry offsets) and of the per-chunk work-unit counts (unit offsets), and
// the unit -> chunk map the attention blocks read.
__global__ void __launch_bounds__(1024) scan_kernel(PrefillArgs a) {
  __shared__ int32_t sa[1024], sb[1024];
  __shared__ int32_t carry_a, carry_b;
  const int64_t bg = blockIdx.x;
  const int32_t* cnt = a.counts + bg * a.n;
  int32_t* offs = a.offs + bg * (a.n + 1);
  int32_t* toff = a.tile_off + bg * (a.n + 1);
  int32_t* tmap = a.tile_chunk + bg * a.tiles_ub;
  const int E = a.entries_per_tile;
  if (threadIdx.x == 0) {
    carry_a = 0;
    carry_b = 0;
  }
  __syncthreads();
  for (int64_t c0 = 0; c0 < a.n; c0 += 1024) {
    const int64_t c = c0 + threadIdx.x;
    const int32_t v = c < a.n ? cnt[c] : 0;
    sa[threadIdx.x] = v;
    sb[threadIdx.x] = (v + E - 1) / E;
    __syncthreads();
    for (int o = 1; o < 1024; o <<= 1) {
      int32_t xa = 0, xb = 0;
      if ((int)threadIdx.x >= o) {
        xa = sa[threadIdx.x - o];
        xb = sb[threadIdx.x - o];
      }
      __syncthreads();
      sa[threadIdx.x] += xa;
      sb[threadIdx.x] += xb;
      __syncthreads();
    }
    if (c < a.n) {
      const int32_t nt = (v + E - 1) / E;
      const int32_t t0 = carry_b + sb[threadIdx.x] - nt;
      offs[c] = carry_a + sa[threadIdx.x] - v;
      toff[c] = t0;
      for (int32_t j = 0; j < nt; ++j) tmap[t0 + j] = (int32_t)c;
    }
    __syncthreads();
    if (threadIdx.x == 1023) {
      carry_a += sa[1023];
      carry_b += sb[1023];
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    offs[a.n] = carry_a;
    toff[a.n] = carry_b;
  }
}

// Selection slot of (token, slot) i = token * topk + slot: the row of the
// token's block start (token / interval) in the selection buffer.
__device__ __forceinline__ int64_t sel_of(const PrefillArgs& a, int64_t i) {
  if (a.interval == 1) return i;
  // per-(b, group) indices stay below L * topk < 2^31: 32-bit division
  const uint32_t u = (uint32_t)i, k = (uint32_t)a.topk;
  const uint32_t tok = u / k;
  return (int64_t)((tok / (uint32_t)a.interval) * k + (u - tok * k));
}
// Selection chunk of entries i = i0 + 256 u (u < 8) of [.., e1): all eight
// loads go out together (past e1: -1, reading the last entry instead).
__device__ __forceinline__ void load_sel8(const PrefillArgs& a, const int32_t* idx, int64_t i0,
                                          int64_t e1, int32_t (&c)[8]) {
#pragma unroll
  for (int u = 0; u < 8; ++u) c[u] = idx[sel_of(a, min(i0 + 256 * u, e1 - 1))];
#pragma unroll
  for (int u = 0; u < 8; ++u)
    if (i0 + 256 * u >= e1) c[u] = -1;
}
constexpr int kInvertLdsBins = 8192;  // chunks whose counters fit in LDS (2 arrays)

// Per-chunk selection counts.  Each block histograms the selections of
// kInvertTokens tokens in LDS and adds one global atomic per touched chunk,
// so hot chunks see a few hundred global atomics instead of one per
// selection (integer sums: the totals do not depend on the order).  For
// ordered lists it also keeps the histogram as its row of blockbase.
__global__ void __launch_bounds__(256) count_kernel(PrefillArgs a, int64_t blocks_per_bg,
                                                    int use_lds) {
  extern __shared__ int32_t hist[];  // [n]
  const int64_t bg = blockIdx.x / blocks_per_bg;
  const int64_t t0 = (blockIdx.x % blocks_per_bg) * kInvertTokens;
  const int64_t t1 = min(t0 + kInvertTokens, a.L);
  const int32_t* idx = a.idx + bg * a.nq * a.topk;
  int32_t* cnt = a.counts + bg * a.n;
  if (use_lds) {
    for (int c = threadIdx.x; c < a.n; c += 256) hist[c] = 0;
    __syncthreads();
  }
  const int64_t e1 = t1 * a.topk;
  for (int64_t i0 = t0 * a.topk + threadIdx.x; i0 < e1; i0 += 8 * 256) {
    int32_t c[8];
    load_sel8(a, idx, i0, e1, c);
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      if (c[u] < 0) continue;
      HSA_DCHECK(c[u] < a.n);
      if (use_lds)
        atomicAdd(&hist[c[u]], 1);
      else
        atomicAdd(&cnt[c[u]], 1);
    }
  }
  if (!use_lds) return;
  __syncthreads();
  if (a.ordered && a.n <= kInvertDetBins) {
    int32_t* row = a.blockbase + blockIdx.x * a.n;  // blocks of one (b, group) are consecutive
    for (int c = threadIdx.x; c < a.n; c += 256) row[c] = hist[c];
  }
  for (int c = threadIdx.x; c < a.n; c += 256)
    if (hist[c] != 0) atomicAdd(&cnt[c], hist[c]);
}

// Lists in token order (ordered lists, up to kInvertDetBins chunks).  A
// block's first position in chunk c's list is offs[c] plus the counts of
// the (b, group)'s earlier blocks (their blockbase rows).  Its tokens then
// go in rounds of 64: every selection sets its token's bit in its chunk's
// 64-bit round mask, and its list position is the block's running position
// for the chunk plus the number of earlier tokens in the mask.  The first
// token of each chunk in the round then advances the running position and
// clears the mask.  A token selects a chunk at most once.
__global__ void __launch_bounds__(256) scatter_ordered_kernel(PrefillArgs a,
                                                              int64_t blocks_per_bg) {
  extern __shared__ int32_t sh[];  // running position [n], then round masks [n][2]
  constexpr int kRound = 64;
  const int64_t bg = blockIdx.x / blocks_per_bg;
  const int64_t t0 = (blockIdx.x % blocks_per_bg) * kInvertTokens;
  const int64_t t1 = min(t0 + kInvertTokens, a.L);
  const int32_t* idx = a.idx + bg * a.nq * a.topk;
  const int32_t* rows0 = a.blockbase + bg * blocks_per_bg * a.n;  // this (b, group)'s rows
  const int nprev = (int)(blockIdx.x % blocks_per_bg);
  const int32_t* offs = a.offs + bg * (a.n + 1);
  int32_t* list = a.list + bg * a.L * a.topk;
  int32_t* epos = a.entry_pos + bg * a.L * a.topk;
  int32_t* run = sh;
  uint32_t* mask = (uint32_t*)(sh + a.n);
  for (int c = threadIdx.x; c < a.n; c += 256) {
    // four rows in flight at a time (rows past nprev read row 0, add 0)
    int32_t acc = offs[c];
    for (int k = 0; k < nprev; k += 4) {
      int32_t h[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) h[j] = rows0[(int64_t)(k + j < nprev ? k + j : 0) * a.n + c];
#pragma unroll
      for (int j = 0; j < 4; ++j) acc += k + j < nprev ? h[j] : 0;
    }
    run[c] = acc;
    mask[2 * c] = 0u;
    mask[2 * c + 1] = 0u;
  }
  __syncthreads();
  const int K = a.topk;
  // the next round's selections load while the current round is placed
  int32_t cn[8];
  load_sel8(a, idx, t0 * K + threadIdx.x, min(t0 + kRound, t1) * K, cn);
  for (int64_t r0 = t0; r0 < t1; r0 += kRound) {
    const int64_t e0 = r0 * K;  // this round's entries: e0 + threadIdx.x + 256 u
    int32_t c[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) c[u] = cn[u];
    const int64_t r1 = r0 + kRound;
    if (r1 < t1) load_sel8(a, idx, r1 * K + threadIdx.x, min(r1 + kRound, t1) * K, cn);
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      if (c[u] < 0) continue;
      const int tl = (int)((threadIdx.x + 256 * u) / K);  // token within the round
      atomicOr(&mask[2 * c[u] + (tl >> 5)], 1u << (tl & 31));
    }
    __syncthreads();
    int rank[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      rank[u] = -1;
      if (c[u] < 0) continue;
      const int e = threadIdx.x + 256 * u;
      const int tl = e / K;
      const uint32_t lo = mask[2 * c[u]], hi = mask[2 * c[u] + 1];
      const uint32_t below = (1u << (tl & 31)) - 1u;
      rank[u] = tl < 32 ? __popc(lo & below) : __popc(lo) + __popc(hi & below);
      const int32_t p = run[c[u]] + rank[u];
      HSA_DCHECK(p >= offs[c[u]] && p < offs[c[u] + 1]);
      const int64_t i = e0 + e;
      list[p] = (int32_t)(((i / K) << kSlotBits) | (i % K));
      epos[i] = p;
    }
    __syncthreads();
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      if (rank[u] != 0) continue;
      const int cc = c[u];
      run[cc] += __popc(mask[2 * cc]) + __popc(mask[2 * cc + 1]);
      mask[2 * cc] = 0u;
      mask[2 * cc + 1] = 0u;
    }
    __syncthreads();
  }
}

// Append (token << kSlotBits | slot) entries to the selected chunks' lists,
// and record where each selection landed (entry_pos).  With
// LDS bins: count locally, reserve one range per touched chunk with a global
// atomic, then place entries by LDS atomics inside the range.  The order
// inside a list does not affect results: every row is computed
// independently of the others that share its chunk.
__global__ void __launch_bounds__(256) scatter_kernel(PrefillArgs a, int64_t blocks_per_bg,
                                                      int use_lds) {
  extern __shared__ int32_t bins[];  // [2][n]: local counts, then running positions
  const int64_t bg = blockIdx.x / blocks_per_bg;
  const int64_t t0 = (blockIdx.x % blocks_per_bg) * kInvertTokens;
  const int64_t t1 = min(t0 + kInvertTokens, a.L);
  const int32_t* idx = a.idx + bg * a.nq * a.topk;
  const int32_t* offs = a.offs + bg * (a.n + 1);
  int32_t* cursor = a.cursor + bg * a.n;
  int32_t* list = a.list + bg * a.L * a.topk;
  int32_t* epos = a.entry_pos + bg * a.L * a.topk;
  if (!use_lds) {
    for (int64_t i = t0 * a.topk + threadIdx.x; i < t1 * a.topk; i += 256) {
      const int32_t c = idx[sel_of(a, i)];
      if (c >= 0) {
        const int32_t p = offs[c] + atomicAdd(&cursor[c], 1);
        HSA_DCHECK(p < offs[c + 1]);
        list[p] = (int32_t)(((i / a.topk) << kSlotBits) | (i % a.topk));
        epos[i] = p;
      }
    }
    return;
  }
  int32_t* local = bins;
  int32_t* pos = bins + a.n;
  for (int c = threadIdx.x; c < a.n; c += 256) local[c] = 0;
  __syncthreads();
  const int64_t e1 = t1 * a.topk;
  for (int64_t i0 = t0 * a.topk + threadIdx.x; i0 < e1; i0 += 8 * 256) {
    int32_t c[8];
    load_sel8(a, idx, i0, e1, c);
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (c[u] >= 0) atomicAdd(&local[c[u]], 1);
  }
  __syncthreads();
  for (int c = threadIdx.x; c < a.n; c += 256)
    pos[c] = local[c] != 0 ? offs[c] + atomicAdd(&cursor[c], local[c]) : 0;
  __syncthreads();
  for (int64_t i0 = t0 * a.topk + threadIdx.x; i0 < e1; i0 += 8 * 256) {
    int32_t c[8];
    load_sel8(a, idx, i0, e1, c);
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      if (c[u] < 0) continue;
      const int64_t i = i0 + 256 * u;
      const int32_t p = atomicAdd(&pos[c[u]], 1);
      HSA_DCHECK(p >= offs[c[u]] && p < offs[c[u] + 1]);
      list[p] = (int32_t)(((i / a.topk) << kSlotBits) | (i % a.topk));
      epos[i] = p;
    }
  }
}

// ---------------------------------------------------------------- attend --

// bf16: 4 waves x 32 rows; a row is (entry, head of the group).
template <int D>
__global__ void __launch_bounds__(kThreads) attend_bf16_kernel(PrefillArgs a, float scale_log2,
                                                               float score_scale) {
  __shared__ KVSmem<D> sm;
  int64_t bg;
  int c, e0, e1;
  if (!locate_tile(a, bg, c, e0, e1)) return;
  const int G = a.Hq / a.Hkv;
  const int b = (int)(bg / a.Hkv), g = (int)(bg % a.Hkv);
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int r = w * 32 + (lane & 31);
  const int e = e0 + r / G;
  const int hh = r % G;
  const bool valid = r < a.entries_per_tile * G && e < e1;
  int32_t entry = 0;
  if (valid) entry = a.list[bg * a.L * a.topk + e];
  const int64_t t = entry >> kSlotBits;
  const int h = g * G + hh;
  const uint16_t* Q = (const uint16_t*)a.Q;
  WaveAttn<D> st;
  wave_attn_init<D>(st, Q + (((int64_t)b * a.Hq + h) * a.L + t) * D, valid);
  const int64_t kv0 = (bg * a.L + (int64_t)c * a.S) * D;
  const bool wave_any = __ballot(valid) != 0;
  for (int kb = 0; kb < a.S; kb += kKeyBlock) {
    const int nk = min(kKeyBlock, a.S - kb);
    __syncthreads();
    load_kv_block<D>(sm, (const uint16_t*)a.K + kv0 + (int64_t)kb * D,
                     (const uint16_t*)a.V + kv0 + (int64_t)kb * D, nk);
    __syncthreads();
    if (wave_any) wave_attn_block<D>(st, sm, nk, valid ? nk : 0, scale_log2);
  }
  if (!wave_any) return;
  float s = wave_q_dot_half<D>(st, a.lmk + (bg * a.n + c) * D);
  s += __shfl_xor(s, 32, kWave);
  if (!valid) return;
  const int64_t row = partial_row(a, bg, e, hh);
  a.part_score[row] = s * score_scale;
  const float inv = st.l > 0.f ? 1.f / st.l : 0.f;
  uint16_t* po = (uint16_t*)a.partial + row * D;
  const int hf = lane >> 5;
#pragma unroll
  for (int bb = 0; bb < D / 32; ++bb)
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const int dd = 32 * bb + 8 * q4 + 4 * hf;
      const u32x2 v = {pack_bf16x2(st.o[bb][4 * q4] * inv, st.o[bb][4 * q4 + 1] * inv),
                       pack_bf16x2(st.o[bb][4 * q4 + 2] * inv, st.o[bb][4 * q4 + 3] * inv)};
      *(u32x2*)(po + dd) = v;
    }
}

// The chunk attention of one block (chunk_attend.h).
template <int D, bool S64>
__global__ void __launch_bounds__(kThreads, 2)
    attend_chunk_bf16_kernel(PrefillArgs a, float scale_log2, float score_scale) {
  __shared__ ChunkSmem<D> smem;
  attend_chunk_body<D, S64>(a, scale_log2, score_scale, blockIdx.x, smem);
}

// fp32: one wave per tile, one row per lane, online softmax on VALU.
template <int D>
__global__ void __launch_bounds__(64) attend_f32_kernel(PrefillArgs a, float scale,
                                                        float score_scale) {
  int64_t bg;
  int c, e0, e1;
  if (!locate_tile(a, bg, c, e0, e1)) return;
  const int G = a.Hq / a.Hkv;
  const int b = (int)(bg / a.Hkv), g = (int)(bg % a.Hkv);
  const int r = threadIdx.x;
  const int e = e0 + r / G;
  if (r >= a.entries_per_tile * G || e >= e1) return;
  const int32_t entry = a.list[bg * a.L * a.topk + e];
  const int64_t t = entry >> kSlotBits;
  const int h = g * G + r % G;
  const float* qrow = (const float*)a.Q + (((int64_t)b * a.Hq + h) * a.L + t) * D;
  float q[D], o[D];
#pragma unroll
  for (int x = 0; x < D; ++x) {
    q[x] = qrow[x];
    o[x] = 0.f;
  }
  const float* Kc = (const float*)a.K + (bg * a.L + (int64_t)c * a.S) * D;
  const float* Vc = (const float*)a.V + (bg * a.L + (int64_t)c * a.S) * D;
  float m = -INFINITY, l = 0.f;
  for (int j = 0; j < a.S; ++j) {
    float dot = 0.f;
#pragma unroll
    for (int x = 0; x < D; ++x) dot += q[x] * Kc[(int64_t)j * D + x];
    dot *= scale;
    const float mn = fmaxf(m, dot);
    const float al = expf(m - mn);
    const float p = expf(dot - mn);
    l = l * al + p;
#pragma unroll
    for (int x = 0; x < D; ++x) o[x] = o[x] * al + p * Vc[(int64_t)j * D + x];
    m = mn;
  }
  const float* lc = a.lmk + (bg * a.n + c) * D;
  float s = 0.f;
#pragma unroll
  for (int x = 0; x < D; ++x) s += q[x] * lc[x];
  const int64_t row = partial_row(a, bg, e, r % G);
  a.part_score[row] = s * score_scale;
  float* po = (float*)a.partial + row * D;
#pragma unroll
  for (int x = 0; x < D; ++x) po[x] = o[x] / l;
}

// ------------------------------------------------------------------ fuse --

// One group of D/VEC threads per (b, group, token, head of the group) row,
// heads fastest: the G heads of one selection entry are adjacent partial
// rows, so a token's gather reads runs of G * d elements.  The row's slot
// loads are all issued before the weighted sum.
template <int D, int DT, int KM>
__global__ void __launch_bounds__(kThreads) fuse_kernel(PrefillArgs a) {
  constexpr int VEC = DT == kF32 ? 4 : 8;
  constexpr int TPR = D / VEC;
  constexpr int RPB = kThreads / TPR;
  const int64_t r = (int64_t)blockIdx.x * RPB + threadIdx.x / TPR;
  const int cg = threadIdx.x % TPR;
  const int64_t total = (int64_t)a.B * a.Hq * a.L;
  if (r >= total) return;
  const int G = a.Hq / a.Hkv;
  const int hh = (int)(r % G);
  const int64_t bgt = r / G;  // (b, group, token)
  const int64_t t = bgt % a.L;
  const int64_t bg = bgt / a.L;
  const int64_t b = bg / a.Hkv;
  const int h = (int)(bg % a.Hkv) * G + hh;
  const int64_t row = (b * a.Hq + h) * a.L + t;  // output row
  const int64_t t0 = t / a.interval * a.interval;  // where the row's selection was made
  const int m = (int)min((int64_t)a.topk, min(t0 / a.S, a.n));
  const int32_t* epos = a.entry_pos + (bg * a.L + t) * a.topk;
  // every load is issued unconditionally (slots past m read row 0 and are
  // dropped afterwards): guarding them per lane would make each wait for
  // the one before
  int32_t ep[KM];
#pragma unroll
  for (int k = 0; k < KM; ++k) ep[k] = epos[min(k, a.topk - 1)];  // in bounds; unused past m
  int64_t pr[KM];
#pragma unroll
  for (int k = 0; k < KM; ++k) {
    HSA_DCHECK(k >= m || (ep[k] >= 0 && (int64_t)ep[k] < a.L * a.topk));
    pr[k] = k < m ? partial_row(a, bg, ep[k], hh) : 0;
  }
  u32x4 x[KM];
  float s[KM];
#pragma unroll
  for (int k = 0; k < KM; ++k) {
    x[k] = __builtin_nontemporal_load(
        (const u32x4*)((const char*)a.partial + (pr[k] * D + cg * VEC) * (DT == kF32 ? 4 : 2)));
    s[k] = a.part_score[pr[k]];
  }
  float smax = -INFINITY;
#pragma unroll
  for (int k = 0; k < KM; ++k) {
    if (k >= m) {
      x[k] = u32x4{0u, 0u, 0u, 0u};
      s[k] = -INFINITY;
    }
    smax = fmaxf(smax, s[k]);
  }
  float z = 0.f;
#pragma unroll
  for (int k = 0; k < KM; ++k) {
    s[k] = k < m ? expf(s[k] - smax) : 0.f;
    z += s[k];
  }
  const float iz = m > 0 ? 1.f / z : 0.f;
  float acc[VEC];
#pragma unroll
  for (int v = 0; v < VEC; ++v) acc[v] = 0.f;
#pragma unroll
  for (int k = 0; k < KM; ++k) {
    const float wk = s[k] * iz;
    if (DT == kF32) {
#pragma unroll
      for (int v = 0; v < 4; ++v) acc[v] += wk * __uint_as_float(x[k][v]);
    } else {
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        acc[2 * v] += wk * bf16_bits_to_f32(x[k][v] & 0xffffu);
        acc[2 * v + 1] += wk * bf16_bits_to_f32(x[k][v] >> 16);
      }
    }
  }
  const int64_t ob = row * D + cg * VEC;
  if (DT == kF32) {
    *(f32x4*)((float*)a.O + ob) = f32x4{acc[0], acc[1], acc[2], acc[3]};
  } else {
    *(u32x4*)((uint16_t*)a.O + ob) =
        u32x4{pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3]),
              pack_bf16x2(acc[4], acc[5]), pack_bf16x2(acc[6], acc[7])};
  }
  if (a.sel_w && cg < a.topk) {
    for (int k = cg; k < a.topk; k += TPR) {
      float wk = 0.f;
#pragma unroll
      for (int j = 0; j < KM; ++j)
        if (j == k) wk = s[j] * iz;
      a.sel_w[row * a.topk + k] = wk;
    }
  }
}

template <int D, int KM>
hipError_t launch_select_dt(const PrefillArgs& a, hipStream_t stream) {
  const int64_t nqt = (a.nq + 63) / 64;
  const int64_t blocks = (int64_t)a.B * a.Hkv * nqt;
  if (a.dtype == kF32)
    launch<select_valu_kernel<D, KM, kF32>>(dim3((unsigned)blocks), dim3(kThreads), 0, stream, a,
                                            nqt);
  else
    launch<select_valu_kernel<D, KM, kBF16>>(dim3((unsigned)blocks), dim3(kThreads), 0, stream, a,
                                             nqt);
  return hipGetLastError();
}

template <int D, int KM>
hipError_t launch_select_mfma(const PrefillArgs& a, hipStream_t stream) {
  const int64_t nqt = (a.nq + 127) / 128;
  const int64_t blocks = (int64_t)a.B * a.Hkv * nqt;
  launch<select_mfma_kernel<D, KM>>(dim3((unsigned)blocks), dim3(kThreads), 0, stream, a, nqt);
  return hipGetLastError();
}

template <int D>
hipError_t launch_select_d(const PrefillArgs& a, hipStream_t stream) {
  if (a.dtype == kBF16) {
    if (a.topk <= 8) return launch_select_mfma<D, 8>(a, stream);
    if (a.topk <= 16) return launch_select_mfma<D, 16>(a, stream);
    return launch_select_mfma<D, 32>(a, stream);
  }
  if (a.topk <= 8) return launch_select_dt<D, 8>(a, stream);
  if (a.topk <= 16) return launch_select_dt<D, 16>(a, stream);
  return launch_select_dt<D, 32>(a, stream);
}

}  // namespace

int prefill_entries_per_tile(int dtype, int G, int S) {
  if (dtype == kF32) return 64 / G;
  if (S <= kKeyBlock) return kChunkUnitRows / G;
  return (kThreads / kWave) * 32 / G;  // one 32-row tile per wave
}

hipError_t prefill_select(const PrefillArgs& a, hipStream_t stream) {
  if (a.L == 0) return hipSuccess;
  return a.d == 64 ? launch_select_d<64>(a, stream) : launch_select_d<128>(a, stream);
}

hipError_t prefill_invert(const PrefillArgs& a, hipStream_t stream) {
  if (a.n == 0) return hipSuccess;
  const int64_t BG = (int64_t)a.B * a.Hkv;
  // counts and cursor were cleared by the select launch
  hipError_t e;
  const int64_t bpb = (a.L + kInvertTokens - 1) / kInvertTokens;
  const int use_lds = a.n <= kInvertLdsBins;
  const bool ordered = a.ordered && a.n <= kInvertDetBins;
  const size_t lds1 = use_lds ? (size_t)a.n * sizeof(int32_t) : 0;
  launch<count_kernel>(dim3((unsigned)(BG * bpb)), dim3(256), lds1, stream, a, bpb, use_lds);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  launch<scan_kernel>(dim3((unsigned)BG), dim3(1024), 0, stream, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (ordered)
    launch<scatter_ordered_kernel>(dim3((unsigned)(BG * bpb)), dim3(256), 3 * lds1, stream, a, bpb);
  else
    launch<scatter_kernel>(dim3((unsigned)(BG * bpb)), dim3(256), 2 * lds1, stream, a, bpb,
                           use_lds);
  return hipGetLastError();
}

hipError_t prefill_attend(const PrefillArgs& a, hipStream_t stream) {
  if (a.n == 0) return hipSuccess;
  const int64_t blocks = (int64_t)a.B * a.Hkv * a.tiles_ub;
  const float scale = 1.0f / sqrtf((float)a.d);
  const float score_scale = scale;
  if (a.dtype == kF32) {
    if (a.d == 64)
      launch<attend_f32_kernel<64>>(dim3((unsigned)blocks), dim3(64), 0, stream, a, scale,
                                    score_scale);
    else
      launch<attend_f32_kernel<128>>(dim3((unsigned)blocks), dim3(64), 0, stream, a, scale,
                                     score_scale);
  } else if (a.S <= kKeyBlock) {
    const float sl2 = scale * 1.4426950408889634f;
    const dim3 grid((unsigned)blocks), block(kThreads);
    if (a.d == 64) {
      if (a.S == kKeyBlock)
        launch<attend_chunk_bf16_kernel<64, true>>(grid, block, 0, stream, a, sl2, score_scale);
      else
        launch<attend_chunk_bf16_kernel<64, false>>(grid, block, 0, stream, a, sl2, score_scale);
    } else {
      if (a.S == kKeyBlock)
        launch<attend_chunk_bf16_kernel<128, true>>(grid, block, 0, stream, a, sl2, score_scale);
      else
        launch<attend_chunk_bf16_kernel<128, false>>(grid, block, 0, stream, a, sl2, score_scale);
    }
  } else {
    const float sl2 = scale * 1.4426950408889634f;
    if (a.d == 64)
      launch<attend_bf16_kernel<64>>(dim3((unsigned)blocks), dim3(kThreads), 0, stream, a, sl2,
                                     score_scale);
    else
      launch<attend_bf16_kernel<128>>(dim3((unsigned)blocks), dim3(kThreads), 0, stream, a, sl2,
                                      score_scale);
  }
  return hipGetLastError();
}

template <int D, int DT>
hipError_t launch_fuse_dt(const PrefillArgs& a, int64_t blocks, hipStream_t stream) {
  if (a.topk <= 8)
    launch<fuse_kernel<D, DT, 8>>(dim3((unsigned)blocks), dim3(kThreads), 0, stream, a);
  else if (a.topk <= 16)
    launch<fuse_kernel<D, DT, 16>>(dim3((unsigned)blocks), dim3(kThreads), 0, stream, a);
  else
    launch<fuse_kernel<D, DT, 32>>(dim3((unsigned)blocks), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

hipError_t prefill_fuse(const PrefillArgs& a, hipStream_t stream) {
  const int64_t rows = (int64_t)a.B * a.Hq * a.L;
  if (rows == 0) return hipSuccess;
  const int VEC = a.dtype == kF32 ? 4 : 8;
  const int rpb = kThreads / (a.d / VEC);
  const int64_t blocks = (rows + rpb - 1) / rpb;
  if (a.dtype == kF32)
    return a.d == 64 ? launch_fuse_dt<64, kF32>(a, blocks, stream)
                     : launch_fuse_dt<128, kF32>(a, blocks, stream);
  return a.d == 64 ? launch_fuse_dt<64, kBF16>(a, blocks, stream)
                   : launch_fuse_dt<128, kBF16>(a, blocks, stream);
}

}  // namespace hsa
