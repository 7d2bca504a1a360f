// decode.hip - HSA decode: one query per sequence against a KV cache
// ([HSA] Methodology: retrieval of the top-K chunks from the landmark memory;
// [HiLS] abstract: per-chunk attention fused by the retrieval scores).
//
//  1. scan   : grid (b, group, slice).  Streams the slice's fp32 landmarks
//              once (the bandwidth-bound step; the next batch of rows loads
//              while the current one is scored), scores them against the
//              group-summed query and keeps the slice's top-K as 64-bit keys
//              (score, then lower index): per-wave bitonic sorts merged into
//              one sorted list.
//  2. attend : chunks of at most 64 keys: R = ceil(K/8) blocks of 8 waves per
//              (b, group), one wave per selected chunk (keys and values in
//              registers); every block merges the slices' candidates into
//              the same ordered top-K; with K <= 8 the block also fuses.
//              Longer chunks: one block per (b, group, rank k) staging the
//              chunk in LDS, every head of the group attending to it.
//  3. fuse   : one block per (b, group): per head, a softmax over the
//              selected chunks' s_h weights the chunk outputs (when the
//              attention blocks did not fuse).
#include <math.h>

#include <type_traits>

#include "hsa_common.h"
#include "kernels.h"

namespace hsa {
namespace {

constexpr int kThreads = 256;
constexpr int kMaxCand = 8192;  // candidates per (b, group) the merge reads
constexpr int kMaxSlice = 4096;

// The K largest of the distinct keys >= lo among keys[0..M) (LDS or
// global), written unordered to out[0..min(K, count)); returns that count.
// Radix select, 8 bits at a time from the top, until the bin holding the
// K-th largest key is needed whole.  Called by all NT (>= 256) threads of
// the block; `hist` is 256 ints of LDS, `sv` 4 ints.
template <int NT>
__device__ int block_topk_ge(const uint64_t* keys, int M, uint64_t lo, int K, uint64_t* out,
                             int* hist, int* sv) {
  const int tid = threadIdx.x;
  if (tid == 0) sv[3] = 0;
  __syncthreads();
  int mine = 0;
  for (int i = tid; i < M; i += NT) mine += keys[i] >= lo;
  if (mine) atomicAdd(&sv[3], mine);
  __syncthreads();
  const int n = sv[3];
  __syncthreads();
  if (n <= K) {
    if (tid == 0) sv[3] = 0;
    __syncthreads();
    for (int i = tid; i < M; i += NT) {
      const uint64_t k = keys[i];
      if (k >= lo) out[atomicAdd(&sv[3], 1)] = k;
    }
    __syncthreads();
    return n;
  }
  uint64_t prefix = 0, mask = 0;
  int need = K;
  for (int shift = 56; shift >= 0; shift -= 8) {
    if (tid < 256) hist[tid] = 0;
    __syncthreads();
    for (int i = tid; i < M; i += NT) {
      const uint64_t k = keys[i];
      if (k >= lo && (k & mask) == prefix) atomicAdd(&hist[(int)((k >> shift) & 255u)], 1);
    }
    __syncthreads();
    if (tid < 64) {
      // lane l owns digits 255-4l .. 252-4l (descending)
      int c[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) c[q] = hist[255 - 4 * tid - q];
      const int s = c[0] + c[1] + c[2] + c[3];
      int incl = s;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int y = __shfl_up(incl, o, kWave);
        if (tid >= o) incl += y;
      }
      const int excl = incl - s;
      if (excl < need && need <= incl) {
        int cum = excl;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          if (cum + c[q] >= need) {
            sv[0] = 255 - 4 * tid - q;
            sv[1] = need - cum;
            sv[2] = c[q];
            break;
          }
          cum += c[q];
        }
      }
    }
    __syncthreads();
    const int digit = sv[0];
    need = sv[1];
    const int bin = sv[2];
    prefix |= (uint64_t)digit << shift;
    mask |= (uint64_t)0xff << shift;
    __syncthreads();
    if (bin == need) break;
  }
  if (tid == 0) sv[3] = 0;
  __syncthreads();
  for (int i = tid; i < M; i += NT) {
    const uint64_t k = keys[i];
    if (k >= lo && (k & mask) >= prefix) out[atomicAdd(&sv[3], 1)] = k;
  }
  __syncthreads();
  return K;
}

// Bitonic sort of one 64-bit key per lane across the wave, descending
// (lane 0 ends with the largest).
__device__ __forceinline__ uint64_t wave_sort_desc_u64(uint64_t x) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int k = 2; k <= kWave; k <<= 1)
#pragma unroll
    for (int j = k >> 1; j > 0; j >>= 1) {
      const uint64_t y = lane_xor_u64(x, j);
      // in a block of k lanes that ends ascending (lane & k set) the lower
      // lane of each pair keeps the smaller key, otherwise the larger
      const bool take_max = ((lane & j) == 0) == ((lane & k) == 0);
      const uint64_t hi = x > y ? x : y, lo = x > y ? y : x;
      x = take_max ? hi : lo;
    }
  return x;
}

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
  for (int o = kWave / 2; o > 0; o >>= 1) {
    const uint64_t y = __shfl_xor(v, o, kWave);
    v = y > v ? y : v;
  }
  return v;
}

// The value of the partner lane whose index differs in bit log2(M) within
// a group of 2M lanes (M = 16: across the two 16-lane rows of a 32-lane
// group; M = 8, 4: the mirrored lane of the 16- or 8-lane half row, which
// differs in that bit and in all lower ones; M = 2, 1: the quad partner).
template <int M>
__device__ __forceinline__ float partner(float v) {
  const int x = __builtin_bit_cast(int, v);
  int y;
  if constexpr (M == 16) y = __shfl_xor(x, 16, kWave);
  else if constexpr (M == 8) y = __builtin_amdgcn_mov_dpp(x, 0x140, 0xF, 0xF, false);
  else if constexpr (M == 4) y = __builtin_amdgcn_mov_dpp(x, 0x141, 0xF, 0xF, false);
  else if constexpr (M == 2) y = __builtin_amdgcn_mov_dpp(x, 0x4E, 0xF, 0xF, false);
  else y = __builtin_amdgcn_mov_dpp(x, 0xB1, 0xF, 0xF, false);
  return __builtin_bit_cast(float, y);
}

// p[0..8) are a lane's partial dot products for 8 rows, each row spread over
// the LPR lanes of its lane group.  Three halving exchanges leave each lane
// one row's partial (row index from bits LPR/2, LPR/4, LPR/8 of the lane),
// the remaining steps finish the sum over the group: 8 rows cost
// 4 + 2 + 1 + log2(LPR/8) exchanges instead of 8 log2(LPR).
template <int LPR>
__device__ __forceinline__ float reduce8_rows(const float (&p)[8], int li, int& row) {
  constexpr int M1 = LPR / 2, M2 = LPR / 4, M3 = LPR / 8;
  const bool h1 = li & M1, h2 = li & M2, h3 = li & M3;
  float q[4], r[2];
#pragma unroll
  for (int j = 0; j < 4; ++j) q[j] = (h1 ? p[j + 4] : p[j]) + partner<M1>(h1 ? p[j] : p[j + 4]);
#pragma unroll
  for (int j = 0; j < 2; ++j) r[j] = (h2 ? q[j + 2] : q[j]) + partner<M2>(h2 ? q[j] : q[j + 2]);
  float s = (h3 ? r[1] : r[0]) + partner<M3>(h3 ? r[0] : r[1]);
  if constexpr (M3 >= 4) s += partner<2>(s);
  if constexpr (M3 >= 2) s += partner<1>(s);
  row = (h3 ? 1 : 0) + (h2 ? 2 : 0) + (h1 ? 4 : 0);
  return s;
}

// Descending bitonic merge of a bitonic sequence of 64 keys, one per lane.
__device__ __forceinline__ uint64_t wave_merge_desc_u64(uint64_t x) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int j = kWave / 2; j > 0; j >>= 1) {
    const uint64_t y = lane_xor_u64(x, j);
    x = ((lane & j) == 0) == (x > y) ? x : y;
  }
  return x;
}

// The K (<= 32) largest of keys[0..M) in LDS, descending in lanes 0..K-1 of
// wave 0 (zeros past the M-th).  Each wave sorts its 64-key pieces and
// merges them into a running top list; wave 0 then merges the four lists.
// `lists` is 4 * 32 keys of LDS.  Called by all threads.
__device__ uint64_t block_topk_sorted(const uint64_t* keys, int M, int K, uint64_t* lists) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  uint64_t run = 0ull;
  for (int c = w; c * kWave < M; c += kThreads / kWave) {
    const int i = c * kWave + lane;
    uint64_t x = wave_sort_desc_u64(i < M ? keys[i] : 0ull);
    // lanes 0..31: the piece's 32 largest, descending; lanes 32..63: the
    // running list reversed (ascending): a bitonic sequence
    const uint64_t rr = __shfl(run, kWave - 1 - lane, kWave);
    x = wave_merge_desc_u64(lane < 32 ? x : rr);
    run = lane < K ? x : 0ull;
  }
  if (lane < 32) lists[w * 32 + lane] = run;
  __syncthreads();
  if (w == 0) {
#pragma unroll 1
    for (int v = 1; v < kThreads / kWave; ++v) {
      const uint64_t x = lane < 32 ? lists[v * 32 + lane] : 0ull;
      const uint64_t rr = __shfl(run, kWave - 1 - lane, kWave);
      run = wave_merge_desc_u64(lane < 32 ? x : rr);
      run = lane < K ? run : 0ull;
    }
  }
  return run;
}

template <int D, int DT>
__global__ void __launch_bounds__(kThreads) scan_kernel(DecodeArgs a) {
  __shared__ float u[D];
  extern __shared__ uint64_t keys[];  // [slice]
  __shared__ uint64_t lists[4 * 32];
  const int64_t bg = blockIdx.x / a.n_slices;
  const int sl = blockIdx.x % a.n_slices;
  const int b = (int)(bg / a.Hkv), g = (int)(bg % a.Hkv);
  const int G = a.Hq / a.Hkv;
  const int64_t c_begin = (int64_t)sl * a.slice;
  const int M = (int)max((int64_t)0, min((int64_t)a.slice, a.n_avail - c_begin));
  constexpr int LPR = D / 4;        // lanes per landmark row (16 bytes each)
  constexpr int RPW = kWave / LPR;  // rows per wave step
  constexpr int U = 8;              // row steps per batch (the reduction takes 8)
  constexpr int STEP = kThreads / kWave * RPW;  // rows per block step
  constexpr int CH = STEP * U;                  // rows per batch
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int li = lane % LPR, sub = lane / LPR;
  const float* lm = a.lmk + (bg * a.lmk_chunks + c_begin) * D + 4 * li;
  auto load = [&](int r0, f32x4 (&x)[U]) {
#pragma unroll
    for (int uu = 0; uu < U; ++uu) {
      const int row = r0 + uu * STEP + w * RPW + sub;
      if (row < M)
        x[uu] = __builtin_nontemporal_load((const f32x4*)(lm + (int64_t)row * D));
      else
        x[uu] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
  };
  // the first batch is in flight while the group's query sum forms
  f32x4 xa[U], xb[U];
  load(0, xa);
  if (threadIdx.x < D) {
    const int x = threadIdx.x;
    const int64_t q0 = ((int64_t)b * a.Hq + g * G) * D + x;
    float acc = 0.f;
    for (int h0 = 0; h0 < G; h0 += 8) {
      float v[8];
      // unguarded loads (heads past G re-read head G - 1 and are not added):
      // guarded ones would each wait for the one before
#pragma unroll
      for (int j = 0; j < 8; ++j) v[j] = load_elem<DT>(a.q, q0 + min(h0 + j, G - 1) * D);
#pragma unroll
      for (int j = 0; j < 8; ++j)
        if (h0 + j < G) acc += v[j];
    }
    u[x] = acc;
  }
  block_sync_lds();
  const f32x4 u4 = *(const f32x4*)(&u[4 * li]);
  auto score = [&](int r0, const f32x4 (&x)[U]) {
    float p[U];
#pragma unroll
    for (int uu = 0; uu < U; ++uu)
      p[uu] = u4[0] * x[uu][0] + u4[1] * x[uu][1] + u4[2] * x[uu][2] + u4[3] * x[uu][3];
    int uu;
    const float s = reduce8_rows<LPR>(p, li, uu);
    const int row = r0 + uu * STEP + w * RPW + sub;
    if (li % (LPR / 8) == 0 && row < M) keys[row] = select_key(s, (uint32_t)(c_begin + row));
  };
  // double-buffered: the next batch loads while the current one is scored
  for (int r0 = 0; r0 < M; r0 += 2 * CH) {
    if (r0 + CH < M) load(r0 + CH, xb);
    score(r0, xa);
    if (r0 + CH >= M) break;
    if (r0 + 2 * CH < M) load(r0 + 2 * CH, xa);
    score(r0 + CH, xb);
  }
  __syncthreads();
  const uint64_t top = block_topk_sorted(keys, M, a.topk, lists);
  if (w == 0) {
    const int got = min(M, a.topk);
    uint64_t* out = a.cand + (bg * a.n_slices + sl) * a.topk;
    if (lane < a.topk) out[lane] = lane < got ? top : 0ull;
    const uint64_t mn = __shfl(top, max(got - 1, 0), kWave);
    if (lane == 0)
      *(u64x2*)(a.cand_mm + (bg * a.n_slices + sl) * 2) =
          u64x2{got > 0 ? top : 0ull, got == a.topk ? mn : 0ull};
  }
}

constexpr int kMergeLds = 1024;  // candidates above the bound kept in LDS

// The ordered top-K chunks of one (b, group) from its slices' candidate
// lists (n_slices lists of K keys, 0 = empty): order[0..K) = chunk indices
// by (score desc, index asc), -1 past the available ones; returns their
// count.  Up to 64 candidates are sorted by one wave in registers.  More
// are first cut at a lower bound of the K-th largest key (the largest
// smallest-kept key of a full slice) and the survivors sorted the same way,
// or, past 64 survivors, radix-selected.  Deterministic: every block of the
// (b, group) gets the same list.  Called by all NT threads of the block.
template <int NT>
__device__ int merge_candidates(const DecodeArgs& a, int64_t bg, uint64_t* ck, uint64_t* top,
                                int32_t* order, int* hist, int* sv, uint64_t* red) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int K = a.topk;
  const int total = a.n_slices * K;
  const uint64_t* cand = a.cand + bg * (int64_t)total;
  const uint64_t* src = cand;
  int n = total;
  uint64_t lb = 1;  // keys are nonzero
  if (total > kWave) {
    // Lower bounds of the K-th largest key: a full slice's smallest kept
    // key, and the K-th largest of the maxima of any 64 slices (K distinct
    // keys reach it).  Lane l of a wave takes slice 64 * grp + l.
    const uint64_t* mm = a.cand_mm + bg * (int64_t)a.n_slices * 2;
    uint64_t m = 0;
    for (int grp = w; grp * kWave < a.n_slices; grp += NT / kWave) {
      const int j = grp * kWave + lane;
      u64x2 v = {0ull, 0ull};
      if (j < a.n_slices) v = *(const u64x2*)(mm + 2 * j);
      m = v[1] > m ? v[1] : m;
      const uint64_t kth = __shfl(wave_sort_desc_u64(v[0]), K - 1, kWave);
      m = kth > m ? kth : m;
    }
    m = wave_max_u64(m);
    if (lane == 0) red[w] = m;
    if (tid == 0) sv[3] = 0;
    __syncthreads();
    for (int x = 0; x < NT / kWave; ++x) lb = red[x] > lb ? red[x] : lb;
    // only slices whose largest key reaches the bound hold survivors; their
    // loads have fixed trip counts (K <= 32 is uniform) so all are in flight
    for (int grp = w; grp * kWave < a.n_slices; grp += NT / kWave) {
      const int j = grp * kWave + lane;
      if (j >= a.n_slices || mm[2 * j] < lb) continue;
      const uint64_t* cs = cand + (int64_t)j * K;
      uint64_t x[32];
#pragma unroll
      for (int kk = 0; kk < 32; ++kk) x[kk] = kk < K ? cs[kk] : 0ull;
#pragma unroll
      for (int kk = 0; kk < 32; ++kk)
        if (x[kk] >= lb) {
          const int p = atomicAdd(&sv[3], 1);
          if (p < kMergeLds) ck[p] = x[kk];
        }
    }
    __syncthreads();
    n = sv[3];
    __syncthreads();
    if (n <= kMergeLds) src = ck;
  }
  if (n <= kWave) {
    if (w == 0) {
      uint64_t x = lane < n ? src[lane] : 0ull;
      if (x < lb) x = 0ull;
      x = wave_sort_desc_u64(x);
      if (lane < K) order[lane] = x != 0ull ? (int32_t)key_index(x) : -1;
      const uint64_t live = __ballot(lane < K && x != 0ull);
      if (lane == 0) sv[0] = __popcll(live);
    }
    __syncthreads();
    const int got = sv[0];
    __syncthreads();
    return got;
  }
  const int got = block_topk_ge<NT>(src, n <= kMergeLds ? n : total, lb, K, top, hist, sv);
  if (tid < K) {
    int32_t idx = -1;
    if (tid < got) {
      const uint64_t k = top[tid];
      int rank = 0;
      for (int j = 0; j < got; ++j) rank += top[j] > k;
      order[rank] = (int32_t)key_index(k);
    } else {
      order[tid] = idx;
    }
  }
  __syncthreads();
  return got;
}

// Per (b, group, rank k): the chunk's keys/values are staged in LDS
// 64 (bf16) or 32 (fp32) rows at a time with 16-byte loads; wave = head
// (looping over the group's heads), lane = key for the logits and lane =
// output columns for the weighted sum (the weights pass through LDS).
template <int D, int DT>
__global__ void __launch_bounds__(kThreads) attend_kernel(DecodeArgs a, float scale) {
  constexpr int KB = DT == kF32 ? 32 : 64;   // keys per LDS block
  constexpr int EB = DT == kF32 ? 4 : 2;     // bytes per element
  constexpr int VE = 16 / EB;                // elements per 16-byte piece
  constexpr int KSTR = D + VE;               // key row stride, padded by 16 bytes
  constexpr int CPL = D / 64;                // output columns per lane: 2 * lane + x
  typedef typename std::conditional<DT == kF32, float, uint16_t>::type T;
  __shared__ __attribute__((aligned(16))) T ks[KB * KSTR];
  __shared__ __attribute__((aligned(16))) T vs[KB * D];
  __shared__ __attribute__((aligned(16))) float ps[kThreads / kWave][KB];
  __shared__ uint64_t top[32];
  __shared__ uint64_t red[kThreads / kWave];
  __shared__ int32_t order[32];
  __shared__ int hist[256];
  __shared__ int sv[4];
  // qs [G * D] fp32, then the merge's candidate buffer when it needs one
  extern __shared__ __attribute__((aligned(16))) float dyn[];
  const int G = a.Hq / a.Hkv;
  float* qs = dyn;
  uint64_t* ck = (uint64_t*)(dyn + ((G * D + 1) & ~1));
  const int64_t bg = blockIdx.x / a.topk;
  const int k = blockIdx.x % a.topk;
  const int b = (int)(bg / a.Hkv), g = (int)(bg % a.Hkv);
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int64_t qrow0 = (int64_t)b * a.Hq + g * G;  // first head row of the group
  for (int e = tid; e < G * D; e += kThreads) qs[e] = load_elem<DT>(a.q, qrow0 * D + e);
  if (a.n_avail == 0) {
    // no chunk lies fully before the query: nothing is selected
    if (k == 0)
      for (int e = tid; e < a.topk; e += kThreads) a.sel[bg * a.topk + e] = -1;
    return;
  }
  const int got = merge_candidates<kThreads>(a, bg, ck, top, order, hist, sv, red);
  if (k == 0)
    for (int e = tid; e < a.topk; e += kThreads) a.sel[bg * a.topk + e] = order[e];
  const int c = k < got ? order[k] : -1;
  if (c < 0 || c >= a.n_avail) return;
  // this lane's landmark columns (for s_h)
  const float* lc = a.lmk + (bg * a.lmk_chunks + c) * D;
  float lmv[CPL];
#pragma unroll
  for (int x = 0; x < CPL; ++x) lmv[x] = lc[CPL * lane + x];
  float m[8], l[8], o[8][CPL];
#pragma unroll
  for (int hi = 0; hi < 8; ++hi) {
    m[hi] = -INFINITY;
    l[hi] = 0.f;
#pragma unroll
    for (int x = 0; x < CPL; ++x) o[hi][x] = 0.f;
  }
  const int64_t base = (bg * a.n_max + (int64_t)c * a.S) * D;
  const T* Kg = (const T*)a.Kc + base;
  const T* Vg = (const T*)a.Vc + base;
  constexpr int PPR = D / VE;  // 16-byte pieces per row
  for (int kb = 0; kb < a.S; kb += KB) {
    const int nk = min(KB, a.S - kb);
    __syncthreads();
    for (int e = tid; e < KB * PPR; e += kThreads) {
      const int row = e / PPR, pc = e % PPR;
      u32x4 kv = {0u, 0u, 0u, 0u}, vv = {0u, 0u, 0u, 0u};
      if (row < nk) {
        kv = *(const u32x4*)(Kg + (int64_t)(kb + row) * D + pc * VE);
        vv = *(const u32x4*)(Vg + (int64_t)(kb + row) * D + pc * VE);
      }
      *(u32x4*)(&ks[row * KSTR + pc * VE]) = kv;
      *(u32x4*)(&vs[row * D + pc * VE]) = vv;
    }
    __syncthreads();
    const int nk4 = (nk + 3) & ~3;  // staged rows past nk are zero
    int hi = 0;
    for (int hh = w; hh < G; hh += kThreads / kWave, ++hi) {
      float dot = -INFINITY;
      if (lane < nk) {
        float acc = 0.f;
        for (int x = 0; x < D; x += VE) {
          const u32x4 kx = *(const u32x4*)(&ks[lane * KSTR + x]);
          if (DT == kF32) {
#pragma unroll
            for (int v = 0; v < 4; ++v) acc += qs[hh * D + x + v] * __uint_as_float(kx[v]);
          } else {
#pragma unroll
            for (int v = 0; v < 4; ++v) {
              acc += qs[hh * D + x + 2 * v] * bf16_bits_to_f32(kx[v] & 0xffffu);
              acc += qs[hh * D + x + 2 * v + 1] * bf16_bits_to_f32(kx[v] >> 16);
            }
          }
        }
        dot = acc * scale;
      }
      const float bm = wave_max(dot);
      const float mn = fmaxf(m[hi], bm);
      const float al = expf(m[hi] - mn);
      const float p = lane < nk ? expf(dot - mn) : 0.f;
      l[hi] = l[hi] * al + wave_sum(p);
      m[hi] = mn;
#pragma unroll
      for (int x = 0; x < CPL; ++x) o[hi][x] *= al;
      // the weights go through this wave's own LDS row
      if (lane < KB) ps[w][lane] = p;
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      for (int j = 0; j < nk4; j += 4) {
        const f32x4 p4 = *(const f32x4*)(&ps[w][j]);
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const T* vr = vs + (j + jj) * D + CPL * lane;
          if (CPL == 2) {
            if (DT == kF32) {
              const f32x2 v2 = *(const f32x2*)vr;
              o[hi][0] += p4[jj] * v2[0];
              o[hi][CPL - 1] += p4[jj] * v2[1];
            } else {
              const uint32_t v2 = *(const uint32_t*)vr;
              o[hi][0] += p4[jj] * bf16_bits_to_f32(v2 & 0xffffu);
              o[hi][CPL - 1] += p4[jj] * bf16_bits_to_f32(v2 >> 16);
            }
          } else {
            o[hi][0] += p4[jj] * load_elem<DT>(vs, (int64_t)(j + jj) * D + lane);
          }
        }
      }
      __builtin_amdgcn_wave_barrier();
    }
  }
  int hi = 0;
  for (int hh = w; hh < G; hh += kThreads / kWave, ++hi) {
    float s = 0.f;
#pragma unroll
    for (int x = 0; x < CPL; ++x) s += qs[hh * D + CPL * lane + x] * lmv[x];
    s = wave_sum(s);
    const int64_t row = (qrow0 + hh) * a.topk + k;
    if (lane == 0) a.part_s[row] = s * scale;
    const float inv = 1.f / l[hi];
    float* po = a.part_o + row * D + CPL * lane;
    if (CPL == 2)
      *(f32x2*)po = f32x2{o[hi][0] * inv, o[hi][CPL - 1] * inv};
    else
      po[0] = o[hi][0] * inv;
  }
}

// Per (b, group): softmax over the selected chunks' per-head scores and the
// weighted sum of the chunk outputs; no selected chunk gives zeros.
template <int D, int DT>
__global__ void __launch_bounds__(kThreads) fuse_kernel(DecodeArgs a) {
  __shared__ float wts[32 * 32];  // [head of the group][rank]
  __shared__ int s_got;
  const int64_t bg = blockIdx.x;
  const int b = (int)(bg / a.Hkv), g = (int)(bg % a.Hkv);
  const int G = a.Hq / a.Hkv;
  const int tid = threadIdx.x;
  const int64_t qrow0 = (int64_t)b * a.Hq + g * G;
  if (tid == 0) {
    const int32_t* sel = a.sel + bg * a.topk;
    int m = 0;
    while (m < a.topk && sel[m] >= 0) ++m;
    s_got = m;
  }
  __syncthreads();
  const int got = s_got;
  for (int e = tid; e < G * a.topk; e += kThreads) {
    const int64_t row = qrow0 + e / a.topk;
    const int kk = e % a.topk;
    const float* sc = a.part_s + row * a.topk;
    float smax = -INFINITY, z = 0.f;
    for (int j = 0; j < got; ++j) smax = fmaxf(smax, sc[j]);
    for (int j = 0; j < got; ++j) z += expf(sc[j] - smax);
    const float wk = kk < got ? expf(sc[kk] - smax) / z : 0.f;
    wts[e] = wk;
    if (a.sel_w) a.sel_w[row * a.topk + kk] = wk;
  }
  __syncthreads();
  for (int e = tid; e < G * D; e += kThreads) {
    const int hh = e / D, x = e % D;
    const int64_t row = qrow0 + hh;
    float acc = 0.f;
    for (int kk = 0; kk < got; ++kk)
      acc += wts[hh * a.topk + kk] * a.part_o[(row * a.topk + kk) * D + x];
    store_elem<DT>(a.o, row * D + x, acc);
  }
}

// Chunks of at most 64 keys: R = ceil(K / 8) blocks of 8 waves per (b,
// group), wave w of block rb taking rank 8 rb + w.  Each block runs the
// merge itself; lane = key for the logits (the key row in registers, packed
// bf16 dot products) and lane = output columns for the weighted value sum
// (the values in registers, the weights broadcast from LDS).  With R = 1 the
// chunk outputs of a round of `fused_heads` heads stay in LDS and the block
// fuses them (the softmax over the ranks' s_h) itself; with R > 1 they go to
// the partial buffers for fuse_kernel.
constexpr int kFusedWaves = 8;
constexpr int kFusedThreads = kFusedWaves * kWave;
constexpr int kFusedPartBytes = 32768;  // LDS for one round's chunk outputs
constexpr int kFusedMaxLds = 61440;  // dynamic LDS bytes (static arrays take ~1.5 KB)

__host__ __device__ inline int fused_heads(int G, int K, int D) {
  int hg = kFusedPartBytes / (K * D * 4);
  hg = hg < 1 ? 1 : hg;
  hg = hg > 8 ? 8 : hg;
  return hg < G ? hg : G;
}

__host__ __device__ inline int round4(int x) { return (x + 3) & ~3; }


// LDS floats before the merge's candidate buffer
__host__ __device__ inline int fused_lds_floats(int G, int K, int D, int dt) {
  const int hg = fused_heads(G, K, D);
  return G * D + (dt == kBF16 ? G * D / 2 : 0) + hg * K * D + 2 * round4(hg * K) +
         kFusedWaves * hg * kWave;
}

// dynamic LDS bytes of the fused kernel, 0 if it does not apply
size_t fused_lds_bytes(const DecodeArgs& a) {
  const int G = a.Hq / a.Hkv;
  if (a.S > kWave) return 0;
  size_t bytes = (size_t)fused_lds_floats(G, a.topk, a.d, a.dtype) * sizeof(float);
  if ((int64_t)a.n_slices * a.topk > kWave) bytes += (size_t)kMergeLds * sizeof(uint64_t);
  return bytes <= (size_t)kFusedMaxLds ? bytes : 0;
}

template <int D, int DT>
__global__ void __launch_bounds__(kFusedThreads) attend_fused_kernel(DecodeArgs a, float scale) {
  constexpr int NW = kFusedWaves, NT = kFusedThreads;
  constexpr int CPL = D / 64;                  // output columns per lane
  constexpr int KV4 = D * (DT == kF32 ? 4 : 2) / 16;  // 16-byte pieces per key row
  __shared__ uint64_t top[32];
  __shared__ uint64_t red[NW];
  __shared__ int32_t order[32];
  __shared__ int hist[256];
  __shared__ int sv[4];
  extern __shared__ __attribute__((aligned(16))) float dyn[];
  const int G = a.Hq / a.Hkv;
  const int K = a.topk;
  const int HG = fused_heads(G, K, D);
  float* qf = dyn;                                             // [G][D] fp32
  uint32_t* qb = (uint32_t*)(qf + G * D);                      // [G][D/2] bf16 pairs
  float* part = (float*)(qb + (DT == kBF16 ? G * D / 2 : 0));  // [HG][K][D]
  float* psc = part + HG * K * D;                              // [HG][K] s_h
  float* wts = psc + round4(HG * K);                           // [HG][K] fusion weights
  float* pbuf = wts + round4(HG * K);                          // [NW][HG][64] key weights
  uint64_t* ck = (uint64_t*)(pbuf + NW * HG * kWave);
  const int R = (K + NW - 1) / NW;  // blocks per (b, group)
  const int64_t bg = blockIdx.x / R;
  const int rb = blockIdx.x % R;
  const int b = (int)(bg / a.Hkv), g = (int)(bg % a.Hkv);
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int64_t qrow0 = (int64_t)b * a.Hq + g * G;  // first head row of the group

  // the group's queries load during the merge
  constexpr int QP = 2;  // query element pairs per thread in flight
  const int npairs = G * D / 2;
  uint32_t qraw[QP];
  f32x2 qpair[QP];
#pragma unroll
  for (int i = 0; i < QP; ++i) {
    const int e2 = tid + i * NT;
    if (e2 < npairs) {
      if (DT == kF32) qpair[i] = ((const f32x2*)a.q)[qrow0 * D / 2 + e2];
      else qraw[i] = ((const uint32_t*)a.q)[qrow0 * D / 2 + e2];
    }
  }
  int got = 0;
  if (a.n_avail > 0) got = merge_candidates<NT>(a, bg, ck, top, order, hist, sv, red);
  for (int i = 0; i < QP; ++i) {
    const int e2 = tid + i * NT;
    if (e2 < npairs) {
      if (DT == kF32) {
        *(f32x2*)(qf + 2 * e2) = qpair[i];
      } else {
        qb[e2] = qraw[i];
        *(f32x2*)(qf + 2 * e2) =
            f32x2{bf16_bits_to_f32(qraw[i] & 0xffffu), bf16_bits_to_f32(qraw[i] >> 16)};
      }
    }
  }
  for (int e2 = tid + QP * NT; e2 < npairs; e2 += NT) {
    if (DT == kF32) {
      *(f32x2*)(qf + 2 * e2) = ((const f32x2*)a.q)[qrow0 * D / 2 + e2];
    } else {
      const uint32_t r = ((const uint32_t*)a.q)[qrow0 * D / 2 + e2];
      qb[e2] = r;
      *(f32x2*)(qf + 2 * e2) = f32x2{bf16_bits_to_f32(r & 0xffffu), bf16_bits_to_f32(r >> 16)};
    }
  }
  if (rb == 0 && tid < K) a.sel[bg * K + tid] = tid < got ? order[tid] : -1;
  __syncthreads();

  const bool key_ok = lane < a.S;
  const int r = rb * NW + w;  // this wave's rank
  float* pw = pbuf + w * HG * kWave;
  for (int h0 = 0; h0 < G; h0 += HG) {
    const int nh = min(HG, G - h0);
    if (r < got) {
      const int c = order[r];
      const int64_t base = (bg * a.n_max + (int64_t)c * a.S) * D;
      // the chunk's rows load again in each round of heads (one round unless
      // the group has more than 8 heads or K * D is large): keeping them
      // across rounds would not fit in registers beside the next loads
      u32x4 kr[KV4];                // this lane's key row
      float lam[CPL];               // this lane's landmark columns
      uint32_t vr[kWave];           // bf16: value columns of key j as loaded
      uint32_t vp[kWave / 2][CPL];  // bf16: values of keys 2m, 2m + 1 in one column
      float vf[kWave][CPL];         // fp32: values of key j
      {
#pragma unroll
        for (int i = 0; i < KV4; ++i)
          kr[i] = key_ok ? *(const u32x4*)((const char*)a.Kc + (base + (int64_t)lane * D) *
                                                                    (DT == kF32 ? 4 : 2) + 16 * i)
                         : u32x4{0u, 0u, 0u, 0u};
        const float* lc = a.lmk + (bg * a.lmk_chunks + c) * D + CPL * lane;
#pragma unroll
        for (int x = 0; x < CPL; ++x) lam[x] = lc[x];
        if (DT == kBF16) {
          // values: lane = output columns, one 2- or 4-byte load per key,
          // in flight with the keys
#pragma unroll
          for (int j = 0; j < kWave; ++j) {
            const int64_t off = base + (int64_t)j * D + CPL * lane;
            vr[j] = 0u;
            if (j < a.S)
              vr[j] = CPL == 2 ? *(const uint32_t*)((const uint16_t*)a.Vc + off)
                               : (uint32_t)((const uint16_t*)a.Vc)[off];
          }
        }
      }
      // logits, softmax over the chunk's keys, s_h: one head at a time; the
      // normalised weights go to this wave's LDS rows (bf16 pairs of
      // consecutive keys, or fp32)
      for (int hh = 0; hh < nh; ++hh) {
        const int h = h0 + hh;
        float acc = 0.f;
        if (DT == kF32) {
          const f32x4* qv = (const f32x4*)(qf + h * D);
#pragma unroll
          for (int i = 0; i < KV4; ++i) {
            const f32x4 q4 = qv[i];
            const f32x4 k4 = __builtin_bit_cast(f32x4, kr[i]);
            acc += q4[0] * k4[0] + q4[1] * k4[1] + q4[2] * k4[2] + q4[3] * k4[3];
          }
        } else {
          const u32x4* qv = (const u32x4*)(qb + h * D / 2);
#pragma unroll
          for (int i = 0; i < KV4; ++i) {
            const u32x4 q4 = qv[i];
#pragma unroll
            for (int v = 0; v < 4; ++v) {
              // copy the elements out first: bit casts of vector-element
              // operands read element 0
              const uint32_t kw = kr[i][v], qw = q4[v];
              acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, kw),
                                                    __builtin_bit_cast(bf16x2, qw), acc, false);
            }
          }
        }
        const float sc = key_ok ? acc * scale : -INFINITY;
        const float mx = wave_max_f32(sc);
        const float p = key_ok ? expf(sc - mx) : 0.f;
        const float pn = p / wave_sum_f32(p);
        if (DT == kF32) {
          pw[hh * kWave + lane] = pn;
        } else {
          const float next = partner<1>(pn);  // the weight of key lane + 1
          if ((lane & 1) == 0) ((uint32_t*)pw)[hh * kWave + lane / 2] = pack_bf16x2(pn, next);
        }
        float sl = 0.f;
#pragma unroll
        for (int x = 0; x < CPL; ++x) sl += qf[h * D + CPL * lane + x] * lam[x];
        sl = wave_sum_f32(sl);
        if (lane == 0) {
          if (R == 1) psc[hh * K + r] = sl * scale;
          else a.part_s[(qrow0 + h) * K + r] = sl * scale;
        }
      }
      {
        if (DT == kBF16) {
          // pair consecutive keys per column for the packed dot products
#pragma unroll
          for (int m = 0; m < kWave / 2; ++m) {
            vp[m][0] = __builtin_amdgcn_perm(vr[2 * m + 1], vr[2 * m], 0x05040100u);
            if (CPL == 2) vp[m][CPL - 1] = __builtin_amdgcn_perm(vr[2 * m + 1], vr[2 * m], 0x07060302u);
          }
        } else {
          // values: lane = output columns, one 4- or 8-byte load per key
#pragma unroll
          for (int j = 0; j < kWave; ++j) {
            const int64_t off = base + (int64_t)j * D + CPL * lane;
#pragma unroll
            for (int x = 0; x < CPL; ++x) vf[j][x] = j < a.S ? ((const float*)a.Vc)[off + x] : 0.f;
          }
        }
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      for (int hh = 0; hh < nh; ++hh) {
        float o[CPL];
#pragma unroll
        for (int x = 0; x < CPL; ++x) o[x] = 0.f;
        if (DT == kF32) {
#pragma unroll
          for (int j = 0; j < kWave; j += 4) {
            const f32x4 p4 = *(const f32x4*)(pw + hh * kWave + j);
#pragma unroll
            for (int jj = 0; jj < 4; ++jj)
#pragma unroll
              for (int x = 0; x < CPL; ++x) o[x] += p4[jj] * vf[j + jj][x];
          }
        } else {
          const uint32_t* pp = (const uint32_t*)pw + hh * kWave;
#pragma unroll
          for (int m = 0; m < kWave / 2; m += 4) {
            const u32x4 p4 = *(const u32x4*)(pp + m);
#pragma unroll
            for (int mm = 0; mm < 4; ++mm) {
              const uint32_t pq = p4[mm];
#pragma unroll
              for (int x = 0; x < CPL; ++x) {
                const uint32_t vq = vp[m + mm][x];
                o[x] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, vq),
                                                       __builtin_bit_cast(bf16x2, pq), o[x], false);
              }
            }
          }
        }
        float* po = (R == 1 ? part + ((int64_t)hh * K + r) * D
                            : a.part_o + ((qrow0 + h0 + hh) * K + r) * D) + CPL * lane;
#pragma unroll
        for (int x = 0; x < CPL; ++x) po[x] = o[x];
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
    if (R > 1) continue;  // fuse_kernel combines the blocks' outputs
    __syncthreads();
    // fusion weights: per head, a softmax over the ranks' s_h
    for (int e = tid; e < nh * K; e += NT) {
      const int hh = e / K, kk = e % K;
      const float* sc = psc + hh * K;
      float smax = -INFINITY, z = 0.f;
      for (int j = 0; j < got; ++j) smax = fmaxf(smax, sc[j]);
      for (int j = 0; j < got; ++j) z += expf(sc[j] - smax);
      const float wk = kk < got ? expf(sc[kk] - smax) / z : 0.f;
      wts[e] = wk;
      if (a.sel_w) a.sel_w[(qrow0 + h0 + hh) * K + kk] = wk;
    }
    __syncthreads();
    for (int e = tid; e < nh * D; e += NT) {
      const int hh = e / D, x = e % D;
      float acc = 0.f;
      for (int kk = 0; kk < got; ++kk) acc += wts[hh * K + kk] * part[(hh * K + kk) * D + x];
      store_elem<DT>(a.o, (qrow0 + h0 + hh) * D + x, acc);
    }
    __syncthreads();
  }
}

template <int D, int DT>
hipError_t stage_dt(const DecodeArgs& a, int stage, hipStream_t stream) {
  const int64_t BG = (int64_t)a.B * a.Hkv;
  const float scale = 1.0f / sqrtf((float)D);
  if (stage == 0) {
    if (a.n_avail > 0)
      scan_kernel<D, DT><<<dim3((unsigned)(BG * a.n_slices)), dim3(kThreads),
                           (size_t)a.slice * sizeof(uint64_t), stream>>>(a);
  } else if (const size_t lds = fused_lds_bytes(a)) {
    // chunks of at most 64 keys: one wave per selected chunk; with K <= 8
    // the attention block also fuses
    const int R = (a.topk + kFusedWaves - 1) / kFusedWaves;
    if (stage == 1)
      attend_fused_kernel<D, DT><<<dim3((unsigned)(BG * R)), dim3(kFusedThreads), lds, stream>>>(
          a, scale);
    else if (R > 1)
      fuse_kernel<D, DT><<<dim3((unsigned)BG), dim3(kThreads), 0, stream>>>(a);
  } else if (stage == 1) {
    attend_kernel<D, DT><<<dim3((unsigned)(BG * a.topk)), dim3(kThreads),
                           decode_attend_lds(a.Hq, a.Hkv, D, a.n_slices, a.topk), stream>>>(a, scale);
  } else {
    fuse_kernel<D, DT><<<dim3((unsigned)BG), dim3(kThreads), 0, stream>>>(a);
  }
  return hipGetLastError();
}

}  // namespace

void decode_plan(int64_t n_avail, int topk, int64_t BHkv, int* n_slices, int* slice) {
  if (n_avail <= 0) {
    *n_slices = 1;
    *slice = 1;
    return;
  }
  int64_t want = (2048 + BHkv - 1) / BHkv;  // aim for ~2048 scan blocks
  int64_t s = (n_avail + want - 1) / want;
  s = (s + 63) / 64 * 64;
  if (s < 256) s = 256;
  if (s > kMaxSlice) s = kMaxSlice;  // the slice's keys live in LDS
  const int64_t max_slices = kMaxCand / topk;
  // the merge holds n_slices * topk keys in LDS; callers guarantee
  // n_avail <= kMaxSlice * max_slices, so this stays <= kMaxSlice
  if ((n_avail + s - 1) / s > max_slices) s = (n_avail + max_slices - 1) / max_slices;
  *slice = (int)s;
  *n_slices = (int)((n_avail + s - 1) / s);
}

int64_t decode_max_chunks(int topk) { return (int64_t)kMaxSlice * (kMaxCand / topk); }

size_t decode_attend_lds(int Hq, int Hkv, int d, int n_slices, int topk) {
  const size_t q = (size_t)(((Hq / Hkv) * d + 1) & ~1) * sizeof(float);
  // the merge stages candidates in LDS only past one wave's worth
  return q + ((int64_t)n_slices * topk > kWave ? (size_t)kMergeLds * sizeof(uint64_t) : 0);
}

hipError_t decode_stage(const DecodeArgs& a, int stage, hipStream_t stream) {
  if (a.d == 64)
    return a.dtype == kF32 ? stage_dt<64, kF32>(a, stage, stream)
                           : stage_dt<64, kBF16>(a, stage, stream);
  return a.dtype == kF32 ? stage_dt<128, kF32>(a, stage, stream)
                         : stage_dt<128, kBF16>(a, stage, stream);
}

}  // namespace hsa
