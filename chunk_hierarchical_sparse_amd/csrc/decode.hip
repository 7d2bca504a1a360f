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
//  2. attend : one block per (b, group, rank k); every block merges the
//              slices' candidates into the same ordered top-K, then attends
//              to the chunk of its rank (coalesced loads, every head of the
//              group); the sliding-window attention of the upper layers can
//              ride in the same launch as extra blocks, one per 64-key piece
//              of the window.
//  3. fuse   : per (b, group) and head, a softmax over the selected
//              chunks' s_h weights the chunk outputs; the window's pieces
//              are merged by their log-sum-exp.  For chunks of at most 64
//              keys it runs in the attend launch itself: the last of the
//              group's blocks to finish does it (attend_fuse_kernel).
#include <math.h>

#include <algorithm>

#include <type_traits>

#include "hsa_common.h"
#include "kernels.h"

namespace hsa {

HSA_DCHECK_SOURCE()
namespace {

constexpr int kThreads = 256;
constexpr int kMaxCand = 8192;  // candidates per (b, group) the merge reads
constexpr int kMaxSlice = 4096;

// Data that other blocks of the same launch read goes through agent-scope
// (device-coherent) loads and stores: they reach every XCD without a
// release fence's write-back of the L2.  A writer waits for its stores to
// complete before it bumps the counter that announces them.
__device__ __forceinline__ void st_agent(uint64_t* p, uint64_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_agent(uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t ld_agent(const uint64_t* p) {
  return __hip_atomic_load(const_cast<uint64_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t ld_agent(const uint32_t* p) {
  return __hip_atomic_load(const_cast<uint32_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// this wave's stores have completed
__device__ __forceinline__ void wait_stores() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

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

// The K (<= 32) largest of the keys get(0..M) (zeros past the M-th),
// descending in lanes 0..K-1 of wave 0.  Each wave sorts its 64-key pieces
// and merges them into a running top list; wave 0 then merges the four
// lists.  `lists` is 4 * 32 keys of LDS.  Called by all threads.
template <typename Get>
__device__ uint64_t block_topk_sorted(Get get, int M, int K, uint64_t* lists) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  uint64_t run = 0ull;
  for (int c = w; c * kWave < M; c += kThreads / kWave) {
    const int i = c * kWave + lane;
    uint64_t x = wave_sort_desc_u64(i < M ? get(i) : 0ull);
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

// Slice sl of (b, group) bg: its candidate list and extremes.  LDS: u [D]
// floats, keys [slice], lists [4 * 32].  Called by all threads.
template <int D, int DT>
__device__ __forceinline__ void scan_body(const DecodeArgs& a, int64_t bg, int sl, float* u,
                                          uint64_t* keys, uint64_t* lists) {
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
  const uint64_t top = block_topk_sorted([&](int i) { return keys[i]; }, M, a.topk, lists);
  if (w == 0) {
    const int got = min(M, a.topk);
    uint64_t* out = a.cand + (bg * a.n_slices + sl) * a.topk;
    if (lane < a.topk) st_agent(&out[lane], lane < got ? top : 0ull);
    const uint64_t mn = __shfl(top, max(got - 1, 0), kWave);
    if (lane == 0)
      *(u64x2*)(a.cand_mm + (bg * a.n_slices + sl) * 2) =
          u64x2{got > 0 ? top : 0ull, got == a.topk ? mn : 0ull};
  }
}

// a.sync (when set): the attention's per-group counters, cleared by block 0.
template <int D, int DT>
__global__ void __launch_bounds__(kThreads) scan_kernel(DecodeArgs a) {
  __shared__ float u[D];
  extern __shared__ uint64_t keys[];  // [slice]
  __shared__ uint64_t lists[4 * 32];
  if (a.sync && blockIdx.x == 0)
    for (int64_t i = threadIdx.x; i < (int64_t)a.B * a.Hkv; i += kThreads) a.sync[i] = 0u;
  scan_body<D, DT>(a, blockIdx.x / a.n_slices, blockIdx.x % a.n_slices, u, keys, lists);
}

// LDS of the candidate merge.
struct MergeLds {
  uint64_t ck[32 * 32];   // candidates at or above the bound (at most K * K)
  uint64_t lists[4 * 32];
  int32_t order[32];
  int sv[4];
};

// The ordered top-K chunks of one (b, group) from its slices' candidate
// lists (n_slices lists of K keys, each the slice's K largest, 0 = empty):
// ml.order[0..K) = chunk indices by (score desc, index asc), -1 past the
// available ones; returns their count.  Up to 64 candidates are sorted by
// one wave.  More are cut first at lb, the K-th largest slice maximum: the
// K largest maxima are K distinct keys at or above it, so every key of the
// global top K is >= lb and lies in a slice whose maximum reaches lb --
// one of those K slices -- and in that slice's list.  At most K * K
// candidates survive; the block takes the K largest.  Deterministic: every
// block of the (b, group) computes the same list.  Called by all threads.
__device__ int merge_sorted(const DecodeArgs& a, int64_t bg, MergeLds& ml) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int K = a.topk, ns = a.n_slices;
  const int total = ns * K;
  const uint64_t* cand = a.cand + bg * (int64_t)total;
  uint64_t top = 0ull;  // wave 0, lanes 0..K-1: the result, descending
  if (total <= kWave) {
    if (w == 0) top = wave_sort_desc_u64(lane < total ? cand[lane] : 0ull);
  } else {
    const uint64_t* mm = a.cand_mm + bg * (int64_t)ns * 2;
    const uint64_t tm =
        block_topk_sorted([&](int i) { return mm[2 * i]; }, ns, K, ml.lists);  // the K largest maxima
    if (w == 0) {
      const uint64_t kth = __shfl(tm, K - 1, kWave);
      // slice of each of the K largest maxima (0: fewer nonempty slices)
      if (lane < K) ml.order[lane] = tm != 0ull ? (int)(key_index(tm) / a.slice) : -1;
      if (lane == 0) {
        ml.sv[0] = 0;
        *(uint64_t*)&ml.sv[2] = kth > 1ull ? kth : 1ull;
      }
    }
    __syncthreads();
    const uint64_t lb = *(const uint64_t*)&ml.sv[2];
    for (int e = tid; e < K * K; e += kThreads) {
      const int j = ml.order[e / K];
      if (j < 0) continue;
      const uint64_t x = cand[(int64_t)j * K + e % K];
      if (x >= lb) ml.ck[atomicAdd(&ml.sv[0], 1)] = x;
    }
    __syncthreads();
    const int n = ml.sv[0];
    top = block_topk_sorted([&](int i) { return ml.ck[i]; }, n, K, ml.lists);
  }
  __syncthreads();  // order[] is rewritten below
  if (w == 0) {
    if (lane < K) ml.order[lane] = top != 0ull ? (int32_t)key_index(top) : -1;
    const uint64_t live = __ballot(lane < K && top != 0ull);
    if (lane == 0) ml.sv[1] = __popcll(live);
  }
  __syncthreads();
  return ml.sv[1];
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
  __shared__ MergeLds ml;
  // qs [G * D] fp32
  extern __shared__ __attribute__((aligned(16))) float dyn[];
  const int G = a.Hq / a.Hkv;
  float* qs = dyn;
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
  const int got = merge_sorted(a, bg, ml);
  if (k == 0)
    for (int e = tid; e < a.topk; e += kThreads) a.sel[bg * a.topk + e] = ml.order[e];
  const int c = k < got ? ml.order[k] : -1;
  HSA_DCHECK(c < a.n_avail);
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

// One unit of the attend stage once its keys are known: keys [row0, row0 +
// nk) of (b, group) bg, either chunk c of rank r or window piece r - K (win).
// qx: this thread's first two 16-byte pieces of the group's queries, already
// loaded.  LDS: kv [64 key rows], lam [D] floats, qs [G * D] elements, ps
// [G * 64] floats.  Called by all threads.
template <int D, int DT>
__device__ __forceinline__ void attend_body(const DecodeArgs& a, int64_t bg, int r, bool win,
                                            int64_t row0, int nk, int c, const u32x4 (&qx)[2],
                                            unsigned char* kv, float* lam, uint32_t* qs,
                                            float* ps, float scale) {
  constexpr int EB = DT == kF32 ? 4 : 2;
  constexpr int ROWB = D * EB;
  constexpr int PPR = ROWB / 16;
  constexpr int NL = kWave * PPR / kThreads;
  constexpr int CPL = D / 64;
  typedef typename std::conditional<DT == kF32, float, uint16_t>::type T;
  const int G = a.Hq / a.Hkv;
  const int K = a.topk;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int64_t qrow0 = (int64_t)((bg / a.Hkv) * a.Hq + (bg % a.Hkv) * G);
  const int nq = G * D * EB / 16;
  const u32x4* qg = (const u32x4*)((const char*)a.q + qrow0 * ROWB);
  const int64_t base = (bg * a.n_max + row0) * ROWB;
  const char* Kg = (const char*)a.Kc + base;
  const char* Vg = (const char*)a.Vc + base;
  // rows past the block's keys (nk < 64) re-read row nk - 1; their weights are zero
  u32x4 kx[NL], vx[NL];
#pragma unroll
  for (int i = 0; i < NL; ++i) {
    const int e = tid + i * kThreads, row = e / PPR, pc = e % PPR;
    const int64_t off = (int64_t)min(row, nk - 1) * ROWB + pc * 16;
    kx[i] = *(const u32x4*)(Kg + off);
    vx[i] = *(const u32x4*)(Vg + off);
  }
  f32x4 lx = {0.f, 0.f, 0.f, 0.f};
  if (!win && tid < D / 4) lx = *(const f32x4*)(a.lmk + (bg * a.lmk_chunks + c) * D + 4 * tid);
  {
    int m = 0;
    for (int i = tid; i < nq; i += kThreads, ++m)
      *(u32x4*)(&qs[4 * i]) = m == 0 ? qx[0] : (m == 1 ? qx[1] : qg[i]);
  }
  // piece pc of key row j sits at piece pc ^ (j % PPR) of the row
#pragma unroll
  for (int i = 0; i < NL; ++i) {
    const int e = tid + i * kThreads, row = e / PPR, pc = e % PPR;
    *(u32x4*)(&kv[row * ROWB + ((pc ^ (row % PPR)) * 16)]) = kx[i];
  }
  if (tid < D / 4) *(f32x4*)(&lam[4 * tid]) = lx;
  __syncthreads();
  const bool key_ok = lane < nk;
  for (int h = w; h < G; h += kThreads / kWave) {
    // logit of key `lane`
    float acc = 0.f;
    const unsigned char* kr = &kv[lane * ROWB];
    const uint32_t* qh = qs + h * D * EB / 4;
#pragma unroll 4
    for (int pc = 0; pc < PPR; ++pc) {
      const u32x4 k4 = *(const u32x4*)(kr + ((pc ^ (lane % PPR)) * 16));
      const u32x4 q4 = *(const u32x4*)(qh + 4 * pc);
      if (DT == kF32) {
#pragma unroll
        for (int v = 0; v < 4; ++v) acc += __uint_as_float(q4[v]) * __uint_as_float(k4[v]);
      } else {
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const uint32_t kw = k4[v], qw = q4[v];
          acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, kw),
                                                __builtin_bit_cast(bf16x2, qw), acc, false);
        }
      }
    }
    const float lg = key_ok ? acc * scale : -INFINITY;
    const float mx = wave_max_f32(lg);
    const float pe = key_ok ? expf(lg - mx) : 0.f;
    const float z = wave_sum_f32(pe);
    ps[h * kWave + lane] = pe / z;
    if (win) {
      if (lane == 0)
        st_agent((uint32_t*)&a.sw_lse[(qrow0 + h) * a.swa_pieces + (r - K)],
                 __float_as_uint(mx + logf(z)));
    } else {
      // s_h: this lane's landmark columns
      float sl = 0.f;
#pragma unroll
      for (int x = 0; x < CPL; ++x) {
        const int col = CPL * lane + x;
        const float qv = DT == kF32 ? __uint_as_float(qh[col])
                                    : bf16_bits_to_f32(((const uint16_t*)qh)[col]);
        sl += qv * lam[col];
      }
      sl = wave_sum_f32(sl);
      if (lane == 0) st_agent((uint32_t*)&a.part_s[(qrow0 + h) * K + r], __float_as_uint(sl * scale));
    }
  }
  __syncthreads();
  // the values replace the keys
#pragma unroll
  for (int i = 0; i < NL; ++i) {
    const int e = tid + i * kThreads, row = e / PPR, pc = e % PPR;
    *(u32x4*)(&kv[row * ROWB + pc * 16]) = vx[i];
  }
  __syncthreads();
  for (int h = w; h < G; h += kThreads / kWave) {
    float o[CPL];
#pragma unroll
    for (int x = 0; x < CPL; ++x) o[x] = 0.f;
    const float* ph = ps + h * kWave;
#pragma unroll 4
    for (int j = 0; j < kWave; j += 4) {
      const f32x4 p4 = *(const f32x4*)(&ph[j]);
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const T* vr = (const T*)&kv[(j + jj) * ROWB] + CPL * lane;
        if (DT == kF32) {
#pragma unroll
          for (int x = 0; x < CPL; ++x) o[x] += p4[jj] * ((const float*)vr)[x];
        } else if (CPL == 2) {
          const uint32_t v2 = *(const uint32_t*)vr;
          o[0] += p4[jj] * bf16_bits_to_f32(v2 & 0xffffu);
          o[CPL - 1] += p4[jj] * bf16_bits_to_f32(v2 >> 16);
        } else {
          o[0] += p4[jj] * bf16_bits_to_f32(*(const uint16_t*)vr);
        }
      }
    }
    float* po = (win ? a.sw_o + ((qrow0 + h) * a.swa_pieces + (r - K)) * D
                     : a.part_o + ((qrow0 + h) * K + r) * D) + CPL * lane;
    if (CPL == 2)
      st_agent((uint64_t*)po, __builtin_bit_cast(uint64_t, f32x2{o[0], o[CPL - 1]}));
    else
      st_agent((uint32_t*)po, __float_as_uint(o[0]));
  }
}

// Per (b, group): per head, a softmax over the selected chunks' s_h (one
// wave per head, lane = rank) and the weighted sum of the normalised chunk
// outputs (16 bytes of columns per thread, all ranks' loads in flight); no
// selected chunk gives zeros.
// LDS: wts [32 * 64] floats, s_got.  Called by all threads.
template <int D, int DT>
__device__ __forceinline__ void fuse_body(const DecodeArgs& a, int64_t bg, float* wts,
                                          int& s_got) {
  const int G = a.Hq / a.Hkv;
  const int K = a.topk;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int64_t qrow0 = (int64_t)((bg / a.Hkv) * a.Hq + (bg % a.Hkv) * G);
  if (w == 0) {
    const int32_t sv = lane < K ? (int32_t)ld_agent((const uint32_t*)&a.sel[bg * K + lane]) : -1;
    const uint64_t live = __ballot(sv >= 0);
    if (lane == 0) s_got = __popcll(live);
  }
  __syncthreads();
  const int got = s_got;
  for (int h = w; h < G; h += kThreads / kWave) {
    const int64_t row = qrow0 + h;
    const float sc =
        lane < got ? __uint_as_float(ld_agent((const uint32_t*)&a.part_s[row * K + lane]))
                   : -INFINITY;
    const float mx = wave_max_f32(sc);
    const float e = lane < got ? expf(sc - mx) : 0.f;
    const float wk = e / wave_sum_f32(e);
    if (lane < K) {
      wts[h * K + lane] = lane < got ? wk : 0.f;
      if (a.sel_w) a.sel_w[row * K + lane] = lane < got ? wk : 0.f;
    }
  }
  __syncthreads();
  for (int e = tid; e < G * D / 4; e += kThreads) {
    const int h = e / (D / 4), x4 = e % (D / 4);
    const int64_t row = qrow0 + h;
    const float* po = a.part_o + row * K * D + 4 * x4;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 8
    for (int kk = 0; kk < got; ++kk) {
      const uint64_t* pv = (const uint64_t*)(po + (int64_t)kk * D);
      const f32x2 v0 = __builtin_bit_cast(f32x2, ld_agent(pv));
      const f32x2 v1 = __builtin_bit_cast(f32x2, ld_agent(pv + 1));
      const f32x4 v = {v0[0], v0[1], v1[0], v1[1]};
      const float wk = wts[h * K + kk];
#pragma unroll
      for (int x = 0; x < 4; ++x) acc[x] += wk * v[x];
    }
#pragma unroll
    for (int x = 0; x < 4; ++x) store_elem<DT>(a.o, row * D + 4 * x4 + x, acc[x]);
  }
  if (a.swa_pieces == 0) return;
  // the window: a softmax merge of the pieces by their log-sum-exp
  const int P = a.swa_pieces;  // <= 64
  __syncthreads();
  for (int h = w; h < G; h += kThreads / kWave) {
    const int64_t row = qrow0 + h;
    const float ls =
        lane < P ? __uint_as_float(ld_agent((const uint32_t*)&a.sw_lse[row * P + lane]))
                 : -INFINITY;
    const float mx = wave_max_f32(ls);
    const float e = lane < P ? expf(ls - mx) : 0.f;
    const float wk = e / wave_sum_f32(e);
    if (lane < P) wts[h * kWave + lane] = wk;
  }
  __syncthreads();
  for (int e = tid; e < G * D / 4; e += kThreads) {
    const int h = e / (D / 4), x4 = e % (D / 4);
    const int64_t row = qrow0 + h;
    const float* po = a.sw_o + row * P * D + 4 * x4;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 8
    for (int pp = 0; pp < P; ++pp) {
      const uint64_t* pv = (const uint64_t*)(po + (int64_t)pp * D);
      const f32x2 v0 = __builtin_bit_cast(f32x2, ld_agent(pv));
      const f32x2 v1 = __builtin_bit_cast(f32x2, ld_agent(pv + 1));
      const f32x4 v = {v0[0], v0[1], v1[0], v1[1]};
      const float wk = wts[h * kWave + pp];
#pragma unroll
      for (int x = 0; x < 4; ++x) acc[x] += wk * v[x];
    }
#pragma unroll
    for (int x = 0; x < 4; ++x) store_elem<DT>(a.o_swa, row * D + 4 * x4 + x, acc[x]);
  }
}

template <int D, int DT>
__global__ void __launch_bounds__(kThreads) fuse_kernel(DecodeArgs a) {
  __shared__ float wts[32 * kWave];  // [head of the group][rank or window piece]
  __shared__ int s_got;
  fuse_body<D, DT>(a, blockIdx.x, wts, s_got);
}

// ---- the attention of chunks of at most 64 keys ------------------------------
//
// With a.sync set (hsa_decode), two launches: the scan (as above; its first
// block also clears the per-group counters of the second launch), then one
// block per (b, group, unit r), the fusion folded in; with a.sync null
// (hsa_swa_decode, whose window merge would lengthen the folded tail) the
// fusion is the third launch.  Units r < K are the selected chunks: every
// such block runs the merge and takes the chunk of rank r.  Units r >= K
// (sliding-window attention in the same launch) are 64-key pieces of the
// window [swa_lo, swa_hi): they need no merge and start at once.  A block
// loads its keys and values into registers with coalesced 16-byte loads
// (each wave instruction reads 1 KB of consecutive bytes: the gather is
// bandwidth-bound and cold in cache, so the loads must be whole lines), and
// a chunk block its landmark row.  The keys go to LDS first (16-byte pieces
// XOR-swizzled by row, so lane = key reads spread over the banks): wave w
// takes heads w, w + 4, ...: lane = key for the logits and a softmax over
// the block's keys, whose weights go to LDS, and for a chunk the head's
// retrieval score s_h = q . lambda / sqrt(d), for a window piece the
// log-sum-exp of its logits.  Then the values replace the keys in the same
// LDS buffer and lane = output columns for the weighted value sum.  One
// 16 KB buffer (bf16, d = 128) keeps the block at about 19 KB of LDS, so 8
// blocks fit on a CU and every block of a batch-32 decode is resident at
// once.  With a.sync set each block counts itself done, and the last block
// of the group to finish runs the fusion.  No block waits for another.

// Grid (b, group, unit).  a.sync [B*Hkv]: blocks of the group done.  LDS
// (dynamic): the merge's MergeLds, then 64 key rows, lam [D] floats, qs
// [G * D] elements, ps [G * 64] floats; the fusion's wts [32 * 64] floats.
template <int D, int DT>
__global__ void __launch_bounds__(kThreads, DT == kF32 ? 4 : 8)
    attend_fuse_kernel(DecodeArgs a, float scale) {
  constexpr int EB = DT == kF32 ? 4 : 2;
  constexpr int ROWB = D * EB;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  __shared__ int32_t s_c;
  __shared__ int s_last;
  __shared__ int s_got;
  const int tid = threadIdx.x;
  const int K = a.topk, G = a.Hq / a.Hkv;
  const int units = K + a.swa_pieces;
  const int64_t bg = blockIdx.x / units;
  const int r = blockIdx.x % units;
  const bool win = r >= K;  // block-uniform
  unsigned char* kv = smem;
  float* lam = (float*)(smem + kWave * ROWB);
  uint32_t* qs = (uint32_t*)(smem + kWave * ROWB + D * 4);
  float* ps = (float*)(smem + kWave * ROWB + D * 4 + G * D * EB);
  const int64_t qrow0 = (int64_t)((bg / a.Hkv) * a.Hq + (bg % a.Hkv) * G);
  // the group's queries load during the merge
  const int nq = G * D * EB / 16;
  const u32x4* qg = (const u32x4*)((const char*)a.q + qrow0 * ROWB);
  u32x4 qx[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) qx[i] = qg[min(tid + i * kThreads, nq - 1)];
  int64_t row0 = 0;  // the block's first key row in the (b, group) cache
  int nk = 0;        // its keys (1..64)
  int c = -1;        // chunk blocks: the chunk
  if (win) {
    row0 = a.swa_lo + (int64_t)(r - K) * kWave;
    nk = (int)min((int64_t)kWave, a.swa_hi - row0);
    HSA_DCHECK(row0 >= 0 && nk >= 1 && row0 + nk <= a.n_max);
  } else {
    if (a.n_avail > 0) {
      MergeLds& ml = *(MergeLds*)smem;
      const int got = merge_sorted(a, bg, ml);
      if (tid == 0) s_c = r < got ? ml.order[r] : -1;
      // the selection goes out from rank 0 (the fusion reads it)
      if (r == 0 && tid < K) st_agent((uint32_t*)&a.sel[bg * K + tid], (uint32_t)ml.order[tid]);
    } else {
      if (tid == 0) s_c = -1;
      if (r == 0 && tid < K) st_agent((uint32_t*)&a.sel[bg * K + tid], 0xffffffffu);
    }
    __syncthreads();
    c = s_c;
    HSA_DCHECK(c < a.n_avail);
    row0 = (int64_t)c * a.S;
    nk = a.S;
  }
  if (win || (c >= 0 && c < a.n_avail))
    attend_body<D, DT>(a, bg, r, win, row0, nk, c, qx, kv, lam, qs, ps, scale);
  if (!a.sync) return;  // the fusion runs as its own launch
  // the last block of bg fuses
  wait_stores();
  __syncthreads();
  if (tid == 0) s_last = atomicAdd(&a.sync[bg], 1u) == (uint32_t)(units - 1);
  __syncthreads();
  if (!s_last) return;
  fuse_body<D, DT>(a, bg, (float*)smem, s_got);
}

template <int D, int DT>
size_t attend_fuse_lds(const DecodeArgs& a) {
  constexpr size_t EB = DT == kF32 ? 4 : 2;
  const size_t G = (size_t)(a.Hq / a.Hkv);
  return std::max<size_t>({kWave * D * EB + D * 4 + G * D * EB + G * kWave * 4,
                           32 * kWave * 4, sizeof(MergeLds)});
}

template <int D, int DT>
hipError_t fused_stage_dt(const DecodeArgs& a, int stage, hipStream_t stream) {
  const int64_t BG = (int64_t)a.B * a.Hkv;
  if (stage == 0) {
    launch<scan_kernel<D, DT>>(dim3((unsigned)(BG * a.n_slices)), dim3(kThreads),
                               (size_t)a.slice * sizeof(uint64_t), stream, a);
  } else {
    const float scale = 1.0f / sqrtf((float)D);
    launch<attend_fuse_kernel<D, DT>>(dim3((unsigned)(BG * (a.topk + a.swa_pieces))),
                                      dim3(kThreads), attend_fuse_lds<D, DT>(a), stream, a,
                                      scale);
  }
  return hipGetLastError();
}

template <int D, int DT>
hipError_t stage_dt(const DecodeArgs& a, int stage, hipStream_t stream) {
  const int64_t BG = (int64_t)a.B * a.Hkv;
  const float scale = 1.0f / sqrtf((float)D);
  const int G = a.Hq / a.Hkv;
  if (stage == 0) {
    if (a.n_avail > 0)
      launch<scan_kernel<D, DT>>(dim3((unsigned)(BG * a.n_slices)), dim3(kThreads),
                                 (size_t)a.slice * sizeof(uint64_t), stream, a);
  } else if (stage == 1) {
    // one block per (b, group, unit); a.sync is null here, so
    // attend_fuse_kernel leaves the fusion to stage 2
    if (a.S <= kWave)
      launch<attend_fuse_kernel<D, DT>>(dim3((unsigned)(BG * (a.topk + a.swa_pieces))),
                                        dim3(kThreads), attend_fuse_lds<D, DT>(a), stream, a,
                                        scale);
    else
      launch<attend_kernel<D, DT>>(dim3((unsigned)(BG * a.topk)), dim3(kThreads),
                                   (size_t)G * D * sizeof(float), stream, a, scale);
  } else {
    launch<fuse_kernel<D, DT>>(dim3((unsigned)BG), dim3(kThreads), 0, stream, a);
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

bool decode_fused_ok(const DecodeArgs& a) {
  // with no chunk available the scan still runs (on empty slices): it
  // clears the counters
  if (a.S > kWave || !a.sync) return false;
  const size_t lds = a.d == 64 ? (a.dtype == kF32 ? attend_fuse_lds<64, kF32>(a)
                                                  : attend_fuse_lds<64, kBF16>(a))
                               : (a.dtype == kF32 ? attend_fuse_lds<128, kF32>(a)
                                                  : attend_fuse_lds<128, kBF16>(a));
  return lds <= 64 * 1024;
}

hipError_t decode_fused_stage(const DecodeArgs& a, int stage, hipStream_t stream) {
  if (a.d == 64)
    return a.dtype == kF32 ? fused_stage_dt<64, kF32>(a, stage, stream)
                           : fused_stage_dt<64, kBF16>(a, stage, stream);
  return a.dtype == kF32 ? fused_stage_dt<128, kF32>(a, stage, stream)
                         : fused_stage_dt<128, kBF16>(a, stage, stream);
}

hipError_t decode_stage(const DecodeArgs& a, int stage, hipStream_t stream) {
  if (a.d == 64)
    return a.dtype == kF32 ? stage_dt<64, kF32>(a, stage, stream)
                           : stage_dt<64, kBF16>(a, stage, stream);
  return a.dtype == kF32 ? stage_dt<128, kF32>(a, stage, stream)
                         : stage_dt<128, kBF16>(a, stage, stream);
}

}  // namespace hsa
