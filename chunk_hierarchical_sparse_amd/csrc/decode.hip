// decode.hip - HSA decode: one query per sequence against a KV cache
// ([HSA] Methodology: retrieval of the top-K chunks from the landmark memory;
// [HiLS] abstract: per-chunk attention fused by the retrieval scores).
//
//  1. scan   : grid (b, group, slice).  Streams the slice's fp32 landmarks
//              once (the bandwidth-bound step), scores them against the
//              group-summed query and keeps the slice's top-K as 64-bit keys
//              (score, then lower index) via an LDS radix select.
//  2. attend : one block per (b, group, rank k).  Every block of a (b, group)
//              merges the slices' candidates into the same ordered top-K
//              (score desc, index asc), stages the chunk of rank k in LDS,
//              lets every head of the group attend to it and scores it
//              against its own query (s_h).
//  3. fuse   : one block per (b, group): per head, a softmax over the
//              selected chunks' s_h weights the chunk outputs.
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
// K-th largest key is needed whole.  Called by all 256 threads; `hist` is
// 256 ints of LDS, `sv` 4 ints.
__device__ int block_topk_ge(const uint64_t* keys, int M, uint64_t lo, int K, uint64_t* out,
                             int* hist, int* sv) {
  const int tid = threadIdx.x;
  if (tid == 0) sv[3] = 0;
  __syncthreads();
  int mine = 0;
  for (int i = tid; i < M; i += kThreads) mine += keys[i] >= lo;
  if (mine) atomicAdd(&sv[3], mine);
  __syncthreads();
  const int n = sv[3];
  __syncthreads();
  if (n <= K) {
    if (tid == 0) sv[3] = 0;
    __syncthreads();
    for (int i = tid; i < M; i += kThreads) {
      const uint64_t k = keys[i];
      if (k >= lo) out[atomicAdd(&sv[3], 1)] = k;
    }
    __syncthreads();
    return n;
  }
  uint64_t prefix = 0, mask = 0;
  int need = K;
  for (int shift = 56; shift >= 0; shift -= 8) {
    hist[tid] = 0;
    __syncthreads();
    for (int i = tid; i < M; i += kThreads) {
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
  for (int i = tid; i < M; i += kThreads) {
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
      const uint64_t y = __shfl_xor(x, j, kWave);
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

template <int D, int DT>
__global__ void __launch_bounds__(kThreads) scan_kernel(DecodeArgs a) {
  __shared__ float u[D];
  extern __shared__ uint64_t keys[];  // [slice]
  __shared__ uint64_t sel[32];
  __shared__ int hist[256];
  __shared__ int sv[4];
  const int64_t bg = blockIdx.x / a.n_slices;
  const int sl = blockIdx.x % a.n_slices;
  const int b = (int)(bg / a.Hkv), g = (int)(bg % a.Hkv);
  const int G = a.Hq / a.Hkv;
  const int64_t c_begin = (int64_t)sl * a.slice;
  const int M = (int)max((int64_t)0, min((int64_t)a.slice, a.n_avail - c_begin));
  for (int x = threadIdx.x; x < D; x += kThreads) {
    float acc = 0.f;
    for (int hh = 0; hh < G; ++hh)
      acc += load_elem<DT>(a.q, ((int64_t)b * a.Hq + g * G + hh) * D + x);
    u[x] = acc;
  }
  __syncthreads();
  constexpr int LPR = D / 4;        // lanes per landmark row
  constexpr int RPW = kWave / LPR;  // rows per wave step
  constexpr int U = 8;              // row steps in flight per wave
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int li = lane % LPR, sub = lane / LPR;
  const f32x4 u4 = *(const f32x4*)(&u[4 * li]);
  const float* lm = a.lmk + (bg * a.lmk_chunks + c_begin) * D + 4 * li;
  constexpr int STEP = 4 * RPW;  // rows per block step
  for (int r0 = 0; r0 < M; r0 += STEP * U) {
    f32x4 x[U];
#pragma unroll
    for (int uu = 0; uu < U; ++uu) {
      const int row = r0 + uu * STEP + w * RPW + sub;
      if (row < M)
        x[uu] = __builtin_nontemporal_load((const f32x4*)(lm + (int64_t)row * D));
      else
        x[uu] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int uu = 0; uu < U; ++uu) {
      const int row = r0 + uu * STEP + w * RPW + sub;
      float p = u4[0] * x[uu][0] + u4[1] * x[uu][1] + u4[2] * x[uu][2] + u4[3] * x[uu][3];
#pragma unroll
      for (int o = LPR / 2; o > 0; o >>= 1) p += __shfl_xor(p, o, kWave);
      if (li == 0 && row < M) keys[row] = select_key(p, (uint32_t)(c_begin + row));
    }
  }
  __syncthreads();
  const int got = block_topk_ge(keys, M, 0ull, a.topk, sel, hist, sv);
  uint64_t* out = a.cand + (bg * a.n_slices + sl) * a.topk;
  for (int k = threadIdx.x; k < a.topk; k += kThreads) out[k] = k < got ? sel[k] : 0ull;
  if (threadIdx.x == 0) {
    uint64_t mx = 0ull, mn = ~0ull;
    for (int k = 0; k < got; ++k) {
      mx = sel[k] > mx ? sel[k] : mx;
      mn = sel[k] < mn ? sel[k] : mn;
    }
    *(u64x2*)(a.cand_mm + (bg * a.n_slices + sl) * 2) = u64x2{mx, got == a.topk ? mn : 0ull};
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
// (b, group) gets the same list.  Called by all 256 threads.
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
    for (int grp = w; grp * kWave < a.n_slices; grp += kThreads / kWave) {
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
    for (int x = 0; x < kThreads / kWave; ++x) lb = red[x] > lb ? red[x] : lb;
    // only slices whose largest key reaches the bound hold survivors; their
    // loads have fixed trip counts (K <= 32 is uniform) so all are in flight
    for (int grp = w; grp * kWave < a.n_slices; grp += kThreads / kWave) {
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
  const int got = block_topk_ge(src, n <= kMergeLds ? n : total, lb, K, top, hist, sv);
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
  const int got = merge_candidates(a, bg, ck, top, order, hist, sv, red);
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

template <int D, int DT>
hipError_t stage_dt(const DecodeArgs& a, int stage, hipStream_t stream) {
  const int64_t BG = (int64_t)a.B * a.Hkv;
  const float scale = 1.0f / sqrtf((float)D);
  if (stage == 0) {
    if (a.n_avail > 0)
      scan_kernel<D, DT><<<dim3((unsigned)(BG * a.n_slices)), dim3(kThreads),
                           (size_t)a.slice * sizeof(uint64_t), stream>>>(a);
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
