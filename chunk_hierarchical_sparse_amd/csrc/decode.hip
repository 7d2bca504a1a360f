// decode.hip - HSA decode: one query per sequence against a KV cache
// ([HSA] Methodology: retrieval of the top-K chunks from the landmark memory;
// [HiLS] abstract: per-chunk attention fused by the retrieval scores).
//
//  1. scan   : grid (b, group, slice).  Streams the slice's fp32 landmarks
//              once (the bandwidth-bound step), scores them against the
//              group-summed query and keeps the slice's top-K as 64-bit keys
//              (score, then lower index) via an LDS radix select.
//  2. merge  : one block per (b, group) selects the top-K of all slices and
//              orders them (score desc, index asc).
//  3. attend : one block per (b, group, selected chunk): the chunk's K/V are
//              staged in LDS, every head of the group attends to it and
//              scores it against its own query (s_h).
//  4. fuse   : per (b, head) softmax over the selected chunks' s_h and the
//              weighted sum of the chunk outputs.
#include <math.h>

#include <type_traits>

#include "hsa_common.h"
#include "kernels.h"

namespace hsa {
namespace {

constexpr int kThreads = 256;
constexpr int kMaxCand = 8192;  // merge buffer (64 KiB of LDS)
constexpr int kMaxSlice = 4096;

// The K largest of M distinct nonzero keys in LDS `keys`, written unordered
// to out[0..min(K,M)).  Radix select, 8 bits at a time from the top, until
// the bin holding the K-th largest key is needed whole.  Called by all 256
// threads; `hist` is 256 ints of LDS, `sv` 4 ints.
__device__ int block_topk_u64(const uint64_t* keys, int M, int K, uint64_t* out, int* hist,
                              int* sv) {
  const int tid = threadIdx.x;
  if (M <= K) {
    for (int i = tid; i < M; i += kThreads) out[i] = keys[i];
    __syncthreads();
    return M;
  }
  uint64_t prefix = 0, mask = 0;
  int need = K;
  for (int shift = 56; shift >= 0; shift -= 8) {
    hist[tid] = 0;
    __syncthreads();
    for (int i = tid; i < M; i += kThreads) {
      const uint64_t k = keys[i];
      if ((k & mask) == prefix) atomicAdd(&hist[(int)((k >> shift) & 255u)], 1);
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
    if ((k & mask) >= prefix) out[atomicAdd(&sv[3], 1)] = k;
  }
  __syncthreads();
  return K;
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
  const int got = block_topk_u64(keys, M, a.topk, sel, hist, sv);
  uint64_t* out = a.cand + (bg * a.n_slices + sl) * a.topk;
  for (int k = threadIdx.x; k < a.topk; k += kThreads) out[k] = k < got ? sel[k] : 0ull;
}

__global__ void __launch_bounds__(kThreads) merge_kernel(DecodeArgs a) {
  __shared__ uint64_t keys[kMaxCand];
  __shared__ uint64_t top[32];
  __shared__ int hist[256];
  __shared__ int sv[4];
  __shared__ int cnt;
  const int64_t bg = blockIdx.x;
  if (threadIdx.x == 0) cnt = 0;
  __syncthreads();
  // With no available chunk the scan does not run and the candidate buffer
  // holds nothing of this call: read none of it.
  const int total = a.n_avail > 0 ? a.n_slices * a.topk : 0;
  const uint64_t* cand = a.cand + bg * (int64_t)a.n_slices * a.topk;
  for (int i = threadIdx.x; i < total; i += kThreads) {
    const uint64_t k = cand[i];
    if (k != 0ull) keys[atomicAdd(&cnt, 1)] = k;
  }
  __syncthreads();
  const int M = cnt;
  const int got = block_topk_u64(keys, M, a.topk, top, hist, sv);
  // order the winners: rank = number of larger keys
  int32_t* sel = a.sel + bg * a.topk;
  __shared__ int32_t sorted[32];
  if (threadIdx.x < got) {
    const uint64_t k = top[threadIdx.x];
    int rank = 0;
    for (int j = 0; j < got; ++j) rank += top[j] > k;
    sorted[rank] = (int32_t)key_index(k);
  }
  __syncthreads();
  if (threadIdx.x < a.topk) sel[threadIdx.x] = threadIdx.x < got ? sorted[threadIdx.x] : -1;
}

// Per (b, group, selected chunk): the chunk's keys/values are staged in LDS
// 64 (bf16) or 32 (fp32) rows at a time with 16-byte loads; wave = head
// (looping over the group's heads), lane = key for the logits and lane =
// output column for the weighted sum.
template <int D, int DT>
__global__ void __launch_bounds__(kThreads) attend_kernel(DecodeArgs a, float scale) {
  constexpr int KB = DT == kF32 ? 32 : 64;   // keys per LDS block
  constexpr int EB = DT == kF32 ? 4 : 2;     // bytes per element
  constexpr int VE = 16 / EB;                // elements per 16-byte piece
  constexpr int KSTR = D + VE;               // key row stride, padded by 16 bytes
  typedef typename std::conditional<DT == kF32, float, uint16_t>::type T;
  __shared__ __attribute__((aligned(16))) T ks[KB * KSTR];
  __shared__ __attribute__((aligned(16))) T vs[KB * D];
  __shared__ __attribute__((aligned(16))) float qs[32 * D];
  const int64_t bg = blockIdx.x / a.topk;
  const int k = blockIdx.x % a.topk;
  const int c = a.sel[bg * a.topk + k];
  if (c < 0 || c >= a.n_avail) return;
  const int b = (int)(bg / a.Hkv), g = (int)(bg % a.Hkv);
  const int G = a.Hq / a.Hkv;
  for (int e = threadIdx.x; e < G * D; e += kThreads)
    qs[e] = load_elem<DT>(a.q, ((int64_t)b * a.Hq + g * G) * D + e);
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  constexpr int CPL = D / 64;  // output columns per lane
  float m[8], l[8], o[8][CPL];
  for (int hi = 0; hi < 8; ++hi) {
    m[hi] = -INFINITY;
    l[hi] = 0.f;
    for (int x = 0; x < CPL; ++x) o[hi][x] = 0.f;
  }
  const int64_t base = (bg * a.n_max + (int64_t)c * a.S) * D;
  const T* Kg = (const T*)a.Kc + base;
  const T* Vg = (const T*)a.Vc + base;
  constexpr int PPR = D / VE;  // 16-byte pieces per row
  for (int kb = 0; kb < a.S; kb += KB) {
    const int nk = min(KB, a.S - kb);
    __syncthreads();
    for (int e = threadIdx.x; e < KB * PPR; e += kThreads) {
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
    int hi = 0;
    for (int hh = w; hh < G; hh += 4, ++hi) {
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
      for (int x = 0; x < CPL; ++x) o[hi][x] *= al;
      for (int j = 0; j < nk; ++j) {
        const float pj = __shfl(p, j, kWave);
        for (int x = 0; x < CPL; ++x)
          o[hi][x] += pj * load_elem<DT>(vs, (int64_t)j * D + lane + 64 * x);
      }
    }
  }
  int hi = 0;
  for (int hh = w; hh < G; hh += 4, ++hi) {
    const float* lc = a.lmk + (bg * a.lmk_chunks + c) * D;
    float s = 0.f;
    for (int x = lane; x < D; x += 64) s += qs[hh * D + x] * lc[x];
    s = wave_sum(s);
    const int64_t row = ((int64_t)b * a.Hq + g * G + hh) * a.topk + k;
    if (lane == 0) a.part_s[row] = s * scale;
    for (int x = 0; x < CPL; ++x) a.part_o[row * D + lane + 64 * x] = o[hi][x] / l[hi];
  }
}

template <int D, int DT>
__global__ void __launch_bounds__(64) fuse_kernel(DecodeArgs a) {
  const int64_t row = blockIdx.x;  // b * Hq + h
  const int b = (int)(row / a.Hq), h = (int)(row % a.Hq);
  const int G = a.Hq / a.Hkv;
  const int g = h / G;
  const int32_t* sel = a.sel + ((int64_t)b * a.Hkv + g) * a.topk;
  int m = 0;
  while (m < a.topk && sel[m] >= 0) ++m;
  const float* sc = a.part_s + row * a.topk;
  float smax = -INFINITY;
  for (int k = 0; k < m; ++k) smax = fmaxf(smax, sc[k]);
  float z = 0.f;
  for (int k = 0; k < m; ++k) z += expf(sc[k] - smax);
  const int lane = threadIdx.x;
  for (int x = lane; x < D; x += 64) {
    float acc = 0.f;
    for (int k = 0; k < m; ++k) acc += expf(sc[k] - smax) / z * a.part_o[(row * a.topk + k) * D + x];
    store_elem<DT>(a.o, row * D + x, acc);
  }
  if (a.sel_w)
    for (int k = lane; k < a.topk; k += 64)
      a.sel_w[row * a.topk + k] = k < m ? expf(sc[k] - smax) / z : 0.f;
}

template <int D, int DT>
hipError_t stage_dt(const DecodeArgs& a, int stage, hipStream_t stream) {
  const int64_t BG = (int64_t)a.B * a.Hkv;
  const float scale = 1.0f / sqrtf((float)D);
  switch (stage) {
    case 0:
      if (a.n_avail > 0)
        scan_kernel<D, DT><<<dim3((unsigned)(BG * a.n_slices)), dim3(kThreads),
                             (size_t)a.slice * sizeof(uint64_t), stream>>>(a);
      break;
    case 1:
      merge_kernel<<<dim3((unsigned)BG), dim3(kThreads), 0, stream>>>(a);
      break;
    case 2:
      attend_kernel<D, DT><<<dim3((unsigned)(BG * a.topk)), dim3(kThreads), 0, stream>>>(a,
                                                                                       scale);
      break;
    default:
      fuse_kernel<D, DT><<<dim3((unsigned)((int64_t)a.B * a.Hq)), dim3(64), 0, stream>>>(a);
      break;
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

hipError_t decode_stage(const DecodeArgs& a, int stage, hipStream_t stream) {
  if (a.d == 64)
    return a.dtype == kF32 ? stage_dt<64, kF32>(a, stage, stream)
                           : stage_dt<64, kBF16>(a, stage, stream);
  return a.dtype == kF32 ? stage_dt<128, kF32>(a, stage, stream)
                         : stage_dt<128, kBF16>(a, stage, stream);
}

}  // namespace hsa
