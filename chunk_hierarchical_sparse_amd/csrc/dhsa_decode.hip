// dhsa_decode.hip - DHSA decode: one new query per (b, head) whose current,
// partial chunk holds it ([DHSA] Referee report, minor comment on
// Algorithm 2: the decode-time update, the last chunk holding the current
// query token; chunk pooling and S_c as in "What carries the argument" and
// Eq. 4; the top-N_b cut of Algorithm 1).
//
//  0. chunk_keys : pooled keys k_hat = sum / sqrt|C| of complete chunks,
//                  kept by the caller as a growing cache.
//  1. score      : one block per (b, head): pooled query and key of the
//                  current chunk, S_c = q_hat . k_hat over the complete chunks
//                  and the current one, chunks ranked by (S_c desc, index asc)
//                  in LDS, and the top-N_b cut as a plan of key runs (whole
//                  chunks in rank order, then the lowest tokens of one).
//  2. attend     : one block per (b, head, run): softmax partials (max, sum,
//                  weighted values) of the new query over the run's keys.
//  3. combine    : per (b, head): the runs' partials into the output.
#include <math.h>

#include "hsa_common.h"
#include "kernels.h"

namespace hsa {
namespace {

constexpr int kThreads = 256;

// out[x] = (sum of rows [0, nrows) of src, row stride D) / sqrt(nrows), in
// LDS.  Thread t sums column piece t % (D / VE) over rows t / (D / VE),
// + RG, ...; the RG partial sums meet in LDS in a fixed order.  Called by
// all threads; ends with a barrier.
template <int D, int DT>
__device__ void pool_rows(const void* src, int64_t row0, int nrows, float* out, float* scratch) {
  constexpr int VE = DT == kF32 ? 4 : 8;  // elements per 16-byte piece
  constexpr int CG = D / VE;              // pieces per row
  constexpr int RG = kThreads / CG;       // row groups
  const int cg = threadIdx.x % CG, rg = threadIdx.x / CG;
  float acc[VE];
#pragma unroll
  for (int v = 0; v < VE; ++v) acc[v] = 0.f;
  for (int r = rg; r < nrows; r += RG) {
    const int64_t e = (row0 + r) * D + cg * VE;
    if (DT == kF32) {
      const f32x4 x = *(const f32x4*)((const float*)src + e);
#pragma unroll
      for (int v = 0; v < 4; ++v) acc[v] += x[v];
    } else {
      const u32x4 x = *(const u32x4*)((const uint16_t*)src + e);
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        acc[2 * v] += bf16_bits_to_f32(x[v] & 0xffffu);
        acc[2 * v + 1] += bf16_bits_to_f32(x[v] >> 16);
      }
    }
  }
#pragma unroll
  for (int v = 0; v < VE; ++v) scratch[rg * D + cg * VE + v] = acc[v];
  __syncthreads();
  const float rs = __fsqrt_rn((float)nrows);
  for (int x = threadIdx.x; x < D; x += kThreads) {
    float s = 0.f;
    for (int g = 0; g < RG; ++g) s += scratch[g * D + x];
    out[x] = __fdiv_rn(s, rs);
  }
  __syncthreads();
}

// One block per (b, head, complete chunk in [chunk_begin, chunk_end)).
template <int D, int DT>
__global__ void __launch_bounds__(kThreads) chunk_keys_kernel(const void* K, float* khat,
                                                              const int32_t* offs, int64_t n_max,
                                                              int n_cap, int chunk_begin,
                                                              int nchunks) {
  __shared__ float scratch[kThreads * (DT == kF32 ? 4 : 8)];
  __shared__ float kh[D];
  const int64_t bh = blockIdx.x / nchunks;
  const int k = chunk_begin + (int)(blockIdx.x % nchunks);
  const int j0 = offs[k - chunk_begin], len = offs[k - chunk_begin + 1] - j0;
  pool_rows<D, DT>(K, bh * n_max + j0, len, kh, scratch);
  for (int x = threadIdx.x; x < D; x += kThreads) khat[(bh * n_cap + k) * D + x] = kh[x];
}

template <int D, int DT>
__global__ void __launch_bounds__(kThreads) score_kernel(DhsaDecodeArgs a) {
  __shared__ float scratch[kThreads * (DT == kF32 ? 4 : 8)];
  __shared__ float qh[D], kc[D];
  __shared__ int32_t part[kThreads];
  __shared__ int s_pw;
  extern __shared__ uint64_t dyn[];
  uint64_t* keys = dyn;                      // [P]
  int32_t* cum = (int32_t*)(dyn + a.P);      // [P + 1]
  const int64_t bh = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int n = a.n, nc = a.n + 1;           // complete chunks, plus the current one
  const int cur0 = a.offs[n];                // first token of the current chunk
  pool_rows<D, DT>(a.qcur, bh * a.m, a.m, qh, scratch);
  pool_rows<D, DT>(a.Kc, bh * a.n_max + cur0, a.m, kc, scratch);
  // S_c[k] = q_hat . k_hat_k: one wave per chunk, lanes split the columns
  constexpr int CPL = D / 64;
  for (int k = w; k < nc; k += kThreads / kWave) {
    const float* kr = k < n ? a.khat + (bh * a.n_cap + k) * D : kc;
    float s = 0.f;
#pragma unroll
    for (int x = 0; x < CPL; ++x) s += qh[CPL * lane + x] * kr[CPL * lane + x];
    s = wave_sum(s);
    if (lane == 0) keys[k] = select_key(s, (uint32_t)k);
  }
  for (int i = nc + tid; i < a.P; i += kThreads) keys[i] = 0ull;
  __syncthreads();
  // bitonic sort, descending: (S_c desc, chunk index asc); padding last
  for (int k = 2; k <= a.P; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      for (int i = tid; i < a.P; i += kThreads) {
        const int ixj = i ^ j;
        if (ixj > i) {
          const uint64_t x = keys[i], y = keys[ixj];
          const bool desc = (i & k) == 0;
          if (desc ? (x < y) : (x > y)) {
            keys[i] = y;
            keys[ixj] = x;
          }
        }
      }
      __syncthreads();
    }
  }
  // cum[p] = tokens of the chunks ranked before p, p = 0..nc
  const int per = (nc + kThreads - 1) / kThreads;
  const int p0 = tid * per;
  int32_t s = 0;
  for (int p = p0; p < min(p0 + per, nc); ++p) {
    const int k = (int)key_index(keys[p]);
    s += k < n ? a.offs[k + 1] - a.offs[k] : a.m;
  }
  part[tid] = s;
  __syncthreads();
  if (tid == 0) {
    int32_t acc = 0;
    for (int t = 0; t < kThreads; ++t) {
      const int32_t v = part[t];
      part[t] = acc;
      acc += v;
    }
  }
  __syncthreads();
  int32_t run = part[tid];
  for (int p = p0; p < min(p0 + per, nc); ++p) {
    cum[p] = run;
    const int k = (int)key_index(keys[p]);
    run += k < n ? a.offs[k + 1] - a.offs[k] : a.m;
  }
  if (p0 < nc && p0 + per >= nc) cum[nc] = run;
  __syncthreads();
  // the cut: pw whole chunks in rank order, then rem lowest tokens of the next
  const int64_t keep = min(a.budget, a.pos + 1);
  if (tid == 0) {
    int lo = 0, hi = nc;  // largest p with cum[p] <= keep
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (cum[mid] <= keep)
        lo = mid;
      else
        hi = mid - 1;
    }
    s_pw = lo;
  }
  __syncthreads();
  const int pw = s_pw;
  const int rem = (int)(keep - cum[pw]);
  int32_t* plan = a.plan + bh * nc * 2;
  for (int p = tid; p < nc; p += kThreads) {
    const int k = (int)key_index(keys[p]);
    const int start = a.offs[k];  // the current chunk starts at offs[n]
    if (p < pw) {
      plan[2 * p] = start;
      plan[2 * p + 1] = k < n ? a.offs[k + 1] - start : a.m;
    } else if (p == pw && rem > 0) {
      plan[2 * p] = start;
      plan[2 * p + 1] = rem;
    }
    if (a.chunk_order) a.chunk_order[bh * nc + p] = k;
  }
  if (tid == 0) a.n_plan[bh] = pw + (pw < nc && rem > 0 ? 1 : 0);
}

// One block per (b, head, run of the plan): keys [start, start + count),
// 64 per wave step; lane = key for the logit, lane = column pair for the
// weighted value sum (weights broadcast from LDS).
template <int D, int DT>
__global__ void __launch_bounds__(kThreads) attend_kernel(DhsaDecodeArgs a, float scale) {
  __shared__ float qs[D];
  __shared__ __attribute__((aligned(16))) float ps[kThreads / kWave][kWave];
  __shared__ float wm[kThreads / kWave], wl[kThreads / kWave];
  __shared__ float wo[kThreads / kWave][D];
  const int nc = a.n + 1;
  const int64_t bh = blockIdx.x / nc;
  const int p = blockIdx.x % nc;
  if (p >= a.n_plan[bh]) return;
  const int start = a.plan[(bh * nc + p) * 2], count = a.plan[(bh * nc + p) * 2 + 1];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  constexpr int CPL = D / 64;
  constexpr int VE = DT == kF32 ? 4 : 8;
  for (int x = tid; x < D; x += kThreads)
    qs[x] = load_elem<DT>(a.qcur, (bh * a.m + a.m - 1) * D + x);
  __syncthreads();
  const int64_t kv0 = bh * a.n_max * D;
  float m = -INFINITY, l = 0.f, o[CPL];
#pragma unroll
  for (int x = 0; x < CPL; ++x) o[x] = 0.f;
  for (int j0 = kWave * w; j0 < count; j0 += kThreads) {
    const int nk = min(kWave, count - j0);
    const int64_t row = start + j0 + lane;
    float dot = -INFINITY;
    if (lane < nk) {
      float acc = 0.f;
#pragma unroll
      for (int x = 0; x < D; x += VE) {
        if (DT == kF32) {
          const f32x4 k4 = *(const f32x4*)((const float*)a.Kc + kv0 + row * D + x);
#pragma unroll
          for (int v = 0; v < 4; ++v) acc += qs[x + v] * k4[v];
        } else {
          const u32x4 k8 = *(const u32x4*)((const uint16_t*)a.Kc + kv0 + row * D + x);
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            acc += qs[x + 2 * v] * bf16_bits_to_f32(k8[v] & 0xffffu);
            acc += qs[x + 2 * v + 1] * bf16_bits_to_f32(k8[v] >> 16);
          }
        }
      }
      dot = acc * scale;
    }
    const float mn = fmaxf(m, wave_max(dot));
    const float al = expf(m - mn);
    const float pj = lane < nk ? expf(dot - mn) : 0.f;
    l = l * al + wave_sum(pj);
    m = mn;
#pragma unroll
    for (int x = 0; x < CPL; ++x) o[x] *= al;
    ps[w][lane] = pj;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    for (int jj = 0; jj < nk; ++jj) {
      const float pw = ps[w][jj];
      const int64_t e = kv0 + (start + j0 + jj) * D + CPL * lane;
#pragma unroll
      for (int x = 0; x < CPL; ++x) o[x] += pw * load_elem<DT>(a.Vc, e + x);
    }
    __builtin_amdgcn_wave_barrier();
  }
  if (lane == 0) {
    wm[w] = m;
    wl[w] = l;
  }
#pragma unroll
  for (int x = 0; x < CPL; ++x) wo[w][CPL * lane + x] = o[x];
  __syncthreads();
  float* part = a.part + (bh * nc + p) * (D + 2);
  float M = -INFINITY;
  for (int v = 0; v < kThreads / kWave; ++v) M = fmaxf(M, wm[v]);
  for (int x = tid; x < D + 1; x += kThreads) {
    float acc = 0.f;
    for (int v = 0; v < kThreads / kWave; ++v) {
      if (wm[v] == -INFINITY) continue;  // a wave without keys
      acc += (x < D ? wo[v][x] : wl[v]) * expf(wm[v] - M);
    }
    if (x < D)
      part[2 + x] = acc;
    else
      part[1] = acc;
  }
  if (tid == 0) part[0] = M;
}

// Per (b, head): out = sum_p o_p e^(m_p - M) / sum_p l_p e^(m_p - M).
template <int D, int DT>
__global__ void __launch_bounds__(D) combine_kernel(DhsaDecodeArgs a) {
  const int nc = a.n + 1;
  const int64_t bh = blockIdx.x;
  const int np = a.n_plan[bh];
  const float* part = a.part + bh * nc * (D + 2);
  float M = -INFINITY;
  for (int p = 0; p < np; ++p) M = fmaxf(M, part[p * (D + 2)]);
  float L = 0.f, O = 0.f;
  const int x = threadIdx.x;
  for (int p = 0; p < np; ++p) {
    const float f = expf(part[p * (D + 2)] - M);
    L += part[p * (D + 2) + 1] * f;
    O += part[p * (D + 2) + 2 + x] * f;
  }
  store_elem<DT>(a.o, bh * D + x, np > 0 ? O / L : 0.f);
}

template <int D, int DT>
hipError_t decode_dt(const DhsaDecodeArgs& a, int stage, hipStream_t stream) {
  const int64_t BH = (int64_t)a.B * a.H;
  const int nc = a.n + 1;
  switch (stage) {
    case 0:
      score_kernel<D, DT><<<dim3((unsigned)BH), dim3(kThreads),
                            (size_t)a.P * sizeof(uint64_t) + (size_t)(a.P + 1) * sizeof(int32_t),
                            stream>>>(a);
      break;
    case 1:
      attend_kernel<D, DT><<<dim3((unsigned)(BH * nc)), dim3(kThreads), 0, stream>>>(
          a, 1.0f / sqrtf((float)D));
      break;
    default:
      combine_kernel<D, DT><<<dim3((unsigned)BH), dim3(D), 0, stream>>>(a);
      break;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t dhsa_decode_stage(const DhsaDecodeArgs& a, int stage, hipStream_t stream) {
  if (a.d == 64)
    return a.dtype == kF32 ? decode_dt<64, kF32>(a, stage, stream)
                           : decode_dt<64, kBF16>(a, stage, stream);
  return a.dtype == kF32 ? decode_dt<128, kF32>(a, stage, stream)
                         : decode_dt<128, kBF16>(a, stage, stream);
}

hipError_t launch_dhsa_chunk_keys(const void* K, float* khat, const int32_t* offs, int dtype,
                                  int64_t BH, int64_t n_max, int d, int n_cap, int chunk_begin,
                                  int chunk_end, hipStream_t stream) {
  const int nchunks = chunk_end - chunk_begin;
  const dim3 grid((unsigned)(BH * nchunks)), block(kThreads);
  if (d == 64) {
    if (dtype == kF32)
      chunk_keys_kernel<64, kF32><<<grid, block, 0, stream>>>(K, khat, offs, n_max, n_cap,
                                                              chunk_begin, nchunks);
    else
      chunk_keys_kernel<64, kBF16><<<grid, block, 0, stream>>>(K, khat, offs, n_max, n_cap,
                                                               chunk_begin, nchunks);
  } else {
    if (dtype == kF32)
      chunk_keys_kernel<128, kF32><<<grid, block, 0, stream>>>(K, khat, offs, n_max, n_cap,
                                                               chunk_begin, nchunks);
    else
      chunk_keys_kernel<128, kBF16><<<grid, block, 0, stream>>>(K, khat, offs, n_max, n_cap,
                                                                chunk_begin, nchunks);
  }
  return hipGetLastError();
}

}  // namespace hsa
