// swa.hip - sliding-window attention, the local part of the upper layers
// ([HSA] Methodology: upper layers pair local self-attention with the HSA
// module; sliding windows of 512 tokens by default).  A query at position t
// attends keys max(0, t-W+1) .. t of its KV head (grouped-query heads share
// one KV head).
//
//  prefill bf16 : MFMA flash attention.  One 256-thread block per (b, KV
//                 head, head block of GT query heads, MQ = 128/GT positions);
//                 each wave owns 32 positions of one head, the GT heads share
//                 the K/V blocks of 128 keys staged in LDS (the next block's
//                 loads in flight while the current one is computed).  Work
//                 units are dealt so that each XCD takes a contiguous run of
//                 positions: neighbouring windows overlap in its L2.
//  prefill fp32 : one lane per (row, head), online softmax on VALU.
//  decode       : one block per (b, KV head, head block): eight waves split
//                 the window into 64-key pieces (lane = key for scores, lane =
//                 column pair for values), merged in LDS.
#include <math.h>

#include <type_traits>

#include "attn_core.h"
#include "hsa_common.h"
#include "kernels.h"
#include "swa_core.h"

namespace hsa {

HSA_DCHECK_SOURCE()
namespace {

constexpr int kThreads = 256;
constexpr int kXcds = 8;

// Heads of a query group handled by one block: 4, 2 or 1, whichever is the
// largest that divides the group size.
int heads_per_block(int G) { return G % 4 == 0 ? 4 : (G % 2 == 0 ? 2 : 1); }

template <int D, int GT>
__global__ void __launch_bounds__(kThreads, 2) prefill_bf16_kernel(SwaArgs a, float scale_log2,
                                                                   int64_t n_units) {
  __shared__ KVSmemWide<D> sm;
  swa_prefill_body<D, GT>(a, scale_log2, n_units, blockIdx.x, sm);
}

// fp32: lane = (b, head, position), positions fastest.
template <int D>
__global__ void __launch_bounds__(64) prefill_f32_kernel(SwaArgs a, float scale) {
  const int64_t r = (int64_t)blockIdx.x * 64 + threadIdx.x;
  if (r >= (int64_t)a.B * a.Hq * a.L) return;
  const int64_t t = r % a.L;
  const int64_t bh = r / a.L;
  const int b = (int)(bh / a.Hq), h = (int)(bh % a.Hq);
  const int G = a.Hq / a.Hkv;
  const float* qrow = (const float*)a.Q + r * D;
  const float* Kb = (const float*)a.K + ((int64_t)b * a.Hkv + h / G) * a.L * D;
  const float* Vb = (const float*)a.V + ((int64_t)b * a.Hkv + h / G) * a.L * D;
  float q[D], o[D];
#pragma unroll
  for (int x = 0; x < D; ++x) {
    q[x] = qrow[x];
    o[x] = 0.f;
  }
  float m = -INFINITY, l = 0.f;
  for (int64_t j = max((int64_t)0, t - a.window + 1); j <= t; ++j) {
    float dot = 0.f;
#pragma unroll
    for (int x = 0; x < D; ++x) dot += q[x] * Kb[j * D + x];
    dot *= scale;
    const float mn = fmaxf(m, dot);
    const float al = expf(m - mn);
    const float p = expf(dot - mn);
    l = l * al + p;
#pragma unroll
    for (int x = 0; x < D; ++x) o[x] = o[x] * al + p * Vb[j * D + x];
    m = mn;
  }
  float* orow = (float*)a.O + r * D;
#pragma unroll
  for (int x = 0; x < D; ++x) orow[x] = o[x] / l;
}

// ------------------------------------------------------------------ decode --

constexpr int kDecWaves = 8;
constexpr int kPiece = 64;

template <int D, int DT, int GT>
__global__ void __launch_bounds__(kDecWaves * kWave) decode_kernel(SwaArgs a, float scale) {
  constexpr int CPL = D / 64;              // value columns per lane
  constexpr int VE = DT == kF32 ? 4 : 8;  // elements per 16-byte piece
  constexpr int EB = DT == kF32 ? 4 : 2;  // bytes per element
  __shared__ float qs[GT][D];
  __shared__ __attribute__((aligned(16))) float ps[kDecWaves][GT][kPiece];
  __shared__ float part[kDecWaves][GT][D + 2];
  const int G = a.Hq / a.Hkv;
  const int nhb = G / GT;
  const int64_t bg = blockIdx.x / nhb;
  const int hb = (int)(blockIdx.x % nhb);
  const int b = (int)(bg / a.Hkv), g = (int)(bg % a.Hkv);
  const int h0 = g * G + hb * GT;
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  for (int x = threadIdx.x; x < GT * D; x += kDecWaves * kWave)
    qs[x / D][x % D] = load_elem<DT>(a.Q, ((int64_t)b * a.Hq + h0 + x / D) * D + x % D);
  __syncthreads();
  const int64_t k0 = max((int64_t)0, a.n_ctx - a.window);
  const int64_t np = (a.n_ctx - k0 + kPiece - 1) / kPiece;  // 64-key pieces of the window
  const int64_t kv0 = bg * a.L * D;
  float m[GT], l[GT], o[GT][CPL];
#pragma unroll
  for (int hh = 0; hh < GT; ++hh) {
    m[hh] = -INFINITY;
    l[hh] = 0.f;
#pragma unroll
    for (int c = 0; c < CPL; ++c) o[hh][c] = 0.f;
  }
  typedef typename std::conditional<
      DT == kF32, typename std::conditional<CPL == 2, f32x2, float>::type,
      typename std::conditional<CPL == 2, uint32_t, uint16_t>::type>::type VT;
  for (int64_t pc = w; pc < np; pc += kDecWaves) {
    const int64_t start = k0 + (int64_t)pc * kPiece;
    const int nk = (int)min((int64_t)kPiece, a.n_ctx - start);
    HSA_DCHECK(start >= 0 && nk >= 1 && start + nk <= a.L);
    // keys past nk re-read the piece's last key (in bounds, weight zero)
    const int64_t row = start + min(lane, nk - 1);
    u32x4 kx[D / VE];
#pragma unroll
    for (int x = 0; x < D / VE; ++x)
      kx[x] = *(const u32x4*)((const char*)a.K + (kv0 + row * D + x * VE) * EB);
    VT vv[kPiece];
#pragma unroll
    for (int jj = 0; jj < kPiece; ++jj)
      vv[jj] = *(const VT*)((const char*)a.V +
                            (kv0 + (start + min(jj, nk - 1)) * D + CPL * lane) * EB);
    float dot[GT];
#pragma unroll
    for (int hh = 0; hh < GT; ++hh) dot[hh] = 0.f;
#pragma unroll
    for (int x = 0; x < D / VE; ++x) {
      float kf[VE];
      if constexpr (DT == kF32) {
#pragma unroll
        for (int v = 0; v < 4; ++v) kf[v] = __uint_as_float(kx[x][v]);
      } else {
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          kf[2 * v] = bf16_bits_to_f32(kx[x][v] & 0xffffu);
          kf[2 * v + 1] = bf16_bits_to_f32(kx[x][v] >> 16);
        }
      }
#pragma unroll
      for (int hh = 0; hh < GT; ++hh)
#pragma unroll
        for (int v = 0; v < VE; ++v) dot[hh] += qs[hh][x * VE + v] * kf[v];
    }
#pragma unroll
    for (int hh = 0; hh < GT; ++hh) {
      const float s = lane < nk ? dot[hh] * scale : -INFINITY;
      const float mn = fmaxf(m[hh], wave_max(s));  // finite: the piece has a key
      const float al = expf(m[hh] - mn);
      const float p = lane < nk ? expf(s - mn) : 0.f;
      l[hh] = l[hh] * al + wave_sum(p);
      m[hh] = mn;
#pragma unroll
      for (int c = 0; c < CPL; ++c) o[hh][c] *= al;
      ps[w][hh][lane] = p;
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
    for (int jj = 0; jj < kPiece; ++jj) {
      float vf[CPL];
      if constexpr (DT == kF32 && CPL == 2) {
        vf[0] = vv[jj][0];
        vf[1] = vv[jj][1];
      } else if constexpr (DT == kF32) {
        vf[0] = vv[jj];
      } else if constexpr (CPL == 2) {
        vf[0] = bf16_bits_to_f32(vv[jj] & 0xffffu);
        vf[1] = bf16_bits_to_f32(vv[jj] >> 16);
      } else {
        vf[0] = bf16_bits_to_f32(vv[jj]);
      }
#pragma unroll
      for (int hh = 0; hh < GT; ++hh) {
        const float pw = ps[w][hh][jj];  // zero past nk
#pragma unroll
        for (int c = 0; c < CPL; ++c) o[hh][c] += pw * vf[c];
      }
    }
    // the next piece overwrites ps only after every lane has read it
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }
#pragma unroll
  for (int hh = 0; hh < GT; ++hh) {
    if (lane == 0) {
      part[w][hh][0] = m[hh];
      part[w][hh][1] = l[hh];
    }
#pragma unroll
    for (int c = 0; c < CPL; ++c) part[w][hh][2 + CPL * lane + c] = o[hh][c];
  }
  __syncthreads();
  // merge the waves' partials: waves without a piece hold m = -inf, l = 0
  const int nw = (int)min(np, (int64_t)kDecWaves);
  for (int x = threadIdx.x; x < GT * D; x += kDecWaves * kWave) {
    const int hh = x / D, dx = x % D;
    float M = -INFINITY;
    for (int v = 0; v < nw; ++v) M = fmaxf(M, part[v][hh][0]);
    float L = 0.f, O = 0.f;
    for (int v = 0; v < nw; ++v) {
      const float f = expf(part[v][hh][0] - M);
      L += part[v][hh][1] * f;
      O += part[v][hh][2 + dx] * f;
    }
    store_elem<DT>(a.O, ((int64_t)b * a.Hq + h0 + hh) * D + dx, O / L);
  }
}

template <int D>
hipError_t prefill_d(const SwaArgs& a, hipStream_t stream) {
  const int G = a.Hq / a.Hkv;
  if (a.dtype == kF32) {
    const int64_t rows = (int64_t)a.B * a.Hq * a.L;
    launch<prefill_f32_kernel<D>>(dim3((unsigned)((rows + 63) / 64)), dim3(64), 0, stream, a,
                                  1.0f / sqrtf((float)D));
    return hipGetLastError();
  }
  const int GT = heads_per_block(G);
  const int MQ = 32 * 4 / GT;
  const int64_t units = (int64_t)a.B * a.Hkv * (G / GT) * ((a.L + MQ - 1) / MQ);
  const int64_t blocks = (units + kXcds - 1) / kXcds * kXcds;
  const float sl2 = 1.4426950408889634f / sqrtf((float)D);
  if (GT == 4)
    launch<prefill_bf16_kernel<D, 4>>(dim3((unsigned)blocks), dim3(kThreads), 0, stream, a, sl2,
                                      units);
  else if (GT == 2)
    launch<prefill_bf16_kernel<D, 2>>(dim3((unsigned)blocks), dim3(kThreads), 0, stream, a, sl2,
                                      units);
  else
    launch<prefill_bf16_kernel<D, 1>>(dim3((unsigned)blocks), dim3(kThreads), 0, stream, a, sl2,
                                      units);
  return hipGetLastError();
}

template <int D, int DT>
hipError_t decode_d(const SwaArgs& a, hipStream_t stream) {
  const int G = a.Hq / a.Hkv;
  const int GT = heads_per_block(G);
  const unsigned blocks = (unsigned)((int64_t)a.B * a.Hkv * (G / GT));
  const float scale = 1.0f / sqrtf((float)D);
  const dim3 th(kDecWaves * kWave);
  if (GT == 4)
    launch<decode_kernel<D, DT, 4>>(dim3(blocks), th, 0, stream, a, scale);
  else if (GT == 2)
    launch<decode_kernel<D, DT, 2>>(dim3(blocks), th, 0, stream, a, scale);
  else
    launch<decode_kernel<D, DT, 1>>(dim3(blocks), th, 0, stream, a, scale);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_swa_prefill(const SwaArgs& a, hipStream_t stream) {
  return a.d == 64 ? prefill_d<64>(a, stream) : prefill_d<128>(a, stream);
}

hipError_t launch_swa_decode(const SwaArgs& a, hipStream_t stream) {
  if (a.d == 64)
    return a.dtype == kF32 ? decode_d<64, kF32>(a, stream) : decode_d<64, kBF16>(a, stream);
  return a.dtype == kF32 ? decode_d<128, kF32>(a, stream) : decode_d<128, kBF16>(a, stream);
}

}  // namespace hsa
