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
//                  in LDS, and the top-N_b cut as runs of keys (whole chunks
//                  in rank order, then the lowest tokens of one), split into
//                  pieces of at most 64 keys.
//  2. attend     : one wave per (b, head, piece): softmax partials (max, sum,
//                  weighted values) of the new query over the piece's keys.
//  3. combine    : per (b, head): the pieces' partials into the output.
#include <math.h>

#include <type_traits>

#include "hsa_common.h"
#include "kernels.h"

namespace hsa {

HSA_DCHECK_SOURCE()
namespace {

constexpr int kThreads = 256;
constexpr int kPiece = 64;  // keys per attention piece (one per lane)

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

// pool_rows over two sources at once (the current chunk's queries and
// keys), their loads in flight together; barriers order LDS only, so
// global loads issued before the call stay in flight.  `scratch` holds
// 2 * kThreads * VE floats.
template <int D, int DT>
__device__ void pool_rows2(const void* srcA, int64_t rowA, const void* srcB, int64_t rowB,
                           int nrows, float* outA, float* outB, float* scratch) {
  constexpr int VE = DT == kF32 ? 4 : 8;  // elements per 16-byte piece
  constexpr int CG = D / VE;              // pieces per row
  constexpr int RG = kThreads / CG;       // row groups
  const int cg = threadIdx.x % CG, rg = threadIdx.x / CG;
  float accA[VE], accB[VE];
#pragma unroll
  for (int v = 0; v < VE; ++v) accA[v] = accB[v] = 0.f;
  for (int r = rg; r < nrows; r += RG) {
    const int64_t ea = (rowA + r) * D + cg * VE, eb = (rowB + r) * D + cg * VE;
    if (DT == kF32) {
      const f32x4 x = *(const f32x4*)((const float*)srcA + ea);
      const f32x4 y = *(const f32x4*)((const float*)srcB + eb);
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        accA[v] += x[v];
        accB[v] += y[v];
      }
    } else {
      const u32x4 x = *(const u32x4*)((const uint16_t*)srcA + ea);
      const u32x4 y = *(const u32x4*)((const uint16_t*)srcB + eb);
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        accA[2 * v] += bf16_bits_to_f32(x[v] & 0xffffu);
        accA[2 * v + 1] += bf16_bits_to_f32(x[v] >> 16);
        accB[2 * v] += bf16_bits_to_f32(y[v] & 0xffffu);
        accB[2 * v + 1] += bf16_bits_to_f32(y[v] >> 16);
      }
    }
  }
#pragma unroll
  for (int v = 0; v < VE; ++v) {
    scratch[rg * D + cg * VE + v] = accA[v];
    scratch[(RG + rg) * D + cg * VE + v] = accB[v];
  }
  block_sync_lds();
  const float rs = __fsqrt_rn((float)nrows);
  for (int x = threadIdx.x; x < D; x += kThreads) {
    float sa = 0.f, sb = 0.f;
    for (int g = 0; g < RG; ++g) {
      sa += scratch[g * D + x];
      sb += scratch[(RG + g) * D + x];
    }
    outA[x] = __fdiv_rn(sa, rs);
    outB[x] = __fdiv_rn(sb, rs);
  }
  block_sync_lds();
}

// Exclusive prefix sum of one int per thread over the block's kThreads
// threads (wave scans, then the four wave totals); *total receives the sum.
// `wsum` is kThreads / 64 ints of LDS.  Called by all threads; contains
// barriers.
__device__ int block_exclusive_scan(int v, int* wsum, int* total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  int incl = v;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const int y = __shfl_up(incl, o, kWave);
    if (lane >= o) incl += y;
  }
  if (lane == kWave - 1) wsum[w] = incl;
  __syncthreads();
  int base = 0, all = 0;
#pragma unroll
  for (int i = 0; i < kThreads / kWave; ++i) {
    base += i < w ? wsum[i] : 0;
    all += wsum[i];
  }
  __syncthreads();
  *total = all;
  return base + incl - v;
}

constexpr int kRankSortMax = 1024;  // chunks ranked by counting (else bitonic)

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

// dynamic LDS of the score kernel: keys [P], cum [P + 1], and with the
// counting rank a second key buffer [P] (8-byte aligned)
size_t dhsa_score_lds(int P) {
  const size_t cum_bytes = ((size_t)(P + 1) * sizeof(int32_t) + 7) / 8 * 8;
  return (size_t)P * sizeof(uint64_t) + cum_bytes +
         (P <= kRankSortMax ? (size_t)P * sizeof(uint64_t) : 0);
}

template <int D, int DT>
__global__ void __launch_bounds__(kThreads) score_kernel(DhsaDecodeArgs a) {
  __shared__ float scratch[2 * kThreads * (DT == kF32 ? 4 : 8)];
  __shared__ __attribute__((aligned(16))) float qh[D], kc[D];
  __shared__ int32_t part[kThreads / kWave];
  __shared__ int s_pw;
  extern __shared__ uint64_t dyn[];
  uint64_t* keys = dyn;                      // [P]
  int32_t* cum = (int32_t*)(dyn + a.P);      // [P + 1]
  const int64_t bh = blockIdx.x;
  const int tid = threadIdx.x;
  const int n = a.n, nc = a.n + 1;           // complete chunks, plus the current one
  const int cur0 = a.offs[n];                // first token of the current chunk
  // S_c[k] = q_hat . k_hat_k: one thread per chunk, its row's loads all in
  // flight at once (the pooled-key stream is this kernel's HBM traffic);
  // the first row of each thread loads while the current chunk is pooled
  f32x4 r[D / 4];
  auto load_khat = [&](int k) {
    const f32x4* kr = (const f32x4*)(a.khat + (bh * a.n_cap + k) * D);
#pragma unroll
    for (int x = 0; x < D / 4; ++x) r[x] = kr[x];
  };
  if (tid < n) load_khat(tid);
  pool_rows2<D, DT>(a.qcur, bh * a.m, a.Kc, bh * a.n_max + cur0, a.m, qh, kc, scratch);
  for (int k = tid; k < nc; k += kThreads) {
    if (k < n) {
      if (k != tid) load_khat(k);
    } else {
#pragma unroll
      for (int x = 0; x < D / 4; ++x) r[x] = *(const f32x4*)(&kc[4 * x]);
    }
    float s = 0.f;
#pragma unroll
    for (int x = 0; x < D / 4; ++x)
#pragma unroll
      for (int v = 0; v < 4; ++v) s += qh[4 * x + v] * r[x][v];
    keys[k] = select_key(s, (uint32_t)k);
  }
  for (int i = nc + tid; i < a.P; i += kThreads) keys[i] = 0ull;
  __syncthreads();
  if (a.P <= kRankSortMax) {
    // rank by counting: each key's position is the number of larger keys
    // (keys are distinct); the ranked keys go to the second buffer
    uint64_t* ranked = (uint64_t*)((char*)cum + ((size_t)(a.P + 1) * sizeof(int32_t) + 7) / 8 * 8);
    for (int i = tid; i < nc; i += kThreads) {
      const uint64_t x = keys[i];
      int r = 0;
      for (int j = 0; j < nc; ++j) r += keys[j] > x;
      ranked[r] = x;
    }
    __syncthreads();
    for (int i = tid; i < nc; i += kThreads) keys[i] = ranked[i];
    __syncthreads();
  } else {
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
  }
  // cum[p] = tokens of the chunks ranked before p, p = 0..nc
  const int per = (nc + kThreads - 1) / kThreads;
  const int p0 = tid * per;
  int32_t s = 0;
  for (int p = p0; p < min(p0 + per, nc); ++p) {
    const int k = (int)key_index(keys[p]);
    s += k < n ? a.offs[k + 1] - a.offs[k] : a.m;
  }
  int32_t tokens_all;  // cum[nc], written below by the thread holding the last rank
  int32_t run = block_exclusive_scan(s, part, &tokens_all);
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
  // runs: p < pw whole chunks, p == pw the first rem tokens; each run is
  // cut into pieces of kPiece keys, numbered by an exclusive scan over runs
  auto run_of = [&](int p, int& start, int& count) {
    const int k = (int)key_index(keys[p]);
    start = a.offs[k];  // the current chunk starts at offs[n]
    count = p < pw ? (k < n ? a.offs[k + 1] - start : a.m) : (p == pw ? rem : 0);
  };
  int32_t pieces = 0;
  for (int p = p0; p < min(p0 + per, nc); ++p) {
    int st, cnt;
    run_of(p, st, cnt);
    pieces += (cnt + kPiece - 1) / kPiece;
  }
  int32_t pieces_all;
  int32_t q = block_exclusive_scan(pieces, part, &pieces_all);
  HSA_DCHECK(pieces_all <= a.max_pieces);
  if (tid == 0) a.n_plan[bh] = pieces_all;
  int32_t* plan = a.plan + bh * a.max_pieces * 2;
  for (int p = p0; p < min(p0 + per, nc); ++p) {
    int st, cnt;
    run_of(p, st, cnt);
    for (int c0 = 0; c0 < cnt; c0 += kPiece, ++q) {
      plan[2 * q] = st + c0;
      plan[2 * q + 1] = min(kPiece, cnt - c0);
    }
  }
  if (a.chunk_order)
    for (int p = tid; p < nc; p += kThreads) a.chunk_order[bh * nc + p] = (int)key_index(keys[p]);
}

// One wave per (b, head, piece of at most 64 keys): every load of the piece
// is issued at once, the key rows with lane = key and the value rows with
// lane = column pair (values stay packed until used); the weights pass
// through LDS.  Writes the piece's (max, sum, weighted values).
template <int D, int DT>
__global__ void __launch_bounds__(kWave) attend_kernel(DhsaDecodeArgs a, float scale) {
  __shared__ float qs[D];
  __shared__ __attribute__((aligned(16))) float ps[kPiece];
  const int64_t bh = blockIdx.x / a.max_pieces;
  const int q = (int)(blockIdx.x % a.max_pieces);
  if (q >= a.n_plan[bh]) return;
  const int start = a.plan[(bh * a.max_pieces + q) * 2];
  const int nk = a.plan[(bh * a.max_pieces + q) * 2 + 1];
  // a piece holds 1..64 keys, all at or before the new query's position
  HSA_DCHECK(start >= 0 && nk >= 1 && nk <= kPiece && start + nk <= a.pos + 1);
  const int lane = threadIdx.x;
  constexpr int CPL = D / 64;
  constexpr int VE = DT == kF32 ? 4 : 8;
  constexpr int EB = DT == kF32 ? 4 : 2;
  const int64_t kv0 = bh * a.n_max * D;
  // keys past nk re-read the piece's last key (in bounds, weight zero)
  const int64_t row = start + min(lane, nk - 1);
  u32x4 kx[D / VE];
#pragma unroll
  for (int x = 0; x < D / VE; ++x)
    kx[x] = *(const u32x4*)((const char*)a.Kc + (kv0 + row * D + x * VE) * EB);
  // value columns CPL*lane .. +CPL-1 of every key of the piece
  typedef typename std::conditional<
      DT == kF32, typename std::conditional<CPL == 2, f32x2, float>::type,
      typename std::conditional<CPL == 2, uint32_t, uint16_t>::type>::type VT;
  VT vv[kPiece];
#pragma unroll
  for (int jj = 0; jj < kPiece; ++jj)
    vv[jj] = *(const VT*)((const char*)a.Vc +
                          (kv0 + (int64_t)(start + min(jj, nk - 1)) * D + CPL * lane) * EB);
  for (int x = lane; x < D; x += kWave)
    qs[x] = load_elem<DT>(a.qcur, (bh * a.m + a.m - 1) * D + x);
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  float dot = -INFINITY;
  if (lane < nk) {
    float acc = 0.f;
#pragma unroll
    for (int x = 0; x < D / VE; ++x) {
      if constexpr (DT == kF32) {
#pragma unroll
        for (int v = 0; v < 4; ++v) acc += qs[x * VE + v] * __uint_as_float(kx[x][v]);
      } else {
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          acc += qs[x * VE + 2 * v] * bf16_bits_to_f32(kx[x][v] & 0xffffu);
          acc += qs[x * VE + 2 * v + 1] * bf16_bits_to_f32(kx[x][v] >> 16);
        }
      }
    }
    dot = acc * scale;
  }
  const float m = wave_max(dot);
  const float pj = lane < nk ? expf(dot - m) : 0.f;
  const float l = wave_sum(pj);
  ps[lane] = pj;
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  float o[CPL];
#pragma unroll
  for (int x = 0; x < CPL; ++x) o[x] = 0.f;
#pragma unroll
  for (int jj = 0; jj < kPiece; ++jj) {
    const float pw = ps[jj];  // zero past nk
    if constexpr (DT == kF32 && CPL == 2) {
      o[0] += pw * vv[jj][0];
      o[1] += pw * vv[jj][1];
    } else if constexpr (DT == kF32) {
      o[0] += pw * vv[jj];
    } else if constexpr (CPL == 2) {
      o[0] += pw * bf16_bits_to_f32(vv[jj] & 0xffffu);
      o[1] += pw * bf16_bits_to_f32(vv[jj] >> 16);
    } else {
      o[0] += pw * bf16_bits_to_f32(vv[jj]);
    }
  }
  float* part = a.part + (bh * a.max_pieces + q) * (D + 2);
  if (lane == 0) {
    part[0] = m;
    part[1] = l;
  }
  if constexpr (CPL == 2)
    *(f32x2*)(part + 2 + 2 * lane) = f32x2{o[0], o[1]};
  else
    part[2 + lane] = o[0];
}

// Per (b, head): out = sum_q o_q e^(m_q - M) / sum_q l_q e^(m_q - M) over
// the pieces q.  The pieces' (max, sum) pairs are read once into LDS by one
// thread each and reduced by waves; then thread t adds column t % D over
// every kThreads / D-th piece with 8 loads in flight, and the column's
// partial sums meet in LDS.
template <int D, int DT>
__global__ void __launch_bounds__(kThreads) combine_kernel(DhsaDecodeArgs a) {
  constexpr int PS = kThreads / D;  // piece subsets
  extern __shared__ float cw[];     // [max_pieces]: e^(m_q - M)
  __shared__ float red[kThreads / kWave];
  __shared__ float acc_s[PS][D];
  const int64_t bh = blockIdx.x;
  const int np = a.n_plan[bh];
  const float* part = a.part + bh * a.max_pieces * (D + 2);
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  float M = -INFINITY;
  for (int q = tid; q < np; q += kThreads) M = fmaxf(M, part[q * (D + 2)]);
  M = wave_max_f32(M);
  if (lane == 0) red[w] = M;
  __syncthreads();
#pragma unroll
  for (int i = 0; i < kThreads / kWave; ++i) M = fmaxf(M, red[i]);
  __syncthreads();
  float L = 0.f;
  for (int q = tid; q < np; q += kThreads) {
    const float f = expf(part[q * (D + 2)] - M);
    cw[q] = f;
    L += part[q * (D + 2) + 1] * f;
  }
  L = wave_sum_f32(L);
  if (lane == 0) red[w] = L;
  __syncthreads();
  L = 0.f;
#pragma unroll
  for (int i = 0; i < kThreads / kWave; ++i) L += red[i];
  const int x = tid % D, sub = tid / D;
  float O = 0.f;
  int q = sub;
  for (; q + 7 * PS < np; q += 8 * PS) {
    float v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = part[(q + u * PS) * (D + 2) + 2 + x];
#pragma unroll
    for (int u = 0; u < 8; ++u) O += v[u] * cw[q + u * PS];
  }
  for (; q < np; q += PS) O += part[q * (D + 2) + 2 + x] * cw[q];
  acc_s[sub][x] = O;
  __syncthreads();
  if (sub == 0) {
    float t = 0.f;
#pragma unroll
    for (int i = 0; i < PS; ++i) t += acc_s[i][x];
    store_elem<DT>(a.o, bh * D + x, np > 0 ? t / L : 0.f);
  }
}

template <int D, int DT>
hipError_t decode_dt(const DhsaDecodeArgs& a, int stage, hipStream_t stream) {
  const int64_t BH = (int64_t)a.B * a.H;
  switch (stage) {
    case 0:
      launch<score_kernel<D, DT>>(dim3((unsigned)BH), dim3(kThreads), dhsa_score_lds(a.P), stream,
                                  a);
      break;
    case 1:
      launch<attend_kernel<D, DT>>(dim3((unsigned)(BH * a.max_pieces)), dim3(kWave), 0, stream, a,
                                   1.0f / sqrtf((float)D));
      break;
    default:
      launch<combine_kernel<D, DT>>(dim3((unsigned)BH), dim3(kThreads),
                                    (size_t)a.max_pieces * sizeof(float), stream, a);
      break;
  }
  return hipGetLastError();
}

}  // namespace

int64_t dhsa_decode_max_pieces(int64_t keep_max, int n_chunks) {
  // each kept run (at most n_chunks + 1) adds at most one partial piece
  return (keep_max + kPiece - 1) / kPiece + n_chunks + 1;
}

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
      launch<chunk_keys_kernel<64, kF32>>(grid, block, 0, stream, K, khat, offs, n_max, n_cap,
                                          chunk_begin, nchunks);
    else
      launch<chunk_keys_kernel<64, kBF16>>(grid, block, 0, stream, K, khat, offs, n_max, n_cap,
                                           chunk_begin, nchunks);
  } else {
    if (dtype == kF32)
      launch<chunk_keys_kernel<128, kF32>>(grid, block, 0, stream, K, khat, offs, n_max, n_cap,
                                           chunk_begin, nchunks);
    else
      launch<chunk_keys_kernel<128, kBF16>>(grid, block, 0, stream, K, khat, offs, n_max, n_cap,
                                            chunk_begin, nchunks);
  }
  return hipGetLastError();
}

}  // namespace hsa
