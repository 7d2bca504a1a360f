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

namespace hsa {
namespace {

constexpr int kThreads = 256;

// ---------------------------------------------------------------- select --

// Keep a descending top-KM list in registers.  Candidates of one lane
// arrive in increasing index order, so a strict '>' places a later
// equal-score candidate after the earlier one (lower index first).
template <int KM>
__device__ __forceinline__ void topk_insert_ordered(float (&ls)[KM], int (&li)[KM], float s,
                                                    int c) {
#pragma unroll
  for (int j = KM - 1; j >= 0; --j) {
    const bool gt_prev = j > 0 ? (s > ls[j > 0 ? j - 1 : 0]) : false;
    const bool gt_cur = s > ls[j];
    const float ns = gt_prev ? ls[j > 0 ? j - 1 : 0] : (gt_cur ? s : ls[j]);
    const int ni = gt_prev ? li[j > 0 ? j - 1 : 0] : (gt_cur ? c : li[j]);
    ls[j] = ns;
    li[j] = ni;
  }
}

// Full (score desc, index asc) comparison for merging lists of different
// lanes/waves.
__device__ __forceinline__ bool better(float s, int c, float t, int d) {
  return s > t || (s == t && c < d);
}

template <int KM>
__device__ __forceinline__ void topk_insert_any(float (&ls)[KM], int (&li)[KM], float s, int c) {
  if (c < 0) return;
#pragma unroll
  for (int j = KM - 1; j >= 0; --j) {
    const bool gt_prev = j > 0 ? better(s, c, ls[j > 0 ? j - 1 : 0], li[j > 0 ? j - 1 : 0])
                               : false;
    const bool gt_cur = better(s, c, ls[j], li[j]);
    const float ns = gt_prev ? ls[j > 0 ? j - 1 : 0] : (gt_cur ? s : ls[j]);
    const int ni = gt_prev ? li[j > 0 ? j - 1 : 0] : (gt_cur ? c : li[j]);
    ls[j] = ns;
    li[j] = ni;
  }
}

// One block = 64 consecutive queries of one (b, group); lane = query.  The
// four waves take interleaved quarters of each 32-landmark tile and merge
// their lists at the end.  Scores are ranked unscaled (u . lmk): the
// positive factor 1/sqrt(d) does not change the order.
template <int D, int KM, int DT>
__global__ void __launch_bounds__(kThreads) select_valu_kernel(PrefillArgs a, int64_t nqt) {
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
  const int64_t t = qt * 64 + lane;
  const bool tvalid = t < a.L;
  const int64_t navail = tvalid ? min(t / a.S, a.n) : 0;
  const int64_t tlast = min(qt * 64 + 63, a.L - 1);
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
      if (c < navail) topk_insert_ordered<KM>(ls, li, dot, (int)c);
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
  int32_t* out = a.idx + (bg * a.L + t) * a.topk;
  int32_t* cnt = a.counts + bg * a.n;
#pragma unroll
  for (int j = 0; j < KM; ++j) {
    if (j < a.topk) {
      out[j] = li[j];
      if (li[j] >= 0) atomicAdd(&cnt[li[j]], 1);
    }
  }
}

// ---------------------------------------------------------------- invert --

// One block per (b, group): exclusive scans of the selection counts
// (entry offsets) and of the per-chunk tile counts (tile offsets).
__global__ void __launch_bounds__(1024) scan_kernel(PrefillArgs a) {
  __shared__ int32_t sa[1024], sb[1024];
  __shared__ int32_t carry_a, carry_b;
  const int64_t bg = blockIdx.x;
  const int32_t* cnt = a.counts + bg * a.n;
  int32_t* offs = a.offs + bg * (a.n + 1);
  int32_t* toff = a.tile_off + bg * (a.n + 1);
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
      offs[c] = carry_a + sa[threadIdx.x] - v;
      toff[c] = carry_b + sb[threadIdx.x] - (v + E - 1) / E;
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

// One thread per (b, group, token, slot): append (token*topk + slot) to the
// selected chunk's list.  The order inside a list does not affect results:
// every row is computed independently of the others in its tile.
__global__ void scatter_kernel(PrefillArgs a) {
  const int64_t total = (int64_t)a.B * a.Hkv * a.L * a.topk;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int32_t c = a.idx[i];
    if (c < 0) continue;
    const int64_t bg = i / (a.L * a.topk);
    const int32_t e = (int32_t)(i % (a.L * a.topk));
    const int32_t pos = a.offs[bg * (a.n + 1) + c] + atomicAdd(&a.cursor[bg * a.n + c], 1);
    a.list[bg * a.L * a.topk + pos] = e;
  }
}

// ---------------------------------------------------------------- attend --

// Locate this block's chunk and entry range.  Returns false for blocks past
// the last tile of their (b, group).
__device__ __forceinline__ bool locate_tile(const PrefillArgs& a, int64_t& bg, int& c, int& e0,
                                            int& e1) {
  bg = blockIdx.x / a.tiles_ub;
  const int64_t tile = blockIdx.x % a.tiles_ub;
  const int32_t* toff = a.tile_off + bg * (a.n + 1);
  if (tile >= toff[a.n]) return false;
  int lo = 0, hi = (int)a.n - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (toff[mid] <= tile)
      lo = mid;
    else
      hi = mid - 1;
  }
  c = lo;
  const int32_t* offs = a.offs + bg * (a.n + 1);
  e0 = offs[c] + (int)(tile - toff[c]) * a.entries_per_tile;
  e1 = min(e0 + a.entries_per_tile, offs[c + 1]);
  return true;
}

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
  const int64_t t = entry / a.topk;
  const int slot = entry % a.topk;
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
    if (wave_any) wave_attn_block<D>(st, sm, valid ? nk : 0, scale_log2);
  }
  if (!wave_any) return;
  float s = wave_q_dot_half<D>(st, a.lmk + (bg * a.n + c) * D);
  s += __shfl_xor(s, 32, kWave);
  if (!valid) return;
  const int64_t row = (((int64_t)b * a.Hq + h) * a.L + t) * a.topk + slot;
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
  const int64_t t = entry / a.topk;
  const int slot = entry % a.topk;
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
  const int64_t row = (((int64_t)b * a.Hq + h) * a.L + t) * a.topk + slot;
  a.part_score[row] = s * score_scale;
  float* po = (float*)a.partial + row * D;
#pragma unroll
  for (int x = 0; x < D; ++x) po[x] = o[x] / l;
}

// ------------------------------------------------------------------ fuse --

// One group of D/VEC threads per (b, head, token) row.
template <int D, int DT>
__global__ void __launch_bounds__(kThreads) fuse_kernel(PrefillArgs a) {
  constexpr int VEC = DT == kF32 ? 4 : 8;
  constexpr int TPR = D / VEC;
  constexpr int RPB = kThreads / TPR;
  const int64_t row = (int64_t)blockIdx.x * RPB + threadIdx.x / TPR;
  const int cg = threadIdx.x % TPR;
  const int64_t total = (int64_t)a.B * a.Hq * a.L;
  if (row >= total) return;
  const int64_t t = row % a.L;
  const int m = (int)min((int64_t)a.topk, min(t / a.S, a.n));
  const float* sc = a.part_score + row * a.topk;
  float smax = -INFINITY;
  for (int k = 0; k < m; ++k) smax = fmaxf(smax, sc[k]);
  float z = 0.f;
  for (int k = 0; k < m; ++k) z += expf(sc[k] - smax);
  float acc[VEC];
#pragma unroll
  for (int v = 0; v < VEC; ++v) acc[v] = 0.f;
  for (int k = 0; k < m; ++k) {
    const float wk = expf(sc[k] - smax) / z;
    const int64_t base = (row * a.topk + k) * D + cg * VEC;
    if (DT == kF32) {
      const f32x4 x = *(const f32x4*)((const float*)a.partial + base);
#pragma unroll
      for (int v = 0; v < 4; ++v) acc[v] += wk * x[v];
    } else {
      const u32x4 x = *(const u32x4*)((const uint16_t*)a.partial + base);
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        acc[2 * v] += wk * bf16_bits_to_f32(x[v] & 0xffffu);
        acc[2 * v + 1] += wk * bf16_bits_to_f32(x[v] >> 16);
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
  if (a.sel_w && cg == 0) {
    for (int k = 0; k < a.topk; ++k)
      a.sel_w[row * a.topk + k] = k < m ? expf(sc[k] - smax) / z : 0.f;
  }
}

template <int D, int KM>
hipError_t launch_select_dt(const PrefillArgs& a, hipStream_t stream) {
  const int64_t nqt = (a.L + 63) / 64;
  const int64_t blocks = (int64_t)a.B * a.Hkv * nqt;
  if (a.dtype == kF32)
    select_valu_kernel<D, KM, kF32><<<dim3((unsigned)blocks), dim3(kThreads), 0, stream>>>(a, nqt);
  else
    select_valu_kernel<D, KM, kBF16><<<dim3((unsigned)blocks), dim3(kThreads), 0, stream>>>(a,
                                                                                           nqt);
  return hipGetLastError();
}

template <int D>
hipError_t launch_select_d(const PrefillArgs& a, hipStream_t stream) {
  if (a.topk <= 8) return launch_select_dt<D, 8>(a, stream);
  if (a.topk <= 16) return launch_select_dt<D, 16>(a, stream);
  return launch_select_dt<D, 32>(a, stream);
}

}  // namespace

int prefill_entries_per_tile(int dtype, int G) { return dtype == kF32 ? 64 / G : 128 / G; }

hipError_t prefill_select(const PrefillArgs& a, hipStream_t stream) {
  hipError_t e = launch_fill_i32(a.counts, (int64_t)a.B * a.Hkv * a.n, 0, stream);
  if (e != hipSuccess) return e;
  if (a.L == 0) return hipSuccess;
  return a.d == 64 ? launch_select_d<64>(a, stream) : launch_select_d<128>(a, stream);
}

hipError_t prefill_invert(const PrefillArgs& a, hipStream_t stream) {
  if (a.n == 0) return hipSuccess;
  hipError_t e = launch_fill_i32(a.cursor, (int64_t)a.B * a.Hkv * a.n, 0, stream);
  if (e != hipSuccess) return e;
  scan_kernel<<<dim3((unsigned)(a.B * a.Hkv)), dim3(1024), 0, stream>>>(a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t total = (int64_t)a.B * a.Hkv * a.L * a.topk;
  int64_t blocks = (total + 255) / 256;
  if (blocks > 16384) blocks = 16384;
  if (blocks > 0) scatter_kernel<<<dim3((unsigned)blocks), dim3(256), 0, stream>>>(a);
  return hipGetLastError();
}

hipError_t prefill_attend(const PrefillArgs& a, hipStream_t stream) {
  if (a.n == 0) return hipSuccess;
  const int64_t blocks = (int64_t)a.B * a.Hkv * a.tiles_ub;
  const float scale = 1.0f / sqrtf((float)a.d);
  const float score_scale = scale;
  if (a.dtype == kF32) {
    if (a.d == 64)
      attend_f32_kernel<64><<<dim3((unsigned)blocks), dim3(64), 0, stream>>>(a, scale,
                                                                             score_scale);
    else
      attend_f32_kernel<128><<<dim3((unsigned)blocks), dim3(64), 0, stream>>>(a, scale,
                                                                              score_scale);
  } else {
    const float sl2 = scale * 1.4426950408889634f;
    if (a.d == 64)
      attend_bf16_kernel<64><<<dim3((unsigned)blocks), dim3(kThreads), 0, stream>>>(a, sl2,
                                                                                    score_scale);
    else
      attend_bf16_kernel<128><<<dim3((unsigned)blocks), dim3(kThreads), 0, stream>>>(
          a, sl2, score_scale);
  }
  return hipGetLastError();
}

hipError_t prefill_fuse(const PrefillArgs& a, hipStream_t stream) {
  const int64_t rows = (int64_t)a.B * a.Hq * a.L;
  if (rows == 0) return hipSuccess;
  const int VEC = a.dtype == kF32 ? 4 : 8;
  const int rpb = kThreads / (a.d / VEC);
  const int64_t blocks = (rows + rpb - 1) / rpb;
  if (a.dtype == kF32) {
    if (a.d == 64)
      fuse_kernel<64, kF32><<<dim3((unsigned)blocks), dim3(kThreads), 0, stream>>>(a);
    else
      fuse_kernel<128, kF32><<<dim3((unsigned)blocks), dim3(kThreads), 0, stream>>>(a);
  } else {
    if (a.d == 64)
      fuse_kernel<64, kBF16><<<dim3((unsigned)blocks), dim3(kThreads), 0, stream>>>(a);
    else
      fuse_kernel<128, kBF16><<<dim3((unsigned)blocks), dim3(kThreads), 0, stream>>>(a);
  }
  return hipGetLastError();
}

}  // namespace hsa
