// dhsa.hip - DHSA prefill ([DHSA] "What carries the argument": chunk queries
// and keys by sqrt|C|-scaled mean pooling (Eq. 4), chunk similarity S_c,
// tiling of S_c into the token map S_t, top-N_b preceding keys per query
// (Algorithm 1), masked softmax attention).
//
// The token map is never materialised.  Every key of chunk k scores
// S_c[l,k] for a query in chunk l, so ordering keys by (score desc, j asc)
// is ordering chunks by (S_c desc, k asc) and then tokens by index: a
// query's kept set is a run of whole chunks in rank order plus the lowest
// tokens of one boundary chunk, with the query's own chunk counting only
// its tokens j <= i.
//
//  1. pool  : q_hat, k_hat per (b, h, chunk), fp32.
//  2. sc    : S_c[l,k] = q_hat_l . k_hat_k for k <= l.
//  3. rank  : per (b, h, l) bitonic sort of 64-bit keys (S_c, then lower k)
//             -> order[p], prefix lengths in rank order, and the rank of l.
//  4. attend: per (b, h, query chunk, 128-row tile): each lane's row finds
//             its cut (number of whole chunks, tokens of the boundary chunk)
//             by binary search, then the block walks the ranked chunks with
//             the MFMA attention core and per-row key limits.
//  5. mask  : optional debug bitmask of the kept keys.
#include <math.h>

#include "attn_core.h"
#include "hsa_common.h"
#include "kernels.h"

namespace hsa {
namespace {

constexpr int kThreads = 256;
// 32-key sub-tiles per online-softmax update in the attention (see
// wave_attn_wide): four, one update per key block of up to 128 keys.
constexpr int kDhsaSub = 4;
constexpr int kRowsPerTile = 128;
constexpr int kMaxSort = 4096;  // 32 KiB of 64-bit sort keys in LDS

template <int DT>
__global__ void __launch_bounds__(kThreads) pool_kernel(DhsaArgs a) {
  constexpr int VEC = DT == kF32 ? 4 : 8;
  extern __shared__ float red[];  // [2][row_sets][d]
  const int d = a.d;
  const int64_t bh = blockIdx.x / a.nc;
  const int l = blockIdx.x % a.nc;
  const int b0 = a.offs[l], b1 = a.offs[l + 1];
  const int groups = d / VEC;
  const int row_sets = kThreads / groups;
  const int cg = threadIdx.x % groups, rs = threadIdx.x / groups;
  float aq[VEC], ak[VEC];
#pragma unroll
  for (int v = 0; v < VEC; ++v) aq[v] = ak[v] = 0.f;
  for (int j = b0 + rs; j < b1; j += row_sets) {
    const int64_t off = (bh * a.L + j) * d + cg * VEC;
#pragma unroll
    for (int v = 0; v < VEC; ++v) {
      aq[v] += load_elem<DT>(a.Q, off + v);
      ak[v] += load_elem<DT>(a.K, off + v);
    }
  }
#pragma unroll
  for (int v = 0; v < VEC; ++v) {
    red[rs * d + cg * VEC + v] = aq[v];
    red[(row_sets + rs) * d + cg * VEC + v] = ak[v];
  }
  __syncthreads();
  const float rsq = __fsqrt_rn((float)(b1 - b0));
  for (int x = threadIdx.x; x < 2 * d; x += kThreads) {
    const int which = x / d, col = x % d;
    float s = 0.f;
    for (int r = 0; r < row_sets; ++r) s += red[(which * row_sets + r) * d + col];
    float* dst = which == 0 ? a.qh : a.kh;
    dst[(bh * a.nc + l) * d + col] = __fdiv_rn(s, rsq);
  }
}

// S_c row l: lanes split d into float4 pieces, reduce with shuffles.
template <int D>
__global__ void __launch_bounds__(kThreads) sc_kernel(DhsaArgs a) {
  const int64_t bh = blockIdx.x / a.nc;
  const int l = blockIdx.x % a.nc;
  constexpr int LPR = D / 4, RPW = kWave / LPR;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int li = lane % LPR, sub = lane / LPR;
  const f32x4 q4 = *(const f32x4*)(a.qh + (bh * a.nc + l) * D + 4 * li);
  // U steps of keys per round, every load issued unconditionally (keys past
  // l read key l and are not stored): loads under a per-lane guard would
  // each be waited for before the next
  constexpr int U = 4;
  for (int k0 = 0; k0 <= l; k0 += U * 4 * RPW) {
    f32x4 x[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int k = min(k0 + u * 4 * RPW + w * RPW + sub, l);
      x[u] = *(const f32x4*)(a.kh + (bh * a.nc + k) * D + 4 * li);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int k = k0 + u * 4 * RPW + w * RPW + sub;
      float p = q4[0] * x[u][0] + q4[1] * x[u][1] + q4[2] * x[u][2] + q4[3] * x[u][3];
#pragma unroll
      for (int o = LPR / 2; o > 0; o >>= 1) p += __shfl_xor(p, o, kWave);
      if (li == 0 && k <= l) a.sc[(bh * a.nc + l) * a.nc + k] = p;
    }
  }
}

__global__ void __launch_bounds__(kThreads) rank_kernel(DhsaArgs a, int P) {
  extern __shared__ uint64_t keys[];  // [P]
  __shared__ int32_t part[kThreads];
  const int64_t bh = blockIdx.x / a.nc;
  const int l = blockIdx.x % a.nc;
  const int n = l + 1;
  const float* sc = a.sc + (bh * a.nc + l) * a.nc;
  for (int i = threadIdx.x; i < P; i += kThreads)
    keys[i] = i < n ? select_key(sc[i], (uint32_t)i) : 0ull;
  __syncthreads();
  // bitonic sort, descending
  for (int k = 2; k <= P; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      for (int i = threadIdx.x; i < P; i += kThreads) {
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
  int32_t* order = a.order + (bh * a.nc + l) * a.nc;
  for (int p = threadIdx.x; p < a.nc; p += kThreads) {
    const int32_t k = p < n ? (int32_t)key_index(keys[p]) : -1;
    order[p] = k;
    if (k == l) a.diag_pos[bh * a.nc + l] = p;
  }
  // cumlen[p] = total length of the chunks ranked before p, p = 0..n
  int32_t* cum = a.cumlen + (bh * a.nc + l) * (a.nc + 1);
  const int per = (n + kThreads - 1) / kThreads;
  const int p0 = threadIdx.x * per;
  int32_t s = 0;
  for (int p = p0; p < min(p0 + per, n); ++p) {
    const int k = (int)key_index(keys[p]);
    s += a.offs[k + 1] - a.offs[k];
  }
  // exclusive scan of the threads' sums: inclusive within each wave by lane
  // shifts, then the totals of the waves before
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  int32_t inc = s;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int32_t y = __shfl_up(inc, o, kWave);
    if (lane >= o) inc += y;
  }
  if (lane == 63) part[w] = inc;
  __syncthreads();
  int32_t run = inc - s;
  for (int v = 0; v < w; ++v) run += part[v];
  for (int p = p0; p < min(p0 + per, n); ++p) {
    cum[p] = run;
    const int k = (int)key_index(keys[p]);
    run += a.offs[k + 1] - a.offs[k];
  }
  if (p0 < n && p0 + per >= n) cum[n] = run;
}

// The cut of query i (in chunk l): how many chunks in rank order are kept
// whole (pw) and how many lowest-index tokens of the next one (rem).
struct Cut {
  int pw;
  int rem;
};

__device__ __forceinline__ Cut row_cut(const DhsaArgs& a, int64_t bh, int l, int i) {
  const int bl = a.offs[l], ll = a.offs[l + 1] - bl;
  const int B = (int)min(a.budget, (int64_t)i + 1);
  const int tail = ll - (i - bl + 1);  // tokens of chunk l after i
  const int dp = a.diag_pos[bh * a.nc + l];
  const int32_t* cum = a.cumlen + (bh * a.nc + l) * (a.nc + 1);
  // E(p) = cum[p] - (p > dp ? tail : 0) is non-decreasing; find the largest
  // p in [0, l+1] with E(p) <= B.
  int lo = 0, hi = l + 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    const int e = cum[mid] - (mid > dp ? tail : 0);
    if (e <= B)
      lo = mid;
    else
      hi = mid - 1;
  }
  Cut c;
  c.pw = lo;
  c.rem = (int)(B - (cum[lo] - (lo > dp ? tail : 0)));
  return c;
}

template <int D>
__global__ void __launch_bounds__(kThreads, 2) attend_kernel(DhsaArgs a, float scale_log2) {
  __shared__ KVSmemWide<D> sm;
  __shared__ int pmax;
  // late query chunks attend the most keys: dispatch them first, with all
  // (b, h) of one chunk next to each other
  const int64_t BH = (int64_t)a.B * a.H;
  const int64_t bh = blockIdx.x % BH;
  const int64_t rest = blockIdx.x / BH;
  const int l = a.nc - 1 - (int)(rest / a.tiles_per_chunk);
  const int tile = (int)(rest % a.tiles_per_chunk);
  const int bl = a.offs[l], bl1 = a.offs[l + 1];
  const int row0 = bl + tile * kRowsPerTile;
  if (row0 >= bl1) return;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  // the tile's 32-row groups go to the waves rotated by block, so the groups
  // past a short chunk's end (idle waves) fall on different SIMDs
  const int wr = (w + (int)(blockIdx.x & 3)) & 3;
  const int i = row0 + wr * 32 + (lane & 31);  // L < 2^31 is checked on the host
  const bool valid = i < bl1;
  Cut cut = {0, 0};
  if (valid) cut = row_cut(a, bh, l, i);
  const int last = valid ? (cut.rem > 0 ? cut.pw : cut.pw - 1) : -1;
  if (threadIdx.x == 0) pmax = -1;
  __syncthreads();
  atomicMax(&pmax, last);
  __syncthreads();
  const int p_end = pmax;
  const uint16_t* Qb = (const uint16_t*)a.Q + bh * a.L * D;
  const uint16_t* Kb = (const uint16_t*)a.K + bh * a.L * D;
  const uint16_t* Vb = (const uint16_t*)a.V + bh * a.L * D;
  WaveAttn<D> st;
  wave_attn_init<D>(st, Qb + (int64_t)min(i, (int)a.L - 1) * D, valid);
  const bool wave_any = __ballot(valid) != 0;
  const int32_t* order = a.order + (bh * a.nc + l) * a.nc;
  // Key blocks in rank order: chunk order[p], keys [kb, kb + 128).  Each
  // step stores the block fetched during the previous step, starts the
  // fetch of the next one, then computes.
  int p = 0, kb = 0, k = 0, bk = 0, lk = 0;
  KVRegsWide<D> rg;
  if (p_end >= 0) {
    k = order[0];
    bk = a.offs[k];
    lk = a.offs[k + 1] - bk;
    fetch_kv_wide<D>(rg, Kb + (int64_t)bk * D, Vb + (int64_t)bk * D, min(kWideBlock, lk));
  }
  while (p <= p_end) {
    const int nk = min(kWideBlock, lk - kb);
    __syncthreads();
    store_kv_wide<D>(sm, rg, nk);
    __syncthreads();
    int np = p, nkb = kb + kWideBlock, nkc = k, nbk = bk, nlk = lk;
    if (nkb >= lk) {
      np = p + 1;
      nkb = 0;
      if (np <= p_end) {
        nkc = order[np];
        nbk = a.offs[nkc];
        nlk = a.offs[nkc + 1] - nbk;
      }
    }
    if (np <= p_end)
      fetch_kv_wide<D>(rg, Kb + (int64_t)(nbk + nkb) * D, Vb + (int64_t)(nbk + nkb) * D,
                       min(kWideBlock, nlk - nkb));
    __builtin_amdgcn_sched_barrier(0);
    const int len_eff = k == l ? i - bl + 1 : lk;
    const int hi = !valid ? 0 : (p < cut.pw ? len_eff : (p == cut.pw ? cut.rem : 0));
    const int nv = max(0, min(hi - kb, nk));
    if (wave_any && __ballot(nv > 0) != 0) wave_attn_wide<D, kDhsaSub>(st, sm, nk, nv, scale_log2);
    p = np;
    kb = nkb;
    k = nkc;
    bk = nbk;
    lk = nlk;
  }
  if (!valid) return;
  const float inv = st.l > 0.f ? 1.f / st.l : 0.f;
  uint16_t* orow = (uint16_t*)a.O + (bh * a.L + i) * D;
  const int hf = lane >> 5;
#pragma unroll
  for (int bb = 0; bb < D / 32; ++bb)
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const int dd = 32 * bb + 8 * q4 + 4 * hf;
      const u32x2 v = {pack_bf16x2(st.o[bb][4 * q4] * inv, st.o[bb][4 * q4 + 1] * inv),
                       pack_bf16x2(st.o[bb][4 * q4 + 2] * inv, st.o[bb][4 * q4 + 3] * inv)};
      *(u32x2*)(orow + dd) = v;
    }
}

// Debug bitmask: one thread per (b, h, row i, 32-key word).
__global__ void mask_kernel(DhsaArgs a) {
  const int64_t words = (a.L + 31) / 32;
  const int64_t total = (int64_t)a.B * a.H * a.L * words;
  for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < total;
       t += (int64_t)gridDim.x * blockDim.x) {
    const int64_t wd = t % words;
    const int64_t i = (t / words) % a.L;
    const int64_t bh = t / (words * a.L);
    // chunk of i
    int lo = 0, hi = a.nc - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (a.offs[mid] <= i) lo = mid; else hi = mid - 1;
    }
    const int l = lo;
    const Cut cut = row_cut(a, bh, l, (int)i);
    const int32_t* order = a.order + (bh * a.nc + l) * a.nc;
    uint32_t bits = 0;
    // rank position of a chunk: scan the (short) kept prefix of the order
    for (int p = 0; p <= min(cut.pw, l); ++p) {
      const int k = order[p];
      const int bk = a.offs[k];
      int lim = p < cut.pw ? a.offs[k + 1] - bk : cut.rem;
      if (k == l) lim = min(lim, (int)(i - bk + 1));
      const int64_t j0 = max((int64_t)bk, wd * 32), j1 = min((int64_t)bk + lim, wd * 32 + 32);
      for (int64_t j = j0; j < j1; ++j) bits |= 1u << (j - wd * 32);
    }
    a.mask_bits[t] = bits;
  }
}

}  // namespace

hipError_t dhsa_stage(const DhsaArgs& a, int stage, hipStream_t stream) {
  const int64_t BH = (int64_t)a.B * a.H;
  const int64_t rows = BH * a.nc;
  if (rows == 0 || a.L == 0) return hipSuccess;
  switch (stage) {
    case 0: {
      const int VEC = a.dtype == kF32 ? 4 : 8;
      const size_t lds = 2 * (size_t)(kThreads / (a.d / VEC)) * a.d * sizeof(float);
      if (a.dtype == kF32)
        pool_kernel<kF32><<<dim3((unsigned)rows), dim3(kThreads), lds, stream>>>(a);
      else
        pool_kernel<kBF16><<<dim3((unsigned)rows), dim3(kThreads), lds, stream>>>(a);
      break;
    }
    case 1:
      if (a.d == 64)
        sc_kernel<64><<<dim3((unsigned)rows), dim3(kThreads), 0, stream>>>(a);
      else
        sc_kernel<128><<<dim3((unsigned)rows), dim3(kThreads), 0, stream>>>(a);
      break;
    case 2: {
      int P = 1;
      while (P < a.nc) P <<= 1;
      rank_kernel<<<dim3((unsigned)rows), dim3(kThreads), (size_t)P * sizeof(uint64_t),
                    stream>>>(a, P);
      break;
    }
    case 3: {
      const float sl2 = 1.4426950408889634f / sqrtf((float)a.d);
      const int64_t blocks = rows * a.tiles_per_chunk;
      if (a.d == 64)
        attend_kernel<64><<<dim3((unsigned)blocks), dim3(kThreads), 0, stream>>>(a, sl2);
      else
        attend_kernel<128><<<dim3((unsigned)blocks), dim3(kThreads), 0, stream>>>(a, sl2);
      break;
    }
    default: {
      if (!a.mask_bits) return hipSuccess;
      const int64_t total = BH * a.L * ((a.L + 31) / 32);
      int64_t nb = (total + 255) / 256;
      if (nb > 65536) nb = 65536;
      mask_kernel<<<dim3((unsigned)nb), dim3(256), 0, stream>>>(a);
      break;
    }
  }
  return hipGetLastError();
}

int dhsa_max_chunks() { return kMaxSort; }

}  // namespace hsa
