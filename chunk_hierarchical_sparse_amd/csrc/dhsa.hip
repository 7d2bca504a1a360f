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
//  2. rank  : per (b, h, l): S_c[l,k] = q_hat_l . k_hat_k for k <= l, as
//             64-bit keys (S_c, then lower k) in LDS, bitonic-sorted
//             -> order[p], prefix lengths in rank order, the rank of l and
//             each rank's (first key, length).
//  3. attend: per (b, h, query chunk, 128-row tile): each lane's row finds
//             its cut (number of whole chunks, tokens of the boundary chunk)
//             by binary search, then the block walks the ranked chunks with
//             the MFMA attention core (bf16) or fp32 VALU dot products
//             (fp32), with per-row key limits.
//  4. mask  : optional debug bitmask of the kept keys.
#include <math.h>

#include "attn_core.h"
#include "hsa_common.h"
#include "kernels.h"

namespace hsa {

HSA_DCHECK_SOURCE()
namespace {

constexpr int kThreads = 256;
// Waves per block of the bf16 attention: each wave owns 32 rows of the
// block's query chunk, and the block walks the ranked key chunks in blocks
// of KB = 32 * kDhsaWaves keys (one online-softmax update each).
constexpr int kDhsaWaves = 4;
// Rows per tile of the host's tile count (tiles_per_chunk): the fp32
// attention's block; the bf16 attention splits each into
// kRowsPerTile / (32 * kDhsaWaves) blocks.
constexpr int kRowsPerTile = 128;
constexpr int kMaxSort = 4096;  // 32 KiB of 64-bit sort keys in LDS

template <int DT>
__global__ void __launch_bounds__(kThreads) pool_kernel(DhsaArgs a) {
  constexpr int VEC = DT == kF32 ? 4 : 8;
  extern __shared__ __attribute__((aligned(16))) float red[];  // [2][row_sets][d]
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
  // four rows per round, all loads issued before any is added (rows past
  // the chunk read its last row and are dropped); the sum still takes the
  // thread's rows in order
  constexpr int U = 4;
  for (int j0 = b0 + rs; j0 < b1; j0 += U * row_sets) {
    float xq[U][VEC], xk[U][VEC];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t off = (bh * a.L + min(j0 + u * row_sets, b1 - 1)) * d + cg * VEC;
#pragma unroll
      for (int v = 0; v < VEC; ++v) {
        xq[u][v] = load_elem<DT>(a.Q, off + v);
        xk[u][v] = load_elem<DT>(a.K, off + v);
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (j0 + u * row_sets < b1) {
#pragma unroll
        for (int v = 0; v < VEC; ++v) {
          aq[v] += xq[u][v];
          ak[v] += xk[u][v];
        }
      }
  }
  // 16-byte stores: a lane's VEC sums are contiguous (scalar stores at a
  // VEC-float stride put VEC lanes on one bank)
#pragma unroll
  for (int v = 0; v < VEC; v += 4) {
    *(f32x4*)&red[rs * d + cg * VEC + v] = f32x4{aq[v], aq[v + 1], aq[v + 2], aq[v + 3]};
    *(f32x4*)&red[(row_sets + rs) * d + cg * VEC + v] =
        f32x4{ak[v], ak[v + 1], ak[v + 2], ak[v + 3]};
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

// Per (b, h, l): the S_c row l (k <= l), straight into LDS as 64-bit sort
// keys (score, then lower k), then ranked.  Lanes split d into float4
// pieces and reduce with shuffles.
template <int D>
__global__ void __launch_bounds__(kThreads) rank_kernel(DhsaArgs a, int P) {
  extern __shared__ uint64_t keys[];  // [P]
  __shared__ int32_t part[kThreads];
  const int64_t bh = blockIdx.x / a.nc;
  const int l = blockIdx.x % a.nc;
  const int n = l + 1;
  {
    constexpr int LPR = D / 4, RPW = kWave / LPR;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int li = lane % LPR, sub = lane / LPR;
    for (int i = n + threadIdx.x; i < P; i += kThreads) keys[i] = 0ull;
    const f32x4 q4 = *(const f32x4*)(a.qh + (bh * a.nc + l) * D + 4 * li);
    // U steps of keys per round, every load issued unconditionally (keys
    // past l read key l and are not stored): loads under a per-lane guard
    // would each be waited for before the next
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
        if (li == 0 && k <= l) keys[k] = select_key(p, (uint32_t)k);
      }
    }
  }
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
  int32_t* ranked = a.ranked + (bh * a.nc + l) * a.nc * 2;
  for (int p = threadIdx.x; p < a.nc; p += kThreads) {
    const int32_t k = p < n ? (int32_t)key_index(keys[p]) : -1;
    order[p] = k;
    if (k == l) a.diag_pos[bh * a.nc + l] = p;
    if (k >= 0) *(u32x2*)(ranked + 2 * p) = u32x2{(uint32_t)a.offs[k],
                                                (uint32_t)(a.offs[k + 1] - a.offs[k])};
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

// cum: the (b, h, l) row of prefix lengths in rank order (global or LDS).
__device__ __forceinline__ Cut row_cut_in(const int32_t* cum, int bl, int ll, int64_t budget,
                                          int dp, int l, int i) {
  const int B = (int)min(budget, (int64_t)i + 1);
  const int tail = ll - (i - bl + 1);  // tokens of chunk l after i
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
  HSA_DCHECK(dp >= 0 && dp <= l && c.pw <= l + 1 && c.rem >= 0);
  return c;
}

__device__ __forceinline__ Cut row_cut(const DhsaArgs& a, int64_t bh, int l, int i) {
  const int bl = a.offs[l], ll = a.offs[l + 1] - bl;
  return row_cut_in(a.cumlen + (bh * a.nc + l) * (a.nc + 1), bl, ll, a.budget,
                    a.diag_pos[bh * a.nc + l], l, i);
}

template <int D, int NW>
__global__ void __launch_bounds__(64 * NW, 2) attend_kernel(DhsaArgs a, float scale_log2) {
  constexpr int KB = 32 * NW, NT = 64 * NW, ROWS = 32 * NW;
  __shared__ KVSmemWide<D, KB> sm;
  __shared__ int pmax;
  // late query chunks attend the most keys: dispatch them first, with all
  // (b, h) of one chunk next to each other
  const int64_t BH = (int64_t)a.B * a.H;
  const int64_t bh = blockIdx.x % BH;
  const int64_t rest = blockIdx.x / BH;
  const int tpc = a.tiles_per_chunk * (kRowsPerTile / ROWS);
  const int l = a.nc - 1 - (int)(rest / tpc);
  const int tile = (int)(rest % tpc);
  const int bl = a.offs[l], bl1 = a.offs[l + 1];
  const int row0 = bl + tile * ROWS;
  if (row0 >= bl1) return;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  // the tile's 32-row groups go to the waves rotated by block, so the groups
  // past a short chunk's end (idle waves) fall on different SIMDs
  const int wr = (w + (int)(blockIdx.x % NW)) % NW;
  const int i = row0 + wr * 32 + (lane & 31);  // L < 2^31 is checked on the host
  const bool valid = i < bl1;
  // Each row's cut searches the (b, h, l) row of prefix lengths: staged in
  // LDS first (the key buffer is free until the first block is stored), so
  // the binary search is not a chain of dependent global loads.
  int32_t* cum_s = reinterpret_cast<int32_t*>(&sm);
  const int32_t* cum_g = a.cumlen + (bh * a.nc + l) * (a.nc + 1);
  static_assert(sizeof(sm) >= (kMaxSort + 2) * sizeof(int32_t), "prefix-length row in LDS");
  for (int x = threadIdx.x; x <= l + 1; x += NT) cum_s[x] = cum_g[x];
  const int dp = a.diag_pos[bh * a.nc + l];
  __syncthreads();
  Cut cut = {0, 0};
  if (valid) cut = row_cut_in(cum_s, bl, bl1 - bl, a.budget, dp, l, i);
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
  // (first key, length) of the chunk at each rank.  The chunk after the
  // current one is looked up a step ahead, with a buffer load (vector
  // memory, so no wait of the LDS work covers it), and the next block's
  // fetch never waits for a lookup.
  const __amdgpu_buffer_rsrc_t rkr =
      buffer_range(a.ranked + (bh * a.nc + l) * a.nc * 2, (l + 1) * 8);
  auto rank_entry = [&](int r) {
    return __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(rkr, r * 8, 0, 0));
  };
  // Key blocks in rank order: the chunk at rank p, keys [kb, kb + 128).
  // Each step stores the block fetched during the previous step, starts the
  // fetch of the next one, then computes.
  int p = 0, kb = 0, bk = 0, lk = 0;
  u32x2 up = {0u, 0u};  // the chunk at rank p + 1
  KVRegsWide<D, KB> rg;
  if (p_end >= 0) {
    const u32x2 e0 = rank_entry(0);
    bk = __builtin_amdgcn_readfirstlane((int)e0[0]);
    lk = __builtin_amdgcn_readfirstlane((int)e0[1]);
    HSA_DCHECK(bk >= 0 && lk >= 1 && bk + lk <= bl1);
    fetch_kv_wide<D, KB>(rg, Kb + (int64_t)bk * D, Vb + (int64_t)bk * D, min(KB, lk));
    if (p_end >= 1) up = rank_entry(1);
  }
  while (p <= p_end) {
    const int nk = min(KB, lk - kb);
    __syncthreads();
    store_kv_wide<D, KB>(sm, rg, nk);
    __syncthreads();
    int np = p, nkb = kb + KB, nbk = bk, nlk = lk;
    if (nkb >= lk) {
      np = p + 1;
      nkb = 0;
      nbk = __builtin_amdgcn_readfirstlane((int)up[0]);
      nlk = __builtin_amdgcn_readfirstlane((int)up[1]);
      HSA_DCHECK(np > p_end || (nbk >= 0 && nlk >= 1 && nbk + nlk <= bl1));
    }
    if (np <= p_end)
      fetch_kv_wide<D, KB>(rg, Kb + (int64_t)(nbk + nkb) * D, Vb + (int64_t)(nbk + nkb) * D,
                           min(KB, nlk - nkb));
    if (np != p && np + 1 <= p_end) up = rank_entry(np + 1);
    __builtin_amdgcn_sched_barrier(0);
    const int len_eff = bk == bl ? i - bl + 1 : lk;  // the query's own chunk starts at bl
    const int hi = !valid ? 0 : (p < cut.pw ? len_eff : (p == cut.pw ? cut.rem : 0));
    const int nv = max(0, min(hi - kb, nk));
    if (wave_any && __ballot(nv > 0) != 0)
      wave_attn_wide<D, NW, false, KB>(st, sm, nk, nv, scale_log2);
    p = np;
    kb = nkb;
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

// fp32 inputs: the same walk over the ranked chunks, on the VALU in fp32.
// Two lanes per query row, 128 rows per block (the bf16 kernel's tiles):
// lane half hf holds the float4 pieces 2u + hf of the row's query and
// output, so the two lanes of a row read 32 consecutive bytes of a key or
// value row and every row of the wave reads the same ones (LDS broadcasts).
// Keys and values are staged 32 rows at a time; rows past the chunk's end
// load its last row and are masked by the row's key count.
constexpr int kF32Keys = 32;

template <int D>
__global__ void __launch_bounds__(kThreads) attend_f32_kernel(DhsaArgs a, float scale_log2) {
  constexpr int P4 = D / 8;  // float4 pieces per lane
  __shared__ f32x4 ks[kF32Keys][D / 4];
  __shared__ f32x4 vs[kF32Keys][D / 4];
  __shared__ int pmax;
  const int64_t BH = (int64_t)a.B * a.H;
  const int64_t bh = blockIdx.x % BH;
  const int64_t rest = blockIdx.x / BH;
  const int l = a.nc - 1 - (int)(rest / a.tiles_per_chunk);
  const int tile = (int)(rest % a.tiles_per_chunk);
  const int bl = a.offs[l], bl1 = a.offs[l + 1];
  const int row0 = bl + tile * kRowsPerTile;
  if (row0 >= bl1) return;
  const int hf = threadIdx.x & 1;
  const int i = row0 + (threadIdx.x >> 1);
  const bool valid = i < bl1;
  Cut cut = {0, 0};
  if (valid) cut = row_cut(a, bh, l, i);
  const int last = valid ? (cut.rem > 0 ? cut.pw : cut.pw - 1) : -1;
  if (threadIdx.x == 0) pmax = -1;
  __syncthreads();
  atomicMax(&pmax, last);
  __syncthreads();
  const int p_end = pmax;
  const float* Kb = (const float*)a.K + bh * a.L * D;
  const float* Vb = (const float*)a.V + bh * a.L * D;
  const float* qrow = (const float*)a.Q + (bh * a.L + min(i, (int)a.L - 1)) * D;
  f32x4 q[P4], o[P4];
#pragma unroll
  for (int u = 0; u < P4; ++u) {
    q[u] = *(const f32x4*)(qrow + 8 * u + 4 * hf);
    o[u] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  float m = -INFINITY, lsum = 0.f;
  const int32_t* order = a.order + (bh * a.nc + l) * a.nc;
  for (int p = 0; p <= p_end; ++p) {
    const int k = order[p];
    HSA_DCHECK(k >= 0 && k <= l);
    const int bk = a.offs[k], lk = a.offs[k + 1] - bk;
    const int len_eff = k == l ? i - bl + 1 : lk;
    const int hi = !valid ? 0 : (p < cut.pw ? len_eff : (p == cut.pw ? cut.rem : 0));
    for (int kb = 0; kb < lk; kb += kF32Keys) {
      const int nk = min(kF32Keys, lk - kb);
      __syncthreads();
      for (int x = threadIdx.x; x < kF32Keys * D / 4; x += kThreads) {
        const int r = x / (D / 4), c4 = x % (D / 4);
        const int64_t row = bk + kb + min(r, nk - 1);
        ks[r][c4] = *(const f32x4*)(Kb + row * D + 4 * c4);
        vs[r][c4] = *(const f32x4*)(Vb + row * D + 4 * c4);
      }
      __syncthreads();
      const int nv = max(0, min(hi - kb, nk));
      float s[kF32Keys];
      float bmax = -INFINITY;
#pragma unroll
      for (int j = 0; j < kF32Keys; ++j) {
        float part = 0.f;
#pragma unroll
        for (int u = 0; u < P4; ++u) {
          const f32x4 kv = ks[j][2 * u + hf];
          part += q[u][0] * kv[0] + q[u][1] * kv[1] + q[u][2] * kv[2] + q[u][3] * kv[3];
        }
        part += __shfl_xor(part, 1, kWave);  // both lanes of the row: the full dot product
        s[j] = j < nv ? part * scale_log2 : -INFINITY;
        bmax = fmaxf(bmax, s[j]);
      }
      if (nv > 0) {
        const float mn = fmaxf(m, bmax);
        const float al = exp2f(m - mn);  // 0 while m is -inf
        lsum *= al;
#pragma unroll
        for (int u = 0; u < P4; ++u) o[u] *= al;
#pragma unroll
        for (int j = 0; j < kF32Keys; ++j) {
          const float pj = exp2f(s[j] - mn);  // 0 for masked keys
          lsum += pj;
#pragma unroll
          for (int u = 0; u < P4; ++u) o[u] += pj * vs[j][2 * u + hf];
        }
        m = mn;
      }
    }
  }
  if (!valid) return;
  const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
  float* orow = (float*)a.O + (bh * a.L + i) * D;
#pragma unroll
  for (int u = 0; u < P4; ++u) *(f32x4*)(orow + 8 * u + 4 * hf) = o[u] * inv;
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
        launch<pool_kernel<kF32>>(dim3((unsigned)rows), dim3(kThreads), lds, stream, a);
      else
        launch<pool_kernel<kBF16>>(dim3((unsigned)rows), dim3(kThreads), lds, stream, a);
      break;
    }
    case 1: {
      int P = 1;
      while (P < a.nc) P <<= 1;
      if (a.d == 64)
        launch<rank_kernel<64>>(dim3((unsigned)rows), dim3(kThreads),
                                (size_t)P * sizeof(uint64_t), stream, a, P);
      else
        launch<rank_kernel<128>>(dim3((unsigned)rows), dim3(kThreads),
                                 (size_t)P * sizeof(uint64_t), stream, a, P);
      break;
    }
    case 2: {
      const float sl2 = 1.4426950408889634f / sqrtf((float)a.d);
      const int64_t blocks = rows * a.tiles_per_chunk;
      if (a.dtype == kF32) {
        const dim3 grid((unsigned)blocks), block(kThreads);
        if (a.d == 64)
          launch<attend_f32_kernel<64>>(grid, block, 0, stream, a, sl2);
        else
          launch<attend_f32_kernel<128>>(grid, block, 0, stream, a, sl2);
      } else {
        constexpr int NW = kDhsaWaves;
        const dim3 grid((unsigned)(blocks * (kRowsPerTile / (32 * NW)))), block(64 * NW);
        if (a.d == 64)
          launch<attend_kernel<64, NW>>(grid, block, 0, stream, a, sl2);
        else
          launch<attend_kernel<128, NW>>(grid, block, 0, stream, a, sl2);
      }
      break;
    }
    default: {
      if (!a.mask_bits) return hipSuccess;
      const int64_t total = BH * a.L * ((a.L + 31) / 32);
      int64_t nb = (total + 255) / 256;
      if (nb > 65536) nb = 65536;
      launch<mask_kernel>(dim3((unsigned)nb), dim3(256), 0, stream, a);
      break;
    }
  }
  return hipGetLastError();
}

int dhsa_max_chunks() { return kMaxSort; }

}  // namespace hsa
