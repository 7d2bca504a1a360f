// prefill_bwd.hip - HSA prefill backward: gradients of the fused output with
// respect to Q, K and V ([HiLS] abstract: retrieval learned end to end, the
// gradient reaching the retrieval scores through the fusion weights; the
// top-K selection itself is piecewise constant and held fixed).
//
// With the forward's selection and chunk-major work list already built:
//  weights: per (token, group), each head: the retrieval scores s_k =
//          q . lambda_ck / sqrt(d) of the kept chunks and the fusion weights
//          w = softmax(s).
//  score : one block per chunk (its whole list of (token, head) rows), the
//          chunk's K and V in LDS, lane = row as in the forward's chunk
//          attention: S^T = K Q^T and dP^T = V dO^T (MFMA), the row's
//          log-sum-exp and dw = dO . o_k = sum_j p_j dP_j, then
//          dS^T = w P^T (dP^T - dw) and the row's dQ piece
//          K^T dS^T / sqrt(d) (MFMA, K^T in the key-quad layout).
//  rows  : per (token, head): ds_k = w_k (dw_k - sum_k' w_k' dw_k').
//  kv    : one block per chunk again, lane = key: each wave owns one 32-key
//          half and walks its own row tiles with no barrier: S = Q K^T,
//          dP = dO V^T, P = exp2(S - lse); Q^T and dO^T come from products
//          with a 0/1 selector; then
//             dV^T += dO^T (w P)                 (MFMA, registers)
//             dK^T += Q^T (dS + ds / sqrt(S))   (MFMA; the landmark term:
//                     lambda_c = sum_j k_j / sqrt(S) gives every key of the
//                     chunk ds q / sqrt(d) / sqrt(S))
//          The block holds the chunk's whole list, so its waves' sums meet
//          in LDS and are written once, as bf16.
//  finish: per (token, head): dQ = sum of its slots' pieces + sum_k ds_k
//          lambda_ck / sqrt(d).
#include <math.h>

#include "attn_core.h"
#include "hsa_common.h"
#include "kernels.h"
#include "prefill_common.h"

namespace hsa {

HSA_DCHECK_SOURCE()
namespace {

constexpr int kThreads = 256;
constexpr int kRowPad = 8;    // LDS row padding (elements) of row-major tiles

// Rows [0, nk) of a [rows, D] bf16 block into LDS, row-major with rows
// padded by kRowPad elements; rows nk..63 are zero.  All threads call.
template <int D>
__device__ __forceinline__ void load_rows(uint16_t* dst, const uint16_t* __restrict__ src,
                                          int nk) {
  constexpr int KPR = D / 8;
  for (int e = threadIdx.x; e < 64 * KPR; e += kThreads) {
    const int row = e / KPR, c8 = e % KPR;
    u32x4 x = {0u, 0u, 0u, 0u};
    if (row < nk) x = *(const u32x4*)(src + (int64_t)row * D + c8 * 8);
    *(u32x4*)(dst + row * (D + kRowPad) + c8 * 8) = x;
  }
}

// The same rows in the key-quad layout [key/4][dim][4 keys]: a lane reads
// four consecutive keys of one dimension as 8 bytes.
template <int D>
__device__ __forceinline__ void load_quads(uint16_t* dst, const uint16_t* __restrict__ src,
                                           int nk) {
  constexpr int VPR = D / 4;
  for (int e = threadIdx.x; e < 16 * VPR; e += kThreads) {
    const int grp = e / VPR, cq = e % VPR;
    u32x2 r[4];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const int key = grp * 4 + kk;
      r[kk] = key < nk ? *(const u32x2*)(src + (int64_t)key * D + cq * 4) : u32x2{0u, 0u};
    }
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      const int w = x >> 1;
      uint32_t lo, hi;
      if ((x & 1) == 0) {
        lo = (r[0][w] & 0xffffu) | (r[1][w] << 16);
        hi = (r[2][w] & 0xffffu) | (r[3][w] << 16);
      } else {
        lo = (r[0][w] >> 16) | (r[1][w] & 0xffff0000u);
        hi = (r[2][w] >> 16) | (r[3][w] & 0xffff0000u);
      }
      *(u32x2*)(&dst[(grp * D + cq * 4 + x) * 4]) = u32x2{lo, hi};
    }
  }
}

__device__ __forceinline__ void wave_sync_lds() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Row r of a unit -> (entry index r / G, head r % G).
__device__ __forceinline__ void split_row(int r, int G, int lg, int& ei, int& hh) {
  if (lg >= 0) {
    ei = r >> lg;
    hh = r & ((1 << lg) - 1);
  } else {
    ei = r / G;
    hh = r - ei * G;
  }
}

// One row's Q and dO as load_row_pair gives them, loaded unconditionally
// (a missing row, entry < 0, reads token 0 and is zeroed by the caller):
// loads guarded per lane would each be waited for before the next.
template <int D>
__device__ __forceinline__ void load_row_pair_nb(const PrefillBwdArgs& ba, int64_t qbase,
                                                 int64_t qplane, int32_t entry, int hh, int hf,
                                                 u32x4 (&q)[D / 16], u32x4 (&o)[D / 16]) {
  const int64_t tok = entry >= 0 ? (int64_t)(entry >> kSlotBits) : 0;
  HSA_DCHECK(tok < ba.p.L);
  const int64_t off = qbase + (int64_t)hh * qplane + tok * D + 8 * hf;
  const uint16_t* qr = (const uint16_t*)ba.p.Q + off;
  const uint16_t* orow = (const uint16_t*)ba.dO + off;
#pragma unroll
  for (int s = 0; s < D / 16; ++s) {
    q[s] = *(const u32x4*)(qr + 16 * s);
    o[s] = *(const u32x4*)(orow + 16 * s);
  }
}

// One row's Q and dO (dims 16s + 8h .. +7 for s = 0 .. D/16-1), zero when
// the row does not exist.
template <int D>
__device__ __forceinline__ void load_row_pair(const PrefillBwdArgs& ba, int64_t qbase,
                                              int64_t qplane, int32_t entry, int hh, int hf,
                                              u32x4 (&q)[D / 16], u32x4 (&o)[D / 16]) {
  if (entry >= 0) {
    HSA_DCHECK((int64_t)(entry >> kSlotBits) < ba.p.L);
    const int64_t off = qbase + (int64_t)hh * qplane + (int64_t)(entry >> kSlotBits) * D + 8 * hf;
    const uint16_t* qr = (const uint16_t*)ba.p.Q + off;
    const uint16_t* orow = (const uint16_t*)ba.dO + off;
#pragma unroll
    for (int s = 0; s < D / 16; ++s) {
      q[s] = *(const u32x4*)(qr + 16 * s);
      o[s] = *(const u32x4*)(orow + 16 * s);
    }
  } else {
#pragma unroll
    for (int s = 0; s < D / 16; ++s) {
      q[s] = u32x4{0u, 0u, 0u, 0u};
      o[s] = u32x4{0u, 0u, 0u, 0u};
    }
  }
}


// ---------------------------------------------------------------- weights --

// One group of D/8 threads per (b, group, token), 8 dims each: the kept
// chunks' landmark segments stay in registers while each head of the group
// takes s_k = q . lambda_ck / sqrt(d) and w = softmax(s), written at the
// slots' list positions.
template <int D, int KM>
__global__ void __launch_bounds__(kThreads) bwd_weights_kernel(PrefillBwdArgs ba, float sc) {
  const PrefillArgs& a = ba.p;
  constexpr int TPR = D / 8;
  constexpr int RPB = kThreads / TPR;
  const int64_t r = (int64_t)blockIdx.x * RPB + threadIdx.x / TPR;
  const int cg = threadIdx.x % TPR;
  if (r >= (int64_t)a.B * a.Hkv * a.L) return;  // whole groups of TPR threads leave together
  const int G = a.Hq / a.Hkv;
  const int64_t t = r % a.L;
  const int64_t bg = r / a.L;
  const int64_t b = bg / a.Hkv;
  const int g = (int)(bg % a.Hkv);
  const int m = (int)min((int64_t)a.topk, min(t / a.S, a.n));
  const int32_t* sel = a.idx + (bg * a.nq + t) * a.topk;
  const int32_t* epos = a.entry_pos + (bg * a.L + t) * a.topk;
  // loads issued unconditionally (slots past m read in-bounds entries,
  // dropped below): per-lane guards would make each wait for the one before
  f32x4 lam[KM][2];
  int32_t ep[KM], ck[KM];
#pragma unroll
  for (int k = 0; k < KM; ++k) {
    const int kk = min(k, a.topk - 1);
    ep[k] = epos[kk];
    ck[k] = sel[kk];
    HSA_DCHECK(k >= m || (ck[k] >= 0 && ck[k] < a.n && ep[k] >= 0 &&
                          (int64_t)ep[k] < a.L * a.topk));
  }
#pragma unroll
  for (int k = 0; k < KM; ++k) {
    const float* lc = a.lmk + (bg * a.n + (k < m ? ck[k] : 0)) * D + cg * 8;
    lam[k][0] = *(const f32x4*)lc;
    lam[k][1] = *(const f32x4*)(lc + 4);
  }
  for (int hh = 0; hh < G; ++hh) {
    const u32x4 qv = *(const u32x4*)((const uint16_t*)a.Q +
                                     ((b * a.Hq + g * G + hh) * a.L + t) * D + cg * 8);
    float qf[8];
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      qf[2 * v] = bf16_bits_to_f32(qv[v] & 0xffffu);
      qf[2 * v + 1] = bf16_bits_to_f32(qv[v] >> 16);
    }
    float s[KM];
    float smax = -INFINITY;
#pragma unroll
    for (int k = 0; k < KM; ++k) {
      float acc = 0.f;
#pragma unroll
      for (int v = 0; v < 4; ++v) acc += qf[v] * lam[k][0][v] + qf[4 + v] * lam[k][1][v];
#pragma unroll
      for (int o = TPR / 2; o > 0; o >>= 1) acc += __shfl_xor(acc, o, kWave);
      s[k] = k < m ? acc * sc : -INFINITY;
      smax = fmaxf(smax, s[k]);
    }
    float z = 0.f;
#pragma unroll
    for (int k = 0; k < KM; ++k) {
      s[k] = k < m ? expf(s[k] - smax) : 0.f;
      z += s[k];
    }
    if (cg == 0) {
#pragma unroll
      for (int k = 0; k < KM; ++k)
        if (k < m) ba.wk[partial_row(a, bg, ep[k], hh)] = s[k] / z;
    }
  }
}

// ----------------------------------------------------------------- score --

template <int D>
struct ScoreSmem {
  uint16_t k[64 * (D + kRowPad)];  // K rows: A operand of S^T = K Q^T
  uint16_t v[64 * (D + kRowPad)];  // V rows: A operand of dP^T = V dO^T
  uint16_t kq[16 * D * 4];         // K, key-quad layout: A operand of K^T dS^T
  uint16_t ostage[kThreads / kWave][16 * (D + 8)];  // each wave's dQ rows, padded
};

// Lane = row (S^T = K Q^T as in the forward's chunk attention): register r
// of lane (i, h) holds the row i's key 8(r/4) + 4h + r%4 (+32 in s1/p1).
template <int D>
__global__ void __launch_bounds__(kThreads, 2) bwd_score_kernel(PrefillBwdArgs ba, float sl2,
                                                                float sc) {
  const PrefillArgs& a = ba.p;
  __shared__ __attribute__((aligned(16))) ScoreSmem<D> sm;
  int64_t bg;
  int c, e_begin, e_end;
  if (!locate_tile(a, bg, c, e_begin, e_end)) return;
  const int G = a.Hq / a.Hkv;
  const int b = (int)(bg / a.Hkv), g = (int)(bg % a.Hkv);
  const int rows = (e_end - e_begin) * G;
  const int ntiles = (rows + 31) / 32;
  const int64_t kv0 = (bg * a.L + (int64_t)c * a.S) * D;
  load_rows<D>(sm.k, (const uint16_t*)a.K + kv0, a.S);
  load_rows<D>(sm.v, (const uint16_t*)a.V + kv0, a.S);
  load_quads<D>(sm.kq, (const uint16_t*)a.K + kv0, a.S);
  __syncthreads();
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int i32 = lane & 31, hf = lane >> 5;
  const int32_t* list = a.list + bg * a.L * a.topk + e_begin;
  const int64_t qplane = a.L * D;
  const int64_t qbase = ((int64_t)b * a.Hq + (int64_t)g * G) * qplane;
  const int64_t row0 = partial_row(a, bg, e_begin, 0);
  const bool two = a.S > 32;
  const f32x16 zero = {};
  const int last_ei = rows > 0 ? (rows - 1) / G : 0;
  for (int tile = w; tile < ntiles; tile += kThreads / kWave) {
    const int r = tile * 32 + i32;
    int ei, hh;
    split_row(r, G, a.log2G, ei, hh);
    // unguarded loads (past the unit: clamped, then dropped)
    const int32_t e_raw = list[min(ei, last_ei)];
    const int32_t entry = r < rows ? e_raw : -1;
    u32x4 q[D / 16], o[D / 16];
    load_row_pair_nb<D>(ba, qbase, qplane, entry, hh, hf, q, o);
    const float wr_raw = ba.wk[row0 + min(r, rows - 1)];
    const float wr = entry >= 0 ? wr_raw : 0.f;
    if (entry < 0) {
#pragma unroll
      for (int s2 = 0; s2 < D / 16; ++s2) q[s2] = o[s2] = u32x4{0u, 0u, 0u, 0u};
    }
    f32x16 s0 = zero, s1 = zero, p0 = zero, p1 = zero;
#pragma unroll
    for (int s = 0; s < D / 16; ++s) {
      const bf16x8 qb = __builtin_bit_cast(bf16x8, q[s]);
      const bf16x8 ob = __builtin_bit_cast(bf16x8, o[s]);
      const int ko = i32 * (D + kRowPad) + 16 * s + 8 * hf;
      s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*(const bf16x8*)&sm.k[ko], qb, s0, 0, 0, 0);
      p0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*(const bf16x8*)&sm.v[ko], ob, p0, 0, 0, 0);
      if (two) {
        const int k1 = ko + 32 * (D + kRowPad);
        s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*(const bf16x8*)&sm.k[k1], qb, s1, 0, 0, 0);
        p1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*(const bf16x8*)&sm.v[k1], ob, p1, 0, 0, 0);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    float mx = -INFINITY;
#pragma unroll
    for (int rr = 0; rr < 16; ++rr) {
      const int key = 8 * (rr >> 2) + 4 * hf + (rr & 3);
      if (key >= a.S) s0[rr] = -INFINITY;
      if (key + 32 >= a.S) s1[rr] = -INFINITY;
      mx = fmaxf(mx, fmaxf(s0[rr], s1[rr]));
    }
    mx = half_pair_max(mx);
    const float mxs = mx * sl2;
    float ps = 0.f, pd = 0.f;
#pragma unroll
    for (int rr = 0; rr < 16; ++rr) {
      s0[rr] = fast_exp2(__builtin_fmaf(s0[rr], sl2, -mxs));
      s1[rr] = fast_exp2(__builtin_fmaf(s1[rr], sl2, -mxs));
      ps += s0[rr] + s1[rr];
      pd += s0[rr] * p0[rr] + s1[rr] * p1[rr];
    }
    ps = half_pair_sum(ps);
    pd = half_pair_sum(pd);
    const float dw = pd / ps;
    // dS^T = w P^T (dP^T - dw), P = exp2(...) / ps; the / sqrt(d) of dQ too
    const float f = wr * sc / ps;
#pragma unroll
    for (int rr = 0; rr < 16; ++rr) {
      s0[rr] = f * s0[rr] * (p0[rr] - dw);
      s1[rr] = f * s1[rr] * (p1[rr] - dw);
    }
    bf16x8 db4[4];
    db4[0] = cvt_bf16x8(s0, 0);
    db4[1] = cvt_bf16x8(s0, 8);
    db4[2] = cvt_bf16x8(s1, 0);
    db4[3] = cvt_bf16x8(s1, 8);
    __builtin_amdgcn_sched_barrier(0);
    // dQ^T = K^T dS^T: B = dS^T straight from the score registers, A = K^T
    // from the key quads in the same k-slot order
    f32x16 dq[D / 32];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      if (kt == 1 && !two) break;
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        const int g0 = 8 * kt + 4 * s2 + hf, g1 = g0 + 2;
#pragma unroll
        for (int bb = 0; bb < D / 32; ++bb) {
          const int dd = 32 * bb + i32;
          const u32x2 k0 = *(const u32x2*)&sm.kq[(g0 * D + dd) * 4];
          const u32x2 k1 = *(const u32x2*)&sm.kq[(g1 * D + dd) * 4];
          dq[bb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
              __builtin_bit_cast(bf16x8, u32x4{k0[0], k0[1], k1[0], k1[1]}), db4[2 * kt + s2],
              kt == 0 && s2 == 0 ? zero : dq[bb], 0, 0, 0);
        }
      }
    }
    if (entry >= 0 && hf == 0) {
      ba.lse2[row0 + r] = mxs + log2f(ps);
      ba.dw[row0 + r] = dw;
    }
    // lane half hf holds dims 32bb + 8q4 + 4hf + 0..3; swapping half of the
    // groups with the partner lane leaves each lane 16 contiguous bytes.
    // The tile's rows are one contiguous run: they go through LDS and leave
    // as 1 KB stores; rows past the unit's end are not written.
    u32x4 outv[D / 32][2];
#pragma unroll
    for (int bb = 0; bb < D / 32; ++bb)
#pragma unroll
      for (int pr = 0; pr < 2; ++pr) {
        const uint32_t e0 = pack_bf16x2(dq[bb][8 * pr], dq[bb][8 * pr + 1]);
        const uint32_t e1 = pack_bf16x2(dq[bb][8 * pr + 2], dq[bb][8 * pr + 3]);
        const uint32_t d0 = pack_bf16x2(dq[bb][8 * pr + 4], dq[bb][8 * pr + 5]);
        const uint32_t d1 = pack_bf16x2(dq[bb][8 * pr + 6], dq[bb][8 * pr + 7]);
        const uint32_t got0 = half_pair_exchange(d0, e0, hf != 0);
        const uint32_t got1 = half_pair_exchange(d1, e1, hf != 0);
        outv[bb][pr] = hf ? u32x4{got0, got1, d0, d1} : u32x4{e0, e1, got0, got1};
      }
    uint16_t* stg = sm.ostage[w];
    const int nrow = min(32, rows - tile * 32);
    constexpr int LPR = D / 8;        // lanes per row (16 bytes each)
    constexpr int RPI = kWave / LPR;  // rows per store instruction
    const int piece = lane % LPR;
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2) {
      wave_sync_lds();
      if (i32 / 16 == h2) {
#pragma unroll
        for (int bb = 0; bb < D / 32; ++bb)
#pragma unroll
          for (int pr = 0; pr < 2; ++pr)
            *(u32x4*)(stg + (i32 % 16) * (D + 8) + 32 * bb + 8 * (2 * pr + hf)) = outv[bb][pr];
      }
      wave_sync_lds();
      uint16_t* base = (uint16_t*)a.partial + (row0 + tile * 32 + h2 * 16) * D;
#pragma unroll
      for (int k = 0; k < 16 / RPI; ++k) {
        const int row = k * RPI + lane / LPR;
        const u32x4 v = *(const u32x4*)(stg + row * (D + 8) + 8 * piece);
        if (h2 * 16 + row < nrow) __builtin_nontemporal_store(v, (u32x4*)(base + (int64_t)row * D + 8 * piece));
      }
    }
  }
}

// ------------------------------------------------------------------ rows --

// One thread per (b, group, token, head of the group) row.
template <int KM>
__global__ void __launch_bounds__(kThreads) bwd_rows_kernel(PrefillBwdArgs ba) {
  const PrefillArgs& a = ba.p;
  const int64_t r = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (r >= (int64_t)a.B * a.Hq * a.L) return;
  const int G = a.Hq / a.Hkv;
  const int hh = (int)(r % G);
  const int64_t t = (r / G) % a.L;
  const int64_t bg = r / G / a.L;
  const int m = (int)min((int64_t)a.topk, min(t / a.S, a.n));
  const int32_t* epos = a.entry_pos + (bg * a.L + t) * a.topk;
  // two rounds of loads, none guarded per lane (slots past m read row 0)
  int32_t ep[KM];
#pragma unroll
  for (int k = 0; k < KM; ++k) ep[k] = epos[min(k, a.topk - 1)];
  int64_t pr[KM];
  float wk[KM], dw[KM];
#pragma unroll
  for (int k = 0; k < KM; ++k) {
    pr[k] = k < m ? partial_row(a, bg, ep[k], hh) : 0;
    wk[k] = ba.wk[pr[k]];
    dw[k] = ba.dw[pr[k]];
  }
  float wdw = 0.f;
#pragma unroll
  for (int k = 0; k < KM; ++k) {
    if (k >= m) wk[k] = dw[k] = 0.f;
    wdw += wk[k] * dw[k];
  }
#pragma unroll
  for (int k = 0; k < KM; ++k)
    if (k < m) ba.ds[pr[k]] = wk[k] * (dw[k] - wdw);
}

// -------------------------------------------------------------------- kv --

constexpr int kRedPitch = 1;  // pad of the [key][dim] fp32 sums (lanes = keys)

template <int D>
struct KvSmem {
  union {
    struct {
      uint16_t k[64 * (D + kRowPad)];
      uint16_t v[64 * (D + kRowPad)];
    } kv;
    float red[64 * (D + kRedPitch)];  // the chunk's dK, then dV sums
  } u;
  float st[kThreads / kWave][4][32];  // per wave, per row: lse2, dw, w, ds
};

// The 0/1 operand that turns a row-major A operand into its transpose: the
// product Q E (E selecting dims 32 bb .. 32 bb + 31 over the k-steps 2 bb and
// 2 bb + 1) leaves Q[row][32 bb + j] in lane j, register r holding row
// 8(r/4) + 4h + r%4 -- the k-slot order of the score registers -- so its
// bf16 packing is the A operand of a product contracted over the tile's
// rows.  Lane (j, h) holds k-slots 8h .. 8h+7 of k-step 2 bb + t: a one
// where 16 t + 8 h + e == j.
__device__ __forceinline__ bf16x8 selector(int t, int j, int h) {
  bf16x8 e8;
#pragma unroll
  for (int e = 0; e < 8; ++e)
    e8[e] = static_cast<__bf16>(16 * t + 8 * h + e == j ? 1.f : 0.f);
  return e8;
}

// Wave w owns keys 32 kt .. 32 kt + 31 (kt = w % 2) and the row tiles
// w / 2, w / 2 + 2, ...; lane = key: register r of lane (j, h) holds row
// 8(r/4) + 4h + r%4 of the tile and key 32 kt + j.  The waves never wait
// for each other inside the loop.
template <int D>
__global__ void __launch_bounds__(kThreads, 2) bwd_kv_kernel(PrefillBwdArgs ba, float sl2,
                                                             float sc, float rs) {
  const PrefillArgs& a = ba.p;
  __shared__ __attribute__((aligned(16))) KvSmem<D> sm;
  int64_t bg;
  int c, e_begin, e_end;
  if (!locate_tile(a, bg, c, e_begin, e_end)) return;
  const int G = a.Hq / a.Hkv;
  const int b = (int)(bg / a.Hkv), g = (int)(bg % a.Hkv);
  const int rows = (e_end - e_begin) * G;
  const int ntiles = (rows + 31) / 32;
  const int64_t kv0 = (bg * a.L + (int64_t)c * a.S) * D;
  load_rows<D>(sm.u.kv.k, (const uint16_t*)a.K + kv0, a.S);
  load_rows<D>(sm.u.kv.v, (const uint16_t*)a.V + kv0, a.S);
  __syncthreads();
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int i32 = lane & 31, hf = lane >> 5;
  const int kt = w & 1, stream = w >> 1;
  const bool keys = 32 * kt < a.S;         // this wave's key half holds keys
  const bool kfull = 32 * kt + 32 <= a.S;  // ... and all 32 of them
  const float kon = 32 * kt + i32 < a.S ? 1.f : 0.f;
  const int32_t* list = a.list + bg * a.L * a.topk + e_begin;
  const int64_t qplane = a.L * D;
  const int64_t qbase = ((int64_t)b * a.Hq + (int64_t)g * G) * qplane;
  const int64_t row0 = partial_row(a, bg, e_begin, 0);
  const bf16x8 sel0 = selector(0, i32, hf), sel1 = selector(1, i32, hf);
  const f32x16 zero = {};
  f32x16 dk[D / 32], dv[D / 32];
#pragma unroll
  for (int bb = 0; bb < D / 32; ++bb) {
    dk[bb] = zero;
    dv[bb] = zero;
  }
  float(&st)[4][32] = sm.st[w];
  const int last_ei = rows > 0 ? (rows - 1) / G : 0;
  for (int tile = stream; keys && tile < ntiles; tile += 2) {
    const int r = tile * 32 + i32;
    int ei, hh;
    split_row(r, G, a.log2G, ei, hh);
    // unguarded loads (past the unit: clamped, then dropped)
    const int32_t e_raw = list[min(ei, last_ei)];
    const int32_t entry = r < rows ? e_raw : -1;
    u32x4 q[D / 16], o[D / 16];
    load_row_pair_nb<D>(ba, qbase, qplane, entry, hh, hf, q, o);
    if (entry < 0) {
#pragma unroll
      for (int s2 = 0; s2 < D / 16; ++s2) q[s2] = o[s2] = u32x4{0u, 0u, 0u, 0u};
    }
    if (hf == 0) {
      const bool ok = entry >= 0;
      const int64_t rr = row0 + min(r, rows - 1);
      const float v0 = ba.lse2[rr], v1 = ba.dw[rr], v2 = ba.wk[rr], v3 = ba.ds[rr];
      st[0][i32] = ok ? v0 : INFINITY;
      st[1][i32] = ok ? v1 : 0.f;
      st[2][i32] = ok ? v2 : 0.f;
      st[3][i32] = ok ? v3 : 0.f;
    }
    f32x16 sa = zero, pa = zero;
#pragma unroll
    for (int s = 0; s < D / 16; ++s) {
      const int ko = (32 * kt + i32) * (D + kRowPad) + 16 * s + 8 * hf;
      sa = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, q[s]),
                                                   *(const bf16x8*)&sm.u.kv.k[ko], sa, 0, 0, 0);
      pa = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, o[s]),
                                                   *(const bf16x8*)&sm.u.kv.v[ko], pa, 0, 0, 0);
    }
    wave_sync_lds();
    // P = exp2(S - lse), w P, dS' = w P (dP - dw) + ds / sqrt(S) (keys past S
    // are 0), packed to bf16 at once
    bf16x8 bp[2], bs[2];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const f32x4 l4 = *(const f32x4*)&st[0][8 * u + 4 * hf];
      const f32x4 d4 = *(const f32x4*)&st[1][8 * u + 4 * hf];
      const f32x4 w4 = *(const f32x4*)&st[2][8 * u + 4 * hf];
      const f32x4 s4 = *(const f32x4*)&st[3][8 * u + 4 * hf];
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int rr = 4 * u + v;
        float p = fast_exp2(__builtin_fmaf(sa[rr], sl2, -l4[v]));
        if (!kfull) p *= kon;
        const float wpv = w4[v] * p;
        float dsk = __builtin_fmaf(s4[v], rs, wpv * (pa[rr] - d4[v]));
        if (!kfull) dsk *= kon;
        bp[u >> 1][4 * (u & 1) + v] = static_cast<__bf16>(wpv);
        bs[u >> 1][4 * (u & 1) + v] = static_cast<__bf16>(dsk);
      }
    }
    // the row statistics of the next tile overwrite st only after every lane
    // has read them
    wave_sync_lds();
    // per dims block: Q^T (then dO^T) from the selector products, and
    // dK^T += Q^T dS' (then dV^T += dO^T (w P)) over the tile's rows; all of
    // dK first, so Q's registers are free during dV's pass
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      const u32x4(&x)[D / 16] = m == 0 ? q : o;
#pragma unroll
      for (int bb = 0; bb < D / 32; ++bb) {
        f32x16 xt = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            __builtin_bit_cast(bf16x8, x[2 * bb]), sel0, zero, 0, 0, 0);
        xt = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, x[2 * bb + 1]),
                                                     sel1, xt, 0, 0, 0);
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
          if (m == 0)
            dk[bb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(cvt_bf16x8(xt, 8 * s2), bs[s2],
                                                             dk[bb], 0, 0, 0);
          else
            dv[bb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(cvt_bf16x8(xt, 8 * s2), bp[s2],
                                                             dv[bb], 0, 0, 0);
        }
      }
    }
  }
  // the chunk's dK, then dV: the two streams of each key half summed in LDS
  // over the K/V area (no longer read), then written once as bf16
  constexpr int RP = D + kRedPitch;
  const int key = 32 * kt + i32;
#pragma unroll
  for (int m = 0; m < 2; ++m) {
    __syncthreads();
    for (int x = threadIdx.x; x < 64 * RP; x += kThreads) sm.u.red[x] = 0.f;
    __syncthreads();
    if (key < a.S) {
#pragma unroll
      for (int bb = 0; bb < D / 32; ++bb)
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) {
          const int dim = 32 * bb + 8 * (rr >> 2) + 4 * hf + (rr & 3);
          atomicAdd(&sm.u.red[key * RP + dim], m == 0 ? dk[bb][rr] : dv[bb][rr]);
        }
    }
    __syncthreads();
    const float scale = m == 0 ? sc : 1.f;
    uint16_t* dst = (uint16_t*)(m == 0 ? ba.dK : ba.dV) + kv0;
    for (int x = threadIdx.x; x < a.S * D / 8; x += kThreads) {
      const int kr = x / (D / 8), d0 = 8 * (x % (D / 8));
      const float* src = &sm.u.red[kr * RP + d0];
      u32x4 out;
#pragma unroll
      for (int j = 0; j < 4; ++j) out[j] = pack_bf16x2(src[2 * j] * scale, src[2 * j + 1] * scale);
      *(u32x4*)(dst + 8 * x) = out;
    }
  }
}

// ---------------------------------------------------------------- finish --

// dQ: one group of D/8 threads per (b, group, token, head) row (8 dims each).
template <int D, int KM>
__global__ void __launch_bounds__(kThreads) bwd_dq_kernel(PrefillBwdArgs ba, float sc) {
  const PrefillArgs& a = ba.p;
  constexpr int TPR = D / 8;
  constexpr int RPB = kThreads / TPR;
  const int64_t r = (int64_t)blockIdx.x * RPB + threadIdx.x / TPR;
  const int cg = threadIdx.x % TPR;
  if (r >= (int64_t)a.B * a.Hq * a.L) return;
  const int G = a.Hq / a.Hkv;
  const int hh = (int)(r % G);
  const int64_t t = (r / G) % a.L;
  const int64_t bg = r / G / a.L;
  const int64_t b = bg / a.Hkv;
  const int h = (int)(bg % a.Hkv) * G + hh;
  const int m = (int)min((int64_t)a.topk, min(t / a.S, a.n));
  const int32_t* epos = a.entry_pos + (bg * a.L + t) * a.topk;
  const int32_t* sel = a.idx + (bg * a.nq + t) * a.topk;
  float acc[8];
#pragma unroll
  for (int v = 0; v < 8; ++v) acc[v] = 0.f;
  // every load is issued unconditionally (slots past m read in-bounds
  // entries and are dropped): per-lane guards would make each wait for the
  // one before.  Round 1: list positions and chunks; round 2: the rest.
  int32_t ep[KM], ck[KM];
#pragma unroll
  for (int k = 0; k < KM; ++k) {
    const int kk = min(k, a.topk - 1);
    ep[k] = epos[kk];
    ck[k] = sel[kk];
    HSA_DCHECK(k >= m || (ck[k] >= 0 && ck[k] < a.n && ep[k] >= 0 &&
                          (int64_t)ep[k] < a.L * a.topk));
  }
  u32x4 x[KM];
  float dsk[KM];
  f32x4 l0[KM], l1[KM];
#pragma unroll
  for (int k = 0; k < KM; ++k) {
    const int64_t pr = k < m ? partial_row(a, bg, ep[k], hh) : 0;
    x[k] = *(const u32x4*)((const uint16_t*)a.partial + pr * D + cg * 8);
    dsk[k] = ba.ds[pr] * sc;
    const float* lc = a.lmk + (bg * a.n + (k < m ? ck[k] : 0)) * D + cg * 8;
    l0[k] = *(const f32x4*)lc;
    l1[k] = *(const f32x4*)(lc + 4);
  }
#pragma unroll
  for (int k = 0; k < KM; ++k) {
    if (k >= m) break;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      acc[2 * v] += bf16_bits_to_f32(x[k][v] & 0xffffu);
      acc[2 * v + 1] += bf16_bits_to_f32(x[k][v] >> 16);
    }
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      acc[v] += dsk[k] * l0[k][v];
      acc[4 + v] += dsk[k] * l1[k][v];
    }
  }
  const int64_t ob = ((b * a.Hq + h) * a.L + t) * D + cg * 8;
  *(u32x4*)((uint16_t*)ba.dQ + ob) =
      u32x4{pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3]), pack_bf16x2(acc[4], acc[5]),
            pack_bf16x2(acc[6], acc[7])};
}

template <int D>
hipError_t finish_d(const PrefillBwdArgs& ba, hipStream_t stream) {
  const PrefillArgs& a = ba.p;
  const int64_t rows = (int64_t)a.B * a.Hq * a.L;
  const int rpb = kThreads / (D / 8);
  const unsigned nb = (unsigned)((rows + rpb - 1) / rpb);
  const float sc = 1.0f / sqrtf((float)D);
  if (a.topk <= 8)
    launch<bwd_dq_kernel<D, 8>>(dim3(nb), dim3(kThreads), 0, stream, ba, sc);
  else if (a.topk <= 16)
    launch<bwd_dq_kernel<D, 16>>(dim3(nb), dim3(kThreads), 0, stream, ba, sc);
  else
    launch<bwd_dq_kernel<D, 32>>(dim3(nb), dim3(kThreads), 0, stream, ba, sc);
  return hipGetLastError();
}


}  // namespace

hipError_t prefill_bwd_weights(const PrefillBwdArgs& ba, hipStream_t stream) {
  const PrefillArgs& a = ba.p;
  if (a.n == 0) return hipSuccess;
  const int64_t groups = (int64_t)a.B * a.Hkv * a.L;  // (b, group, token)
  const int rpb = kThreads / (a.d / 8);
  const unsigned nb = (unsigned)((groups + rpb - 1) / rpb);
  const float sc = 1.0f / sqrtf((float)a.d);
  if (a.d == 64) {
    if (a.topk <= 8)
      launch<bwd_weights_kernel<64, 8>>(dim3(nb), dim3(kThreads), 0, stream, ba, sc);
    else if (a.topk <= 16)
      launch<bwd_weights_kernel<64, 16>>(dim3(nb), dim3(kThreads), 0, stream, ba, sc);
    else
      launch<bwd_weights_kernel<64, 32>>(dim3(nb), dim3(kThreads), 0, stream, ba, sc);
  } else {
    if (a.topk <= 8)
      launch<bwd_weights_kernel<128, 8>>(dim3(nb), dim3(kThreads), 0, stream, ba, sc);
    else if (a.topk <= 16)
      launch<bwd_weights_kernel<128, 16>>(dim3(nb), dim3(kThreads), 0, stream, ba, sc);
    else
      launch<bwd_weights_kernel<128, 32>>(dim3(nb), dim3(kThreads), 0, stream, ba, sc);
  }
  return hipGetLastError();
}

hipError_t prefill_bwd_score(const PrefillBwdArgs& ba, hipStream_t stream) {
  const PrefillArgs& a = ba.p;
  if (a.n == 0) return hipSuccess;
  const int64_t blocks = (int64_t)a.B * a.Hkv * a.tiles_ub;
  const float sc = 1.0f / sqrtf((float)a.d);
  const float sl2 = sc * 1.4426950408889634f;
  if (a.d == 64)
    launch<bwd_score_kernel<64>>(dim3((unsigned)blocks), dim3(kThreads), 0, stream, ba, sl2, sc);
  else
    launch<bwd_score_kernel<128>>(dim3((unsigned)blocks), dim3(kThreads), 0, stream, ba, sl2, sc);
  return hipGetLastError();
}

hipError_t prefill_bwd_rows(const PrefillBwdArgs& ba, hipStream_t stream) {
  const PrefillArgs& a = ba.p;
  if (a.n == 0) return hipSuccess;
  const int64_t rows = (int64_t)a.B * a.Hq * a.L;
  const unsigned nb = (unsigned)((rows + kThreads - 1) / kThreads);
  if (a.topk <= 8)
    launch<bwd_rows_kernel<8>>(dim3(nb), dim3(kThreads), 0, stream, ba);
  else if (a.topk <= 16)
    launch<bwd_rows_kernel<16>>(dim3(nb), dim3(kThreads), 0, stream, ba);
  else
    launch<bwd_rows_kernel<32>>(dim3(nb), dim3(kThreads), 0, stream, ba);
  return hipGetLastError();
}

hipError_t prefill_bwd_kv(const PrefillBwdArgs& ba, hipStream_t stream) {
  const PrefillArgs& a = ba.p;
  // keys of chunks no row selected (and of a trailing partial chunk) get zero
  const int64_t words = (int64_t)a.B * a.Hkv * a.L * a.d / 2;  // bf16 pairs
  hipError_t e = launch_fill_i32((int32_t*)ba.dK, words, 0, stream);
  if (e != hipSuccess) return e;
  if ((e = launch_fill_i32((int32_t*)ba.dV, words, 0, stream)) != hipSuccess) return e;
  if (a.n == 0) return hipSuccess;
  const int64_t blocks = (int64_t)a.B * a.Hkv * a.tiles_ub;
  const float sc = 1.0f / sqrtf((float)a.d);
  const float sl2 = sc * 1.4426950408889634f;
  const float rs = 1.0f / sqrtf((float)a.S);
  if (a.d == 64)
    launch<bwd_kv_kernel<64>>(dim3((unsigned)blocks), dim3(kThreads), 0, stream, ba, sl2, sc, rs);
  else
    launch<bwd_kv_kernel<128>>(dim3((unsigned)blocks), dim3(kThreads), 0, stream, ba, sl2, sc, rs);
  return hipGetLastError();
}

hipError_t prefill_bwd_finish(const PrefillBwdArgs& ba, hipStream_t stream) {
  if ((int64_t)ba.p.B * ba.p.L == 0) return hipSuccess;
  return ba.p.d == 64 ? finish_d<64>(ba, stream) : finish_d<128>(ba, stream);
}

}  // namespace hsa
