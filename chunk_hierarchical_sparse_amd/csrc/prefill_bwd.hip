// prefill_bwd.hip - HSA prefill backward: gradients of the fused output with
// respect to Q, K and V ([HiLS] abstract: retrieval learned end to end, the
// gradient reaching the retrieval scores through the fusion weights; the
// top-K selection itself is piecewise constant and held fixed).
//
// With the forward's selection and chunk-major work list already built:
//  score : one block per work unit (a run of one chunk's (token, head) rows)
//          recomputes, on MFMA, each row's in-chunk logits S^T = K Q^T, its
//          log-sum-exp, its retrieval score s = q . lambda_c (split-bf16
//          landmark rows, fp32 accurate) and dw = dO . o_k = sum_j p_j
//          (dO . v_j) from dP^T = V dO^T.  Nothing of size d is written.
//  rows  : per (token, head): w = softmax(s) over the kept slots and
//          ds_k = w_k (dw_k - sum_k' w_k' dw_k').
//  chunk : per chunk, its K and V stay in LDS and wave pairs walk 32-row
//          tiles with the key on the lane (one wave per 32-key half):
//          S = Q K^T and dP = dO V^T (MFMA), P = exp2(S - lse),
//          dS = w P (dP - dw); then
//             dV^T += dO^T (w P)                 (MFMA, registers)
//             dK^T += Q^T (dS + ds / sqrt(S))   (MFMA; the landmark term:
//                     lambda_c = sum_j k_j / sqrt(S) gives every key of the
//                     chunk ds q / sqrt(d) / sqrt(S))
//             dQ^T piece = K^T dS^T / sqrt(d)    (MFMA, dS through LDS)
//          A work unit holds a chunk's whole list, so the waves' dK/dV sums
//          meet in LDS and are written once, as bf16.
//  finish: per (token, head): dQ = sum of its slots' pieces + sum_k ds_k
//          lambda_ck / sqrt(d).
#include <math.h>

#include "attn_core.h"
#include "hsa_common.h"
#include "kernels.h"
#include "prefill_common.h"

namespace hsa {
namespace {

constexpr int kThreads = 256;
constexpr int kRowPad = 8;    // LDS row padding (elements) of row-major tiles
constexpr int kDsPitch = 72;  // LDS row pitch of a wave's dS tile (64 keys + pad)

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

// The value of the neighbouring lane (lane ^ 1), by a DPP quad permute.
__device__ __forceinline__ uint32_t swap_adjacent_lanes(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, false);
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

// One row's Q and dO (dims 16s + 8h .. +7 for s = 0 .. D/16-1), zero when
// the row does not exist.
template <int D>
__device__ __forceinline__ void load_row_pair(const PrefillBwdArgs& ba, int64_t qbase,
                                              int64_t qplane, int32_t entry, int hh, int hf,
                                              u32x4 (&q)[D / 16], u32x4 (&o)[D / 16]) {
  if (entry >= 0) {
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

// ----------------------------------------------------------------- score --

template <int D>
struct ScoreSmem {
  uint16_t k[64 * (D + kRowPad)];
  uint16_t v[64 * (D + kRowPad)];
  uint16_t lsplit[3][D];
};

// Lane = query row (S^T = K Q^T as in the forward's chunk attention).
template <int D>
__global__ void __launch_bounds__(kThreads, 2) bwd_score_kernel(PrefillBwdArgs ba, float sl2,
                                                                float score_scale) {
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
  for (int x = threadIdx.x; x < D; x += kThreads) {
    // the fp32 landmark as three bf16 parts hi + lo + lo2 (exact)
    const float v = a.lmk[(bg * a.n + c) * D + x];
    const __bf16 h = static_cast<__bf16>(v);
    const float r1 = v - static_cast<float>(h);
    const __bf16 l = static_cast<__bf16>(r1);
    const __bf16 m = static_cast<__bf16>(r1 - static_cast<float>(l));
    sm.lsplit[0][x] = __builtin_bit_cast(uint16_t, h);
    sm.lsplit[1][x] = __builtin_bit_cast(uint16_t, l);
    sm.lsplit[2][x] = __builtin_bit_cast(uint16_t, m);
  }
  __syncthreads();
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int i32 = lane & 31, hf = lane >> 5;
  const int32_t* list = a.list + bg * a.L * a.topk + e_begin;
  const int64_t qplane = a.L * D;
  const int64_t qbase = ((int64_t)b * a.Hq + (int64_t)g * G) * qplane;
  const bool two = a.S > 32;
  for (int tile = w; tile < ntiles; tile += kThreads / kWave) {
    const int r = tile * 32 + i32;
    int ei, hh;
    split_row(r, G, a.log2G, ei, hh);
    const int32_t entry = r < rows ? list[ei] : -1;
    u32x4 q[D / 16], o[D / 16];
    load_row_pair<D>(ba, qbase, qplane, entry, hh, hf, q, o);
    const f32x16 zero = {};
    f32x16 s0 = zero, s1 = zero, p0 = zero, p1 = zero, sl = zero;
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
      u32x4 la = {0u, 0u, 0u, 0u};
      if (i32 < 3) la = *(const u32x4*)(&sm.lsplit[i32][16 * s + 8 * hf]);
      sl = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, la), qb, sl, 0, 0,
                                                   0);
    }
    const float sh = (sl[2] + sl[1]) + sl[0];
    float mx = -INFINITY;
#pragma unroll
    for (int rr = 0; rr < 16; ++rr) {
      const int key = 8 * (rr >> 2) + 4 * hf + (rr & 3);
      if (key >= a.S) s0[rr] = -INFINITY;
      if (key + 32 >= a.S) s1[rr] = -INFINITY;
      mx = fmaxf(mx, fmaxf(s0[rr], s1[rr]));
    }
    mx = fmaxf(mx, __shfl_xor(mx, 32, kWave));
    const float mxs = mx * sl2;
    float ps = 0.f, pd = 0.f;
#pragma unroll
    for (int rr = 0; rr < 16; ++rr) {
      const float e0 = fast_exp2(__builtin_fmaf(s0[rr], sl2, -mxs));
      const float e1 = fast_exp2(__builtin_fmaf(s1[rr], sl2, -mxs));
      ps += e0 + e1;
      pd += e0 * p0[rr] + e1 * p1[rr];
    }
    ps += __shfl_xor(ps, 32, kWave);
    pd += __shfl_xor(pd, 32, kWave);
    if (entry >= 0 && hf == 0) {
      const int64_t row = partial_row(a, bg, e_begin, 0) + r;
      a.part_score[row] = sh * score_scale;
      ba.lse2[row] = mxs + log2f(ps);
      ba.dw[row] = pd / ps;
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
  int64_t pr[KM];
  float s[KM], dw[KM];
  float smax = -INFINITY;
#pragma unroll
  for (int k = 0; k < KM; ++k) {
    pr[k] = k < m ? partial_row(a, bg, epos[k], hh) : 0;
    s[k] = k < m ? a.part_score[pr[k]] : -INFINITY;
    dw[k] = k < m ? ba.dw[pr[k]] : 0.f;
    smax = fmaxf(smax, s[k]);
  }
  float z = 0.f;
#pragma unroll
  for (int k = 0; k < KM; ++k) {
    s[k] = k < m ? expf(s[k] - smax) : 0.f;
    z += s[k];
  }
  const float iz = m > 0 ? 1.f / z : 0.f;
  float wdw = 0.f;
#pragma unroll
  for (int k = 0; k < KM; ++k) wdw += s[k] * iz * dw[k];
#pragma unroll
  for (int k = 0; k < KM; ++k)
    if (k < m) {
      const float wk = s[k] * iz;
      ba.wk[pr[k]] = wk;
      ba.ds[pr[k]] = wk * (dw[k] - wdw);
    }
}

// ----------------------------------------------------------------- chunk --

constexpr int kTPitch = 36;  // [dim][row] tiles: 32 rows + 4 pad (18 dwords: rows of
                             // dims 8 apart fall 16 banks apart)
constexpr int kRedPitch = 1;  // pad of the [key][dim] fp32 sums (lanes = keys)

// A wave pair's tile buffers: the tile's Q and dO transposed as [dim][row]
// (the A operand of dV^T and dK^T reads 4 consecutive rows of one dim), dS
// as [row][key] (the B operand of dQ^T) and the rows' statistics.
template <int D>
struct PairTiles {
  uint16_t qt[D * kTPitch];
  uint16_t ot[D * kTPitch];
  uint16_t dsl[32 * kDsPitch];
  float st[4][32];  // per row: lse2, dw, w, ds
};

template <int D>
struct ChunkSmem {
  uint16_t k[64 * (D + kRowPad)];
  uint16_t v[64 * (D + kRowPad)];
  uint16_t kq[16 * D * 4];
  union {
    PairTiles<D> t[2][2];                // [pair][iteration parity]
    float red[2][64 * (D + kRedPitch)];  // the chunk's dK, dV sums
  } u;
};

// Waves form two pairs; pair p takes row tiles p, p + 2, ...  Within a
// pair, the wave of key half kt computes S = Q K^T and dP = dO V^T for keys
// 32 kt .. 32 kt + 31 (key on the lane: accumulator register r of lane
// (j, h) holds row 8(r/4) + 4h + r%4 of the tile and key 32 kt + j), keeps
// that half's dK^T and dV^T in registers, and produces dQ^T for dims
// 64 kt .. 64 kt + 63 from the pair's whole dS tile.  The pair's tile
// buffers alternate with the iteration parity, so a buffer is rewritten
// only after the barrier that follows its last read.
template <int D>
__global__ void __launch_bounds__(kThreads, 1) bwd_chunk_kernel(PrefillBwdArgs ba, float sl2,
                                                                float sc, float rs) {
  const PrefillArgs& a = ba.p;
  __shared__ __attribute__((aligned(16))) ChunkSmem<D> sm;
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
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int i32 = lane & 31, hf = lane >> 5;
  const int pair = w >> 1, kt = w & 1;
  const bool keys = 32 * kt < a.S;         // this wave's key half holds keys
  const bool kval = 32 * kt + i32 < a.S;  // this lane's key exists
  const int nks = a.S > 32 ? 4 : 2;       // 16-key steps of dQ
  const int32_t* list = a.list + bg * a.L * a.topk + e_begin;
  const int64_t qplane = a.L * D;
  const int64_t qbase = ((int64_t)b * a.Hq + (int64_t)g * G) * qplane;
  const int64_t row0 = partial_row(a, bg, e_begin, 0);
  const f32x16 zero = {};
  f32x16 dk[D / 32], dv[D / 32];
#pragma unroll
  for (int bb = 0; bb < D / 32; ++bb) {
    dk[bb] = zero;
    dv[bb] = zero;
  }
  const int iters = (ntiles + 1) / 2;
  // rows of iteration i: list entries run two iterations ahead, Q / dO rows
  // and the row statistics one iteration ahead of their use
  auto entry_of = [&](int i) -> int32_t {
    const int r = (2 * i + pair) * 32 + i32;
    if (i >= iters || r >= rows) return -1;
    int ei, hh;
    split_row(r, G, a.log2G, ei, hh);
    return list[ei];
  };
  auto head_of = [&](int i) -> int {
    int ei, hh;
    split_row((2 * i + pair) * 32 + i32, G, a.log2G, ei, hh);
    return hh;
  };
  const bool stat_lane = kt == 1 && hf == 0;
  auto load_stats = [&](int i, int32_t e, f32x4& st4) {
    const int64_t pr = row0 + (2 * i + pair) * 32 + i32;
    st4 = f32x4{INFINITY, 0.f, 0.f, 0.f};
    if (stat_lane && e >= 0) st4 = f32x4{ba.lse2[pr], ba.dw[pr], ba.wk[pr], ba.ds[pr]};
  };
  // one tile of the pair: rows of iteration it with their Q / dO rows and
  // statistics already in registers
  auto body = [&](int it, int32_t entry, const u32x4 (&q)[D / 16], const u32x4 (&o)[D / 16],
                  const f32x4& st4) {
    PairTiles<D>& pt = sm.u.t[pair][it & 1];
    const int r = (2 * it + pair) * 32 + i32;
    // the pair's tile buffers: Q rows from the kt = 0 wave, dO rows and the
    // row statistics from the kt = 1 wave.  Lanes i32 and i32 ^ 1 hold
    // adjacent rows: per pair of dims (2x, 2x+1) they swap one value so the
    // even lane writes dim 2x of both rows and the odd lane dim 2x+1, one
    // dword each.
    uint16_t* tt = kt == 0 ? pt.qt : pt.ot;
    const int odd = i32 & 1;
    // v_perm_b32 picks bytes of {got, own}: the even lane keeps the low
    // halves (own, then the partner's), the odd lane the high halves
    const uint32_t psel = odd ? 0x03020706u : 0x05040100u;
#pragma unroll
    for (int s = 0; s < D / 16; ++s)
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        const uint32_t wv = kt == 0 ? q[s][x] : o[s][x];  // dims 2x, 2x+1 of this row
        const uint32_t word = __builtin_amdgcn_perm(swap_adjacent_lanes(wv), wv, psel);
        const int dim = 16 * s + 8 * hf + 2 * x + odd;
        *(uint32_t*)&tt[dim * kTPitch + (i32 & ~1)] = word;
      }
    if (stat_lane) {
#pragma unroll
      for (int f = 0; f < 4; ++f) pt.st[f][i32] = st4[f];
    }
    // S = Q K^T and dP = dO V^T for this wave's 32 keys
    f32x16 sa = zero, pa = zero;
    if (keys) {
#pragma unroll
      for (int s = 0; s < D / 16; ++s) {
        const int ko = (32 * kt + i32) * (D + kRowPad) + 16 * s + 8 * hf;
        sa = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, q[s]),
                                                     *(const bf16x8*)&sm.k[ko], sa, 0, 0, 0);
        pa = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, o[s]),
                                                     *(const bf16x8*)&sm.v[ko], pa, 0, 0, 0);
      }
    }
    block_sync_lds();  // the pair's Q/dO tiles and statistics are in LDS
    if (keys) {
      // P = exp2(S - lse), w P, dS = w P (dP - dw), dS' = dS + ds / sqrt(S)
      // (keys past S are 0; no masking when the wave's 32 keys all exist),
      // packed to bf16 at once; dS / sqrt(d) to LDS for dQ
      const bool kfull = 32 * kt + 32 <= a.S;
      const float kon = kval ? 1.f : 0.f;
      bf16x8 bp[2], bs[2];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const f32x4 l4 = *(const f32x4*)&pt.st[0][8 * u + 4 * hf];
        const f32x4 d4 = *(const f32x4*)&pt.st[1][8 * u + 4 * hf];
        const f32x4 w4 = *(const f32x4*)&pt.st[2][8 * u + 4 * hf];
        const f32x4 s4 = *(const f32x4*)&pt.st[3][8 * u + 4 * hf];
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int rr = 4 * u + v;
          float p = fast_exp2(__builtin_fmaf(sa[rr], sl2, -l4[v]));
          if (!kfull) p *= kon;
          const float wpv = w4[v] * p;
          const float dsv = wpv * (pa[rr] - d4[v]);
          float dsk = __builtin_fmaf(s4[v], rs, dsv);
          if (!kfull) dsk *= kon;
          bp[u >> 1][4 * (u & 1) + v] = static_cast<__bf16>(wpv);
          bs[u >> 1][4 * (u & 1) + v] = static_cast<__bf16>(dsk);
          pt.dsl[(8 * u + 4 * hf + v) * kDsPitch + 32 * kt + i32] =
              __builtin_bit_cast(uint16_t, static_cast<__bf16>(dsv * sc));
        }
      }
      // dV^T += dO^T (w P), dK^T += Q^T dS' (the tile's rows are the
      // contraction, in the k-slot order of the score registers)
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        // k-slots 0..3 are rows 16 s2 + 4 hf + 0..3, k-slots 4..7 rows + 8
        const int r0 = 16 * s2 + 4 * hf;
#pragma unroll
        for (int bb = 0; bb < D / 32; ++bb) {
          const int dd = 32 * bb + i32;
          const u32x2 o0 = *(const u32x2*)&pt.ot[dd * kTPitch + r0];
          const u32x2 o1 = *(const u32x2*)&pt.ot[dd * kTPitch + r0 + 8];
          const u32x2 q0 = *(const u32x2*)&pt.qt[dd * kTPitch + r0];
          const u32x2 q1 = *(const u32x2*)&pt.qt[dd * kTPitch + r0 + 8];
          dv[bb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
              __builtin_bit_cast(bf16x8, u32x4{o0[0], o0[1], o1[0], o1[1]}), bp[s2], dv[bb], 0, 0,
              0);
          dk[bb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
              __builtin_bit_cast(bf16x8, u32x4{q0[0], q0[1], q1[0], q1[1]}), bs[s2], dk[bb], 0, 0,
              0);
        }
      }
    }
    block_sync_lds();  // the pair's dS tile is complete
    // dQ^T = K^T dS^T for dims 64 kt .. 64 kt + 63 over all keys
    f32x16 dq[D / 64];
#pragma unroll
    for (int b2 = 0; b2 < D / 64; ++b2) {
      const int bb = (D / 64) * kt + b2;
      dq[b2] = zero;
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        if (s >= nks) break;
        const bf16x8 bsv = *(const bf16x8*)&pt.dsl[i32 * kDsPitch + 16 * s + 8 * hf];
        const int g0 = 4 * s + 2 * hf, g1 = g0 + 1;
        const int dd = 32 * bb + i32;
        const u32x2 k0 = *(const u32x2*)&sm.kq[(g0 * D + dd) * 4];
        const u32x2 k1 = *(const u32x2*)&sm.kq[(g1 * D + dd) * 4];
        dq[b2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            __builtin_bit_cast(bf16x8, u32x4{k0[0], k0[1], k1[0], k1[1]}), bsv, dq[b2], 0, 0, 0);
      }
    }
    if (entry >= 0) {
      uint16_t* po = (uint16_t*)a.partial + (row0 + r) * D;
#pragma unroll
      for (int b2 = 0; b2 < D / 64; ++b2)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const int dd = 32 * ((D / 64) * kt + b2) + 8 * q4 + 4 * hf;
          const u32x2 v = {pack_bf16x2(dq[b2][4 * q4], dq[b2][4 * q4 + 1]),
                           pack_bf16x2(dq[b2][4 * q4 + 2], dq[b2][4 * q4 + 3])};
          *(u32x2*)(po + dd) = v;
        }
    }
  };
  // two register sets: the next tile's rows load during the current tile,
  // list entries run one tile further ahead
  int32_t ea = entry_of(0), eb = entry_of(1);
  u32x4 qa[D / 16], oa[D / 16], qb[D / 16], ob[D / 16];
  f32x4 sta, stb;
  load_row_pair<D>(ba, qbase, qplane, ea, head_of(0), hf, qa, oa);
  load_stats(0, ea, sta);
  for (int it = 0; it < iters; it += 2) {
    const int32_t ec = entry_of(it + 2);
    load_row_pair<D>(ba, qbase, qplane, eb, head_of(it + 1), hf, qb, ob);
    load_stats(it + 1, eb, stb);
    body(it, ea, qa, oa, sta);
    if (it + 1 >= iters) break;
    const int32_t ed = entry_of(it + 3);
    load_row_pair<D>(ba, qbase, qplane, ec, head_of(it + 2), hf, qa, oa);
    load_stats(it + 2, ec, sta);
    body(it + 1, eb, qb, ob, stb);
    ea = ec;
    eb = ed;
  }
  // the chunk's dK / dV: the two pairs' halves summed in LDS
  constexpr int RP = D + kRedPitch;
  __syncthreads();
  for (int x = threadIdx.x; x < 2 * 64 * RP; x += kThreads) (&sm.u.red[0][0])[x] = 0.f;
  __syncthreads();
  if (kval) {
    const int key = 32 * kt + i32;
#pragma unroll
    for (int bb = 0; bb < D / 32; ++bb)
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) {
        const int dim = 32 * bb + 8 * (rr >> 2) + 4 * hf + (rr & 3);
        atomicAdd(&sm.u.red[0][key * RP + dim], dk[bb][rr]);
        atomicAdd(&sm.u.red[1][key * RP + dim], dv[bb][rr]);
      }
  }
  __syncthreads();
  // the block holds the chunk's whole list: its rows of dK and dV are final
  for (int x = threadIdx.x; x < a.S * D / 8; x += kThreads) {
    const int key = x / (D / 8), d0 = 8 * (x % (D / 8));
    const float* kr = &sm.u.red[0][key * RP + d0];
    const float* vr = &sm.u.red[1][key * RP + d0];
    u32x4 ko, vo;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      ko[j] = pack_bf16x2(kr[2 * j] * sc, kr[2 * j + 1] * sc);
      vo[j] = pack_bf16x2(vr[2 * j], vr[2 * j + 1]);
    }
    *(u32x4*)((uint16_t*)ba.dK + kv0 + 8 * x) = ko;
    *(u32x4*)((uint16_t*)ba.dV + kv0 + 8 * x) = vo;
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
  u32x4 x[KM];
  float dsk[KM];
  int32_t ck[KM];
#pragma unroll
  for (int k = 0; k < KM; ++k) {
    const int64_t pr = k < m ? partial_row(a, bg, epos[k], hh) : 0;
    x[k] = k < m ? *(const u32x4*)((const uint16_t*)a.partial + pr * D + cg * 8)
                 : u32x4{0u, 0u, 0u, 0u};
    dsk[k] = k < m ? ba.ds[pr] * sc : 0.f;
    ck[k] = k < m ? sel[k] : 0;
  }
#pragma unroll
  for (int k = 0; k < KM; ++k) {
    if (k >= m) break;
    const float* lc = a.lmk + (bg * a.n + ck[k]) * D + cg * 8;
    const f32x4 l0 = *(const f32x4*)lc, l1 = *(const f32x4*)(lc + 4);
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      acc[2 * v] += bf16_bits_to_f32(x[k][v] & 0xffffu);
      acc[2 * v + 1] += bf16_bits_to_f32(x[k][v] >> 16);
    }
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      acc[v] += dsk[k] * l0[v];
      acc[4 + v] += dsk[k] * l1[v];
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
    bwd_dq_kernel<D, 8><<<dim3(nb), dim3(kThreads), 0, stream>>>(ba, sc);
  else if (a.topk <= 16)
    bwd_dq_kernel<D, 16><<<dim3(nb), dim3(kThreads), 0, stream>>>(ba, sc);
  else
    bwd_dq_kernel<D, 32><<<dim3(nb), dim3(kThreads), 0, stream>>>(ba, sc);
  return hipGetLastError();
}

}  // namespace

hipError_t prefill_bwd_score(const PrefillBwdArgs& ba, hipStream_t stream) {
  const PrefillArgs& a = ba.p;
  if (a.n == 0) return hipSuccess;
  const int64_t blocks = (int64_t)a.B * a.Hkv * a.tiles_ub;
  const float sc = 1.0f / sqrtf((float)a.d);
  const float sl2 = sc * 1.4426950408889634f;
  if (a.d == 64)
    bwd_score_kernel<64><<<dim3((unsigned)blocks), dim3(kThreads), 0, stream>>>(ba, sl2, sc);
  else
    bwd_score_kernel<128><<<dim3((unsigned)blocks), dim3(kThreads), 0, stream>>>(ba, sl2, sc);
  return hipGetLastError();
}

hipError_t prefill_bwd_rows(const PrefillBwdArgs& ba, hipStream_t stream) {
  const PrefillArgs& a = ba.p;
  if (a.n == 0) return hipSuccess;
  const int64_t rows = (int64_t)a.B * a.Hq * a.L;
  const unsigned nb = (unsigned)((rows + kThreads - 1) / kThreads);
  if (a.topk <= 8)
    bwd_rows_kernel<8><<<dim3(nb), dim3(kThreads), 0, stream>>>(ba);
  else if (a.topk <= 16)
    bwd_rows_kernel<16><<<dim3(nb), dim3(kThreads), 0, stream>>>(ba);
  else
    bwd_rows_kernel<32><<<dim3(nb), dim3(kThreads), 0, stream>>>(ba);
  return hipGetLastError();
}

hipError_t prefill_bwd_chunk(const PrefillBwdArgs& ba, hipStream_t stream) {
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
    bwd_chunk_kernel<64><<<dim3((unsigned)blocks), dim3(kThreads), 0, stream>>>(ba, sl2, sc, rs);
  else
    bwd_chunk_kernel<128><<<dim3((unsigned)blocks), dim3(kThreads), 0, stream>>>(ba, sl2, sc,
                                                                                 rs);
  return hipGetLastError();
}

hipError_t prefill_bwd_finish(const PrefillBwdArgs& ba, hipStream_t stream) {
  if ((int64_t)ba.p.B * ba.p.L == 0) return hipSuccess;
  return ba.p.d == 64 ? finish_d<64>(ba, stream) : finish_d<128>(ba, stream);
}

}  // namespace hsa
