// chunk_attend.h - the bf16 chunk attention of HSA prefill ([HiLS]
// abstract: each query attends independently inside every retrieved chunk,
// and the chunk outputs are later fused by the retrieval scores), as a
// block-level device function: the chunk-major prefill launch runs it for
// every block, and the upper layers' fused launch runs it for the blocks
// it gives to HSA.
#pragma once

#include "attn_core.h"
#include "hsa_common.h"
#include "kernels.h"
#include "prefill_common.h"

namespace hsa {

HSA_DCHECK_SOURCE()

constexpr int kChunkThreads = 256;

// LDS of one block of the chunk attention.
template <int D>
struct ChunkSmem {
  KVSmem<D> kv;
  // the landmark's three bf16 parts, then a zero row that lanes 3..31 read;
  // rows padded by 16 bytes, so the four rows' reads fall on different banks
  __attribute__((aligned(16))) uint16_t lsplit[4][D + 8];
  // each wave's tile of partial rows, rows padded by 16 bytes (conflict-free)
  __attribute__((aligned(16))) uint16_t ostage[kChunkThreads / kWave][32 * (D + 8)];
};

// bf16, S <= 64: one block per work unit, a run of at most
// kChunkUnitRows (token, head) rows of one chunk's list, so hot chunks spread
// over several blocks.  The chunk's K/V are staged in LDS once per block;
// each wave then walks 32-row tiles of the unit's rows.  A row sees exactly this chunk, so its softmax is over
// at most 64 keys held in registers: no online rescaling.  The per-head
// retrieval score s_h = q . lmk_c runs on MFMA too: the fp32 landmark is
// split into three bf16 rows (hi + lo + lo2 == the fp32 value) that act as
// extra "keys", so q (exact in bf16) meets an exact landmark and s_h keeps
// fp32 accuracy.  Q rows are double-buffered: a tile's rows load during the
// whole previous tile.  S64: chunks of exactly 64 keys (both key halves, no
// masking), fixed at compile time.
template <int D, bool S64>
__device__ __forceinline__ void attend_chunk_body(const PrefillArgs& a, float scale_log2,
                                                  float score_scale, int64_t blk,
                                                  ChunkSmem<D>& smem) {
  constexpr int kThreads = kChunkThreads;
  KVSmem<D>& sm = smem.kv;
  auto& lsplit = smem.lsplit;
  auto& ostage = smem.ostage;
  int64_t bg;
  int c, e_begin, e_end;
  if (!locate_tile(a, blk, bg, c, e_begin, e_end)) return;
  const int cnt = e_end - e_begin;
  const int G = a.Hq / a.Hkv;
  const int b = (int)(bg / a.Hkv), g = (int)(bg % a.Hkv);
  const int rows = cnt * G;
  const int ntiles = (rows + 31) / 32;
  const int64_t kv0 = (bg * a.L + (int64_t)c * a.S) * D;
  load_kv_block<D>(sm, (const uint16_t*)a.K + kv0, (const uint16_t*)a.V + kv0, a.S);
  for (int x = threadIdx.x; x < D; x += kThreads) {
    const float v = a.lmk[(bg * a.n + c) * D + x];
    const __bf16 h = static_cast<__bf16>(v);
    const float r1 = v - static_cast<float>(h);
    const __bf16 l = static_cast<__bf16>(r1);
    const __bf16 m = static_cast<__bf16>(r1 - static_cast<float>(l));
    lsplit[0][x] = __builtin_bit_cast(uint16_t, h);
    lsplit[1][x] = __builtin_bit_cast(uint16_t, l);
    lsplit[2][x] = __builtin_bit_cast(uint16_t, m);
    lsplit[3][x] = 0;
  }
  __syncthreads();

  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int i32 = lane & 31, hf = lane >> 5;
  const int32_t* list = a.list + bg * a.L * a.topk + e_begin;
  const uint16_t* Q = (const uint16_t*)a.Q;
  const int64_t qplane = (int64_t)a.L * D;  // stride between heads
  const int64_t qbase = (int64_t)b * a.Hq * qplane + (int64_t)g * G * qplane;
  const int lg = a.log2G;

  // row r of the chunk -> (entry index r / G, head r % G)
  auto split_row = [&](int r, int& ei, int& hh) {
    if (lg >= 0) {
      ei = r >> lg;
      hh = r & ((1 << lg) - 1);
    } else {
      ei = r / G;
      hh = r - ei * G;
    }
  };
  // Loads are issued unconditionally (indices clamped in bounds, values
  // dropped afterwards): a load under a per-lane guard makes the compiler
  // count outstanding loads for the path without it, so the next wait would
  // also cover the prefetch it was meant to overlap.
  // A tile's row exists when row_ok; entry_raw and load_q read clamped,
  // always-valid indices for the others (values unused), also for tiles
  // past the last, so no load is issued conditionally.
  const int last_e = max(cnt - 1, 0);
  auto row_ok = [&](int tile) { return tile * 32 + i32 < rows; };
  auto entry_raw = [&](int tile) -> int32_t {
    int ei, hh;
    split_row(tile * 32 + i32, ei, hh);
    return list[min(ei, last_e)];
  };
  auto load_q = [&](int tile, int32_t entry, u32x4 (&q)[D / 16]) {
    int ei, hh;
    split_row(tile * 32 + i32, ei, hh);
    const int64_t t = row_ok(tile) ? (int64_t)(entry >> kSlotBits) : 0;
    // a listed token sees the chunk whole: (c + 1) S <= t < L
    HSA_DCHECK(!row_ok(tile) || (t >= (int64_t)(c + 1) * a.S && t < a.L));
    const uint16_t* qrow = Q + qbase + (int64_t)hh * qplane + t * D + 8 * hf;
#pragma unroll
    for (int s2 = 0; s2 < D / 16; ++s2) q[s2] = *(const u32x4*)(qrow + 16 * s2);
  };

  const bool two = S64 || a.S > 32;
  const bool full = S64 || a.S == kKeyBlock;  // no key masking needed
  auto compute_tile = [&](int tile, int32_t ent_cur, const u32x4 (&q)[D / 16]) {
    // S^T = K Q^T (keys 0..63) and L^T = LMK3 Q^T (rows 0..2: landmark parts)
    // the first k-step takes a zero accumulator operand: no register fill
    f32x16 s0, s1, sl;
#pragma unroll
    for (int s2 = 0; s2 < D / 16; ++s2) {
      const f32x16 zero = {};
      const bf16x8 qb = __builtin_bit_cast(bf16x8, q[s2]);
      const bf16x8 a0 = *(const bf16x8*)(&sm.k[i32 * (D + 8) + 16 * s2 + 8 * hf]);
      s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, qb, s2 == 0 ? zero : s0, 0, 0, 0);
      if (two) {
        const bf16x8 a1 = *(const bf16x8*)(&sm.k[(32 + i32) * (D + 8) + 16 * s2 + 8 * hf]);
        s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, qb, s2 == 0 ? zero : s1, 0, 0, 0);
      } else if (s2 == 0) {
        s1 = zero;
      }
      const bf16x8 la = *(const bf16x8*)(&lsplit[min(i32, 3)][16 * s2 + 8 * hf]);
      sl = __builtin_amdgcn_mfma_f32_32x32x16_bf16(la, qb, s2 == 0 ? zero : sl, 0, 0, 0);
    }
    // rows 0..2 of L^T sit in registers 0..2 of the lanes of half 0
    const float sh = (sl[2] + sl[1]) + sl[0];
    __builtin_amdgcn_sched_barrier(0);
    // softmax over the chunk's keys: p = exp2((s - max) * scale), normalised
    float mx = -INFINITY;
    if (!full) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = 8 * (r >> 2) + 4 * hf + (r & 3);
        s0[r] = key < a.S ? s0[r] : -INFINITY;
        s1[r] = key + 32 < a.S ? s1[r] : -INFINITY;
      }
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, fmaxf(s0[r], s1[r]));
    mx = half_pair_max(mx);
    const float mxs = mx * scale_log2;
    float ps = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      s0[r] = fast_exp2(__builtin_fmaf(s0[r], scale_log2, -mxs));
      s1[r] = fast_exp2(__builtin_fmaf(s1[r], scale_log2, -mxs));
      ps += s0[r] + s1[r];
    }
    ps = half_pair_sum(ps);
    const float inv = 1.f / ps;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      s0[r] *= inv;
      s1[r] *= inv;
    }
    bf16x8 pb4[4];
    pb4[0] = cvt_bf16x8(s0, 0);
    pb4[1] = cvt_bf16x8(s0, 8);
    pb4[2] = cvt_bf16x8(s1, 0);
    pb4[3] = cvt_bf16x8(s1, 8);
    __builtin_amdgcn_sched_barrier(0);
    // O^T = V^T P^T (already normalised)
    f32x16 o[D / 32];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      if (kt == 1 && !two) break;
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        const bf16x8 pb = pb4[2 * kt + s2];
        const int g0 = 8 * kt + 4 * s2 + hf, g1 = g0 + 2;
#pragma unroll
        for (int bb = 0; bb < D / 32; ++bb) {
          const int dd = 32 * bb + i32;
          const u32x2 v0 = *(const u32x2*)(&sm.v[(g0 * D + dd) * 4]);
          const u32x2 v1 = *(const u32x2*)(&sm.v[(g1 * D + dd) * 4]);
          const u32x4 av = {v0[0], v0[1], v1[0], v1[1]};
          if (kt == 0 && s2 == 0) {
            const f32x16 zero = {};
            o[bb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, av), pb,
                                                            zero, 0, 0, 0);
          } else {
            o[bb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, av), pb,
                                                            o[bb], 0, 0, 0);
          }
        }
      }
    }
    // lane half hf holds columns 32bb + 8q4 + 4hf + 0..3; swapping half of
    // the groups with the partner lane leaves each lane 16 contiguous bytes
    // (columns 32bb + 8(2pr + hf) + 0..7) to store
    u32x4 outv[D / 32][2];
#pragma unroll
    for (int bb = 0; bb < D / 32; ++bb)
#pragma unroll
      for (int pr = 0; pr < 2; ++pr) {
        const int q_even = 2 * pr, q_odd = 2 * pr + 1;
        const uint32_t e0 = pack_bf16x2(o[bb][4 * q_even], o[bb][4 * q_even + 1]);
        const uint32_t e1 = pack_bf16x2(o[bb][4 * q_even + 2], o[bb][4 * q_even + 3]);
        const uint32_t d0 = pack_bf16x2(o[bb][4 * q_odd], o[bb][4 * q_odd + 1]);
        const uint32_t d1 = pack_bf16x2(o[bb][4 * q_odd + 2], o[bb][4 * q_odd + 3]);
        // half 0 keeps the even group and sends the odd one; half 1 the reverse
        const uint32_t got0 = half_pair_exchange(d0, e0, hf != 0);
        const uint32_t got1 = half_pair_exchange(d1, e1, hf != 0);
        outv[bb][pr] = hf ? u32x4{got0, got1, d0, d1} : u32x4{e0, e1, got0, got1};
      }
    // rows of a tile are consecutive: (entry e_begin + r / G, head r % G),
    // so the tile's partials are one contiguous run of up to 32 rows.  They
    // go through LDS and leave as 1 KB stores; rows past the unit's end
    // belong to the next unit and are not written.
    const int64_t row0 = partial_row(a, bg, e_begin, 0) + tile * 32;
    if (ent_cur >= 0 && hf == 0) a.part_score[row0 + i32] = sh * score_scale;
    uint16_t* stg = ostage[w];
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
    for (int bb = 0; bb < D / 32; ++bb)
#pragma unroll
      for (int pr = 0; pr < 2; ++pr)
        *(u32x4*)(stg + i32 * (D + 8) + 32 * bb + 8 * (2 * pr + hf)) = outv[bb][pr];
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    const int nrow = min(32, rows - tile * 32);
    constexpr int LPR = D / 8;        // lanes per row (16 bytes each)
    constexpr int RPI = kWave / LPR;  // rows per store instruction
    uint16_t* base = (uint16_t*)a.partial + row0 * D;
    const int piece = lane % LPR;
#pragma unroll
    for (int k = 0; k < 32 / RPI; ++k) {
      const int row = k * RPI + lane / LPR;
      const u32x4 v = *(const u32x4*)(stg + row * (D + 8) + 8 * piece);
      if (row < nrow) __builtin_nontemporal_store(v, (u32x4*)(base + (int64_t)row * D + 8 * piece));
    }
  };

  // Double-buffered Q: the next tile's rows load during the whole current
  // tile.  List entries run one tile further ahead.
  // Every load is unconditional: a load issued on one path only makes the
  // compiler count outstanding loads for the other path, and the next wait
  // would then cover the prefetch too.
  u32x4 qa[D / 16], qb[D / 16];
  int tile = w;
  int32_t ea = entry_raw(tile);
  int32_t eb = entry_raw(tile + 4);
  load_q(tile, ea, qa);
  for (; tile < ntiles; tile += 8) {
    const int32_t ec = entry_raw(tile + 8);
    load_q(tile + 4, eb, qb);
    compute_tile(tile, row_ok(tile) ? ea : -1, qa);
    if (tile + 4 >= ntiles) break;
    const int32_t ed = entry_raw(tile + 12);
    load_q(tile + 8, ec, qa);
    compute_tile(tile + 4, row_ok(tile + 4) ? eb : -1, qb);
    ea = ec;
    eb = ed;
  }
}

}  // namespace hsa
