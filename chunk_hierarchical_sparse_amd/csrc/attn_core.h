// attn_core.h - bf16 MFMA softmax attention of 32 query rows per wave over
// key blocks of up to 64 keys staged in LDS, with an online softmax across
// blocks.  Used by the HSA chunk attention (one chunk per row, [HiLS]
// abstract: attention independently inside each retrieved chunk) and by the
// DHSA masked attention (several key chunks per row).
//
// Layout (v_mfma_f32_32x32x16_bf16, lane l, half h = l/32, row i = l%32):
//  * scores are computed transposed, S^T = K Q^T: A = 32 keys x 16 dims from
//    LDS, B = Q^T with lane l holding query l%32 (dims 16s+8h..+7 of k-step
//    s).  The accumulator gives lane l the query l%32 and keys
//    8*(r/4) + 4h + r%4 (r = 0..15), so each lane owns one query's row
//    statistics and only lanes l and l^32 share a query.
//  * O^T = V^T P^T: B = P^T straight from the score registers (registers
//    8s'..8s'+7 form k-step s'; the k-slot -> key map is the one the score
//    layout gives, and A uses the same map), A = V^T read from LDS where V
//    is stored as [key/4][dim][4 keys], so each lane reads 8 contiguous
//    bytes per key quad.  The output accumulator again has lane l = query,
//    so the online-softmax rescale is a per-lane scalar.
#pragma once

#include "hsa_common.h"

namespace hsa {

constexpr int kKeyBlock = 64;

template <int D>
struct KVSmem {
  uint16_t k[kKeyBlock * (D + 8)];  // row-major, rows padded by 16 bytes
  uint16_t v[(kKeyBlock / 4) * D * 4];
};

// Stage keys/values rows [0, nk) (1 <= nk <= 64) of a block (row stride D
// elements) into LDS; rows nk..63 are zero so masked keys never meet
// non-finite data.  Every load is issued before any store (rows past nk
// re-read row nk - 1 and are zeroed): guarded loads would each wait for
// the one before.  Called by all threads of a 256-thread block.
template <int D>
__device__ __forceinline__ void load_kv_block(KVSmem<D>& sm, const uint16_t* __restrict__ Kg,
                                              const uint16_t* __restrict__ Vg, int nk) {
  const int tid = threadIdx.x;
  constexpr int KPR = D / 8;                        // 16-byte pieces per key row
  constexpr int NKL = kKeyBlock * KPR / 256;        // key loads per thread
  constexpr int VPR = D / 4;                        // 8-byte pieces per value row
  constexpr int NVL = (kKeyBlock / 4) * VPR / 256;  // value quads per thread
  u32x4 kx[NKL];
#pragma unroll
  for (int i = 0; i < NKL; ++i) {
    const int e = tid + i * 256, row = e / KPR, c8 = e % KPR;
    kx[i] = *(const u32x4*)(Kg + (int64_t)min(row, nk - 1) * D + c8 * 8);
  }
  u32x2 vr[NVL][4];
#pragma unroll
  for (int i = 0; i < NVL; ++i) {
    const int e = tid + i * 256, grp = e / VPR, cq = e % VPR;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
      vr[i][kk] = *(const u32x2*)(Vg + (int64_t)min(grp * 4 + kk, nk - 1) * D + cq * 4);
  }
#pragma unroll
  for (int i = 0; i < NKL; ++i) {
    const int e = tid + i * 256, row = e / KPR, c8 = e % KPR;
    *(u32x4*)(&sm.k[row * (D + 8) + c8 * 8]) = row < nk ? kx[i] : u32x4{0u, 0u, 0u, 0u};
  }
#pragma unroll
  for (int i = 0; i < NVL; ++i) {
    const int e = tid + i * 256, grp = e / VPR, cq = e % VPR;
    u32x2 r[4];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) r[kk] = grp * 4 + kk < nk ? vr[i][kk] : u32x2{0u, 0u};
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
      *(u32x2*)(&sm.v[(grp * D + cq * 4 + x) * 4]) = u32x2{lo, hi};
    }
  }
}

template <int D>
struct WaveAttn {
  bf16x8 qf[D / 16];  // Q^T operand, k-step s: dims 16s + 8h .. 16s + 8h + 7
  f32x16 o[D / 32];   // O^T accumulator, block b: dims 32b + 8(r/4) + 4h + r%4
  float m;            // running max of log2-domain logits (this lane's query)
  float l;            // running sum of exp2(logit - m)
};

// qrow must point at a readable row even when !valid (the row is loaded and
// then zeroed: loads guarded per lane would each wait for the one before).
template <int D>
__device__ __forceinline__ void wave_attn_init(WaveAttn<D>& st, const uint16_t* qrow,
                                               bool valid) {
  const int h = (threadIdx.x & 63) >> 5;
  u32x4 x[D / 16];
#pragma unroll
  for (int s = 0; s < D / 16; ++s) x[s] = *(const u32x4*)(qrow + 16 * s + 8 * h);
#pragma unroll
  for (int s = 0; s < D / 16; ++s)
    st.qf[s] = __builtin_bit_cast(bf16x8, valid ? x[s] : u32x4{0u, 0u, 0u, 0u});
#pragma unroll
  for (int b = 0; b < D / 32; ++b)
#pragma unroll
    for (int r = 0; r < 16; ++r) st.o[b][r] = 0.f;
  st.m = -INFINITY;
  st.l = 0.f;
  // wait for the query rows here: left outstanding into a key loop, they
  // make the compiler's wait before the loop's first MFMA cover every load
  // issued since, including the next key block's prefetch
  __builtin_amdgcn_s_waitcnt(0);
}

__device__ __forceinline__ bf16x8 cvt_bf16x8(const f32x16& p, int base) {
  bf16x8 r;
#pragma unroll
  for (int e = 0; e < 8; ++e) r[e] = static_cast<__bf16>(p[base + e]);
  return r;
}

// One key block of nkeys (<= 64, the same for the whole block) staged keys:
// keys with in-block index < nvalid are attended by this lane's query
// (nvalid <= nkeys may differ per lane; 0 = none).  scale_log2 =
// log2(e)/sqrt(d).  Must be called by every lane of the wave.
template <int D>
__device__ __forceinline__ void wave_attn_block(WaveAttn<D>& st, const KVSmem<D>& sm, int nkeys,
                                                int nvalid, float scale_log2) {
  const int lane = threadIdx.x & 63;
  const int h = lane >> 5;
  const int i32 = lane & 31;
  // keys 32..63 of the block exist only when the block holds more than 32
  // (block-uniform, so the branch does not diverge)
  const bool two = nkeys > 32;
  f32x16 s0, s1;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    s0[r] = 0.f;
    s1[r] = 0.f;
  }
#pragma unroll
  for (int s = 0; s < D / 16; ++s) {
    const bf16x8 a0 = *(const bf16x8*)(&sm.k[i32 * (D + 8) + 16 * s + 8 * h]);
    s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, st.qf[s], s0, 0, 0, 0);
    if (two) {
      const bf16x8 a1 = *(const bf16x8*)(&sm.k[(32 + i32) * (D + 8) + 16 * s + 8 * h]);
      s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, st.qf[s], s1, 0, 0, 0);
    }
  }
  __builtin_amdgcn_sched_barrier(0);
  float mx = -INFINITY;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int key = 8 * (r >> 2) + 4 * h + (r & 3);
    const float x0 = key < nvalid ? s0[r] * scale_log2 : -INFINITY;
    const float x1 = key + 32 < nvalid ? s1[r] * scale_log2 : -INFINITY;
    s0[r] = x0;
    s1[r] = x1;
    mx = fmaxf(mx, fmaxf(x0, x1));
  }
  mx = half_pair_max(mx);
  const float m_new = fmaxf(st.m, mx);
  const float m_use = m_new == -INFINITY ? 0.f : m_new;
  const float alpha = fast_exp2(st.m - m_use);
  float ps = 0.f;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    s0[r] = fast_exp2(s0[r] - m_use);
    s1[r] = fast_exp2(s1[r] - m_use);
    ps += s0[r] + s1[r];
  }
  ps = half_pair_sum(ps);
  st.l = st.l * alpha + ps;
  st.m = m_new;
  bf16x8 pb4[4];
  pb4[0] = cvt_bf16x8(s0, 0);
  pb4[1] = cvt_bf16x8(s0, 8);
  pb4[2] = cvt_bf16x8(s1, 0);
  pb4[3] = cvt_bf16x8(s1, 8);
#pragma unroll
  for (int b = 0; b < D / 32; ++b)
#pragma unroll
    for (int r = 0; r < 16; ++r) st.o[b][r] *= alpha;
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int kt = 0; kt < 2; ++kt) {
    if (kt == 1 && !two) break;
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
      const bf16x8 pb = pb4[2 * kt + s2];
      const int g0 = 8 * kt + 4 * s2 + h;  // key quad of k-slots 0..3
      const int g1 = g0 + 2;               // key quad of k-slots 4..7
#pragma unroll
      for (int b = 0; b < D / 32; ++b) {
        const int dd = 32 * b + i32;
        const u32x2 v0 = *(const u32x2*)(&sm.v[(g0 * D + dd) * 4]);
        const u32x2 v1 = *(const u32x2*)(&sm.v[(g1 * D + dd) * 4]);
        const u32x4 av = {v0[0], v0[1], v1[0], v1[1]};
        st.o[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, av), pb,
                                                          st.o[b], 0, 0, 0);
      }
    }
  }
}

// ---------------------------------------------------------------------
// Variable-length key blocks of up to 128 keys (DHSA: one chunk per block;
// the sliding-window attention: 128-key blocks of the window).
//
// V layout of these blocks: row-major, the 16-byte units of value row r at
// unit ^ wide_vswz(r), and the A operand of O^T = V^T P^T (lane = column,
// eight keys) taken by two transposed reads (ds_read_b64_tr_b16), so that
// staging is a plain 16-byte copy of each row piece.

constexpr int kWideBlock = 128;

template <int D, int KB = kWideBlock>
struct KVSmemWide {
  uint16_t k[KB * (D + 8)];
  uint16_t v[KB * D];  // row-major, 16-byte units swizzled by wide_vswz
};

// XOR applied to the 16-byte unit index of value row r.  A transposed read
// takes 32 bytes from each of four consecutive rows (a multiple of four on)
// per 16 lanes; with the four rows' units moved by 0, 4, 8, 12 (two values
// for the 8-unit rows of d = 64) the read touches every bank once.
template <int D>
__device__ __forceinline__ constexpr int wide_vswz(int r) {
  return D >= 128 ? 4 * (r & 3) : 4 * (r & 1);
}

typedef short s16x4 __attribute__((ext_vector_type(4)));

// Transposed 8-byte LDS read (ds_read_b64_tr_b16): in each 16-lane group,
// lane i receives element i % 4 of the 8-byte pieces addressed by lanes
// i / 4 + 4 j, as its value j (j = 0..3).
__device__ __forceinline__ u32x2 lds_read_tr16(const uint16_t* p) {
  const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4*)(p));
  return __builtin_bit_cast(u32x2, v);
}

// One thread's share of a KB-key block held in registers between its global
// load and its LDS store, so the next block's loads can be in flight while
// the current block is computed.  NT = 2 KB threads (256 for 128 keys); K
// and V as 16-byte row pieces (thread t: piece t % KPR of rows t / KPR +
// i * (NT / KPR)).
template <int D, int KB = kWideBlock>
struct KVRegsWide {
  static constexpr int NT = 2 * KB;
  static constexpr int KPR = D / 8;  // 16-byte pieces per row
  static constexpr int NK = KB * KPR / NT;
  u32x4 k[NK];
  u32x4 v[NK];
};

// Raw buffer resource over [base, base + bytes): buffer loads at offsets
// past the range return zero instead of touching memory.  Word 3 holds the
// CDNA default (32-bit data format, no swizzle).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_range(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, 0x00020000);
}

// Loads of rows [0, nk) (nk <= KB) of a key/value block into registers;
// rows past nk read as zero (buffer range check, no branches).  Called by
// all NT threads of the block.  The range check of a raw buffer load
// covers the lane offset (and the instruction's immediate) but not the
// scalar offset, so the whole offset is in the lane operand: load i reads
// rows i * (NT / KPR) further on by moving its buffer's base there (scalar
// registers) and shrinking its range to match.
template <int D, int KB = kWideBlock>
__device__ __forceinline__ void fetch_kv_wide(KVRegsWide<D, KB>& r,
                                              const uint16_t* __restrict__ Kg,
                                              const uint16_t* __restrict__ Vg, int nk) {
  using R = KVRegsWide<D, KB>;
  const int tid = threadIdx.x;
  const int bytes = nk * D * 2;
  const char* kg = (const char*)Kg;
  const char* vg = (const char*)Vg;
  const int off = ((tid / R::KPR) * D + (tid % R::KPR) * 8) * 2;  // bytes
#pragma unroll
  for (int i = 0; i < R::NK; ++i) {
    constexpr int step = (R::NT / R::KPR) * D * 2;
    const int left = max(bytes - i * step, 0);
    r.k[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                           buffer_range(kg + i * step, left), off, 0, 0));
    r.v[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                           buffer_range(vg + i * step, left), off, 0, 0));
  }
}

// LDS store of a fetched block: rows up to the next multiple of 32 above nk
// (zeros past nk) are written, rows beyond that are never read.  A thread's
// rows are all one residue mod 4 (NT / KPR is a multiple of 4), so its V
// pieces share one swizzle.
template <int D, int KB = kWideBlock>
__device__ __forceinline__ void store_kv_wide(KVSmemWide<D, KB>& sm, const KVRegsWide<D, KB>& r,
                                              int nk) {
  using R = KVRegsWide<D, KB>;
  constexpr int RS = R::NT / R::KPR;  // rows between a thread's pieces
  const int tid = threadIdx.x;
  const int rows = (nk + 31) & ~31;
  const int krow = tid / R::KPR, c = tid % R::KPR;
  uint16_t* ks = &sm.k[krow * (D + 8) + c * 8];
  uint16_t* vs = &sm.v[krow * D + ((c ^ wide_vswz<D>(krow)) * 8)];
#pragma unroll
  for (int i = 0; i < R::NK; ++i)
    if (krow + i * RS < rows) {
      *(u32x4*)(ks + i * RS * (D + 8)) = r.k[i];
      *(u32x4*)(vs + i * RS * D) = r.v[i];
    }
}

// One staged block of nkeys (<= 128, block-uniform) keys: this lane's query
// attends keys with in-block index < nvalid (<= nkeys; may differ per lane)
// and, with BAND, also >= nlo (a sliding window's lower edge).
// The block is taken SUB 32-key sub-tiles at a time (SUB = 4: one update
// for the whole block; SUB = 2: two, with half the score registers), each
// with one online-softmax update; the accumulator is rescaled only when
// some lane's running maximum grew.
template <int D, int SUB, bool BAND = false, int KB = kWideBlock>
__device__ __forceinline__ void wave_attn_wide(WaveAttn<D>& st, const KVSmemWide<D, KB>& sm,
                                               int nkeys, int nvalid, float scale_log2,
                                               int nlo = 0) {
  const int lane = threadIdx.x & 63;
  const int h = lane >> 5;
  const int i32 = lane & 31;
  const int nsub_all = (nkeys + 31) >> 5;  // 1..4
#pragma nounroll
  for (int t0 = 0; t0 < nsub_all; t0 += SUB) {
    const int nsub = min(SUB, nsub_all - t0);
    const int nv = nvalid - 32 * t0;  // valid keys of this lane from sub-tile t0 on
    const int nl = nlo - 32 * t0;     // first valid key relative to sub-tile t0
    // the valid keys end before nvalid, so once no lane has any left none follow
    if (__ballot(nv > 0) == 0) break;
    // sub-tiles wholly below every lane's window hold no valid key
    if (BAND && __ballot(nl < 32 * nsub) == 0) continue;
    // the first k-step takes a zero accumulator operand: no register fill
    f32x16 sc[SUB];
#pragma unroll
    for (int t = 0; t < SUB; ++t) {
      if (t >= nsub) break;
      const f32x16 zero = {};
      const bf16x8 a0 = *(const bf16x8*)(&sm.k[(32 * (t0 + t) + i32) * (D + 8) + 8 * h]);
      sc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, st.qf[0], zero, 0, 0, 0);
#pragma unroll
      for (int s = 1; s < D / 16; ++s) {
        const bf16x8 a1 =
            *(const bf16x8*)(&sm.k[(32 * (t0 + t) + i32) * (D + 8) + 16 * s + 8 * h]);
        sc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, st.qf[s], sc[t], 0, 0, 0);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    // keys at or past nvalid (and padding past nkeys) take no weight; only
    // the sub-tiles some lane's valid keys end in or before need the mask
#pragma unroll
    for (int t = 0; t < SUB; ++t) {
      if (t >= nsub) break;
      if (__ballot(nv < 32 * (t + 1) || (BAND && nl > 32 * t)) != 0) {
        if (BAND) {
          // key = 32 t + 4 h + c_r with c_r = 8 (r / 4) + r % 4 a constant:
          // compare c_r against the lane's bounds moved by 32 t + 4 h
          // (measured faster for the band, slower without it)
          const int hi = nv - 32 * t - 4 * h, lo = nl - 32 * t - 4 * h;
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int cr = 8 * (r >> 2) + (r & 3);
            if (cr >= hi || cr < lo) sc[t][r] = -INFINITY;
          }
        } else {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = 32 * t + 8 * (r >> 2) + 4 * h + (r & 3);
            if (key >= nv) sc[t][r] = -INFINITY;
          }
        }
      }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int t = 0; t < SUB; ++t) {
      if (t >= nsub) break;
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sc[t][r]);
    }
    mx = half_pair_max(mx) * scale_log2;
    const float m_new = fmaxf(st.m, mx);
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    float ps = 0.f;
#pragma unroll
    for (int t = 0; t < SUB; ++t) {
      if (t >= nsub) break;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        sc[t][r] = fast_exp2(__builtin_fmaf(sc[t][r], scale_log2, -m_use));
        ps += sc[t][r];
      }
    }
    ps = half_pair_sum(ps);
    if (__ballot(m_new > st.m) != 0) {
      const float alpha = fast_exp2(st.m - m_use);
      st.l *= alpha;
#pragma unroll
      for (int b = 0; b < D / 32; ++b)
#pragma unroll
        for (int r = 0; r < 16; ++r) st.o[b][r] *= alpha;
    }
    st.l += ps;
    st.m = m_new;
    __builtin_amdgcn_sched_barrier(0);
    // value operand of k-step (t, s2), column block b: lane (16-lane group
    // g, index i) reads row key0 + i / 4 at logical columns 32 b + 16 (g % 2)
    // + 4 (i % 4); key0 = 32 (t0 + t) + 16 s2 + 4 h (+ 8 for the operand's
    // upper half) is a multiple of 4, so the row's swizzle is the lane's own
    // The unit of column block b is (4 b + u0) ^ sw = 4 (b ^ (sw / 4)) + u0
    // (sw a multiple of 4, u0 < 4), so the element offset of block b is the
    // lane's offset for block 0 XOR 32 b: one XOR per block and read pair,
    // and a single address register.
    const int tg = (lane >> 4) & 1, ti = lane & 15, vr = ti >> 2, vc4 = ti & 3;
    const int va = (4 * h + vr) * D + 4 * (vc4 & 1) + ((2 * tg + (vc4 >> 1)) ^ wide_vswz<D>(vr)) * 8;
#pragma unroll
    for (int t = 0; t < SUB; ++t) {
      if (t >= nsub) break;
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        const bf16x8 pb = cvt_bf16x8(sc[t], 8 * s2);
        const uint16_t* vk = &sm.v[(32 * (t0 + t) + 16 * s2) * D];
#pragma unroll
        for (int b = 0; b < D / 32; ++b) {
          const int vo = va ^ (32 * b);
          const u32x2 lo = lds_read_tr16(vk + vo);
          const u32x2 hi = lds_read_tr16(vk + 8 * D + vo);
          const bf16x8 av = __builtin_bit_cast(bf16x8, u32x4{lo[0], lo[1], hi[0], hi[1]});
          st.o[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, pb, st.o[b], 0, 0, 0);
        }
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  }
}

// Dot product of this lane's query half with an fp32 vector (dims
// 16s + 8h + 0..7); the caller adds the partner lane (l ^ 32).
template <int D>
__device__ __forceinline__ float wave_q_dot_half(const WaveAttn<D>& st, const float* vec) {
  const int h = (threadIdx.x & 63) >> 5;
  float acc = 0.f;
#pragma unroll
  for (int s = 0; s < D / 16; ++s) {
    const f32x4 a = *(const f32x4*)(vec + 16 * s + 8 * h);
    const f32x4 b = *(const f32x4*)(vec + 16 * s + 8 * h + 4);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      acc += (float)st.qf[s][e] * a[e];
      acc += (float)st.qf[s][e + 4] * b[e];
    }
  }
  return acc;
}

}  // namespace hsa
