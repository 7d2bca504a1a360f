// swa_core.h - the bf16 sliding-window prefill attention of the upper
// layers ([HSA] Methodology: upper layers pair local sliding-window
// self-attention, 512-token windows, with the HSA module) as a block-level
// device function: the sliding-window launch runs it for every block, and
// the upper layers' fused launch runs it for the blocks it gives to the
// window.  One block per (b, KV head, head block of GT query heads, 128/GT
// positions); each wave owns 32 positions of one head and the GT heads
// share the 128-key K/V blocks staged in LDS (the next block's loads in
// flight while the current one is computed).  Work units are dealt so that
// each XCD takes a contiguous run of positions: neighbouring windows overlap
// in its L2.
#pragma once

#include "attn_core.h"
#include "hsa_common.h"
#include "kernels.h"

namespace hsa {

HSA_DCHECK_SOURCE()

constexpr int kSwaXcds = 8;

template <int D, int GT>
__device__ __forceinline__ void swa_prefill_body(const SwaArgs& a, float scale_log2,
                                                 int64_t n_units, int64_t blk,
                                                 KVSmemWide<D>& sm) {
  constexpr int MQ = 32 * 4 / GT;  // positions per block
  // block i runs on XCD i % 8; XCD x takes units [x * per, (x + 1) * per)
  const int64_t per = (n_units + kSwaXcds - 1) / kSwaXcds;
  const int64_t unit = (blk % kSwaXcds) * per + blk / kSwaXcds;
  if (unit >= n_units) return;
  const int G = a.Hq / a.Hkv;
  const int64_t P = (a.L + MQ - 1) / MQ;
  const int64_t grp = unit / P;  // (b, g, head block)
  const int64_t t0 = (unit % P) * MQ;
  const int nhb = G / GT;
  const int64_t bg = grp / nhb;
  const int hb = (int)(grp % nhb);
  const int b = (int)(bg / a.Hkv), g = (int)(bg % a.Hkv);
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int h = g * G + hb * GT + w % GT;
  // positions in 32 bits (B * Hq * L < 2^31 is checked on the host); a
  // window reaching past the sequence start is the whole prefix
  const int Li = (int)a.L, W = (int)min(a.window, a.L);
  const int tb = (int)t0;
  const int t = tb + (w / GT) * 32 + (lane & 31);
  const bool valid = t < Li;
  const uint16_t* Kb = (const uint16_t*)a.K + bg * a.L * D;
  const uint16_t* Vb = (const uint16_t*)a.V + bg * a.L * D;
  WaveAttn<D> st;
  wave_attn_init<D>(st, (const uint16_t*)a.Q + (((int64_t)b * a.Hq + h) * a.L + min(t, Li - 1)) * D,
                    valid);
  const int t_end = min(Li, tb + MQ);
  const int k_lo = max(0, tb - W + 1);
  HSA_DCHECK(tb >= 0 && tb < Li && k_lo <= tb && t_end <= Li);
  KVRegsWide<D> rg;
  fetch_kv_wide<D>(rg, Kb + (int64_t)k_lo * D, Vb + (int64_t)k_lo * D,
                   min(kWideBlock, t_end - k_lo));
  for (int kb = k_lo; kb < t_end; kb += kWideBlock) {
    const int nk = min(kWideBlock, t_end - kb);
    __syncthreads();
    store_kv_wide<D>(sm, rg, nk);
    __syncthreads();
    const int nkb = kb + kWideBlock;
    if (nkb < t_end)
      fetch_kv_wide<D>(rg, Kb + (int64_t)nkb * D, Vb + (int64_t)nkb * D,
                       min(kWideBlock, t_end - nkb));
    __builtin_amdgcn_sched_barrier(0);
    // this lane's keys in the block: [lo, hi) in-block indices.  t - kb lies
    // in (-128, 2^31); lo = t - kb - (W - 1) clamped to [-1, 129], the
    // difference taken unsigned so the branch not chosen cannot overflow
    const int dk = t - kb;
    const int hi = valid ? min(nk, dk + 1) : 0;
    const int lo = dk >= W - 1 ? min(kWideBlock + 1, (int)((unsigned)dk - (unsigned)(W - 1))) : -1;
    if (__ballot(hi > 0 && hi > lo) != 0)
      wave_attn_wide<D, 4, true>(st, sm, nk, max(hi, 0), scale_log2, lo);
  }
  if (!valid) return;
  const float inv = st.l > 0.f ? 1.f / st.l : 0.f;
  uint16_t* orow = (uint16_t*)a.O + (((int64_t)b * a.Hq + h) * a.L + t) * D;
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

}  // namespace hsa
