// prefill_common.h - device helpers of the chunk-major prefill work list,
// shared by the forward (prefill.hip) and backward (prefill_bwd.hip)
// kernels: where a list entry's per-row values live and which chunk and
// entry range a block of the chunk-major launch covers.
#pragma once

#include "hsa_common.h"
#include "kernels.h"

namespace hsa {

HSA_DCHECK_SOURCE()

// Partial outputs and their retrieval scores share one row index, in list
// order: row (e * G + head of the group) for entry e of the (b, group)'s
// chunk lists.  A tile's rows are consecutive entries of one list, so the
// attention writes its partials as one contiguous run; the fusion finds a
// token's entries through entry_pos.
__device__ __forceinline__ int64_t partial_row(const PrefillArgs& a, int64_t bg, int64_t e,
                                               int hh) {
  const int G = a.Hq / a.Hkv;
  return (bg * a.L * a.topk + e) * G + hh;
}

// Locate this block's chunk and entry range.  Blocks interleave the (b,
// group) pairs (b, group = fastest index) and walk each pair's work units in
// chunk order, so the early, most-selected chunks start first.  Returns false
// for blocks past the last unit of their (b, group).
__device__ __forceinline__ bool locate_tile(const PrefillArgs& a, int64_t blk, int64_t& bg,
                                            int& c, int& e0, int& e1) {
  const int64_t BG = (int64_t)a.B * a.Hkv;
  bg = blk % BG;
  const int64_t tile = blk / BG;
  const int32_t* toff = a.tile_off + bg * (a.n + 1);
  if (tile >= toff[a.n]) return false;
  c = a.tile_chunk[bg * a.tiles_ub + tile];
  HSA_DCHECK(c >= 0 && c < a.n);
  const int32_t* offs = a.offs + bg * (a.n + 1);
  e0 = offs[c] + (int)(tile - toff[c]) * a.entries_per_tile;
  e1 = min(e0 + a.entries_per_tile, offs[c + 1]);
  HSA_DCHECK(e0 >= offs[c] && e0 < e1 && (int64_t)e1 <= a.L * a.topk);
  return true;
}

__device__ __forceinline__ bool locate_tile(const PrefillArgs& a, int64_t& bg, int& c, int& e0,
                                            int& e1) {
  return locate_tile(a, (int64_t)blockIdx.x, bg, c, e0, e1);
}

}  // namespace hsa
