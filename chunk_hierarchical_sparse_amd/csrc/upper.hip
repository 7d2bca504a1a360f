// upper.hip - the upper layers' two attentions of a sequence in one launch
// ([HSA] Methodology: the upper layers pair local sliding-window
// self-attention with the HSA module).  After HSA's selection and list
// building, one grid runs both the HSA chunk attention (chunk_attend.h,
// memory-bound: partial outputs and gathered query rows) and the
// sliding-window attention (swa_core.h, bound by MFMA issue and softmax
// arithmetic), so each role's blocks fill the time the other's wait.
//
// Block roles alternate by XCD round: block i runs on XCD i % 8, and its
// round i / 8 goes to HSA when even and to the window when odd (while both
// have blocks left), so every XCD gets both kinds and each role's i-th
// block still lands on XCD i % 8 -- which the window's unit mapping relies
// on.  The two roles share one LDS buffer (their own layouts in a union).
#include <math.h>

#include "chunk_attend.h"
#include "hsa_common.h"
#include "kernels.h"
#include "swa_core.h"

namespace hsa {
namespace {

template <int D, bool S64, int GT>
__global__ void __launch_bounds__(kChunkThreads, 2)
    upper_attend_kernel(PrefillArgs pa, SwaArgs sa, float scale_log2, float score_scale,
                        int64_t n_hsa8, int64_t n_swa_units, int64_t n_swa8) {
  union Smem {
    ChunkSmem<D> chunk;
    KVSmemWide<D> win;
  };
  __shared__ Smem sm;
  const int64_t idx = blockIdx.x;
  const int64_t xcd = idx & 7, round = idx >> 3;
  const int64_t pairs = min(n_hsa8, n_swa8) / 8;  // rounds of either kind while both last
  bool win;
  int64_t v;
  if (round < 2 * pairs) {
    win = (round & 1) != 0;
    v = (round >> 1) * 8 + xcd;
  } else {
    win = n_swa8 > n_hsa8;
    v = (pairs + (round - 2 * pairs)) * 8 + xcd;
  }
  if (win)
    swa_prefill_body<D, GT>(sa, scale_log2, n_swa_units, v, sm.win);
  else
    attend_chunk_body<D, S64>(pa, scale_log2, score_scale, v, sm.chunk);
}

int heads_per_swa_block(int G) { return G % 4 == 0 ? 4 : (G % 2 == 0 ? 2 : 1); }

template <int D, bool S64>
hipError_t launch_d(const PrefillArgs& pa, const SwaArgs& sa, hipStream_t stream) {
  const int G = sa.Hq / sa.Hkv;
  const int GT = heads_per_swa_block(G);
  const int MQ = 32 * 4 / GT;
  const int64_t n_swa_units = (int64_t)sa.B * sa.Hkv * (G / GT) * ((sa.L + MQ - 1) / MQ);
  const int64_t n_swa8 = (n_swa_units + 7) / 8 * 8;
  const int64_t n_hsa = pa.n > 0 ? (int64_t)pa.B * pa.Hkv * pa.tiles_ub : 0;
  const int64_t n_hsa8 = (n_hsa + 7) / 8 * 8;
  const float scale = 1.0f / sqrtf((float)D);
  const float sl2 = scale * 1.4426950408889634f;
  const dim3 grid((unsigned)(n_hsa8 + n_swa8)), block(kChunkThreads);
  if (GT == 4)
    launch<upper_attend_kernel<D, S64, 4>>(grid, block, 0, stream, pa, sa, sl2, scale, n_hsa8,
                                           n_swa_units, n_swa8);
  else if (GT == 2)
    launch<upper_attend_kernel<D, S64, 2>>(grid, block, 0, stream, pa, sa, sl2, scale, n_hsa8,
                                           n_swa_units, n_swa8);
  else
    launch<upper_attend_kernel<D, S64, 1>>(grid, block, 0, stream, pa, sa, sl2, scale, n_hsa8,
                                           n_swa_units, n_swa8);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_upper_attend(const PrefillArgs& pa, const SwaArgs& sa, hipStream_t stream) {
  if (pa.d == 64)
    return pa.S == kKeyBlock ? launch_d<64, true>(pa, sa, stream)
                             : launch_d<64, false>(pa, sa, stream);
  return pa.S == kKeyBlock ? launch_d<128, true>(pa, sa, stream)
                           : launch_d<128, false>(pa, sa, stream);
}

}  // namespace hsa
