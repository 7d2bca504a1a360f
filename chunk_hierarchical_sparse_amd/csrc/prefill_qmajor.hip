// prefill_qmajor.hip - HSA prefill with retrieval every R tokens, run query
// by query ([HSA] Key Contributions: the retrieval frequency; Main Findings:
// per-token against per-8-token retrieval).  The R tokens after a selection
// row share its chunks, so with R * G = 32 the rows of one selection row
// (R tokens x the G heads of the group) fill one 32-row MFMA tile, and the
// whole path after the selection runs in one wave with the fusion in
// registers ([HSA] Methodology in Plain English: attention inside each
// retrieved chunk, then the chunk outputs weighted by a softmax over the
// retrieval scores).  No per-chunk partial outputs are written and no
// separate fusion pass runs.
//
// Per wave (b, group, selection row r; rows t = rR .. rR + R - 1, heads of
// the group):
//  1. the retrieval scores s_k = q . lambda_k / sqrt(d) of all selected
//     chunks at once: the landmarks, split into three bf16 parts each
//     (split3_bf16, exact), are the rows of one MFMA tile against Q^T, so
//     s_k is fp32-accurate; w_k = softmax_k(s_k) before any chunk is read;
//  2. per chunk k: S^T = K Q^T with K read straight into the MFMA operand
//     registers (the next chunk's keys load while this one is finished),
//     the chunk's own softmax (max m, sum l), P scaled by w_k / l and
//     rounded to bf16, O^T += V^T P^T with V loaded into the wave's own LDS
//     buffer by buffer-to-LDS loads (row-major, swizzled) and its operand
//     taken by transposed LDS reads.  The sum over chunks is then the fused
//     output itself.
// The waves of a block are independent (no block barriers): two blocks of
// four waves share a CU, and the waves' loads overlap one another's work.
#include <math.h>

#include "attn_core.h"
#include "hsa_common.h"
#include "kernels.h"

namespace hsa {

HSA_DCHECK_SOURCE()
namespace {

constexpr int kWaves = 4;     // independent waves (selection rows) per block
constexpr int kMaxSlots = 8;  // three landmark parts per slot fill one 32-row tile

// Landmarks split into three bf16 parts: out[bg][c][p][d] for p = hi, lo, lo2.
__global__ void __launch_bounds__(256) split_landmarks_kernel(const float* __restrict__ lmk,
                                                              uint16_t* __restrict__ out,
                                                              int64_t rows, int d) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= rows * d) return;
  const int64_t row = i / d;
  const int dd = (int)(i % d);
  uint16_t hi, lo, lo2;
  split3_bf16(lmk[i], hi, lo, lo2);
  uint16_t* o = out + row * 3 * d + dd;
  o[0] = hi;
  o[d] = lo;
  o[2 * d] = lo2;
}

// Value of landmark-tile row j (0..31) from the accumulator registers of both
// lane halves: row 8 (r / 4) + 4 h + r % 4 sits in register r of half h.
template <int J>
__device__ __forceinline__ float tile_row(const float (&lo)[16], const float (&hi)[16]) {
  constexpr int h = (J >> 2) & 1;
  constexpr int r = 4 * (J >> 3) + (J & 3);
  return h ? hi[r] : lo[r];
}

template <int D>
__global__ void __launch_bounds__(64 * kWaves, 2) qmajor_kernel(PrefillArgs a,
                                                                const uint16_t* __restrict__ lsplit,
                                                                float sl2) {
  __shared__ __attribute__((aligned(16))) uint16_t vsm[kWaves][64 * D];  // one chunk's values
  // each lane's fusion weights, [slot][lane] per wave
  __shared__ float wsm[kWaves][kMaxSlots][64];
  const int lane = threadIdx.x & 63;
  // the wave index is uniform in a wave: in a scalar register, so are the
  // task, its (b, group) and every buffer base derived from them
  const int w = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int h = lane >> 5, i32 = lane & 31;
  const int64_t BG = (int64_t)a.B * a.Hkv;
  const int64_t task = (int64_t)blockIdx.x * kWaves + w;
  if (task >= BG * a.nq) return;  // the whole wave: no block barrier follows
  const int64_t bg = task / a.nq;
  const int64_t r = task % a.nq;
  const int G = a.Hq / a.Hkv;  // R * G == 32 (checked on the host)
  const int64_t b = bg / a.Hkv;
  const int hd = (int)(bg % a.Hkv) * G + i32 % G;
  const int64_t t0 = r * a.interval;
  const int64_t t = t0 + i32 / G;
  const bool valid = t < a.L;
  // chunks available at t0 and selected there (slots past m hold -1)
  const int m = (int)min((int64_t)a.topk, min(t0 / a.S, a.n));
  const int32_t* selp = a.idx + (bg * a.nq + r) * a.topk;
  const int64_t qrow = (b * a.Hq + hd) * a.L + min(t, a.L - 1);
  WaveAttn<D> st;
  wave_attn_init<D>(st, (const uint16_t*)a.Q + qrow * D, valid);

  // --- 1. retrieval scores and fusion weights -----------------------------
  float wk[kMaxSlots];
#pragma unroll
  for (int k = 0; k < kMaxSlots; ++k) wk[k] = 0.f;
  if (m > 0) {
    // tile row j = 3 k + p: part p of the landmark of slot k (zero past 3m)
    const int j = i32, ks = j / 3, p = j % 3;
    const bool live = j < 3 * m;
    const int c = live ? selp[ks] : 0;
    HSA_DCHECK(!live || (c >= 0 && c < a.n));
    const uint16_t* lr = lsplit + ((bg * a.n + (live ? c : 0)) * 3 + p) * D + 8 * h;
    f32x16 acc = {};
#pragma unroll
    for (int s = 0; s < D / 16; ++s) {
      const u32x4 x = *(const u32x4*)(lr + 16 * s);
      const bf16x8 av = __builtin_bit_cast(bf16x8, live ? x : u32x4{0u, 0u, 0u, 0u});
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, st.qf[s], acc, 0, 0, 0);
    }
    // every lane gets both halves' rows
    float lo[16], hi[16];
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const f32x2 v = lane_halves(acc[q]);
      lo[q] = v[0];
      hi[q] = v[1];
    }
    float s2[kMaxSlots];
    // s = lo2 + lo + hi parts, smallest first; log2 domain with 1/sqrt(d)
#define HSA_QM_SLOT(K)                                                                    \
  s2[K] = K < m ? ((tile_row<3 * K + 2>(lo, hi) + tile_row<3 * K + 1>(lo, hi)) +        \
                   tile_row<3 * K>(lo, hi)) * sl2                                        \
                : -INFINITY;
    HSA_QM_SLOT(0)
    HSA_QM_SLOT(1)
    HSA_QM_SLOT(2)
    HSA_QM_SLOT(3)
    HSA_QM_SLOT(4)
    HSA_QM_SLOT(5)
    HSA_QM_SLOT(6)
    HSA_QM_SLOT(7)
#undef HSA_QM_SLOT
    float mx = s2[0];
#pragma unroll
    for (int k = 1; k < kMaxSlots; ++k) mx = fmaxf(mx, s2[k]);
    float z = 0.f;
#pragma unroll
    for (int k = 0; k < kMaxSlots; ++k) {
      wk[k] = k < m ? fast_exp2(s2[k] - mx) : 0.f;
      z += wk[k];
    }
    const float iz = 1.f / z;
#pragma unroll
    for (int k = 0; k < kMaxSlots; ++k) wk[k] *= iz;
  }
  // kept in LDS for the chunk loop and the end (registers are short there)
#pragma unroll
  for (int k = 0; k < kMaxSlots; ++k) wsm[w][k][lane] = wk[k];

  // --- 2. the chunks --------------------------------------------------------
  const uint16_t* Kb = (const uint16_t*)a.K + bg * a.L * D;
  const uint16_t* Vb = (const uint16_t*)a.V + bg * a.L * D;
  uint16_t* vs = vsm[w];
  const bool two = a.S > 32;  // keys 32..63 exist (uniform)
  const int S = a.S;
  const int cbytes = S * D * 2;  // one chunk of keys or values
  // keys of slot k as the A operands of S^T = K Q^T: sub-tile u, k-step s.
  // Raw buffer loads over the chunk: rows past it read as zero, and each
  // sub-tile's buffer starts at its first row (scalar registers), so every
  // load takes one lane offset plus an immediate.
  u32x4 kop[2][D / 16];
  const int koff = (i32 * D + 8 * h) * 2;
  auto fetch_k = [&](int c) {
    const char* kc = (const char*)(Kb + (int64_t)c * S * D);
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const __amdgpu_buffer_rsrc_t rs =
          buffer_range(kc + u * 32 * D * 2, max(cbytes - u * 32 * D * 2, 0));
#pragma unroll
      for (int s = 0; s < D / 16; ++s)
        kop[u][s] = __builtin_bit_cast(
            u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, koff + 32 * s, 0, 0));
    }
  };
  // Values: each chunk's rows go straight to the wave's LDS buffer by
  // buffer-to-LDS loads (no registers, no byte permutation), row-major with
  // the 16-byte units of row r XOR-swizzled by sw(r), so that the transposed
  // reads of the value operand (four rows x 32 bytes per 16 lanes) spread
  // over the banks.  Load i writes LDS bytes [1 KB i, 1 KB (i + 1)): lane p
  // lands at 16 p, i.e. row RPI i + p / NUNIT, unit p % NUNIT, and fetches
  // that unit's logical source (unit ^ sw(row)).
  constexpr int NUNIT = D / 8;          // 16-byte units of a row
  constexpr int RPI = 1024 / (2 * D);   // rows per 1 KB load
  constexpr int NLD = 64 / RPI;         // loads per 64-row chunk
  constexpr int SWM = NUNIT >= 16 ? 3 : 1;  // row bits that select the swizzle
  const int prow = lane / NUNIT;        // this lane's row within each load
  // RPI is a multiple of 4, so row & SWM = prow & SWM for every load
  const int vsrc = (prow * D + (((lane % NUNIT) ^ (4 * (prow & SWM))) * 8)) * 2;
  auto fetch_v = [&](int c) {
    const char* vc = (const char*)(Vb + (int64_t)c * S * D);
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
      const int ib = i * 1024;
      const __amdgpu_buffer_rsrc_t rs = buffer_range(vc + ib, max(cbytes - ib, 0));
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rs, (__attribute__((address_space(3))) void*)(vs + i * 512), 16, vsrc, 0, 0, 0);
    }
  };
  // transposed-read addresses of the value operand (see the loop): lane
  // (16-lane group g, index ti) reads row key0 + ti / 4, logical columns
  // 32 b + 16 (g % 2) + 4 (ti % 4), whose unit 4 b + 2 (g % 2) + (ti % 4) / 2
  // sits at that ^ 4 (row & SWM); key0 is a multiple of 4, so the swizzle is
  // the lane's own: one offset per column block b
  const int tg = (lane >> 4) & 1, ti = lane & 15, vr = ti >> 2, vc4 = ti & 3;
  int voffb[D / 32];
#pragma unroll
  for (int bb = 0; bb < D / 32; ++bb)
    voffb[bb] = (4 * h + vr) * D +
                ((4 * bb + 2 * tg + (vc4 >> 1)) ^ (4 * (vr & SWM))) * 8 + 4 * (vc4 & 1);
  int cnext = 0;
  if (m > 0) {
    cnext = __builtin_amdgcn_readfirstlane(selp[0]);
    HSA_DCHECK(cnext >= 0 && cnext < a.n);
    fetch_k(cnext);
  }
#pragma nounroll
  for (int k = 0; k < m; ++k) {
    const int c = cnext;
    const float wcur = wsm[w][k][lane];  // this slot's weight
    if (k + 1 < m) cnext = __builtin_amdgcn_readfirstlane(selp[k + 1]);
    HSA_DCHECK(k + 1 >= m || (cnext >= 0 && cnext < a.n));
    __builtin_amdgcn_sched_barrier(0);
    // this chunk's values (the last step's reads of the buffer have all
    // returned: their products were taken before the loop came round)
    fetch_v(c);
    __builtin_amdgcn_sched_barrier(0);
    f32x16 s0 = {}, s1 = {};
#pragma unroll
    for (int s = 0; s < D / 16; ++s) {
      s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, kop[0][s]),
                                                   st.qf[s], s0, 0, 0, 0);
      if (two)
        s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, kop[1][s]),
                                                     st.qf[s], s1, 0, 0, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
    // the next chunk's keys load while this one is finished
    if (k + 1 < m) fetch_k(cnext);
    __builtin_amdgcn_sched_barrier(0);
    // the chunk's own softmax (log2 domain), then P scaled by w_k / l
    float mx = -INFINITY;
    // key = 4 h + c_q (+ 32) with c_q = 8 (q / 4) + q % 4 a constant
    const int kr = S - 4 * h;
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const int cq = 8 * (q >> 2) + (q & 3);
      const float x0 = cq < kr ? s0[q] * sl2 : -INFINITY;
      const float x1 = cq + 32 < kr ? s1[q] * sl2 : -INFINITY;
      s0[q] = x0;
      s1[q] = x1;
      mx = fmaxf(mx, fmaxf(x0, x1));
    }
    mx = half_pair_max(mx);
    float ps = 0.f;
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      s0[q] = fast_exp2(s0[q] - mx);
      s1[q] = fast_exp2(s1[q] - mx);
      ps += s0[q] + s1[q];
    }
    ps = half_pair_sum(ps);
    const float beta = wcur / ps;
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      s0[q] *= beta;
      s1[q] *= beta;
    }
    bf16x8 pb4[4];
    pb4[0] = cvt_bf16x8(s0, 0);
    pb4[1] = cvt_bf16x8(s0, 8);
    pb4[2] = cvt_bf16x8(s1, 0);
    pb4[3] = cvt_bf16x8(s1, 8);
    __builtin_amdgcn_sched_barrier(0);
    // the values have landed once every load older than the key prefetch
    // has: at most the prefetch's 2 D / 16 loads may still be in flight
    // (vmcnt, with expcnt and lgkmcnt left at their maxima)
    if (k + 1 < m) {
      constexpr int N = 2 * (D / 16);
      __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
    } else {
      __builtin_amdgcn_s_waitcnt((7 << 4) | (15 << 8));  // vmcnt(0)
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      if (kt == 1 && !two) break;
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        const bf16x8 pb = pb4[2 * kt + s2];
        const int key0 = 32 * kt + 16 * s2;  // + 4 h (in voffb); + 8 for slots 4..7
#pragma unroll
        for (int bb = 0; bb < D / 32; ++bb) {
          const u32x2 lo = lds_read_tr16(vs + voffb[bb] + key0 * D);
          const u32x2 hi = lds_read_tr16(vs + voffb[bb] + (key0 + 8) * D);
          const u32x4 av = {lo[0], lo[1], hi[0], hi[1]};
          st.o[bb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, av), pb,
                                                             st.o[bb], 0, 0, 0);
        }
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  }

  // --- 3. the fused rows (the weights sum to one: no normalisation left) -----
  if (!valid) return;
  uint16_t* orow = (uint16_t*)a.O + qrow * D;
#pragma unroll
  for (int bb = 0; bb < D / 32; ++bb)
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const int dd = 32 * bb + 8 * q4 + 4 * h;
      const u32x2 v = {pack_bf16x2(st.o[bb][4 * q4], st.o[bb][4 * q4 + 1]),
                       pack_bf16x2(st.o[bb][4 * q4 + 2], st.o[bb][4 * q4 + 3])};
      *(u32x2*)(orow + dd) = v;
    }
  if (a.sel_w && h == 0) {
    float* wr = a.sel_w + qrow * a.topk;
#pragma unroll
    for (int k = 0; k < kMaxSlots; ++k)
      if (k < a.topk) wr[k] = wsm[w][k][lane];
    for (int k = kMaxSlots; k < a.topk; ++k) wr[k] = 0.f;
  }
}

}  // namespace

bool prefill_query_major(const PrefillArgs& a) {
  return a.dtype == kBF16 && a.interval > 1 && a.Hkv > 0 &&
         a.interval * (a.Hq / a.Hkv) == 32 && a.topk <= kMaxSlots && a.S <= 64 &&
         (a.d == 64 || a.d == 128) &&
         (int64_t)a.B * a.Hkv * a.nq < ((int64_t)1 << 31) * kWaves;  // one launch
}

size_t prefill_query_major_scratch(int64_t BHkv, int64_t n, int d) {
  return (size_t)BHkv * n * 3 * d * sizeof(uint16_t);
}

hipError_t prefill_attend_query_major(const PrefillArgs& a, void* scratch, hipStream_t stream) {
  const int64_t BG = (int64_t)a.B * a.Hkv;
  const int64_t tasks = BG * a.nq;
  if (tasks == 0) return hipSuccess;
  uint16_t* lsplit = (uint16_t*)scratch;
  const int64_t rows = BG * a.n;
  if (rows > 0)
    launch<split_landmarks_kernel>(dim3((unsigned)((rows * a.d + 255) / 256)), dim3(256), 0,
                                   stream, a.lmk, lsplit, rows, a.d);
  const float sl2 = 1.4426950408889634f / sqrtf((float)a.d);
  const dim3 grid((unsigned)((tasks + kWaves - 1) / kWaves)), block(64 * kWaves);
  if (a.d == 64)
    launch<qmajor_kernel<64>>(grid, block, 0, stream, a, (const uint16_t*)lsplit, sl2);
  else
    launch<qmajor_kernel<128>>(grid, block, 0, stream, a, (const uint16_t*)lsplit, sl2);
  return hipGetLastError();
}

}  // namespace hsa
