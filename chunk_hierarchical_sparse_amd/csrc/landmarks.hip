// landmarks.hip - landmark pooling: one fp32 vector per chunk, the sum of the
// chunk's S keys divided by sqrt(S) ([HSA] Methodology, landmark per chunk;
// sqrt-scaled mean pooling as in [DHSA] Eq. 4).
//
// Pure stream: K is read once, coalesced; the output is 1/S of the input.
// One 256-thread block per chunk: threads split the columns into 16-byte
// groups and the S rows into 256/(d/VEC) interleaved row sets, then reduce
// the row sets through LDS.
#include "hsa_common.h"
#include "kernels.h"

namespace hsa {

HSA_DCHECK_SOURCE()
namespace {

constexpr int kThreads = 256;

template <int DT>
__global__ void __launch_bounds__(kThreads)
    landmark_kernel(const void* __restrict__ K, float* __restrict__ lmk, int64_t slab_tokens,
                    int64_t lmk_chunks, int d, int S, int64_t c0, int64_t nchunks) {
  constexpr int VEC = DT == kF32 ? 4 : 8;  // elements per 16-byte load
  extern __shared__ float red[];           // [row_sets][d]
  const int64_t blk = blockIdx.x;
  const int64_t bh = blk / nchunks;
  const int64_t c = c0 + blk % nchunks;
  const int groups = d / VEC;
  const int row_sets = kThreads / groups;
  const int cg = threadIdx.x % groups;
  const int rs = threadIdx.x / groups;

  float acc[VEC];
#pragma unroll
  for (int v = 0; v < VEC; ++v) acc[v] = 0.f;

  const int64_t row0 = bh * slab_tokens + c * (int64_t)S;
  HSA_DCHECK(c < lmk_chunks && (c + 1) * S <= slab_tokens);
#pragma unroll 4
  for (int j = rs; j < S; j += row_sets) {
    const int64_t off = (row0 + j) * d + cg * VEC;
    if (DT == kF32) {
      const f32x4 x = *(const f32x4*)((const float*)K + off);
#pragma unroll
      for (int v = 0; v < 4; ++v) acc[v] += x[v];
    } else {
      const u32x4 x = *(const u32x4*)((const uint16_t*)K + off);
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        acc[2 * v] += bf16_bits_to_f32(x[v] & 0xffffu);
        acc[2 * v + 1] += bf16_bits_to_f32(x[v] >> 16);
      }
    }
  }
#pragma unroll
  for (int v = 0; v < VEC; ++v) red[rs * d + cg * VEC + v] = acc[v];
  __syncthreads();
  const float rsq = __fsqrt_rn((float)S);
  for (int x = threadIdx.x; x < d; x += kThreads) {
    float s = 0.f;
    for (int r = 0; r < row_sets; ++r) s += red[r * d + x];
    lmk[(bh * lmk_chunks + c) * d + x] = __fdiv_rn(s, rsq);
  }
}

}  // namespace

hipError_t launch_landmarks(const void* K, int dtype, float* lmk, int64_t BH, int64_t slab_tokens,
                            int64_t lmk_chunks, int d, int S, int64_t c0, int64_t c1,
                            hipStream_t stream) {
  const int64_t nchunks = c1 - c0;
  if (nchunks <= 0 || BH <= 0) return hipSuccess;
  const int64_t blocks = BH * nchunks;
  const int VEC = dtype == kF32 ? 4 : 8;
  const size_t lds = (size_t)(kThreads / (d / VEC)) * d * sizeof(float);
  if (dtype == kF32)
    launch<landmark_kernel<kF32>>(dim3((unsigned)blocks), dim3(kThreads), lds, stream, K, lmk,
                                  slab_tokens, lmk_chunks, d, S, c0, nchunks);
  else
    launch<landmark_kernel<kBF16>>(dim3((unsigned)blocks), dim3(kThreads), lds, stream, K, lmk,
                                   slab_tokens, lmk_chunks, d, S, c0, nchunks);
  return hipGetLastError();
}

namespace {
__global__ void fill_i32_kernel(int32_t* p, int64_t n, int32_t value) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x)
    p[i] = value;
}

// One thread checks that `fail` is zero: the debug library's self-test of
// the device-check path (no memory is touched either way).
__global__ void check_selftest_kernel(int fail) {
  if (threadIdx.x == 0) HSA_DCHECK(fail == 0);
}
}  // namespace

hipError_t launch_check_selftest(int fail, hipStream_t stream) {
  launch<check_selftest_kernel>(dim3(1), dim3(64), 0, stream, fail);
  return hipGetLastError();
}

hipError_t launch_fill_i32(int32_t* p, int64_t n, int32_t value, hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  int64_t blocks = (n + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  launch<fill_i32_kernel>(dim3((unsigned)blocks), dim3(256), 0, stream, p, n, value);
  return hipGetLastError();
}

}  // namespace hsa
