// synth_device.hip - device side of the seeded input generator (see
// synth_core.h).  Produces the same bits as synth_fill_normal() on the host,
// so a tensor too large to generate and upload from the host can be filled in
// place on the GPU while the CPU regenerates only the pieces it needs.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "synth_core.h"

namespace {

constexpr int kThreads = 256;

template <int DT>
__global__ void __launch_bounds__(kThreads)
    fill_normal_kernel(void* out, uint64_t first, uint64_t n, uint64_t seed, uint32_t tid,
                       double scale) {
  // One thread per Philox block of four elements.
  const uint64_t b0 = first >> 2;
  const uint64_t nb = ((first + n - 1) >> 2) - b0 + 1;
  const uint64_t stride = (uint64_t)gridDim.x * kThreads;
  for (uint64_t t = (uint64_t)blockIdx.x * kThreads + threadIdx.x; t < nb; t += stride) {
    const uint64_t b = b0 + t;
    double z[4];
    synth_normal4(seed, tid, b, z);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint64_t e = b * 4u + (uint64_t)j;
      if (e < first || e >= first + n) continue;
      const uint64_t i = e - first;
      const double v = scale * z[j];
      if (DT == 0)
        ((float*)out)[i] = (float)v;
      else
        ((uint16_t*)out)[i] = synth_f32_to_bf16((float)v);
    }
  }
}

}  // namespace

// dtype 0 = fp32, 1 = bf16.  `out` is device memory holding n elements.
// Returns 0, -1 for a bad argument, or the HIP error code of the launch.
extern "C" int synth_fill_normal_device(void* out, int dtype, uint64_t first, uint64_t n,
                                        uint64_t seed, uint32_t tid, double scale,
                                        hipStream_t stream) {
  if (n == 0) return 0;
  if (out == nullptr || (dtype != 0 && dtype != 1)) return -1;
  const uint64_t nb = ((first + n - 1) >> 2) - (first >> 2) + 1;
  uint64_t blocks = (nb + kThreads - 1) / kThreads;
  if (blocks > 65536) blocks = 65536;
  if (dtype == 0)
    fill_normal_kernel<0><<<dim3((unsigned)blocks), dim3(kThreads), 0, stream>>>(
        out, first, n, seed, tid, scale);
  else
    fill_normal_kernel<1><<<dim3((unsigned)blocks), dim3(kThreads), 0, stream>>>(
        out, first, n, seed, tid, scale);
  hipError_t e = hipGetLastError();
  return e == hipSuccess ? 0 : (int)e;
}
