// hsa_common.h - device helpers shared by the gfx950 kernels of libhsa_attn.
//
// Nothing here is shared with the CPU oracle.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels.h"

namespace hsa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint64_t u64x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

// The values of lanes l % 32 and 32 + l % 32 of x, in every lane l: one
// v_permlane32_swap of x with itself (no LDS round trip, no lane index).
__device__ __forceinline__ f32x2 lane_halves(float x) {
  const auto r =
      __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return f32x2{__uint_as_float(r[0]), __uint_as_float(r[1])};
}

// x[l] + x[l ^ 32] and max(x[l], x[l ^ 32]), in every lane (both lanes of a
// pair get the same bits: the sum is taken in one order for both).
__device__ __forceinline__ float half_pair_sum(float x) {
  const f32x2 h = lane_halves(x);
  return h[0] + h[1];
}
__device__ __forceinline__ float half_pair_max(float x) {
  const f32x2 h = lane_halves(x);
  return fmaxf(h[0], h[1]);
}

// The partner lane's (l ^ 32) value where lanes 0..31 offer lo_send and
// lanes 32..63 offer hi_send: lanes 0..31 receive hi_send of lane l + 32,
// lanes 32..63 receive lo_send of lane l - 32.
__device__ __forceinline__ uint32_t half_pair_exchange(uint32_t lo_send, uint32_t hi_send,
                                                       bool upper) {
  const auto a = __builtin_amdgcn_permlane32_swap(hi_send, hi_send, false, false);
  const auto b = __builtin_amdgcn_permlane32_swap(lo_send, lo_send, false, false);
  return upper ? b[0] : a[1];
}

// Every kernel of the library is launched through launch<Kernel>(grid,
// block, dynamic LDS bytes, stream, kernel arguments...), which prints the
// launch when HSA_ATTN_LOG is set (launch_log_enabled, kernels.h).
// HSA_DCHECK(cond): in the debug library a failed condition is counted, and
// the source line and a tag of the source file of the first failure are
// kept in this translation unit's own counters; the kernel carries on (no
// trap).  Every file with checks names itself once with HSA_DCHECK_SOURCE()
// so the tag maps back to its path.  The release library compiles both away.
constexpr uint32_t source_tag(const char* s, uint32_t h = 2166136261u) {  // FNV-1a
  return *s ? source_tag(s + 1, (h ^ (uint32_t)(unsigned char)*s) * 16777619u) : h;
}
#define HSA_DCHECK_CAT2(a, b) a##b
#define HSA_DCHECK_CAT(a, b) HSA_DCHECK_CAT2(a, b)
#if HSA_DEVICE_CHECKS
namespace {
__device__ uint32_t g_checks[3];  // failures, line of the first, its source tag
hipError_t read_checks(uint32_t counters[3]) {
  return hipMemcpyFromSymbol(counters, HIP_SYMBOL(g_checks), sizeof(g_checks));
}
hipError_t clear_checks() {
  const uint32_t zero[3] = {0u, 0u, 0u};
  return hipMemcpyToSymbol(HIP_SYMBOL(g_checks), zero, sizeof(zero));
}
const bool g_checks_registered = register_device_checks(read_checks, clear_checks);
}  // namespace
#define HSA_DCHECK(cond)                                            \
  do {                                                              \
    if (!(cond)) {                                                  \
      constexpr uint32_t tag_ = ::hsa::source_tag(__FILE__);        \
      if (atomicAdd(&::hsa::g_checks[0], 1u) == 0u) {               \
        ::hsa::g_checks[1] = __LINE__;                              \
        ::hsa::g_checks[2] = tag_;                                  \
      }                                                             \
    }                                                               \
  } while (0)
#define HSA_DCHECK_SOURCE()                                                       \
  namespace {                                                                     \
  const bool HSA_DCHECK_CAT(g_source_, __LINE__) =                                \
      ::hsa::register_check_source(::hsa::source_tag(__FILE__), __FILE__);        \
  }
#else
#define HSA_DCHECK(cond) \
  do {                   \
  } while (0)
#define HSA_DCHECK_SOURCE()
#endif

template <auto Kern, typename... Args>
inline void launch(dim3 grid, dim3 block, size_t lds, hipStream_t stream, const Args&... args) {
  if (launch_log_enabled()) log_launch((const void*)Kern, grid, block, lds, stream);
  Kern<<<grid, block, lds, stream>>>(args...);
}

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) {
  return __uint_as_float(b << 16);
}

// Round to nearest even; NaN stays NaN.
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  uint32_t b = __float_as_uint(f);
  if ((b & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((b >> 16) | 0x40u);
  b += 0x7fffu + ((b >> 16) & 1u);
  return (uint16_t)(b >> 16);
}

// Two floats -> packed bf16 pair (low half = a), round to nearest even
// (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  const bf16x2 v = {static_cast<__bf16>(a), static_cast<__bf16>(b)};
  return __builtin_bit_cast(uint32_t, v);
}

// Element i of an fp32 or bf16 array as float.
template <int DT>
__device__ __forceinline__ float load_elem(const void* p, int64_t i) {
  if (DT == kF32) return ((const float*)p)[i];
  return bf16_bits_to_f32(((const uint16_t*)p)[i]);
}

template <int DT>
__device__ __forceinline__ void store_elem(void* p, int64_t i, float v) {
  if (DT == kF32)
    ((float*)p)[i] = v;
  else
    ((uint16_t*)p)[i] = f32_to_bf16_bits(v);
}

// Order-preserving map of a float onto uint32 (larger float -> larger
// integer).  -0 is folded onto +0 so that equal scores tie exactly.
__device__ __forceinline__ uint32_t ordered_bits(float f) {
  f = f + 0.0f;
  uint32_t b = __float_as_uint(f);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

__device__ __forceinline__ float ordered_to_float(uint32_t o) {
  uint32_t b = (o & 0x80000000u) ? (o & 0x7fffffffu) : ~o;
  return __uint_as_float(b);
}

// 64-bit selection key: score first, then the lower index.  Distinct
// indices give distinct keys; 0 is below every real key.
__device__ __forceinline__ uint64_t select_key(float score, uint32_t idx) {
  return ((uint64_t)ordered_bits(score) << 32) | (uint64_t)(0xffffffffu - idx);
}

__device__ __forceinline__ uint32_t key_index(uint64_t key) {
  return 0xffffffffu - (uint32_t)key;
}

__device__ __forceinline__ float key_score(uint64_t key) {
  return ordered_to_float((uint32_t)(key >> 32));
}

template <typename T>
__device__ __forceinline__ T wave_max(T v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    T w = __shfl_xor(v, o, kWave);
    v = v > w ? v : w;
  }
  return v;
}

template <typename T>
__device__ __forceinline__ T wave_sum(T v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

// The value of lane (this lane ^ j), j a power of two below 64 known at
// compile time after unrolling.  j <= 8 stays in the lane's 16-lane row and
// goes through DPP moves: the quad permutations give j = 1, 2, and j = 4, 8
// compose two mirrors (lane ^ 3 then ^ 7, lane ^ 7 then ^ 15).  j = 16, 32
// cross rows and use the LDS permute.
__device__ __forceinline__ uint32_t lane_xor(uint32_t v, int j) {
  const int x = (int)v;
  if (j == 1) return (uint32_t)__builtin_amdgcn_mov_dpp(x, 0xB1, 0xF, 0xF, false);
  if (j == 2) return (uint32_t)__builtin_amdgcn_mov_dpp(x, 0x4E, 0xF, 0xF, false);
  if (j == 4)
    return (uint32_t)__builtin_amdgcn_mov_dpp(__builtin_amdgcn_mov_dpp(x, 0x1B, 0xF, 0xF, false),
                                              0x141, 0xF, 0xF, false);
  if (j == 8)
    return (uint32_t)__builtin_amdgcn_mov_dpp(__builtin_amdgcn_mov_dpp(x, 0x141, 0xF, 0xF, false),
                                              0x140, 0xF, 0xF, false);
  return (uint32_t)__shfl_xor(x, j, kWave);
}

__device__ __forceinline__ uint64_t lane_xor_u64(uint64_t v, int j) {
  return (uint64_t)lane_xor((uint32_t)v, j) | ((uint64_t)lane_xor((uint32_t)(v >> 32), j) << 32);
}

__device__ __forceinline__ float lane_xor_f32(float v, int j) {
  return __builtin_bit_cast(float, lane_xor(__builtin_bit_cast(uint32_t, v), j));
}

// Wave-wide maximum and sum: butterflies inside each 16-lane row, then the
// four row results read out of lanes 0, 16, 32, 48.
__device__ __forceinline__ float wave_max_f32(float v) {
#pragma unroll
  for (int j = 1; j < 16; j <<= 1) v = fmaxf(v, lane_xor_f32(v, j));
  const float a0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 0));
  const float a1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 16));
  const float a2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 32));
  const float a3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 48));
  return fmaxf(fmaxf(a0, a1), fmaxf(a2, a3));
}

__device__ __forceinline__ float wave_sum_f32(float v) {
#pragma unroll
  for (int j = 1; j < 16; j <<= 1) v += lane_xor_f32(v, j);
  const float a0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 0));
  const float a1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 16));
  const float a2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 32));
  const float a3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 48));
  return (a0 + a1) + (a2 + a3);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// x = hi + lo + lo2 exactly for finite fp32 x: three bf16 parts, each the
// round-to-nearest-even of what the previous ones leave.  Products of a
// bf16 value with each part are exact in fp32, so three bf16 MFMA products
// summed smallest first give an fp32-accurate dot product.
__device__ __forceinline__ void split3_bf16(float x, uint16_t& hi, uint16_t& lo, uint16_t& lo2) {
  const __bf16 h = static_cast<__bf16>(x);  // round to nearest even
  const float r1 = x - static_cast<float>(h);
  const __bf16 l = static_cast<__bf16>(r1);
  const float r2 = r1 - static_cast<float>(l);
  const __bf16 m = static_cast<__bf16>(r2);
  hi = __builtin_bit_cast(uint16_t, h);
  lo = __builtin_bit_cast(uint16_t, l);
  lo2 = __builtin_bit_cast(uint16_t, m);
}

// Block barrier ordering LDS accesses only: unlike __syncthreads(), global
// loads issued before it (prefetches) stay in flight across it.
__device__ __forceinline__ void block_sync_lds() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

}  // namespace hsa
