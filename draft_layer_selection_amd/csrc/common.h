// Device-side helpers shared by the HIP kernels of the library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ks {

typedef __bf16 bf16;
typedef bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16 x) { return (float)x; }

template <class T>
__device__ __forceinline__ T from_f32(float x);
template <>
__device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <>
__device__ __forceinline__ bf16 from_f32<bf16>(float x) { return (bf16)x; }  // RNE

__device__ __forceinline__ float warp_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

__device__ __forceinline__ float warp_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

__device__ __forceinline__ float silu_f(float z) { return z / (1.0f + expf(-z)); }

// Map the hardware workgroup id onto a logical tile id so that consecutive logical tiles
// land on the same XCD (workgroups are dealt to the 8 XCDs round-robin by id).
__device__ __forceinline__ int xcd_tile(int bid, int per_xcd) {
  return (bid & 7) * per_xcd + (bid >> 3);
}

}  // namespace ks
