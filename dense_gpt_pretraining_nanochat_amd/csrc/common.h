// Device-side helpers shared by the HIP kernels of the library: element types,
// 16-byte vector access, conversions and wavefront reductions for CDNA4
// (gfx950, 64-wide wavefronts).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nc {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

// ---- scalar conversions (round to nearest even, as the hardware does) ----
__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16 x) { return static_cast<float>(x); }
template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float x) { return static_cast<bf16>(x); }

// ---- 16-byte vectors of T: 8 bf16 or 4 float -----------------------------
template <typename T> struct Vec16;
template <> struct Vec16<bf16> {
  static constexpr int N = 8;
  typedef bf16x8 type;
};
template <> struct Vec16<float> {
  static constexpr int N = 4;
  typedef f32x4 type;
};

template <typename T>
__device__ __forceinline__ void load16_f32(const T* p, float* out) {
  typedef typename Vec16<T>::type V;
  V v = *reinterpret_cast<const V*>(p);
#pragma unroll
  for (int i = 0; i < Vec16<T>::N; ++i) out[i] = to_f32(v[i]);
}
template <typename T>
__device__ __forceinline__ void store16_f32(T* p, const float* in) {
  typedef typename Vec16<T>::type V;
  V v;
#pragma unroll
  for (int i = 0; i < Vec16<T>::N; ++i) v[i] = from_f32<T>(in[i]);
  *reinterpret_cast<V*>(p) = v;
}

// ---- wavefront reductions (all 64 lanes get the result) -------------------
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}
// reduce over the 4 lane groups of 16 (lanes l, l^16, l^32, l^48)
__device__ __forceinline__ float group4_sum(float v) {
  v += __shfl_xor(v, 16, kWave);
  v += __shfl_xor(v, 32, kWave);
  return v;
}
__device__ __forceinline__ float group4_max(float v) {
  v = fmaxf(v, __shfl_xor(v, 16, kWave));
  v = fmaxf(v, __shfl_xor(v, 32, kWave));
  return v;
}
// reduce over the 16 lanes of a lane group (lanes sharing l / 16)
__device__ __forceinline__ float lane16_sum(float v) {
#pragma unroll
  for (int o = 8; o >= 1; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

// sum over the 16 lanes of a DPP row (lanes sharing l / 16), in registers:
// rotations of the row by 8, 4, 2 and 1 lanes (DPP row_ror, controls
// 0x128 / 0x124 / 0x122 / 0x121). Every lane gets the row's sum; lanes may
// differ in the last bit (each adds in its own order), so a caller stores the
// value of one fixed lane.
__device__ __forceinline__ float row16_sum(float v) {
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x128, 0xf, 0xf, false));
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x124, 0xf, 0xf, false));
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x122, 0xf, 0xf, false));
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x121, 0xf, 0xf, false));
  return v;
}

// Block-wide sum for blockDim.x threads (a multiple of 64, <= 1024); every
// thread gets the result. `red` must hold 16 floats of shared memory.
__device__ __forceinline__ float block_sum(float v, float* red) {
  v = wave_sum(v);
  const int w = threadIdx.x / kWave, nw = blockDim.x / kWave;
  __syncthreads();
  if ((threadIdx.x % kWave) == 0) red[w] = v;
  __syncthreads();
  float s = 0.f;
  for (int i = 0; i < nw; ++i) s += red[i];   // fixed order: deterministic
  return s;
}

// ---- device status bits ---------------------------------------------------
enum : uint32_t {
  kStatusTokenRange = 1u,      // a token id outside [0, V) was clamped
  kStatusTargetRange = 2u,     // a target id outside [0, V) was clamped
  kStatusNonFiniteLoss = 4u,   // the mean loss is not finite
};

}  // namespace nc
