// Out-of-place matrix transpose, out[c][r] = in[r][c], for 2- and 4-byte
// elements. Puts the contraction index of weight- and input-gradient products
// innermost, so every contraction of the step runs as one K-contiguous
// matrix-core kernel.
//
// 64x64 tiles through LDS: 16-byte coalesced loads along input rows, 16-byte
// coalesced stores along output rows; the LDS tile is padded by one 4-byte
// word per row so the column reads spread over the banks. Bandwidth-bound.
#include "common.h"
#include "launch.h"

namespace nc {
namespace {

constexpr int kTile = 64;

template <typename T>
__global__ __launch_bounds__(256) void transpose_kernel(const T* __restrict__ in, int R, int C,
                                                        int ld_in, T* __restrict__ out,
                                                        int ld_out) {
  constexpr int VEC = Vec16<T>::N;
  constexpr int CH = kTile / VEC;                       // 16-byte chunks per tile row
  constexpr int PAD = 4 / sizeof(T);                    // one 4-byte word
  typedef typename Vec16<T>::type V;
  __shared__ T tile[kTile][kTile + PAD];

  const int r0 = blockIdx.y * kTile, c0 = blockIdx.x * kTile;
  for (int i = threadIdx.x; i < kTile * CH; i += 256) {
    const int r = i / CH, c = (i % CH) * VEC;
    if (r0 + r < R && c0 + c < C) {
      const V v = *reinterpret_cast<const V*>(in + (size_t)(r0 + r) * ld_in + c0 + c);
#pragma unroll
      for (int e = 0; e < VEC; ++e) tile[r][c + e] = v[e];
    }
  }
  __syncthreads();
  for (int i = threadIdx.x; i < kTile * CH; i += 256) {
    const int c = i / CH, r = (i % CH) * VEC;         // output row c, columns r..r+VEC
    if (c0 + c < C && r0 + r < R) {
      V v;
#pragma unroll
      for (int e = 0; e < VEC; ++e) v[e] = tile[r + e][c];
      *reinterpret_cast<V*>(out + (size_t)(c0 + c) * ld_out + r0 + r) = v;
    }
  }
}

}  // namespace

hipError_t transpose(DType t, const void* in, int R, int C, int ld_in, void* out, int ld_out,
                     hipStream_t s) {
  const int vec = t == DType::BF16 ? 8 : 4;
  if (R <= 0 || C <= 0 || R % vec || C % vec || ld_in % vec || ld_out % vec)
    return hipErrorInvalidValue;
  dim3 grid((C + kTile - 1) / kTile, (R + kTile - 1) / kTile), block(256);
  if (t == DType::BF16)
    hipLaunchKernelGGL(transpose_kernel<bf16>, grid, block, 0, s, static_cast<const bf16*>(in), R, C,
                       ld_in, static_cast<bf16*>(out), ld_out);
  else
    hipLaunchKernelGGL(transpose_kernel<float>, grid, block, 0, s, static_cast<const float*>(in), R,
                       C, ld_in, static_cast<float*>(out), ld_out);
  return hipGetLastError();
}

}  // namespace nc
