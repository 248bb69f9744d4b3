// Parameter initialisation from a counter-based generator.
//
// The pages do not state an initialisation; the rule implemented here is:
// element i of the flat buffer gets std * N_i with N_i ~ N(0, 1), std = 0.02
// (divided by sqrt(2 * depth) on the attention and MLP output projections, as
// the workload descriptions ask), padding is 0. N_i is the Box-Muller
// transform (Box and Muller, 1958) of SplitMix64 outputs 2i and 2i+1
// (Steele, Lea and Flood, OOPSLA 2014) for the user seed, in float64:
//   u1 = ((z >> 11) + 1) * 2^-53,  u2 = (z' >> 11) * 2^-53,
//   N  = sqrt(-2 ln u1) * cos(2 pi u2);
// the float64 product std * N is rounded to float32, then to bf16 in bf16
// mode (round to nearest even both times). Every element is a pure function
// of (seed, index), so the result does not depend on the launch shape.
#include <math.h>

#include "common.h"
#include "launch.h"

namespace nc {
namespace {

__device__ __forceinline__ uint64_t splitmix64_out(uint64_t seed, uint64_t n) {
  uint64_t z = seed + (n + 1) * 0x9E3779B97F4A7C15ull;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

template <typename T>
__global__ void init_kernel(T* __restrict__ out, uint64_t seed, size_t begin, size_t end,
                            double std) {
  const double two_pi = 2.0 * 3.141592653589793;
  for (size_t i = begin + blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < end;
       i += (size_t)gridDim.x * blockDim.x) {
    const uint64_t z1 = splitmix64_out(seed, 2 * (uint64_t)i);
    const uint64_t z2 = splitmix64_out(seed, 2 * (uint64_t)i + 1);
    const double u1 = ((double)(z1 >> 11) + 1.0) * 0x1p-53;
    const double u2 = (double)(z2 >> 11) * 0x1p-53;
    const double n = sqrt(-2.0 * log(u1)) * cos(two_pi * u2);
    out[i] = from_f32<T>((float)(std * n));
  }
}

}  // namespace

hipError_t init_params(DType t, uint64_t seed, const InitSeg* segs, int nseg, size_t total,
                       void* params, hipStream_t s) {
  const size_t esz = t == DType::BF16 ? 2 : 4;
  hipError_t e = fill_zero(params, total * esz, s);     // padding
  if (e != hipSuccess) return e;
  for (int k = 0; k < nseg; ++k) {
    const size_t n = segs[k].end - segs[k].begin;
    if (n == 0) continue;
    const size_t want = (n + 255) / 256;
    const int grid = (int)(want < 16384 ? want : 16384);
    if (t == DType::BF16)
      hipLaunchKernelGGL(init_kernel<bf16>, dim3(grid), dim3(256), 0, s, static_cast<bf16*>(params),
                         seed, segs[k].begin, segs[k].end, segs[k].std);
    else
      hipLaunchKernelGGL(init_kernel<float>, dim3(grid), dim3(256), 0, s, static_cast<float*>(params),
                         seed, segs[k].begin, segs[k].end, segs[k].std);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace nc
