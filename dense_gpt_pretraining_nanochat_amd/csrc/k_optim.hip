// Optimizer step kernels: the global gradient norm and clip factor, AdamW for
// the embedding and lm_head, and the elementwise parts of Muon for the block
// matrices (momentum, normalisation, the Newton-Schulz linear combinations
// and the final update). Muon's matrix products run on the GEMM kernels.
//
// The pairing of Muon with AdamW follows the followin.io release article
// (paragraph after the architecture list); clipping by global norm, the
// wmrh.cn tutorial, section 5.1. The update rules themselves are the public
// descriptions of AdamW (decoupled weight decay, with Adam's bias correction)
// and of Muon (Nesterov momentum, then a quintic Newton-Schulz iteration
// X <- a X + (b A + c A^2) X with A = X X^T); the pages do not define them.
//
// Every reduction has a fixed grid and a fixed summation order, so a step is
// bitwise reproducible.
#include <math.h>

#include "common.h"
#include "launch.h"

namespace nc {
namespace {

constexpr int kOptThreads = 256;

// fp64 block sum (thread 0 holds the result)
__device__ __forceinline__ double block_sum_f64(double v, double* red) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  const int w = threadIdx.x >> 6, nw = blockDim.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  double s = 0.0;
  for (int i = 0; i < nw; ++i) s += red[i];
  return s;
}

// partial[r * gridDim.x + blockIdx.x] = sum of squares of this block's share
// of range r (grid-stride in fp64)
__global__ __launch_bounds__(kOptThreads) void sumsq_ranges_kernel(const float* __restrict__ x,
                                                                   OptRanges rg,
                                                                   double* __restrict__ partial) {
  __shared__ double red[kOptThreads / 64];
  const int r = blockIdx.y;
  const f32x4* p = reinterpret_cast<const f32x4*>(x + rg.off[r]);   // ranges are 16-byte aligned
  const size_t n4 = rg.cnt[r] / 4;                                    // and multiples of 4
  const size_t stride = (size_t)gridDim.x * kOptThreads;
  double s = 0.0;
  size_t i = blockIdx.x * (size_t)kOptThreads + threadIdx.x;
  for (; i + 3 * stride < n4; i += 4 * stride) {      // four 16-byte loads in flight
    f32x4 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) v[u] = p[i + u * stride];
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int e = 0; e < 4; ++e) s += (double)v[u][e] * v[u][e];
  }
  for (; i < n4; i += stride) {
    const f32x4 v = p[i];
#pragma unroll
    for (int e = 0; e < 4; ++e) s += (double)v[e] * v[e];
  }
  s = block_sum_f64(s, red);
  if (threadIdx.x == 0) partial[(size_t)r * gridDim.x + blockIdx.x] = s;
}

// norm_scale[0] = sqrt(sum of partials), norm_scale[1] = clip factor
__global__ __launch_bounds__(kOptThreads) void norm_finish_kernel(const double* __restrict__ partial,
                                                                  int n, float max_norm,
                                                                  float* __restrict__ norm_scale) {
  __shared__ double red[kOptThreads / 64];
  // fixed order: thread t sums t, t + 256, ...; then the block sum in wave order
  double s = 0.0;
  for (int i = threadIdx.x; i < n; i += kOptThreads) s += partial[i];
  s = block_sum_f64(s, red);
  if (threadIdx.x == 0) {
    const double norm = sqrt(s);
    norm_scale[0] = (float)norm;
    norm_scale[1] = max_norm > 0.f ? (float)fmin(1.0, (double)max_norm / (norm + 1e-6)) : 1.0f;
  }
}

template <typename T>
__global__ __launch_bounds__(kOptThreads) void adamw_kernel(T* __restrict__ p,
                                                            const float* __restrict__ g,
                                                            float* __restrict__ m,
                                                            float* __restrict__ v, size_t n,
                                                            AdamWArgs a,
                                                            const float* __restrict__ norm_scale) {
  const float s = norm_scale[1];
  for (size_t i = blockIdx.x * (size_t)kOptThreads + threadIdx.x; i < n;
       i += (size_t)gridDim.x * kOptThreads) {
    const float gi = g[i] * s;
    const float mi = a.beta1 * m[i] + (1.0f - a.beta1) * gi;
    const float vi = a.beta2 * v[i] + (1.0f - a.beta2) * gi * gi;
    m[i] = mi;
    v[i] = vi;
    const float mh = mi * a.bc1, vh = vi * a.bc2;
    const float pi = to_f32(p[i]) * a.decay - a.lr * mh / (sqrtf(vh) + a.eps);
    p[i] = from_f32<T>(pi);
  }
}

// Item y of a batch of matrices (gradient and momentum at stride `gs`, u
// packed): buf = mu buf + s g;  u = s g + mu buf;  partial[y][block] = the
// block's share of ||u||^2 (fp64)
__global__ __launch_bounds__(kOptThreads) void muon_momentum_kernel(
    const float* __restrict__ g, float* __restrict__ buf, size_t gs, float* __restrict__ u,
    size_t n, float mu, const float* __restrict__ norm_scale, double* __restrict__ partial) {
  __shared__ double red[kOptThreads / 64];
  const float s = norm_scale[1];
  const size_t y = blockIdx.y;
  const f32x4* gy = reinterpret_cast<const f32x4*>(g + y * gs);
  f32x4* by = reinterpret_cast<f32x4*>(buf + y * gs);
  f32x4* uy = reinterpret_cast<f32x4*>(u + y * n);
  double acc = 0.0;
  for (size_t i = blockIdx.x * (size_t)kOptThreads + threadIdx.x; i < n / 4;
       i += (size_t)gridDim.x * kOptThreads) {
    const f32x4 gi = gy[i] * s;
    const f32x4 bi = mu * by[i] + gi;
    by[i] = bi;
    const f32x4 ui = gi + mu * bi;
    uy[i] = ui;
#pragma unroll
    for (int e = 0; e < 4; ++e) acc += (double)ui[e] * ui[e];
  }
  acc = block_sum_f64(acc, red);
  if (threadIdx.x == 0) partial[y * gridDim.x + blockIdx.x] = acc;
}

// x = T(u / (||u||_F + 1e-7)), ||u|| from the momentum kernel's partials
template <typename T>
__global__ __launch_bounds__(kOptThreads) void muon_normalize_kernel(
    const float* __restrict__ u, size_t n, const double* __restrict__ partial, int nparts,
    T* __restrict__ x) {
  __shared__ double red[kOptThreads / 64];
  __shared__ float inv_s;
  const size_t y = blockIdx.y;                   // batch item: u, x packed, partials per item
  u += y * n;
  x += y * n;
  partial += y * nparts;
  double s = 0.0;
  for (int i = threadIdx.x; i < nparts; i += kOptThreads) s += partial[i];
  s = block_sum_f64(s, red);
  if (threadIdx.x == 0) inv_s = (float)(1.0 / (sqrt(s) + 1e-7));
  __syncthreads();
  const float inv = inv_s;
  for (size_t i = blockIdx.x * (size_t)kOptThreads + threadIdx.x; i < n;
       i += (size_t)gridDim.x * kOptThreads)
    x[i] = from_f32<T>(u[i] * inv);
}

// p = p * decay - coef * x  (x fp32 in the parameter's layout)
template <typename T>
__global__ __launch_bounds__(kOptThreads) void muon_update_kernel(T* __restrict__ p, size_t ps,
                                                                  const float* __restrict__ x,
                                                                  size_t n, float decay, float coef) {
  p += blockIdx.y * ps;                          // batch item: p at stride ps, x packed
  x += blockIdx.y * n;
  for (size_t i = blockIdx.x * (size_t)kOptThreads + threadIdx.x; i < n;
       i += (size_t)gridDim.x * kOptThreads)
    p[i] = from_f32<T>(to_f32(p[i]) * decay - coef * x[i]);
}

int grid_for(size_t n, int cap = 4096) {
  const size_t want = (n + kOptThreads - 1) / kOptThreads;
  return (int)(want < (size_t)cap ? (want > 0 ? want : 1) : cap);
}

}  // namespace

hipError_t grad_norm(const float* grads, const OptRanges& rg, double* partial, float max_norm,
                     float* norm_scale, hipStream_t s) {
  if (rg.n <= 0 || rg.n > kOptMaxRanges) return hipErrorInvalidValue;
  for (int i = 0; i < rg.n; ++i)
    if (rg.off[i] % 4 || rg.cnt[i] % 4) return hipErrorInvalidValue;
  hipLaunchKernelGGL(sumsq_ranges_kernel, dim3(kNormBlocksPerRange, rg.n), dim3(kOptThreads), 0, s,
                     grads, rg, partial);
  hipLaunchKernelGGL(norm_finish_kernel, dim3(1), dim3(kOptThreads), 0, s, partial,
                     rg.n * kNormBlocksPerRange, max_norm, norm_scale);
  return hipGetLastError();
}

hipError_t adamw(DType t, void* p, const float* g, float* m, float* v, size_t n, const AdamWArgs& a,
                 const float* norm_scale, hipStream_t s) {
  if (t == DType::BF16)
    hipLaunchKernelGGL(adamw_kernel<bf16>, dim3(grid_for(n)), dim3(kOptThreads), 0, s,
                       static_cast<bf16*>(p), g, m, v, n, a, norm_scale);
  else
    hipLaunchKernelGGL(adamw_kernel<float>, dim3(grid_for(n)), dim3(kOptThreads), 0, s,
                       static_cast<float*>(p), g, m, v, n, a, norm_scale);
  return hipGetLastError();
}

hipError_t muon_momentum(const float* g, float* buf, size_t gs, float* u, size_t n, int items,
                         float mu, const float* norm_scale, double* partial, hipStream_t s) {
  if (n % 4 || gs % 4 || items < 1) return hipErrorInvalidValue;
  hipLaunchKernelGGL(muon_momentum_kernel, dim3(kMuonParts, items), dim3(kOptThreads), 0, s, g, buf,
                     gs, u, n, mu, norm_scale, partial);
  return hipGetLastError();
}

hipError_t muon_normalize(DType t, const float* u, size_t n, int items, const double* partial,
                          void* x, hipStream_t s) {
  const dim3 grid(grid_for(n, 1024), items);
  if (t == DType::BF16)
    hipLaunchKernelGGL(muon_normalize_kernel<bf16>, grid, dim3(kOptThreads), 0, s, u, n, partial,
                       kMuonParts, static_cast<bf16*>(x));
  else
    hipLaunchKernelGGL(muon_normalize_kernel<float>, grid, dim3(kOptThreads), 0, s, u, n, partial,
                       kMuonParts, static_cast<float*>(x));
  return hipGetLastError();
}

hipError_t muon_update(DType t, void* p, size_t ps, const float* x, size_t n, int items, float decay,
                       float coef, hipStream_t s) {
  const dim3 grid(grid_for(n, 1024), items);
  if (t == DType::BF16)
    hipLaunchKernelGGL(muon_update_kernel<bf16>, grid, dim3(kOptThreads), 0, s,
                       static_cast<bf16*>(p), ps, x, n, decay, coef);
  else
    hipLaunchKernelGGL(muon_update_kernel<float>, grid, dim3(kOptThreads), 0, s,
                       static_cast<float*>(p), ps, x, n, decay, coef);
  return hipGetLastError();
}

}  // namespace nc
