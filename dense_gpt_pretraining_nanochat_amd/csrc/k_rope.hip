// Rotary position embedding fused with QK-norm, forward and backward.
//
// Position enters only through rotary embeddings, and the query and key
// vectors are RMS-normalised (followin.io release article, architecture list).
// Convention used (the pages leave it open): half-split pairs (j, j + 64) of
// each 128-dim head vector are rotated by +theta, theta = t * base^(-2j/128),
// t the position inside the sequence; then the head vector is normalised by
// its RMS (the two steps commute exactly, rotation being orthogonal).
//
// One wavefront per head vector: lane j holds elements j and j + 64, so the
// rotation is lane-local and the norm is one shuffle-tree reduction.
// The kernels work in place on the fused [tokens, q heads | k | v] buffer.
#include "common.h"
#include "launch.h"

namespace nc {
namespace {

constexpr int kHalf = 64;   // head_dim / 2

__global__ void rope_table_kernel(int T, int half, double base, float* __restrict__ cs) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= T * half) return;
  const int t = i / half, j = i % half;
  const double inv_freq = pow(base, -2.0 * j / (2.0 * half));
  const double th = (double)t * inv_freq;
  cs[i] = (float)cos(th);
  cs[(size_t)T * half + i] = (float)sin(th);
}

template <typename T>
__global__ __launch_bounds__(256) void rope_qknorm_fwd_kernel(T* __restrict__ qkv, int ldq, int M,
                                                              int Tlen, int H,
                                                              const float* __restrict__ cs,
                                                              float eps,
                                                              float* __restrict__ rinv_qk) {
  const int lane = threadIdx.x & 63;
  const int w = blockIdx.x * 4 + (threadIdx.x >> 6);     // (token, head) pair
  const int nh = H + 1;
  if (w >= M * nh) return;
  const int m = w / nh, h = w % nh;
  const int t = m % Tlen;
  T* p = qkv + (size_t)m * ldq + h * 128;
  const float a = to_f32(p[lane]), b = to_f32(p[lane + kHalf]);
  const float c = cs[t * kHalf + lane], s = cs[(size_t)Tlen * kHalf + t * kHalf + lane];
  const float ra = a * c - b * s, rb = a * s + b * c;
  const float ss = wave_sum(ra * ra + rb * rb);
  const float r = 1.0f / sqrtf(ss * (1.0f / 128.0f) + eps);
  p[lane] = from_f32<T>(ra * r);
  p[lane + kHalf] = from_f32<T>(rb * r);
  if (lane == 0) rinv_qk[(size_t)m * nh + h] = r;
}

// dz' = r (dy - y mean(dy y)) with y the saved normalised vector, then rotate by -theta
template <typename T>
__global__ __launch_bounds__(256) void rope_qknorm_bwd_kernel(T* __restrict__ dqkv, int ldd,
                                                              const T* __restrict__ qkv, int ldq,
                                                              int M, int Tlen, int H,
                                                              const float* __restrict__ cs,
                                                              const float* __restrict__ rinv_qk) {
  const int lane = threadIdx.x & 63;
  const int w = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int nh = H + 1;
  if (w >= M * nh) return;
  const int m = w / nh, h = w % nh;
  const int t = m % Tlen;
  T* g = dqkv + (size_t)m * ldd + h * 128;
  const T* y = qkv + (size_t)m * ldq + h * 128;
  const float ga = to_f32(g[lane]), gb = to_f32(g[lane + kHalf]);
  const float ya = to_f32(y[lane]), yb = to_f32(y[lane + kHalf]);
  const float dot = wave_sum(ga * ya + gb * yb) * (1.0f / 128.0f);
  const float r = rinv_qk[(size_t)m * nh + h];
  const float da = r * (ga - ya * dot), db = r * (gb - yb * dot);
  const float c = cs[t * kHalf + lane], s = cs[(size_t)Tlen * kHalf + t * kHalf + lane];
  g[lane] = from_f32<T>(da * c + db * s);
  g[lane + kHalf] = from_f32<T>(-da * s + db * c);
}

}  // namespace

hipError_t rope_table(int T, int half, double base, float* cs, hipStream_t s) {
  const int n = T * half;
  hipLaunchKernelGGL(rope_table_kernel, dim3((n + 255) / 256), dim3(256), 0, s, T, half, base, cs);
  return hipGetLastError();
}

hipError_t rope_qknorm_fwd(DType t, void* qkv, int ldq, int M, int T, int H, const float* cs,
                           float eps, float* rinv_qk, hipStream_t s) {
  const int waves = M * (H + 1);
  dim3 grid((waves + 3) / 4), block(256);
  if (t == DType::BF16)
    hipLaunchKernelGGL(rope_qknorm_fwd_kernel<bf16>, grid, block, 0, s, static_cast<bf16*>(qkv), ldq,
                       M, T, H, cs, eps, rinv_qk);
  else
    hipLaunchKernelGGL(rope_qknorm_fwd_kernel<float>, grid, block, 0, s, static_cast<float*>(qkv),
                       ldq, M, T, H, cs, eps, rinv_qk);
  return hipGetLastError();
}

hipError_t rope_qknorm_bwd(DType t, void* dqkv, int ldd, const void* qkv, int ldq, int M, int T,
                           int H, const float* cs, const float* rinv_qk, hipStream_t s) {
  const int waves = M * (H + 1);
  dim3 grid((waves + 3) / 4), block(256);
  if (t == DType::BF16)
    hipLaunchKernelGGL(rope_qknorm_bwd_kernel<bf16>, grid, block, 0, s, static_cast<bf16*>(dqkv), ldd,
                       static_cast<const bf16*>(qkv), ldq, M, T, H, cs, rinv_qk);
  else
    hipLaunchKernelGGL(rope_qknorm_bwd_kernel<float>, grid, block, 0, s, static_cast<float*>(dqkv),
                       ldd, static_cast<const float*>(qkv), ldq, M, T, H, cs, rinv_qk);
  return hipGetLastError();
}

}  // namespace nc
