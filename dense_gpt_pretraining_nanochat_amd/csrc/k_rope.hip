// Rotary position embedding fused with QK-norm, forward and backward.
//
// Position enters only through rotary embeddings, and the query and key
// vectors are RMS-normalised (followin.io release article, architecture list).
// Convention used (the pages leave it open): half-split pairs (j, j + 64) of
// each 128-dim head vector are rotated by +theta, theta = t * base^(-2j/128),
// t the position inside the sequence; then the head vector is normalised by
// its RMS (the two steps commute exactly, rotation being orthogonal).
//
// Sixteen lanes per head vector, each holding four elements of either half, so
// the rotation is lane-local and the norm is a 16-lane shuffle reduction.
// The kernels work in place on the fused [tokens, q heads | k | v] buffer.
#include "common.h"
#include "launch.h"

namespace nc {
namespace {

constexpr int kHalf = 64;   // head_dim / 2

// rows t = 0..T-1 of the table hold position t0 + t
__global__ void rope_table_kernel(int T, int t0, int half, double base, float* __restrict__ cs) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= T * half) return;
  const int t = i / half, j = i % half;
  const double inv_freq = pow(base, -2.0 * j / (2.0 * half));
  const double th = (double)(t0 + t) * inv_freq;
  cs[i] = (float)cos(th);
  cs[(size_t)T * half + i] = (float)sin(th);
}

// 16 lanes per head vector: lane s holds elements 4s..4s+3 and 64+4s..64+4s+3,
// so every rotation pair (j, j+64) stays in one lane; a wavefront covers four
// head vectors with 8-byte accesses.
template <typename T>
struct Quad {
  typedef T T4 __attribute__((ext_vector_type(4)));
  __device__ __forceinline__ static void load(const T* p, float* o) {
    const T4 v = *reinterpret_cast<const T4*>(p);
    o[0] = to_f32(v[0]); o[1] = to_f32(v[1]); o[2] = to_f32(v[2]); o[3] = to_f32(v[3]);
  }
  __device__ __forceinline__ static void store(T* p, const float* o) {
    const T4 v = {from_f32<T>(o[0]), from_f32<T>(o[1]), from_f32<T>(o[2]), from_f32<T>(o[3])};
    *reinterpret_cast<T4*>(p) = v;
  }
};

template <typename T>
__global__ __launch_bounds__(256) void rope_qknorm_fwd_kernel(T* __restrict__ qkv, int ldq, int M,
                                                              int Tlen, int H,
                                                              const float* __restrict__ cs,
                                                              float eps,
                                                              float* __restrict__ rinv_qk,
                                                              T* __restrict__ cache, int max_seq,
                                                              int pos0) {
  const int sl = threadIdx.x & 15;
  const size_t w = (size_t)blockIdx.x * 16 + (threadIdx.x >> 4);   // (token, head) pair
  const int nh = H + 1;
  if (w >= (size_t)M * nh) return;                                  // whole 16-lane groups
  const size_t m = w / nh;
  const int h = (int)(w % nh);
  const int t = (int)(m % Tlen);
  T* p = qkv + m * ldq + h * 128 + 4 * sl;
  float a[4], b[4];
  Quad<T>::load(p, a);
  Quad<T>::load(p + kHalf, b);
  const f32x4 c = *reinterpret_cast<const f32x4*>(cs + t * kHalf + 4 * sl);
  const f32x4 sn = *reinterpret_cast<const f32x4*>(cs + (size_t)Tlen * kHalf + t * kHalf + 4 * sl);
  float ra[4], rb[4], ss = 0.f;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    ra[e] = a[e] * c[e] - b[e] * sn[e];
    rb[e] = a[e] * sn[e] + b[e] * c[e];
    ss += ra[e] * ra[e] + rb[e] * rb[e];
  }
  ss = lane16_sum(ss);
  const float r = 1.0f / sqrtf(ss * (1.0f / 128.0f) + eps);
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    ra[e] *= r;
    rb[e] *= r;
  }
  Quad<T>::store(p, ra);
  Quad<T>::store(p + kHalf, rb);
  if (rinv_qk && sl == 0) rinv_qk[m * nh + h] = r;
  if (cache && h == H) {
    // KV cache row of (sequence m / Tlen, position pos0 + t): k-hat, then v
    T* dst = cache + ((m / Tlen) * (size_t)max_seq + pos0 + t) * 256 + 4 * sl;
    Quad<T>::store(dst, ra);
    Quad<T>::store(dst + kHalf, rb);
    float v[4];
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      Quad<T>::load(p + 128 + half * kHalf, v);
      Quad<T>::store(dst + 128 + half * kHalf, v);
    }
  }
}

// dz' = r (dy - y mean(dy y)) with y the saved normalised vector, then rotate by -theta.
// RS: the result is then multiplied by rs[m] (the row scale of the RMSNorm folded
// into the QKV product; the attention backward applies it to the value gradient).
template <typename T, bool RS>
__global__ __launch_bounds__(256) void rope_qknorm_bwd_kernel(T* __restrict__ dqkv, int ldd,
                                                              const T* __restrict__ qkv, int ldq,
                                                              int M, int Tlen, int H,
                                                              const float* __restrict__ cs,
                                                              const float* __restrict__ rinv_qk,
                                                              const float* __restrict__ rs) {
  const int sl = threadIdx.x & 15;
  const size_t w = (size_t)blockIdx.x * 16 + (threadIdx.x >> 4);
  const int nh = H + 1;
  if (w >= (size_t)M * nh) return;
  const size_t m = w / nh;
  const int h = (int)(w % nh);
  const int t = (int)(m % Tlen);
  T* g = dqkv + m * ldd + h * 128 + 4 * sl;
  const T* y = qkv + m * ldq + h * 128 + 4 * sl;
  float ga[4], gb[4], ya[4], yb[4];
  Quad<T>::load(g, ga);
  Quad<T>::load(g + kHalf, gb);
  Quad<T>::load(y, ya);
  Quad<T>::load(y + kHalf, yb);
  float dot = 0.f;
#pragma unroll
  for (int e = 0; e < 4; ++e) dot += ga[e] * ya[e] + gb[e] * yb[e];
  dot = lane16_sum(dot) * (1.0f / 128.0f);
  const float r = rinv_qk[m * nh + h];
  const f32x4 c = *reinterpret_cast<const f32x4*>(cs + t * kHalf + 4 * sl);
  const f32x4 sn = *reinterpret_cast<const f32x4*>(cs + (size_t)Tlen * kHalf + t * kHalf + 4 * sl);
  float oa[4], ob[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const float da = r * (ga[e] - ya[e] * dot), db = r * (gb[e] - yb[e] * dot);
    oa[e] = da * c[e] + db * sn[e];
    ob[e] = -da * sn[e] + db * c[e];
  }
  if constexpr (RS) {
    const float f = rs[m];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      oa[e] *= f;
      ob[e] *= f;
    }
  }
  Quad<T>::store(g, oa);
  Quad<T>::store(g + kHalf, ob);
}

}  // namespace

hipError_t rope_table(int T, int half, double base, float* cs, hipStream_t s, int t0) {
  const int n = T * half;
  hipLaunchKernelGGL(rope_table_kernel, dim3((n + 255) / 256), dim3(256), 0, s, T, t0, half, base,
                     cs);
  return hipGetLastError();
}

hipError_t rope_qknorm_fwd(DType t, void* qkv, int ldq, int M, int T, int H, const float* cs,
                           float eps, float* rinv_qk, hipStream_t s, void* cache, int max_seq,
                           int pos0) {
  if (cache && (M % T || pos0 < 0 || pos0 + T > max_seq)) return hipErrorInvalidValue;
  const size_t vecs = (size_t)M * (H + 1);
  dim3 grid((unsigned)((vecs + 15) / 16)), block(256);
  if (t == DType::BF16)
    hipLaunchKernelGGL(rope_qknorm_fwd_kernel<bf16>, grid, block, 0, s, static_cast<bf16*>(qkv), ldq,
                       M, T, H, cs, eps, rinv_qk, static_cast<bf16*>(cache), max_seq, pos0);
  else
    hipLaunchKernelGGL(rope_qknorm_fwd_kernel<float>, grid, block, 0, s, static_cast<float*>(qkv),
                       ldq, M, T, H, cs, eps, rinv_qk, static_cast<float*>(cache), max_seq, pos0);
  return hipGetLastError();
}

template <typename T>
static void launch_rope_bwd(void* dqkv, int ldd, const void* qkv, int ldq, int M, int Tlen, int H,
                            const float* cs, const float* rinv_qk, const float* rs, hipStream_t s) {
  const size_t vecs = (size_t)M * (H + 1);
  dim3 grid((unsigned)((vecs + 15) / 16)), block(256);
  if (rs)
    hipLaunchKernelGGL((rope_qknorm_bwd_kernel<T, true>), grid, block, 0, s, static_cast<T*>(dqkv), ldd,
                       static_cast<const T*>(qkv), ldq, M, Tlen, H, cs, rinv_qk, rs);
  else
    hipLaunchKernelGGL((rope_qknorm_bwd_kernel<T, false>), grid, block, 0, s, static_cast<T*>(dqkv), ldd,
                       static_cast<const T*>(qkv), ldq, M, Tlen, H, cs, rinv_qk, rs);
}

hipError_t rope_qknorm_bwd(DType t, void* dqkv, int ldd, const void* qkv, int ldq, int M, int T,
                           int H, const float* cs, const float* rinv_qk, hipStream_t s, const float* rs) {
  if (t == DType::BF16) launch_rope_bwd<bf16>(dqkv, ldd, qkv, ldq, M, T, H, cs, rinv_qk, rs, s);
  else launch_rope_bwd<float>(dqkv, ldd, qkv, ldq, M, T, H, cs, rinv_qk, rs, s);
  return hipGetLastError();
}

}  // namespace nc
