// Fused logit softcap + log-softmax + cross-entropy, forward and backward in
// one pass over a chunk of lm_head logits.
//
// Logits are capped as z = c * tanh(l / c) before the softmax (followin.io
// release article, architecture list: logit softcap; c = 15), and the loss is
// the next-token cross-entropy averaged over all positions (wmrh.cn tutorial,
// section 2.3). Per row:
//   lse     = log sum_v exp(z_v)
//   loss    = lse - z[target]
//   dl_v    = w * (softmax(z)_v - [v == target]) * (1 - (z_v / c)^2)
// with w = 1 / (number of positions in the batch).
//
// Logits arrive in the step's activation type (bf16 in bf16 mode, like every
// other inter-kernel activation). One workgroup per row holds the whole row in
// fp32 registers (up to 64 values per thread at V = 65,536), so each logit is
// read once from HBM and each gradient written once (4 bytes per logit in
// bf16 mode). Because
// |z| <= c, exp(z - c) never overflows and needs no running maximum. tanh is
// evaluated from one exponential (see tanh_fast) to keep the pass bound by
// memory rather than by transcendental throughput.
#include <math.h>

#include "common.h"
#include "launch.h"

namespace nc {
namespace {

constexpr int kMaxChunks = 16;   // float4 chunks per thread: 16 * 4 * 1024 = 65,536

// tanh(x) = sign(x) (1 - e) / (1 + e) with e = exp(-2|x|): one exponential and
// one reciprocal; e in (0, 1] so nothing overflows.
__device__ __forceinline__ float tanh_fast(float x) {
  const float e = __expf(-2.0f * fabsf(x));
  return copysignf((1.0f - e) * __frcp_rn(1.0f + e), x);
}

template <typename T>
__global__ __launch_bounds__(1024) void softcap_ce_kernel(const T* __restrict__ logits,
                                                          const int32_t* __restrict__ tgt, int V,
                                                          int nch, float cap, float w,
                                                          float* __restrict__ loss_rows,
                                                          T* __restrict__ dl,
                                                          uint32_t* status) {
  __shared__ float red[16];
  const int row = blockIdx.x;
  const int tid = threadIdx.x, nt = blockDim.x;
  const T* src = logits + (size_t)row * V;
  typedef T T4 __attribute__((ext_vector_type(4)));
  const float inv_cap = 1.0f / cap;

  // t = tanh(l / c) = z / c is kept per logit; exp(z - c) = exp(c (t - 1))
  f32x4 tz[kMaxChunks];
  float se = 0.f;
#pragma unroll
  for (int i = 0; i < kMaxChunks; ++i) {
    const int c = (i * nt + tid) * 4;
    if (i < nch && c < V) {
      const T4 l = *reinterpret_cast<const T4*>(src + c);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        tz[i][e] = tanh_fast(to_f32(l[e]) * inv_cap);
        se += __expf(cap * (tz[i][e] - 1.0f));
      }
    }
  }
  const float sum = block_sum(se, red);
  const float inv_sum = 1.0f / sum;
  int t = tgt[row];
  if (t < 0 || t >= V) {
    if (tid == 0) atomicOr(status, kStatusTargetRange);
    t = t < 0 ? 0 : V - 1;
  }
  if (tid == 0) {
    const float zt = cap * tanh_fast(to_f32(src[t]) * inv_cap);
    loss_rows[row] = cap + logf(sum) - zt;
  }
  if (dl == nullptr) return;                       // loss only
  T* dst = dl + (size_t)row * V;
#pragma unroll
  for (int i = 0; i < kMaxChunks; ++i) {
    const int c = (i * nt + tid) * 4;
    if (i < nch && c < V) {
      float g[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float tc = tz[i][e];
        const float p = __expf(cap * (tc - 1.0f)) * inv_sum - (c + e == t ? 1.0f : 0.0f);
        g[e] = w * p * (1.0f - tc * tc);
      }
      T4 v = {from_f32<T>(g[0]), from_f32<T>(g[1]), from_f32<T>(g[2]), from_f32<T>(g[3])};
      *reinterpret_cast<T4*>(dst + c) = v;
    }
  }
}

}  // namespace

hipError_t softcap_ce(DType t, const void* logits, const int32_t* tgt, int R, int V, float cap,
                      float w, float* loss_rows, void* dlogits, uint32_t* status, hipStream_t s) {
  if (V % 4 || V > 65536 || R <= 0) return hipErrorInvalidValue;
  int nt = ((V / 4 + 63) / 64) * 64;
  if (nt > 1024) nt = 1024;
  const int nch = (V + 4 * nt - 1) / (4 * nt);
  if (nch > kMaxChunks) return hipErrorInvalidValue;
  if (t == DType::BF16)
    hipLaunchKernelGGL(softcap_ce_kernel<bf16>, dim3(R), dim3(nt), 0, s, static_cast<const bf16*>(logits), tgt, V, nch, cap, w,
                       loss_rows, static_cast<bf16*>(dlogits), status);
  else
    hipLaunchKernelGGL(softcap_ce_kernel<float>, dim3(R), dim3(nt), 0, s, static_cast<const float*>(logits), tgt, V, nch, cap, w,
                       loss_rows, static_cast<float*>(dlogits), status);
  return hipGetLastError();
}

}  // namespace nc
