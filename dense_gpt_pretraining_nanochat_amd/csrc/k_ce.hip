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
// other inter-kernel activation). One workgroup per row keeps the row's raw
// logits in registers (16-byte chunks: 32 registers per thread at V = 65,536
// in bf16), so each logit is read once from HBM and each gradient written once
// (4 bytes per logit in bf16 mode). The capped values are recomputed in the
// gradient pass instead of being kept in fp32: the kernel then fits in 64
// registers and two rows are in flight per compute unit, so one row's loads
// overlap another's reduction and stores. Because |z| <= c, exp(z - c) never
// overflows and needs no running maximum. tanh is evaluated from one
// exponential and a hardware reciprocal (see capped_unit) to keep the pass
// bound by memory rather than by arithmetic.
#include <math.h>

#include "common.h"
#include "launch.h"

namespace nc {
namespace {

constexpr int kCeThreads = 1024;
constexpr int kCeMaxV = 65536;

// Capped logit in units of the cap, t = tanh(l / c) = z / c, from one base-2
// exponential and one hardware reciprocal: tanh(x) = sign(x) (1 - e) / (1 + e)
// with e = exp(-2|x|) = exp2(k1 |l|), k1 = -2 log2(e) / c; e in (0, 1] so
// nothing overflows.
struct CapConsts {
  float k1;        // -2 log2(e) / c
  float k2;        // c log2(e): exp(z - c) = exp2(k2 t - k2)
};
__device__ __forceinline__ float capped_unit(float l, const CapConsts& q) {
  const float e = __builtin_amdgcn_exp2f(q.k1 * fabsf(l));
  return copysignf((1.0f - e) * __builtin_amdgcn_rcpf(1.0f + e), l);
}
// exp(z - c) for z = c t
__device__ __forceinline__ float shifted_exp(float t, const CapConsts& q) {
  return __builtin_amdgcn_exp2f(fmaf(q.k2, t, -q.k2));
}

// CB: bytes per chunk (16, or 8 when a bf16 row is only 8-byte aligned).
template <typename T, int CB>
__global__ __launch_bounds__(kCeThreads, sizeof(T) == 2 && CB == 16 ? 8 : 4) void softcap_ce_kernel(
    const T* __restrict__ logits, const int32_t* __restrict__ tgt, int V, int nch, float cap,
    float w, float* __restrict__ loss_rows, T* __restrict__ dl, uint32_t* status) {
  constexpr int E = CB / (int)sizeof(T);                       // logits per chunk
  constexpr int NCH = kCeMaxV / (kCeThreads * E);              // chunks per thread, at most
  typedef T TV __attribute__((ext_vector_type(E)));
  __shared__ float red[16];
  const int row = blockIdx.x;
  const int tid = threadIdx.x, nt = blockDim.x;
  const T* src = logits + (size_t)row * V;
  const CapConsts q = {-2.0f * 1.44269504088896341f / cap, cap * 1.44269504088896341f};

  // every chunk that starts inside the row is whole (V is a multiple of E)
  TV raw[NCH];
  float se = 0.f;
#pragma unroll
  for (int i = 0; i < NCH; ++i) {
    const int c = (i * nt + tid) * E;
    if (i < nch && c < V) raw[i] = *reinterpret_cast<const TV*>(src + c);
  }
#pragma unroll
  for (int i = 0; i < NCH; ++i) {
    const int c = (i * nt + tid) * E;
    if (i < nch && c < V) {
#pragma unroll
      for (int e = 0; e < E; ++e) se += shifted_exp(capped_unit(to_f32(raw[i][e]), q), q);
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
    const float zt = cap * capped_unit(to_f32(src[t]), q);
    loss_rows[row] = cap + logf(sum) - zt;
  }
  if (dl == nullptr) return;                       // loss only
  T* dst = dl + (size_t)row * V;
#pragma unroll
  for (int i = 0; i < NCH; ++i) {
    const int c = (i * nt + tid) * E;
    if (i < nch && c < V) {
      TV v;
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const float tc = capped_unit(to_f32(raw[i][e]), q);
        const float p = shifted_exp(tc, q) * inv_sum - (c + e == t ? 1.0f : 0.0f);
        v[e] = from_f32<T>(w * p * fmaf(-tc, tc, 1.0f));
      }
      *reinterpret_cast<TV*>(dst + c) = v;
    }
  }
}

template <typename T, int CB>
hipError_t launch_ce(const void* logits, const int32_t* tgt, int R, int V, float cap, float w,
                     float* loss_rows, void* dlogits, uint32_t* status, hipStream_t s) {
  constexpr int E = CB / (int)sizeof(T);
  int nt = ((V / E + 63) / 64) * 64;
  if (nt > kCeThreads) nt = kCeThreads;
  const int nch = (V + E * nt - 1) / (E * nt);
  if (nch > kCeMaxV / (kCeThreads * E)) return hipErrorInvalidValue;
  hipLaunchKernelGGL((softcap_ce_kernel<T, CB>), dim3(R), dim3(nt), 0, s,
                     static_cast<const T*>(logits), tgt, V, nch, cap, w, loss_rows,
                     static_cast<T*>(dlogits), status);
  return hipGetLastError();
}

}  // namespace

hipError_t softcap_ce(DType t, const void* logits, const int32_t* tgt, int R, int V, float cap,
                      float w, float* loss_rows, void* dlogits, uint32_t* status, hipStream_t s) {
  if (V % 4 || V > kCeMaxV || V <= 0 || R <= 0) return hipErrorInvalidValue;
  if (t == DType::BF16) {
    if (V % 8 == 0)
      return launch_ce<bf16, 16>(logits, tgt, R, V, cap, w, loss_rows, dlogits, status, s);
    return launch_ce<bf16, 8>(logits, tgt, R, V, cap, w, loss_rows, dlogits, status, s);
  }
  return launch_ce<float, 16>(logits, tgt, R, V, cap, w, loss_rows, dlogits, status, s);
}

}  // namespace nc
