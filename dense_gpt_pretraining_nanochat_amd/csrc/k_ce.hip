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
// (4 bytes per logit in bf16 mode). The gradient may be written in place over
// the logits: every read of the row happens before the row's reduction
// barrier (the target's logit reaches the other threads through LDS), every
// write after it.
//
// Per logit the capped value comes from one base-2 exponential and one
// hardware reciprocal (see capped_unit), the shifted softmax numerator from a
// second exponential: because |z| <= c, exp(z - c) never overflows and needs
// no running maximum. With e = exp(-2|l|/c) and r = 1/(1+e), the softcap's
// derivative is 1 - (z/c)^2 = 4 e r^2, so the first pass also forms
// q = exp(z - c) e r^2 and keeps it, in the activation type, in the registers
// the raw logit occupied; the gradient pass is then one multiply per logit,
// dl = (4 w / sum) q, plus an fp32 correction of the target's element. This
// keeps the kernel's arithmetic (three transcendentals and about a dozen other
// operations per logit) below its memory traffic.
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
// GRAD: also write the logit gradient (dl may equal logits).
template <typename T, int CB, bool GRAD>
__global__ __launch_bounds__(kCeThreads, sizeof(T) == 2 && CB == 16 ? 8 : 4) void softcap_ce_kernel(
    const T* logits, const int32_t* __restrict__ tgt, int V, int nch, float cap, float w0,
    float* __restrict__ loss_rows, T* dl, uint32_t* status, const float* __restrict__ rs) {
  constexpr int E = CB / (int)sizeof(T);                       // logits per chunk
  constexpr int NCH = kCeMaxV / (kCeThreads * E);              // chunks per thread, at most
  typedef T TV __attribute__((ext_vector_type(E)));
  __shared__ float red[16];
  __shared__ float lt_s;                          // the target's logit
  const int row = blockIdx.x;
  const int tid = threadIdx.x, nt = blockDim.x;
  // the final RMSNorm's row scale, folded into the lm_head, carried by the gradient
  const float w = (GRAD && rs) ? w0 * rs[row] : w0;
  const T* src = logits + (size_t)row * V;
  const CapConsts q = {-2.0f * 1.44269504088896341f / cap, cap * 1.44269504088896341f};

  int t = tgt[row];
  const bool bad = t < 0 || t >= V;
  t = t < 0 ? 0 : (t >= V ? V - 1 : t);

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
      // the chunk holding the target hands its logit over through LDS (no
      // thread reads the row from memory after the barrier below)
      if ((unsigned)(t - c) < (unsigned)E) {
#pragma unroll
        for (int e = 0; e < E; ++e)
          if (c + e == t) lt_s = to_f32(raw[i][e]);
      }
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const float l = to_f32(raw[i][e]);
        const float u = __builtin_amdgcn_exp2f(q.k1 * fabsf(l));
        const float r = __builtin_amdgcn_rcpf(1.0f + u);
        const float ur = u * r;                   // (1 - u) r = r - u r
        const float ez = shifted_exp(copysignf(r - ur, l), q);
        se += ez;
        if constexpr (GRAD) raw[i][e] = from_f32<T>((ez * ur) * r);
      }
    }
  }
  const float sum = block_sum(se, red);           // barrier: the row has been read
  const float inv_sum = 1.0f / sum;
  const float tct = capped_unit(lt_s, q);
  if (tid == 0) {
    if (bad) atomicOr(status, kStatusTargetRange);
    loss_rows[row] = cap + logf(sum) - cap * tct;
  }
  if constexpr (GRAD) {
    T* dst = dl + (size_t)row * V;
    const float sc = 4.0f * w * inv_sum;
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int c = (i * nt + tid) * E;
      if (i < nch && c < V) {
        TV v;
#pragma unroll
        for (int e = 0; e < E; ++e) v[e] = from_f32<T>(sc * to_f32(raw[i][e]));
        if (t >= c && t < c + E) {
          // the target's element, w (p - 1) (1 - (z/c)^2), from the fp32 logit
          const float gt = w * fmaf(shifted_exp(tct, q), inv_sum, -1.0f) * fmaf(-tct, tct, 1.0f);
#pragma unroll
          for (int e = 0; e < E; ++e)
            if (c + e == t) v[e] = from_f32<T>(gt);
        }
        *reinterpret_cast<TV*>(dst + c) = v;
      }
    }
  }
}

template <typename T, int CB>
hipError_t launch_ce(const void* logits, const int32_t* tgt, int R, int V, float cap, float w,
                     float* loss_rows, void* dlogits, uint32_t* status, const float* rs, hipStream_t s) {
  constexpr int E = CB / (int)sizeof(T);
  int nt = ((V / E + 63) / 64) * 64;
  if (nt > kCeThreads) nt = kCeThreads;
  const int nch = (V + E * nt - 1) / (E * nt);
  if (nch > kCeMaxV / (kCeThreads * E)) return hipErrorInvalidValue;
  if (dlogits)
    hipLaunchKernelGGL((softcap_ce_kernel<T, CB, true>), dim3(R), dim3(nt), 0, s,
                       static_cast<const T*>(logits), tgt, V, nch, cap, w, loss_rows,
                       static_cast<T*>(dlogits), status, rs);
  else
    hipLaunchKernelGGL((softcap_ce_kernel<T, CB, false>), dim3(R), dim3(nt), 0, s,
                       static_cast<const T*>(logits), tgt, V, nch, cap, w, loss_rows,
                       static_cast<T*>(nullptr), status, rs);
  return hipGetLastError();
}

}  // namespace

hipError_t softcap_ce(DType t, const void* logits, const int32_t* tgt, int R, int V, float cap,
                      float w, float* loss_rows, void* dlogits, uint32_t* status, hipStream_t s,
                      const float* rs) {
  if (V % 4 || V > kCeMaxV || V <= 0 || R <= 0) return hipErrorInvalidValue;
  if (t == DType::BF16) {
    if (V % 8 == 0)
      return launch_ce<bf16, 16>(logits, tgt, R, V, cap, w, loss_rows, dlogits, status, rs, s);
    return launch_ce<bf16, 8>(logits, tgt, R, V, cap, w, loss_rows, dlogits, status, rs, s);
  }
  return launch_ce<float, 16>(logits, tgt, R, V, cap, w, loss_rows, dlogits, status, rs, s);
}

}  // namespace nc
