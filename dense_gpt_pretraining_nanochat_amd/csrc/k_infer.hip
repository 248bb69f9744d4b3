// Inference with a KV cache: the prompt's forward fills the cache (prefill),
// then each decoding step runs one new token per sequence through the blocks
// and attends over the cached keys and values. The project's feature list
// names an inference engine with a KV cache and a simple prefill / decode flow
// (followin.io release article, section "花半天用 100 美元訓練的模型， 打敗了
// GPT-2"; vnrom.net, section "Cấu trúc thư mục và module chính"); the model is
// the training step's, so a decoded position gives the logits the
// full-sequence forward gives there (the mask is causal).
//
// Multi-query attention means one cached K/V head per layer serves every
// query head: a decoding workgroup stages 64 cached keys once and scores all
// H heads against them. Scores are bounded by sqrt(128) (QK-norm), so the
// softmax is shifted by the same fixed bound as in training and the chunk
// partials sum_u p v and sum_u p simply add; they are combined in chunk order
// (bitwise reproducible).
#include <math.h>

#include "common.h"
#include "launch.h"

namespace nc {
namespace {

constexpr int kKvW = 256;          // cached values per position: k-hat then v
constexpr int kKeyChunk = 64;      // keys per decoding workgroup
constexpr int kMaxHeads = 16;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kScoreMax2 = 17.0f;   // > sqrt(128) log2(e): exponents stay <= 0

template <typename T>
__global__ __launch_bounds__(256) void kv_store_kernel(const T* __restrict__ qkv, int ldq, int H,
                                                       int M, int Tseq, int pos0,
                                                       T* __restrict__ cache, int max_seq) {
  typedef typename Vec16<T>::type V;
  constexpr int E = Vec16<T>::N;            // elements per 16-byte chunk
  constexpr int C = kKvW / E;               // chunks per position
  const size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x;
  if (i >= (size_t)M * C) return;
  const int m = (int)(i / C), c = (int)(i % C);
  const int b = m / Tseq, t = m % Tseq;
  *reinterpret_cast<V*>(cache + ((size_t)b * max_seq + pos0 + t) * kKvW + c * E) =
      *reinterpret_cast<const V*>(qkv + (size_t)m * ldq + H * 128 + c * E);
}

// grid (B, chunks): partial sums of chunk `blockIdx.y` of row `blockIdx.x`
template <typename T>
__global__ __launch_bounds__(256) void decode_attn_partial_kernel(
    const T* __restrict__ qkv, int ldq, int H, const T* __restrict__ cache, int max_seq, int pos,
    float* __restrict__ part) {
  __shared__ float qs[kMaxHeads][128];
  __shared__ float ks[kKeyChunk][129];      // padded: score reads of 64 keys hit 64 banks
  __shared__ float vs[kKeyChunk][128];
  __shared__ float ps[kMaxHeads][kKeyChunk];
  const int b = blockIdx.x, ch = blockIdx.y, nch = gridDim.y;
  const int tid = threadIdx.x;
  const int u0 = ch * kKeyChunk;
  for (int i = tid; i < H * 128; i += 256) qs[i / 128][i % 128] = to_f32(qkv[(size_t)b * ldq + i]);
  const T* cb = cache + ((size_t)b * max_seq + u0) * kKvW;
  for (int i = tid; i < kKeyChunk * kKvW; i += 256) {
    const int k = i / kKvW, j = i % kKvW;
    const int kc = min(k, pos - u0);          // keys past pos: read the last valid one, then drop it
    const float raw = to_f32(cb[(size_t)kc * kKvW + j]);
    const float v = (u0 + k <= pos) ? raw : 0.f;
    if (j < 128) ks[k][j] = v;
    else vs[k][j - 128] = v;
  }
  __syncthreads();
  const float sc = kLog2e / sqrtf(128.0f);
  for (int i = tid; i < H * kKeyChunk; i += 256) {
    const int h = i / kKeyChunk, k = i % kKeyChunk;
    float sdot = 0.f;
#pragma unroll 8
    for (int j = 0; j < 128; ++j) sdot += qs[h][j] * ks[k][j];
    ps[h][k] = (u0 + k <= pos) ? exp2f(fmaf(sdot, sc, -kScoreMax2)) : 0.f;
  }
  __syncthreads();
  float* pb = part + ((size_t)b * nch + ch) * H * 129;
  for (int i = tid; i < H * 128; i += 256) {
    const int h = i / 128, dcol = i % 128;
    float acc = 0.f;
#pragma unroll 8
    for (int k = 0; k < kKeyChunk; ++k) acc += ps[h][k] * vs[k][dcol];
    pb[h * 129 + dcol] = acc;
  }
  if (tid < H) {
    float l = 0.f;
    for (int k = 0; k < kKeyChunk; ++k) l += ps[tid][k];
    pb[tid * 129 + 128] = l;
  }
}

template <typename T>
__global__ __launch_bounds__(256) void decode_attn_combine_kernel(const float* __restrict__ part,
                                                                  int nch, int H, T* __restrict__ o,
                                                                  int ldo) {
  const int b = blockIdx.x;
  for (int i = threadIdx.x; i < H * 128; i += 256) {
    const int h = i / 128, dcol = i % 128;
    float acc = 0.f, l = 0.f;
    for (int c = 0; c < nch; ++c) {
      const float* pb = part + ((size_t)b * nch + c) * H * 129 + h * 129;
      acc += pb[dcol];
      l += pb[128];
    }
    o[(size_t)b * ldo + i] = from_f32<T>(acc / l);
  }
}

template <typename T>
__global__ __launch_bounds__(256) void gather_last_rows_kernel(const T* __restrict__ src, int stride,
                                                               int rows, int rows_pad, int d,
                                                               T* __restrict__ dst) {
  const size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x;
  if (i >= (size_t)rows_pad * d) return;
  const int r = (int)(i / d), c = (int)(i % d);
  dst[i] = r < rows ? src[((size_t)(r + 1) * stride - 1) * d + c] : from_f32<T>(0.f);
}

__global__ __launch_bounds__(256) void softcap_rows_kernel(const float* __restrict__ in, size_t n,
                                                           float cap, float* __restrict__ out) {
  const float inv = 1.0f / cap;
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n;
       i += (size_t)gridDim.x * blockDim.x)
    out[i] = cap * tanhf(in[i] * inv);
}

}  // namespace

hipError_t kv_store(DType t, const void* qkv, int ldq, int H, int M, int Tseq, int pos0, void* cache,
                    int max_seq, hipStream_t s) {
  if (M <= 0 || Tseq <= 0 || pos0 < 0 || pos0 + Tseq > max_seq || M % Tseq) return hipErrorInvalidValue;
  const int per = kKvW / (t == DType::BF16 ? 8 : 4);
  const size_t n = (size_t)M * per;
  const dim3 grid((unsigned)((n + 255) / 256));
  if (t == DType::BF16)
    hipLaunchKernelGGL(kv_store_kernel<bf16>, grid, dim3(256), 0, s, static_cast<const bf16*>(qkv), ldq,
                       H, M, Tseq, pos0, static_cast<bf16*>(cache), max_seq);
  else
    hipLaunchKernelGGL(kv_store_kernel<float>, grid, dim3(256), 0, s, static_cast<const float*>(qkv),
                       ldq, H, M, Tseq, pos0, static_cast<float*>(cache), max_seq);
  return hipGetLastError();
}

hipError_t decode_attn(DType t, const void* qkv, int ldq, int B, int H, const void* cache,
                       int max_seq, int pos, float* part, void* o, int ldo, hipStream_t s) {
  if (B <= 0 || H < 1 || H > kMaxHeads || pos < 0 || pos >= max_seq) return hipErrorInvalidValue;
  const int nch = (pos + 1 + kKeyChunk - 1) / kKeyChunk;
  if (t == DType::BF16) {
    hipLaunchKernelGGL(decode_attn_partial_kernel<bf16>, dim3(B, nch), dim3(256), 0, s,
                       static_cast<const bf16*>(qkv), ldq, H, static_cast<const bf16*>(cache), max_seq,
                       pos, part);
    hipLaunchKernelGGL(decode_attn_combine_kernel<bf16>, dim3(B), dim3(256), 0, s, part, nch, H,
                       static_cast<bf16*>(o), ldo);
  } else {
    hipLaunchKernelGGL(decode_attn_partial_kernel<float>, dim3(B, nch), dim3(256), 0, s,
                       static_cast<const float*>(qkv), ldq, H, static_cast<const float*>(cache),
                       max_seq, pos, part);
    hipLaunchKernelGGL(decode_attn_combine_kernel<float>, dim3(B), dim3(256), 0, s, part, nch, H,
                       static_cast<float*>(o), ldo);
  }
  return hipGetLastError();
}

hipError_t gather_last_rows(DType t, const void* src, int stride, int rows, int rows_pad, int d,
                            void* dst, hipStream_t s) {
  const size_t n = (size_t)rows_pad * d;
  const dim3 grid((unsigned)((n + 255) / 256));
  if (t == DType::BF16)
    hipLaunchKernelGGL(gather_last_rows_kernel<bf16>, grid, dim3(256), 0, s,
                       static_cast<const bf16*>(src), stride, rows, rows_pad, d, static_cast<bf16*>(dst));
  else
    hipLaunchKernelGGL(gather_last_rows_kernel<float>, grid, dim3(256), 0, s,
                       static_cast<const float*>(src), stride, rows, rows_pad, d,
                       static_cast<float*>(dst));
  return hipGetLastError();
}

hipError_t softcap_rows(const float* in, int rows, int V, float cap, float* out, hipStream_t s) {
  const size_t n = (size_t)rows * V;
  const size_t want = (n + 255) / 256;
  hipLaunchKernelGGL(softcap_rows_kernel, dim3((unsigned)(want < 8192 ? want : 8192)), dim3(256), 0,
                     s, in, n, cap, out);
  return hipGetLastError();
}

}  // namespace nc
