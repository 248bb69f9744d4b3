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

// bf16 decoding attention on the matrix cores. grid (B, nwg): workgroup c
// takes the 64-key chunks c, c + nwg, ... up to pos. Per chunk each
// wavefront scores 16 keys against all heads (v_mfma_f32_16x16x32_bf16, the
// cached k-hat rows as the 16-row operand, the query heads as the 16-column
// one), writes its probabilities to LDS as P^T [head][key], and then
// multiplies P by two 16-column tiles of V over all 64 keys
// (v_mfma_f32_16x16x16_bf16, V staged transposed in LDS so both operands are
// key-contiguous). Heads past H and keys past pos carry probability 0; their
// cache reads are clamped to row pos, so every value read is finite.
__global__ __launch_bounds__(256) void decode_attn_mfma_kernel(const bf16* __restrict__ qkv, int ldq,
                                                               int H, const bf16* __restrict__ cache,
                                                               int max_seq, int pos,
                                                               float* __restrict__ part) {
  typedef short s16x4 __attribute__((ext_vector_type(4)));
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  constexpr int KR = 72;                       // LDS row: 64 keys + 16-byte pad
  __shared__ __align__(16) bf16 vt[128][KR];   // V^T of the chunk: [dcol][key]
  __shared__ __align__(16) bf16 pt[16][KR];    // P^T: [head][key]
  __shared__ float lsum[4][16];
  const int b = blockIdx.x, c0 = blockIdx.y, nwg = gridDim.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, lg = lane >> 4;
  const int nchunks = pos / kKeyChunk + 1;
  const float sc = kLog2e / sqrtf(128.0f);

  bf16x8 qf[4];
#pragma unroll
  for (int s = 0; s < 4; ++s)
    qf[s] = l16 < H ? *reinterpret_cast<const bf16x8*>(qkv + (size_t)b * ldq + l16 * 128 + 32 * s + 8 * lg)
                    : bf16x8{};
  f32x4 oacc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
  float lpart = 0.f;
  const bf16* cb = cache + (size_t)b * max_seq * kKvW;

  for (int ch = c0; ch < nchunks; ch += nwg) {
    const int u0 = ch * kKeyChunk;
    // V^T: thread takes keys 2kp, 2kp + 1 and dcol chunks cc, cc + 8
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int kp = tid & 31, cc = (tid >> 5) + 8 * j;
      const int k0 = min(u0 + 2 * kp, pos), k1 = min(u0 + 2 * kp + 1, pos);
      const bf16x8 v0 = *reinterpret_cast<const bf16x8*>(cb + (size_t)k0 * kKvW + 128 + 8 * cc);
      const bf16x8 v1 = *reinterpret_cast<const bf16x8*>(cb + (size_t)k1 * kKvW + 128 + 8 * cc);
#pragma unroll
      for (int e = 0; e < 8; ++e)
        *reinterpret_cast<bf16x2*>(&vt[8 * cc + e][2 * kp]) = bf16x2{v0[e], v1[e]};
    }
    // scores of keys u0 + 16 wave + (0..15) against heads 0..15
    const int krow = min(u0 + 16 * wave + l16, pos);
    f32x4 s4 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const bf16x8 kf = *reinterpret_cast<const bf16x8*>(cb + (size_t)krow * kKvW + 32 * s + 8 * lg);
      s4 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[s], s4, 0, 0, 0);
    }
    // lane holds key 16 wave + 4 lg + r for head l16
    float p[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int key = u0 + 16 * wave + 4 * lg + r;
      p[r] = (key <= pos && l16 < H) ? exp2f(fmaf(s4[r], sc, -kScoreMax2)) : 0.f;
      lpart += p[r];
    }
    *reinterpret_cast<bf16x4*>(&pt[l16][16 * wave + 4 * lg]) =
        bf16x4{(bf16)p[0], (bf16)p[1], (bf16)p[2], (bf16)p[3]};
    __syncthreads();
    // O[h][dcol] += P[h][key] V[key][dcol], dcol tiles 2 wave and 2 wave + 1
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
      const s16x4 a = *reinterpret_cast<const s16x4*>(&pt[l16][16 * kt + 4 * lg]);
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const s16x4 v = *reinterpret_cast<const s16x4*>(&vt[16 * (2 * wave + t) + l16][16 * kt + 4 * lg]);
        oacc[t] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, v, oacc[t], 0, 0, 0);
      }
    }
    __syncthreads();
  }
  lpart += __shfl_xor(lpart, 16, 64);
  lpart += __shfl_xor(lpart, 32, 64);
  if (lane < 16) lsum[wave][lane] = lpart;
  __syncthreads();
  float* pb = part + ((size_t)b * nwg + c0) * H * 129;
  // oacc[t] lane holds O[head 4 lg + r][dcol 16 (2 wave + t) + l16]
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int h = 4 * lg + r;
      if (h < H) pb[h * 129 + 16 * (2 * wave + t) + l16] = oacc[t][r];
    }
  if (tid < H) pb[tid * 129 + 128] = lsum[0][tid] + lsum[1][tid] + lsum[2][tid] + lsum[3][tid];
}

// grid (B, H), 128 threads: o[b][h][dcol] = sum_c acc / sum_c l in chunk order
template <typename T>
__global__ __launch_bounds__(128) void decode_combine_kernel(const float* __restrict__ part, int nwg,
                                                             int H, T* __restrict__ o, int ldo) {
  const int b = blockIdx.x, h = blockIdx.y, dcol = threadIdx.x;
  float acc = 0.f, l = 0.f;
  const float* pb = part + ((size_t)b * nwg * H + h) * 129;
#pragma unroll 4
  for (int c = 0; c < nwg; ++c) {
    acc += pb[(size_t)c * H * 129 + dcol];
    l += pb[(size_t)c * H * 129 + 128];
  }
  o[(size_t)b * ldo + h * 128 + dcol] = from_f32<T>(acc / l);
}

// ---------------------------------------------------------------------------
// Products with a handful of rows (decoding: one row per sequence), bf16:
// C[m, n] (epilogue) sum_k X[m, k] W[n, k], m < M <= 32. The product is a
// stream over W, so a workgroup owns just 16 output columns (many
// workgroups, short dependency chains); its 8 wavefronts take interleaved
// 32-wide k steps, so together they read each W row front to back, and
// multiply with v_mfma_f32_16x16x32_bf16 (16 W rows as the row operand, 16
// rows of X as the column operand). The wavefronts' partial tiles are added
// through LDS in wavefront order (bitwise reproducible).
constexpr int kSkWaves = 8;

template <int MT, SkEpi EPI>
__global__ __launch_bounds__(512) void skinny_kernel(const bf16* __restrict__ W, int ldw,
                                                     const bf16* __restrict__ X, int ldx,
                                                     void* __restrict__ Cv, int ldc, int M, int K,
                                                     float cap) {
  __shared__ __align__(16) float red[kSkWaves * MT * 256];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, lg = lane >> 4;
  const int n0 = blockIdx.x * 16;
  const int nsteps = K >> 5;
  const bf16* wrow = W + (size_t)(n0 + l16) * ldw + 8 * lg;
  f32x4 acc[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) acc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
  constexpr int U = 4;
  for (int s0 = wave; s0 < nsteps; s0 += kSkWaves * U) {
    bf16x8 a[U], x[U][MT];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int s = s0 + kSkWaves * u;
      if (s < nsteps) {
        a[u] = *reinterpret_cast<const bf16x8*>(wrow + 32 * s);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          const int m = 16 * mt + l16;
          x[u][mt] = m < M ? *reinterpret_cast<const bf16x8*>(X + (size_t)m * ldx + 32 * s + 8 * lg)
                           : bf16x8{};
        }
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (s0 + kSkWaves * u < nsteps)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
          acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[u], x[u][mt], acc[mt], 0, 0, 0);
  }
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
    *reinterpret_cast<f32x4*>(red + ((wave * MT + mt) * 64 + lane) * 4) = acc[mt];
  __syncthreads();
  // lane ln of tile mt holds C[16 mt + (ln & 15)][n0 + 4 (ln >> 4) + r]
  for (int e = tid; e < MT * 64; e += 512) {
    const int mt = e >> 6, ln = e & 63;
    f32x4 v = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int w = 0; w < kSkWaves; ++w) v += *reinterpret_cast<const f32x4*>(red + ((w * MT + mt) * 64 + ln) * 4);
    const int m = 16 * mt + (ln & 15), n = n0 + 4 * (ln >> 4);
    if (m >= M) continue;
    const size_t off = (size_t)m * ldc + n;
    if constexpr (EPI == SkEpi::StoreT) {
      *reinterpret_cast<bf16x4*>(static_cast<bf16*>(Cv) + off) =
          bf16x4{(bf16)v[0], (bf16)v[1], (bf16)v[2], (bf16)v[3]};
    } else if constexpr (EPI == SkEpi::Relu2) {
      bf16x4 w;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float r = fmaxf(v[i], 0.f);
        w[i] = (bf16)(r * r);
      }
      *reinterpret_cast<bf16x4*>(static_cast<bf16*>(Cv) + off) = w;
    } else if constexpr (EPI == SkEpi::AddF32) {
      f32x4* c = reinterpret_cast<f32x4*>(static_cast<float*>(Cv) + off);
      *c = *c + v;
    } else {
      const float inv = 1.0f / cap;
      f32x4 z;
#pragma unroll
      for (int i = 0; i < 4; ++i) z[i] = cap * tanhf(v[i] * inv);
      *reinterpret_cast<f32x4*>(static_cast<float*>(Cv) + off) = z;
    }
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
    // about two workgroups per CU over the batch; never more than the chunks
    const int want = (2 * 256 + B - 1) / B;
    const int nwg = want < nch ? want : nch;
    hipLaunchKernelGGL(decode_attn_mfma_kernel, dim3(B, nwg), dim3(256), 0, s,
                       static_cast<const bf16*>(qkv), ldq, H, static_cast<const bf16*>(cache), max_seq,
                       pos, part);
    hipLaunchKernelGGL(decode_combine_kernel<bf16>, dim3(B, H), dim3(128), 0, s, part, nwg, H,
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

hipError_t skinny_gemm(const void* W, int ldw, const void* X, int ldx, void* C, int ldc, int M, int N,
                       int K, SkEpi epi, float cap, hipStream_t s) {
  if (M < 1 || M > kSkinnyMaxRows || N < 16 || N % 16 || K < 32 || K % 32 || ldw % 8 || ldx % 8 ||
      ldc % 4 || ldw < K || ldx < K || ldc < N)
    return hipErrorInvalidValue;
  const dim3 grid(N / 16), block(512);
  const bf16* w = static_cast<const bf16*>(W);
  const bf16* x = static_cast<const bf16*>(X);
#define NC_SKINNY(MT, E)                                                                      \
  hipLaunchKernelGGL((skinny_kernel<MT, E>), grid, block, 0, s, w, ldw, x, ldx, C, ldc, M, K, cap)
#define NC_SKINNY_EPI(MT)                                       \
  switch (epi) {                                                \
    case SkEpi::StoreT: NC_SKINNY(MT, SkEpi::StoreT); break;    \
    case SkEpi::AddF32: NC_SKINNY(MT, SkEpi::AddF32); break;    \
    case SkEpi::Relu2: NC_SKINNY(MT, SkEpi::Relu2); break;      \
    case SkEpi::SoftcapF32: NC_SKINNY(MT, SkEpi::SoftcapF32); break; \
  }
  if (M <= 16) {
    NC_SKINNY_EPI(1)
  } else {
    NC_SKINNY_EPI(2)
  }
#undef NC_SKINNY_EPI
#undef NC_SKINNY
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
