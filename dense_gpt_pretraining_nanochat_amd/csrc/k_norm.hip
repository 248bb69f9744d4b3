// Bandwidth-bound row kernels: embedding gather + RMSNorm, RMSNorm forward and
// backward, the embedding backward scatter, the loss mean and a zero fill.
//
// RMSNorm has no learnable parameters and the token embedding output is
// normalised (followin.io release article, architecture list). The norm is
// n(v) = v / sqrt(mean(v^2) + eps); its gradient is
// dv = rinv * (dy - y * mean(dy * y)) with y = n(v), rinv = 1/sqrt(mean+eps).
//
// One 64-lane wavefront owns one row (d <= 2048 floats): each lane keeps up to
// 8 float4 of the row in registers, so a row is read from HBM once and written
// once, with 16-byte coalesced accesses and a shuffle-tree reduction.
#include "common.h"
#include "launch.h"

namespace nc {
namespace {

constexpr int kRowsPerBlock = 4;          // 4 wavefronts, one row each
constexpr int kMaxVec = 8;                // d <= 8 * 256 = 2048

template <typename T>
__device__ __forceinline__ void load4(const T* p, float* o) {
  typedef T T4 __attribute__((ext_vector_type(4)));
  T4 v = *reinterpret_cast<const T4*>(p);
  o[0] = to_f32(v[0]); o[1] = to_f32(v[1]); o[2] = to_f32(v[2]); o[3] = to_f32(v[3]);
}
template <typename T>
__device__ __forceinline__ void store4(T* p, const float* o) {
  typedef T T4 __attribute__((ext_vector_type(4)));
  T4 v = {from_f32<T>(o[0]), from_f32<T>(o[1]), from_f32<T>(o[2]), from_f32<T>(o[3])};
  *reinterpret_cast<T4*>(p) = v;
}

// x[m] = n(E[tok[m]]) in fp32, rinv[m]
template <typename T>
__global__ __launch_bounds__(256) void embed_norm_fwd_kernel(const T* __restrict__ E,
                                                             const int32_t* __restrict__ tok,
                                                             int M, int d, int V, float eps,
                                                             float* __restrict__ x,
                                                             float* __restrict__ rinv,
                                                             uint32_t* status) {
  const int lane = threadIdx.x & 63;
  const int m = blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6);
  if (m >= M) return;
  int id = tok[m];
  if (id < 0 || id >= V) {
    if (lane == 0) atomicOr(status, kStatusTokenRange);
    id = id < 0 ? 0 : V - 1;
  }
  const T* src = E + (size_t)id * d;
  float v[kMaxVec][4];
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < kMaxVec; ++i) {
    const int c = (i * 64 + lane) * 4;
    if (c < d) {
      load4(src + c, v[i]);
      ss += v[i][0] * v[i][0] + v[i][1] * v[i][1] + v[i][2] * v[i][2] + v[i][3] * v[i][3];
    }
  }
  ss = wave_sum(ss);
  const float r = 1.0f / sqrtf(ss / d + eps);
  float* dst = x + (size_t)m * d;
#pragma unroll
  for (int i = 0; i < kMaxVec; ++i) {
    const int c = (i * 64 + lane) * 4;
    if (c < d) {
      f32x4 o = {v[i][0] * r, v[i][1] * r, v[i][2] * r, v[i][3] * r};
      *reinterpret_cast<f32x4*>(dst + c) = o;
    }
  }
  if (lane == 0) rinv[m] = r;
}

template <typename T>
__global__ __launch_bounds__(256) void rmsnorm_fwd_kernel(const float* __restrict__ x, int M, int d,
                                                          float eps, T* __restrict__ y,
                                                          float* __restrict__ rinv) {
  const int lane = threadIdx.x & 63;
  const int m = blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6);
  if (m >= M) return;
  const float* src = x + (size_t)m * d;
  f32x4 v[kMaxVec];
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < kMaxVec; ++i) {
    const int c = (i * 64 + lane) * 4;
    if (c < d) {
      v[i] = *reinterpret_cast<const f32x4*>(src + c);
      ss += v[i][0] * v[i][0] + v[i][1] * v[i][1] + v[i][2] * v[i][2] + v[i][3] * v[i][3];
    }
  }
  ss = wave_sum(ss);
  const float r = 1.0f / sqrtf(ss / d + eps);
  T* dst = y + (size_t)m * d;
#pragma unroll
  for (int i = 0; i < kMaxVec; ++i) {
    const int c = (i * 64 + lane) * 4;
    if (c < d) {
      float o[4] = {v[i][0] * r, v[i][1] * r, v[i][2] * r, v[i][3] * r};
      store4(dst + c, o);
    }
  }
  if (lane == 0) rinv[m] = r;
}

template <typename T, bool ACC, bool WRITE_G>
__global__ __launch_bounds__(256) void rmsnorm_bwd_kernel(const T* __restrict__ dy,
                                                          const T* __restrict__ y,
                                                          const float* __restrict__ rinv, int M,
                                                          int d, float* __restrict__ dx,
                                                          T* __restrict__ g) {
  const int lane = threadIdx.x & 63;
  const int m = blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6);
  if (m >= M) return;
  const size_t base = (size_t)m * d;
  float gy[kMaxVec][4];
  float yy[kMaxVec][4];
  float dot = 0.f;
#pragma unroll
  for (int i = 0; i < kMaxVec; ++i) {
    const int c = (i * 64 + lane) * 4;
    if (c < d) {
      load4(dy + base + c, gy[i]);
      load4(y + base + c, yy[i]);
      dot += gy[i][0] * yy[i][0] + gy[i][1] * yy[i][1] + gy[i][2] * yy[i][2] + gy[i][3] * yy[i][3];
    }
  }
  dot = wave_sum(dot) / d;
  const float r = rinv[m];
#pragma unroll
  for (int i = 0; i < kMaxVec; ++i) {
    const int c = (i * 64 + lane) * 4;
    if (c < d) {
      f32x4 o;
#pragma unroll
      for (int e = 0; e < 4; ++e) o[e] = r * (gy[i][e] - yy[i][e] * dot);
      f32x4* p = reinterpret_cast<f32x4*>(dx + base + c);
      if (ACC) o += *p;
      *p = o;
      if (WRITE_G) {
        float oo[4] = {o[0], o[1], o[2], o[3]};
        store4(g + base + c, oo);
      }
    }
  }
}

// ---- embedding backward -----------------------------------------------------
// de[m] = n'(dx[m]) with y = x0 = E[tok[m]] * rinv0[m] recomputed; counts[tok]++
template <typename T>
__global__ __launch_bounds__(256) void embed_de_kernel(const T* __restrict__ E,
                                                       const int32_t* __restrict__ tok,
                                                       const float* __restrict__ rinv0,
                                                       const float* __restrict__ dx, int M, int d,
                                                       int V, float* __restrict__ de,
                                                       int32_t* __restrict__ counts) {
  const int lane = threadIdx.x & 63;
  const int m = blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6);
  if (m >= M) return;
  int id = tok[m];
  id = id < 0 ? 0 : (id >= V ? V - 1 : id);
  const T* src = E + (size_t)id * d;
  const float r = rinv0[m];
  const size_t base = (size_t)m * d;
  f32x4 gy[kMaxVec];
  float yy[kMaxVec][4];
  float dot = 0.f;
#pragma unroll
  for (int i = 0; i < kMaxVec; ++i) {
    const int c = (i * 64 + lane) * 4;
    if (c < d) {
      gy[i] = *reinterpret_cast<const f32x4*>(dx + base + c);
      load4(src + c, yy[i]);
#pragma unroll
      for (int e = 0; e < 4; ++e) yy[i][e] *= r;
      dot += gy[i][0] * yy[i][0] + gy[i][1] * yy[i][1] + gy[i][2] * yy[i][2] + gy[i][3] * yy[i][3];
    }
  }
  dot = wave_sum(dot) / d;
#pragma unroll
  for (int i = 0; i < kMaxVec; ++i) {
    const int c = (i * 64 + lane) * 4;
    if (c < d) {
      f32x4 o;
#pragma unroll
      for (int e = 0; e < 4; ++e) o[e] = r * (gy[i][e] - yy[i][e] * dot);
      *reinterpret_cast<f32x4*>(de + base + c) = o;
    }
  }
  if (lane == 0) atomicAdd(&counts[id], 1);
}

// exclusive scan of counts[0..V) into offsets[0..V] and cursor[0..V), one block
__global__ __launch_bounds__(1024) void scan_counts_kernel(const int32_t* __restrict__ counts,
                                                           int V, int32_t* __restrict__ offsets,
                                                           int32_t* __restrict__ cursor) {
  __shared__ int32_t part[1024];
  const int tid = threadIdx.x;
  const int per = (V + 1023) / 1024;
  const int b = tid * per, e = min(b + per, V);
  int s = 0;
  for (int i = b; i < e; ++i) s += counts[i];
  part[tid] = s;
  __syncthreads();
  for (int o = 1; o < 1024; o <<= 1) {     // Hillis-Steele inclusive scan
    const int v = tid >= o ? part[tid - o] : 0;
    __syncthreads();
    part[tid] += v;
    __syncthreads();
  }
  int run = tid ? part[tid - 1] : 0;
  for (int i = b; i < e; ++i) {
    offsets[i] = run;
    cursor[i] = run;
    run += counts[i];
  }
  if (tid == 1023) offsets[V] = part[1023];
}

__global__ void fill_list_kernel(const int32_t* __restrict__ tok, int M, int V,
                                 int32_t* __restrict__ cursor, int32_t* __restrict__ list) {
  const int m = blockIdx.x * blockDim.x + threadIdx.x;
  if (m >= M) return;
  int id = tok[m];
  id = id < 0 ? 0 : (id >= V ? V - 1 : id);
  list[atomicAdd(&cursor[id], 1)] = m;
}

constexpr int kSortCap = 4096;   // buckets up to this size are sorted in LDS

// One block per vocabulary row: dE[v] = sum of de[m] over tok[m] == v, in
// increasing m (a fixed order, so the result is bitwise reproducible).
__global__ __launch_bounds__(256) void segment_sum_kernel(const int32_t* __restrict__ tok,
                                                          const int32_t* __restrict__ offsets,
                                                          const int32_t* __restrict__ list,
                                                          const float* __restrict__ de, int M,
                                                          int d, int V, float* __restrict__ dE) {
  __shared__ int32_t idx[kSortCap];
  __shared__ int32_t runc[256];
  const int v = blockIdx.x;
  const int tid = threadIdx.x;
  const int beg = offsets[v], n = offsets[v + 1] - beg;
  float* dst = dE + (size_t)v * d;
  const int ncol4 = d / 4;                       // d <= 2048 -> <= 2 float4 per thread
  f32x4 acc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
  if (n == 0) {
  } else if (n <= kSortCap) {
    int np2 = 1;
    while (np2 < n) np2 <<= 1;
    for (int i = tid; i < np2; i += 256) idx[i] = i < n ? list[beg + i] : INT32_MAX;
    __syncthreads();
    for (int k = 2; k <= np2; k <<= 1) {          // bitonic sort, ascending
      for (int j = k >> 1; j > 0; j >>= 1) {
        for (int i = tid; i < np2; i += 256) {
          const int p = i ^ j;
          if (p > i) {
            const int a = idx[i], b = idx[p];
            const bool up = (i & k) == 0;
            if ((a > b) == up) { idx[i] = b; idx[p] = a; }
          }
        }
        __syncthreads();
      }
    }
    for (int s = 0; s < n; ++s) {
      const float* row = de + (size_t)idx[s] * d;
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const int c4 = tid + q * 256;
        if (c4 < ncol4) acc[q] += reinterpret_cast<const f32x4*>(row)[c4];
      }
    }
  } else {
    // large bucket: walk the token array in order, compacting matches per chunk
    auto id_at = [&](int i) {
      const int t = tok[i];
      return t < 0 ? 0 : (t >= V ? V - 1 : t);
    };
    for (int c0 = 0; c0 < M; c0 += kSortCap) {
      // ordered compaction: each thread scans a contiguous run of 16 positions
      const int rb = c0 + tid * 16;
      int local = 0;
      for (int i = rb; i < min(rb + 16, M); ++i) local += (id_at(i) == v) ? 1 : 0;
      runc[tid] = local;
      __syncthreads();
      for (int o = 1; o < 256; o <<= 1) {
        const int t2 = tid >= o ? runc[tid - o] : 0;
        __syncthreads();
        runc[tid] += t2;
        __syncthreads();
      }
      int w = runc[tid] - local;
      for (int i = rb; i < min(rb + 16, M); ++i)
        if (id_at(i) == v) idx[w++] = i;
      const int total = runc[255];
      __syncthreads();
      for (int s = 0; s < total; ++s) {
        const float* row = de + (size_t)idx[s] * d;
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          const int c4 = tid + q * 256;
          if (c4 < ncol4) acc[q] += reinterpret_cast<const f32x4*>(row)[c4];
        }
      }
      __syncthreads();
    }
  }
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int c4 = tid + q * 256;
    if (c4 < ncol4) reinterpret_cast<f32x4*>(dst)[c4] = acc[q];
  }
}

__global__ __launch_bounds__(1024) void loss_mean_kernel(const float* __restrict__ loss_rows,
                                                         int M, float* __restrict__ out,
                                                         uint32_t* status) {
  __shared__ float red[16];
  float s = 0.f;
  for (int i = threadIdx.x; i < M; i += 1024) s += loss_rows[i];
  s = block_sum(s, red);
  if (threadIdx.x == 0) {
    const float mean = s / (float)M;
    *out = mean;
    if (!isfinite(mean)) atomicOr(status, kStatusNonFiniteLoss);
  }
}

__global__ void fill_zero_kernel(uint32_t* __restrict__ p, size_t n) {
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n;
       i += (size_t)gridDim.x * blockDim.x)
    p[i] = 0u;
}

inline int row_grid(int M) { return (M + kRowsPerBlock - 1) / kRowsPerBlock; }

}  // namespace

hipError_t embed_norm_fwd(DType t, const void* E, const int32_t* tok, int M, int d, int V,
                          float eps, float* x, float* rinv, uint32_t* status, hipStream_t s) {
  if (d % 4 || d > 2048) return hipErrorInvalidValue;
  if (t == DType::BF16)
    hipLaunchKernelGGL(embed_norm_fwd_kernel<bf16>, dim3(row_grid(M)), dim3(256), 0, s,
                       static_cast<const bf16*>(E), tok, M, d, V, eps, x, rinv, status);
  else
    hipLaunchKernelGGL(embed_norm_fwd_kernel<float>, dim3(row_grid(M)), dim3(256), 0, s,
                       static_cast<const float*>(E), tok, M, d, V, eps, x, rinv, status);
  return hipGetLastError();
}

hipError_t rmsnorm_fwd(DType t, const float* x, int M, int d, float eps, void* y, float* rinv,
                       hipStream_t s) {
  if (d % 4 || d > 2048) return hipErrorInvalidValue;
  if (t == DType::BF16)
    hipLaunchKernelGGL(rmsnorm_fwd_kernel<bf16>, dim3(row_grid(M)), dim3(256), 0, s, x, M, d, eps,
                       static_cast<bf16*>(y), rinv);
  else
    hipLaunchKernelGGL(rmsnorm_fwd_kernel<float>, dim3(row_grid(M)), dim3(256), 0, s, x, M, d, eps,
                       static_cast<float*>(y), rinv);
  return hipGetLastError();
}

template <typename T>
static void launch_norm_bwd(const void* dyv, const void* y, const float* rinv, int M, int d,
                            float* dx, bool acc, void* g, hipStream_t s) {
  const T* dy = static_cast<const T*>(dyv);
  const T* yt = static_cast<const T*>(y);
  T* gt = static_cast<T*>(g);
  dim3 grid(row_grid(M)), block(256);
  if (acc && g) hipLaunchKernelGGL((rmsnorm_bwd_kernel<T, true, true>), grid, block, 0, s, dy, yt, rinv, M, d, dx, gt);
  else if (acc) hipLaunchKernelGGL((rmsnorm_bwd_kernel<T, true, false>), grid, block, 0, s, dy, yt, rinv, M, d, dx, gt);
  else if (g) hipLaunchKernelGGL((rmsnorm_bwd_kernel<T, false, true>), grid, block, 0, s, dy, yt, rinv, M, d, dx, gt);
  else hipLaunchKernelGGL((rmsnorm_bwd_kernel<T, false, false>), grid, block, 0, s, dy, yt, rinv, M, d, dx, gt);
}

hipError_t rmsnorm_bwd(DType t, const void* dy, const void* y, const float* rinv, int M, int d,
                       float* dx, bool accumulate, void* g, hipStream_t s) {
  if (d % 4 || d > 2048) return hipErrorInvalidValue;
  if (t == DType::BF16) launch_norm_bwd<bf16>(dy, y, rinv, M, d, dx, accumulate, g, s);
  else launch_norm_bwd<float>(dy, y, rinv, M, d, dx, accumulate, g, s);
  return hipGetLastError();
}

hipError_t embed_bwd(DType t, const void* E, const int32_t* tok, const float* rinv0,
                     const float* dx, int M, int d, int V, EmbedBwdScratch ws, float* dE,
                     hipStream_t s) {
  if (d % 4 || d > 2048) return hipErrorInvalidValue;
  hipError_t e = fill_zero(ws.counts, sizeof(int32_t) * (V + 1), s);
  if (e != hipSuccess) return e;
  if (t == DType::BF16)
    hipLaunchKernelGGL(embed_de_kernel<bf16>, dim3(row_grid(M)), dim3(256), 0, s,
                       static_cast<const bf16*>(E), tok, rinv0, dx, M, d, V, ws.de, ws.counts);
  else
    hipLaunchKernelGGL(embed_de_kernel<float>, dim3(row_grid(M)), dim3(256), 0, s,
                       static_cast<const float*>(E), tok, rinv0, dx, M, d, V, ws.de, ws.counts);
  hipLaunchKernelGGL(scan_counts_kernel, dim3(1), dim3(1024), 0, s, ws.counts, V, ws.offsets,
                     ws.cursor);
  hipLaunchKernelGGL(fill_list_kernel, dim3((M + 255) / 256), dim3(256), 0, s, tok, M, V,
                     ws.cursor, ws.list);
  hipLaunchKernelGGL(segment_sum_kernel, dim3(V), dim3(256), 0, s, tok, ws.offsets, ws.list, ws.de,
                     M, d, V, dE);
  return hipGetLastError();
}

hipError_t loss_mean(const float* loss_rows, int M, float* out, uint32_t* status, hipStream_t s) {
  hipLaunchKernelGGL(loss_mean_kernel, dim3(1), dim3(1024), 0, s, loss_rows, M, out, status);
  return hipGetLastError();
}

hipError_t fill_zero(void* p, size_t bytes, hipStream_t s) {
  if (bytes % 4) return hipErrorInvalidValue;
  const size_t n = bytes / 4;
  if (n == 0) return hipSuccess;
  const size_t want = (n + 255) / 256;
  const int grid = (int)(want < 8192 ? want : 8192);
  hipLaunchKernelGGL(fill_zero_kernel, dim3(grid), dim3(256), 0, s, static_cast<uint32_t*>(p), n);
  return hipGetLastError();
}

}  // namespace nc
