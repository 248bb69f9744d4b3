// Bandwidth-bound row kernels: embedding gather + RMSNorm, RMSNorm forward and
// backward, the embedding backward scatter, the loss mean and a zero fill.
//
// RMSNorm has no learnable parameters and the token embedding output is
// normalised (followin.io release article, architecture list). The norm is
// n(v) = v / sqrt(mean(v^2) + eps); its gradient is
// dv = rinv * (dy - y * mean(dy * y)) with y = n(v), rinv = 1/sqrt(mean+eps).
// In the training step the norms in front of the blocks and the lm_head are
// folded into the products (the consumer scales its output rows by rinv, the
// gradients arriving there carry rinv), so the backward here also takes the
// prescaled form dv = dy' - rinv^2 * v * mean(dy' * v) with dy' = rinv * dy,
// and rinv itself comes from per-64-column sums of squares (ssq_rinv).
//
// One 64-lane wavefront owns one row (d <= 2048 floats): each lane keeps up to
// 8 float4 of the row in registers, so a row is read from HBM once and written
// once, with 16-byte coalesced accesses and a shuffle-tree reduction.
#include <algorithm>

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

// x[m] = n(E[tok[m]]) in fp32, rinv[m]; with XB also xb[m] = T(x[m]) and
// rinv_x[m] = 1/sqrt(mean(x[m]^2) + eps), the first block's norm of x folded
// into its QKV product
template <typename T, bool XB>
__global__ __launch_bounds__(256) void embed_norm_fwd_kernel(const T* __restrict__ E,
                                                             const int32_t* __restrict__ tok,
                                                             int M, int d, int V, float eps,
                                                             float* __restrict__ x,
                                                             float* __restrict__ rinv,
                                                             uint32_t* status, T* __restrict__ xb,
                                                             float* __restrict__ rinv_x) {
  const int lane = threadIdx.x & 63;
  const int m = blockIdx.x * kRowsPerBlock + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
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
  float ss2 = 0.f;
#pragma unroll
  for (int i = 0; i < kMaxVec; ++i) {
    const int c = (i * 64 + lane) * 4;
    if (c < d) {
      f32x4 o = {v[i][0] * r, v[i][1] * r, v[i][2] * r, v[i][3] * r};
      *reinterpret_cast<f32x4*>(dst + c) = o;
      if constexpr (XB) {
        float oo[4] = {o[0], o[1], o[2], o[3]};
        store4(xb + (size_t)m * d + c, oo);
        ss2 += o[0] * o[0] + o[1] * o[1] + o[2] * o[2] + o[3] * o[3];
      }
    }
  }
  if (lane == 0) rinv[m] = r;
  if constexpr (XB) {
    ss2 = wave_sum(ss2);
    if (lane == 0) rinv_x[m] = 1.0f / sqrtf(ss2 / d + eps);
  }
}

// rinv[m] = 1/sqrt(sum_p ssq[m][p] / d + eps), the partial sums of squares
// (per 64 columns, written by the residual-add product) added in column order.
// One thread per row; its P loads are independent and issued together.
constexpr int kSsqMaxP = 32;                   // d <= 2048
__global__ __launch_bounds__(128) void ssq_rinv_kernel(const float* __restrict__ ssq, int M, int P, int d,
                                                       float eps, float* __restrict__ rinv) {
  const int m = blockIdx.x * 128 + threadIdx.x;
  if (m >= M) return;
  const float* p = ssq + (size_t)m * P;
  float v[kSsqMaxP];
#pragma unroll
  for (int i = 0; i < kSsqMaxP; ++i) v[i] = i < P ? p[i] : 0.f;
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < kSsqMaxP; ++i)
    if (i < P) ss += v[i];
  rinv[m] = 1.0f / sqrtf(ss / d + eps);
}

template <typename T>
__global__ __launch_bounds__(256) void rmsnorm_fwd_kernel(const float* __restrict__ x, int M, int d,
                                                          float eps, T* __restrict__ y,
                                                          float* __restrict__ rinv) {
  const int lane = threadIdx.x & 63;
  const int m = blockIdx.x * kRowsPerBlock + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
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

// PRE: y is the unnormalised input v and dy already carries the factor rinv
// (the norm folded into the products): dx = dy - rinv^2 v mean(dy v), the same
// gradient as rinv (dy0 - y0 mean(dy0 y0)) for dy0 = dy / rinv, y0 = rinv v.
template <typename T, bool ACC, bool WRITE_G, bool PRE>
__global__ __launch_bounds__(256) void rmsnorm_bwd_kernel(const T* __restrict__ dy,
                                                          const T* __restrict__ y,
                                                          const float* __restrict__ rinv, int M,
                                                          int d, float* __restrict__ dx,
                                                          T* __restrict__ g) {
  const int lane = threadIdx.x & 63;
  const int m = blockIdx.x * kRowsPerBlock + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
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
      for (int e = 0; e < 4; ++e) {
        if constexpr (PRE) o[e] = gy[i][e] - yy[i][e] * (r * r * dot);
        else o[e] = r * (gy[i][e] - yy[i][e] * dot);
      }
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
// ---- embedding backward --------------------------------------------------
// Every occurrence of token v normalises the same row E[v] (same rinv, same
// y = E[v] * rinv), and the norm gradient is linear in the upstream gradient,
// so dE[v] = rinv * (S - y * mean(S * y)) with S = sum of dx[m] over tok[m] == v.
// S is summed in increasing m in fixed-size pieces whose partial sums are then
// added in piece order, so the result is bitwise reproducible. Steps: count
// tokens per id, scan the counts, bucket positions by id, sort each bucket,
// sum pieces of kSeg rows (one workgroup each), add the pieces of long buckets
// and apply the norm gradient.
constexpr int kSeg = 64;         // rows of one bucket summed by one workgroup
constexpr int kSortCap = 4096;   // buckets up to this size are sorted in LDS

__device__ __forceinline__ int clamp_id(int t, int V) { return t < 0 ? 0 : (t >= V ? V - 1 : t); }

__global__ void embed_count_kernel(const int32_t* __restrict__ tok, int M, int V,
                                   int32_t* __restrict__ counts) {
  const int m = blockIdx.x * blockDim.x + threadIdx.x;
  if (m < M) atomicAdd(&counts[clamp_id(tok[m], V)], 1);
}

// Exclusive scans over ids of (rows, pieces, pieces of multi-piece buckets),
// in two coalesced passes over blocks of 1024 ids: the first writes each
// block's three sums, the second adds the earlier blocks' sums to a
// block-wide scan and writes the offsets, cursors, piece offsets and the
// owning id of every piece.
constexpr int kScanBlock = 1024;
__device__ __forceinline__ void scan_counts_of(int n, int* v) {
  const int it = (n + kSeg - 1) / kSeg;
  v[0] = n;
  v[1] = it;
  v[2] = it > 1 ? it : 0;
}

__global__ __launch_bounds__(kScanBlock) void embed_scan_blocks_kernel(const int32_t* __restrict__ counts,
                                                                       int V, int32_t* __restrict__ blocks) {
  __shared__ int red[3][kScanBlock / 64];
  const int i = blockIdx.x * kScanBlock + threadIdx.x;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  int v[3];
  scan_counts_of(i < V ? counts[i] : 0, v);
#pragma unroll
  for (int k = 0; k < 3; ++k) {
    int x = v[k];
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o, 64);
    if (lane == 0) red[k][w] = x;
  }
  __syncthreads();
  if (threadIdx.x < 3) {
    int t = 0;
    for (int j = 0; j < kScanBlock / 64; ++j) t += red[threadIdx.x][j];
    blocks[blockIdx.x * 3 + threadIdx.x] = t;
  }
}

__global__ __launch_bounds__(kScanBlock) void embed_scan_kernel(const int32_t* __restrict__ counts, int V,
                                                                const int32_t* __restrict__ blocks,
                                                                EmbedBwdScratch ws) {
  __shared__ int wtot[3][kScanBlock / 64];
  __shared__ int carry[3];
  const int i = blockIdx.x * kScanBlock + threadIdx.x;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  if (threadIdx.x < 3) {
    int c = 0;
    for (int b = 0; b < (int)blockIdx.x; ++b) c += blocks[b * 3 + threadIdx.x];
    carry[threadIdx.x] = c;
  }
  int v[3], inc[3];
  scan_counts_of(i < V ? counts[i] : 0, v);
#pragma unroll
  for (int k = 0; k < 3; ++k) {                // inclusive scan inside the wavefront
    int x = v[k];
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(x, o, 64);
      if (lane >= o) x += y;
    }
    inc[k] = x;
    if (lane == 63) wtot[k][w] = x;
  }
  __syncthreads();
  int ex[3];
#pragma unroll
  for (int k = 0; k < 3; ++k) {
    int before = carry[k];
    for (int j = 0; j < w; ++j) before += wtot[k][j];
    ex[k] = before + inc[k] - v[k];
  }
  if (i < V) {
    ws.offsets[i] = ex[0];
    ws.cursor[i] = ex[0];
    ws.item_off[i] = ex[1];
    ws.part_off[i] = ex[2];
    for (int j = 0; j < v[1]; ++j) ws.item_bucket[ex[1] + j] = i;
    if (i == V - 1) {
      ws.offsets[V] = ex[0] + v[0];
      ws.item_off[V] = ex[1] + v[1];
      ws.part_off[V] = ex[2] + v[2];
    }
  }
}

__global__ void fill_list_kernel(const int32_t* __restrict__ tok, int M, int V,
                                 int32_t* __restrict__ cursor, int32_t* __restrict__ list) {
  const int m = blockIdx.x * blockDim.x + threadIdx.x;
  if (m >= M) return;
  list[atomicAdd(&cursor[clamp_id(tok[m], V)], 1)] = m;
}

// One block per id: put the bucket's positions in increasing order (the atomic
// fill leaves them in arbitrary order). Small buckets: bitonic sort in LDS;
// large ones: an ordered compaction of the token array, chunk by chunk.
__global__ __launch_bounds__(256) void embed_sort_kernel(const int32_t* __restrict__ tok, int M,
                                                         int V, const int32_t* __restrict__ offsets,
                                                         int32_t* __restrict__ list) {
  __shared__ int32_t idx[kSortCap];
  __shared__ int32_t runc[256];
  const int v = blockIdx.x;
  const int tid = threadIdx.x;
  const int beg = offsets[v], n = offsets[v + 1] - beg;
  if (n <= 1) return;
  if (n <= kSortCap) {
    int np2 = 1;
    while (np2 < n) np2 <<= 1;
    for (int i = tid; i < np2; i += 256) idx[i] = i < n ? list[beg + i] : INT32_MAX;
    __syncthreads();
    for (int k = 2; k <= np2; k <<= 1) {
      for (int j = k >> 1; j > 0; j >>= 1) {
        for (int i = tid; i < np2; i += 256) {
          const int p = i ^ j;
          if (p > i) {
            const int x = idx[i], y = idx[p];
            const bool up = (i & k) == 0;
            if ((x > y) == up) { idx[i] = y; idx[p] = x; }
          }
        }
        __syncthreads();
      }
    }
    for (int i = tid; i < n; i += 256) list[beg + i] = idx[i];
    return;
  }
  constexpr int kRun = 32;                       // positions per thread per chunk
  int w0 = beg;
  for (int c0 = 0; c0 < M; c0 += 256 * kRun) {
    const int rb = c0 + tid * kRun, re = min(rb + kRun, M);
    int local = 0;
    for (int i = rb; i < re; ++i) local += clamp_id(tok[i], V) == v ? 1 : 0;
    runc[tid] = local;
    __syncthreads();
    for (int o = 1; o < 256; o <<= 1) {
      const int t2 = tid >= o ? runc[tid - o] : 0;
      __syncthreads();
      runc[tid] += t2;
      __syncthreads();
    }
    int w = w0 + runc[tid] - local;
    for (int i = rb; i < re; ++i)
      if (clamp_id(tok[i], V) == v) list[w++] = i;
    w0 += runc[255];
    __syncthreads();
  }
}

// dE[v] = rinv * (S - y * mean(S * y)), y = E[v] * rinv; all threads call it
template <typename T>
__device__ __forceinline__ void embed_finish_row(const T* __restrict__ E, int v, int d, float r,
                                                 f32x4 S, bool active, float* __restrict__ dE,
                                                 bool accumulate) {
  __shared__ float red[16];
  const int c = threadIdx.x * 4;
  float y[4] = {0.f, 0.f, 0.f, 0.f};
  if (active) {
    load4(E + (size_t)v * d + c, y);
#pragma unroll
    for (int k = 0; k < 4; ++k) y[k] *= r;
  }
  float dot = S[0] * y[0] + S[1] * y[1] + S[2] * y[2] + S[3] * y[3];
  dot = block_sum(dot, red) / d;
  if (active) {
    f32x4 o;
#pragma unroll
    for (int k = 0; k < 4; ++k) o[k] = r * (S[k] - y[k] * dot);
    f32x4* dst = reinterpret_cast<f32x4*>(dE + (size_t)v * d + c);
    if (accumulate) o += *dst;
    *dst = o;
  }
}

// One block per piece of <= kSeg rows of one bucket; thread t owns columns
// 4t..4t+3. Single-piece buckets are finished here, the others leave a partial.
template <typename T>
__global__ __launch_bounds__(512) void embed_sum_kernel(const T* __restrict__ E,
                                                        const float* __restrict__ rinv0,
                                                        const float* __restrict__ dx, int d, int V,
                                                        EmbedBwdScratch ws, float* __restrict__ dE,
                                                        bool accumulate) {
  __shared__ int32_t rows[kSeg];
  const int i = blockIdx.x;
  if (i >= ws.item_off[V]) return;
  const int tid = threadIdx.x;
  const int v = ws.item_bucket[i];
  const int j = i - ws.item_off[v];
  const int beg = ws.offsets[v], n = ws.offsets[v + 1] - beg;
  const int cnt = min(kSeg, n - j * kSeg);
  if (tid < cnt) rows[tid] = ws.list[beg + j * kSeg + tid];
  __syncthreads();
  const bool active = tid * 4 < d;
  const size_t c = active ? (size_t)tid * 4 : 0;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  int s = 0;
  for (; s + 8 <= cnt; s += 8) {                 // eight rows in flight, added in order
    f32x4 t[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) t[u] = *reinterpret_cast<const f32x4*>(dx + (size_t)rows[s + u] * d + c);
#pragma unroll
    for (int u = 0; u < 8; ++u) acc += t[u];
  }
  for (; s < cnt; ++s) acc += *reinterpret_cast<const f32x4*>(dx + (size_t)rows[s] * d + c);
  if (n <= kSeg) {
    embed_finish_row(E, v, d, rinv0[rows[0]], acc, active, dE, accumulate);
  } else if (active) {
    *reinterpret_cast<f32x4*>(ws.part + (size_t)(ws.part_off[v] + j) * d + c) = acc;
  }
}

// One block per id: zero rows for unused ids; multi-piece buckets add their
// partials in piece order and apply the norm gradient.
template <typename T>
__global__ __launch_bounds__(512) void embed_finish_kernel(const T* __restrict__ E,
                                                           const float* __restrict__ rinv0, int d,
                                                           EmbedBwdScratch ws,
                                                           float* __restrict__ dE,
                                                           bool accumulate) {
  const int v = blockIdx.x;
  const int tid = threadIdx.x;
  const int beg = ws.offsets[v], n = ws.offsets[v + 1] - beg;
  const bool active = tid * 4 < d;
  const size_t c = active ? (size_t)tid * 4 : 0;
  if (n == 0) {                                  // unused id: dE row is 0 (nothing to add)
    if (active && !accumulate) *reinterpret_cast<f32x4*>(dE + (size_t)v * d + c) = f32x4{0.f, 0.f, 0.f, 0.f};
    return;
  }
  if (n <= kSeg) return;
  const int items = (n + kSeg - 1) / kSeg;
  const float* p = ws.part + (size_t)ws.part_off[v] * d + c;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  int k = 0;
  for (; k + 4 <= items; k += 4) {
    f32x4 t[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) t[u] = *reinterpret_cast<const f32x4*>(p + (size_t)(k + u) * d);
#pragma unroll
    for (int u = 0; u < 4; ++u) acc += t[u];
  }
  for (; k < items; ++k) acc += *reinterpret_cast<const f32x4*>(p + (size_t)k * d);
  embed_finish_row(E, v, d, rinv0[ws.list[beg]], acc, active, dE, accumulate);
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

// Bits per byte of a batch: the summed loss of the positions whose target has
// a nonzero byte length, those lengths summed, and their ratio in bits, all in
// fp64 and a fixed order (one workgroup). Targets are clamped as the loss
// kernel clamps them.
__device__ __forceinline__ double block_sum_f64(double v, double* red) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, kWave);
  const int w = threadIdx.x / kWave, nw = blockDim.x / kWave;
  __syncthreads();
  if ((threadIdx.x % kWave) == 0) red[w] = v;
  __syncthreads();
  double s = 0.0;
  for (int i = 0; i < nw; ++i) s += red[i];
  return s;
}

__global__ __launch_bounds__(1024) void bpb_kernel(const float* __restrict__ loss_rows,
                                                   const int32_t* __restrict__ targets, int M,
                                                   const int32_t* __restrict__ token_bytes, int V,
                                                   double* __restrict__ out) {
  __shared__ double red[16];
  double nats = 0.0, bytes = 0.0;
  for (int i = threadIdx.x; i < M; i += 1024) {
    int t = targets[i];
    t = t < 0 ? 0 : (t >= V ? V - 1 : t);
    const int b = token_bytes[t];
    if (b > 0) {
      nats += (double)loss_rows[i];
      bytes += (double)b;
    }
  }
  nats = block_sum_f64(nats, red);
  bytes = block_sum_f64(bytes, red);
  if (threadIdx.x == 0) {
    out[0] = nats;
    out[1] = bytes;
    out[2] = bytes > 0.0 ? nats / (0.69314718055994530942 * bytes) : __builtin_nan("");
  }
}

__global__ void fill_zero_kernel(uint32_t* __restrict__ p, size_t n) {
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n;
       i += (size_t)gridDim.x * blockDim.x)
    p[i] = 0u;
}

inline int row_grid(int M) { return (M + kRowsPerBlock - 1) / kRowsPerBlock; }

}  // namespace

template <typename T>
static void launch_embed_norm(const void* E, const int32_t* tok, int M, int d, int V, float eps, float* x,
                              float* rinv, uint32_t* status, void* xb, float* rinv_x, hipStream_t s) {
  if (xb && rinv_x)
    hipLaunchKernelGGL((embed_norm_fwd_kernel<T, true>), dim3(row_grid(M)), dim3(256), 0, s,
                       static_cast<const T*>(E), tok, M, d, V, eps, x, rinv, status, static_cast<T*>(xb),
                       rinv_x);
  else
    hipLaunchKernelGGL((embed_norm_fwd_kernel<T, false>), dim3(row_grid(M)), dim3(256), 0, s,
                       static_cast<const T*>(E), tok, M, d, V, eps, x, rinv, status, static_cast<T*>(nullptr),
                       static_cast<float*>(nullptr));
}

hipError_t embed_norm_fwd(DType t, const void* E, const int32_t* tok, int M, int d, int V,
                          float eps, float* x, float* rinv, uint32_t* status, hipStream_t s, void* xb,
                          float* rinv_x) {
  if (d % 4 || d > 2048) return hipErrorInvalidValue;
  if (t == DType::BF16) launch_embed_norm<bf16>(E, tok, M, d, V, eps, x, rinv, status, xb, rinv_x, s);
  else launch_embed_norm<float>(E, tok, M, d, V, eps, x, rinv, status, xb, rinv_x, s);
  return hipGetLastError();
}

hipError_t ssq_rinv(const float* ssq, int M, int P, int d, float eps, float* rinv, hipStream_t s) {
  if (M <= 0 || P <= 0 || P > kSsqMaxP || d <= 0) return hipErrorInvalidValue;
  hipLaunchKernelGGL(ssq_rinv_kernel, dim3((M + 127) / 128), dim3(128), 0, s, ssq, M, P, d, eps, rinv);
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

template <typename T, bool PRE>
static void launch_norm_bwd(const void* dyv, const void* y, const float* rinv, int M, int d,
                            float* dx, bool acc, void* g, hipStream_t s) {
  const T* dy = static_cast<const T*>(dyv);
  const T* yt = static_cast<const T*>(y);
  T* gt = static_cast<T*>(g);
  dim3 grid(row_grid(M)), block(256);
  if (acc && g) hipLaunchKernelGGL((rmsnorm_bwd_kernel<T, true, true, PRE>), grid, block, 0, s, dy, yt, rinv, M, d, dx, gt);
  else if (acc) hipLaunchKernelGGL((rmsnorm_bwd_kernel<T, true, false, PRE>), grid, block, 0, s, dy, yt, rinv, M, d, dx, gt);
  else if (g) hipLaunchKernelGGL((rmsnorm_bwd_kernel<T, false, true, PRE>), grid, block, 0, s, dy, yt, rinv, M, d, dx, gt);
  else hipLaunchKernelGGL((rmsnorm_bwd_kernel<T, false, false, PRE>), grid, block, 0, s, dy, yt, rinv, M, d, dx, gt);
}

hipError_t rmsnorm_bwd(DType t, const void* dy, const void* y, const float* rinv, int M, int d,
                       float* dx, bool accumulate, void* g, hipStream_t s, bool prescaled) {
  if (d % 4 || d > 2048) return hipErrorInvalidValue;
  if (t == DType::BF16) {
    if (prescaled) launch_norm_bwd<bf16, true>(dy, y, rinv, M, d, dx, accumulate, g, s);
    else launch_norm_bwd<bf16, false>(dy, y, rinv, M, d, dx, accumulate, g, s);
  } else {
    if (prescaled) launch_norm_bwd<float, true>(dy, y, rinv, M, d, dx, accumulate, g, s);
    else launch_norm_bwd<float, false>(dy, y, rinv, M, d, dx, accumulate, g, s);
  }
  return hipGetLastError();
}

uint64_t embed_bwd_max_pieces(int64_t M, int V) {
  return (uint64_t)std::min<int64_t>(M, V) + (uint64_t)(M / kSeg) + 1;
}
uint64_t embed_bwd_max_parts(int64_t M) { return 2 * (uint64_t)(M / kSeg) + 1; }
uint64_t embed_bwd_scan_blocks(int V) { return 3 * (uint64_t)((V + kScanBlock - 1) / kScanBlock); }

hipError_t embed_bwd(DType t, const void* E, const int32_t* tok, const float* rinv0,
                     const float* dx, int M, int d, int V, EmbedBwdScratch ws, float* dE,
                     bool accumulate, hipStream_t s) {
  if (d % 4 || d > 2048 || M <= 0 || V <= 0) return hipErrorInvalidValue;
  hipError_t e = fill_zero(ws.counts, sizeof(int32_t) * (V + 1), s);
  if (e != hipSuccess) return e;
  const int nthr = ((d / 4 + 63) / 64) * 64;
  const unsigned pieces = (unsigned)embed_bwd_max_pieces(M, V);
  hipLaunchKernelGGL(embed_count_kernel, dim3((M + 255) / 256), dim3(256), 0, s, tok, M, V,
                     ws.counts);
  const unsigned sblocks = (unsigned)((V + kScanBlock - 1) / kScanBlock);
  hipLaunchKernelGGL(embed_scan_blocks_kernel, dim3(sblocks), dim3(kScanBlock), 0, s, ws.counts, V,
                     ws.scan_blocks);
  hipLaunchKernelGGL(embed_scan_kernel, dim3(sblocks), dim3(kScanBlock), 0, s, ws.counts, V,
                     ws.scan_blocks, ws);
  hipLaunchKernelGGL(fill_list_kernel, dim3((M + 255) / 256), dim3(256), 0, s, tok, M, V,
                     ws.cursor, ws.list);
  hipLaunchKernelGGL(embed_sort_kernel, dim3(V), dim3(256), 0, s, tok, M, V, ws.offsets, ws.list);
  if (t == DType::BF16) {
    const bf16* Eb = static_cast<const bf16*>(E);
    hipLaunchKernelGGL(embed_sum_kernel<bf16>, dim3(pieces), dim3(nthr), 0, s, Eb, rinv0, dx, d, V,
                       ws, dE, accumulate);
    hipLaunchKernelGGL(embed_finish_kernel<bf16>, dim3(V), dim3(nthr), 0, s, Eb, rinv0, d, ws, dE,
                       accumulate);
  } else {
    const float* Ef = static_cast<const float*>(E);
    hipLaunchKernelGGL(embed_sum_kernel<float>, dim3(pieces), dim3(nthr), 0, s, Ef, rinv0, dx, d,
                       V, ws, dE, accumulate);
    hipLaunchKernelGGL(embed_finish_kernel<float>, dim3(V), dim3(nthr), 0, s, Ef, rinv0, d, ws, dE,
                       accumulate);
  }
  return hipGetLastError();
}

hipError_t loss_mean(const float* loss_rows, int M, float* out, uint32_t* status, hipStream_t s) {
  hipLaunchKernelGGL(loss_mean_kernel, dim3(1), dim3(1024), 0, s, loss_rows, M, out, status);
  return hipGetLastError();
}

hipError_t bits_per_byte(const float* loss_rows, const int32_t* targets, int M, const int32_t* token_bytes,
                         int V, double* out, hipStream_t s) {
  if (M < 1 || V < 1) return hipErrorInvalidValue;
  hipLaunchKernelGGL(bpb_kernel, dim3(1), dim3(1024), 0, s, loss_rows, targets, M, token_bytes, V, out);
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
