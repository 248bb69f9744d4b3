// Causal multi-query attention on the CDNA4 matrix cores: forward, the
// delta = <dO, O> preprocess, and a two-kernel backward without atomics.
//
// All query heads share one key/value head (followin.io release article,
// architecture list: multi-query attention); the objective is next-token
// prediction, so position t attends to keys u <= t (wmrh.cn tutorial, section
// 2.3). Scale 1/sqrt(128).
//
// Layout: the fused projection buffer holds, per token, H query heads, then
// the key head, then the value head, 128 values each (after rotary + QK-norm).
//
// Forward (flash style, online softmax in the log2 domain): a workgroup owns
// 32 query tokens and a group of up to 8 heads, one wavefront per head. Each
// K/V tile of 64 keys is staged in LDS once and read by every head's
// wavefront: K row-major, V transposed. The wavefront computes S^T = K Q^T so
// that each lane column is one query row; its softmax statistics then live in
// the lane, and P^T feeds O^T += V^T P^T straight from registers.
//
// Backward: dK/dV are summed over all heads and all later queries by the
// workgroup that owns a 64-key block (16 keys per wavefront, accumulators in
// registers); dQ is produced by a second kernel shaped like the forward.
// Neither uses atomics, so results are bitwise reproducible.
#include <math.h>

#include "common.h"
#include "launch.h"

namespace nc {
namespace {

constexpr int D = 128;
constexpr int BQ = 32;      // query tokens per workgroup (fwd, dQ)
constexpr int BKV = 64;     // keys per tile (fwd, dQ) and per workgroup (dK/dV)
constexpr int kMaxHeadsPerWG = 8;     // forward
constexpr int kMaxHeadsPerWGdQ = 4;   // dQ holds Q, dO and dQ tiles: fewer, fatter waves
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

template <typename T> struct Mma;
template <> struct Mma<bf16> {
  __device__ __forceinline__ static void run(f32x4& acc, const bf16x8& a, const bf16x8& b) {
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc, 0, 0, 0);
  }
};
template <> struct Mma<float> {
  __device__ __forceinline__ static void run(f32x4& acc, const f32x4& a, const f32x4& b) {
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[0], b[0], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[1], b[1], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[2], b[2], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[3], b[3], acc, 0, 0, 0);
  }
};

// A fragment whose contraction index runs over 16*NPT accumulator rows, built
// from NPT accumulator tiles held by this lane (lane group g owns rows
// 4g..4g+3 of each 16-row tile). bf16 takes two tiles (32 rows), fp32 one.
template <typename T> struct CFrag;
template <> struct CFrag<bf16> {
  static constexpr int NPT = 2;
  __device__ __forceinline__ static bf16x8 pack(const f32x4* t) {
    bf16x8 r;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      r[e] = static_cast<bf16>(t[0][e]);
      r[e + 4] = static_cast<bf16>(t[1][e]);
    }
    return r;
  }
  // matching operand from a [row][k] LDS array (k contiguous): k = 4g..4g+3 of
  // tile 0, then of tile 1
  __device__ __forceinline__ static bf16x8 read(const bf16* row, int k0, int lg) {
    const bf16x4 a = *reinterpret_cast<const bf16x4*>(row + k0 + 4 * lg);
    const bf16x4 b = *reinterpret_cast<const bf16x4*>(row + k0 + 16 + 4 * lg);
    return bf16x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  }
};
template <> struct CFrag<float> {
  static constexpr int NPT = 1;
  __device__ __forceinline__ static f32x4 pack(const f32x4* t) { return t[0]; }
  __device__ __forceinline__ static f32x4 read(const float* row, int k0, int lg) {
    return *reinterpret_cast<const f32x4*>(row + k0 + 4 * lg);
  }
};

template <typename T>
struct AttnTypes {
  static constexpr int VEC = Vec16<T>::N;
  static constexpr int KB = 4 * VEC;           // contraction per fragment
  static constexpr int NS = D / KB;            // fragments along the head dim
  static constexpr int KSTR = D + VEC;         // [key][d] rows, 16-byte pad
  static constexpr int TSTR64 = BKV + VEC;     // [d][64 keys] rows
  static constexpr int TSTR32 = BQ + VEC;      // [d][32 rows] rows
  typedef typename Vec16<T>::type V;
  typedef T T4 __attribute__((ext_vector_type(4)));
};

// Stage `nrows` rows (a multiple of 4) of 128 values from global (row stride ld)
// into LDS row-major [row][KSTR] and/or transposed [d][tstr].
template <typename T, bool ROWMAJOR, bool TRANS>
__device__ __forceinline__ void stage_rows(const T* __restrict__ src, size_t ld, int nrows,
                                           T* rm, T* tr, int tstr, int tid, int nthr) {
  typedef AttnTypes<T> A;
  constexpr int DC = D / A::VEC;
  const int units = DC * (nrows / 4);
  for (int u = tid; u < units; u += nthr) {
    const int dc = u % DC, rg = u / DC;
    typename A::V r4[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
      r4[j] = *reinterpret_cast<const typename A::V*>(src + (size_t)(rg * 4 + j) * ld + dc * A::VEC);
    if (ROWMAJOR) {
#pragma unroll
      for (int j = 0; j < 4; ++j)
        *reinterpret_cast<typename A::V*>(rm + (rg * 4 + j) * A::KSTR + dc * A::VEC) = r4[j];
    }
    if (TRANS) {
#pragma unroll
      for (int e = 0; e < A::VEC; ++e) {
        typename A::T4 w = {r4[0][e], r4[1][e], r4[2][e], r4[3][e]};
        *reinterpret_cast<typename A::T4*>(tr + (dc * A::VEC + e) * tstr + rg * 4) = w;
      }
    }
  }
}

// workgroup -> (batch, query block, head group); heavy (late) query blocks first
struct QBlock {
  int b, qb, hg;
};
__device__ __forceinline__ QBlock qblock_of(int bid, int nqb, int ngroups) {
  const int per_b = nqb * ngroups;
  QBlock q;
  q.b = bid / per_b;
  const int r = bid % per_b;
  q.qb = nqb - 1 - r / ngroups;
  q.hg = r % ngroups;
  return q;
}

// --------------------------------------------------------------------------
// forward
// --------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(kMaxHeadsPerWG * 64) void attn_fwd_kernel(
    const T* __restrict__ qkv, int ldq, int Tn, int H, int hpg, T* __restrict__ o,
    float* __restrict__ lse) {
  typedef AttnTypes<T> A;
  typedef typename A::V V;
  __shared__ __align__(16) T Ks[BKV * A::KSTR];
  __shared__ __align__(16) T Vt[D * A::TSTR64];

  const int ngroups = (H + hpg - 1) / hpg;
  const QBlock qbk = qblock_of(blockIdx.x, Tn / BQ, ngroups);
  const int tq0 = qbk.qb * BQ;
  const int tid = threadIdx.x, nthr = blockDim.x;
  const int wave = tid >> 6, lane = tid & 63, l16 = lane & 15, lg = lane >> 4;
  const int h = qbk.hg * hpg + wave;
  const bool active = h < H;
  const size_t row0 = (size_t)qbk.b * Tn;
  const T* kbase = qkv + H * D;
  const T* vbase = qkv + (H + 1) * D;

  V qf[2][A::NS];
#pragma unroll
  for (int c = 0; c < 2; ++c)
#pragma unroll
    for (int s = 0; s < A::NS; ++s)
      qf[c][s] = active ? *reinterpret_cast<const V*>(qkv + (row0 + tq0 + c * 16 + l16) * ldq +
                                                      h * D + s * A::KB + lg * A::VEC)
                        : V{};

  f32x4 oacc[8][2];
#pragma unroll
  for (int i = 0; i < 8; ++i) oacc[i][0] = oacc[i][1] = f32x4{0.f, 0.f, 0.f, 0.f};
  float mrow[2] = {-INFINITY, -INFINITY}, lrow[2] = {0.f, 0.f};
  const float sc = kLog2e / sqrtf((float)D);

  const int kv_end = tq0 + BQ;
  for (int kv0 = 0; kv0 < kv_end; kv0 += BKV) {
    __syncthreads();
    stage_rows<T, true, false>(kbase + (row0 + kv0) * ldq, ldq, BKV, Ks, nullptr, 0, tid, nthr);
    stage_rows<T, false, true>(vbase + (row0 + kv0) * ldq, ldq, BKV, nullptr, Vt, A::TSTR64, tid, nthr);
    __syncthreads();
    if (!active) continue;

    f32x4 st[4][2];
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) st[kt][0] = st[kt][1] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < A::NS; ++s)
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) {
        const V kf = *reinterpret_cast<const V*>(Ks + (kt * 16 + l16) * A::KSTR + s * A::KB + lg * A::VEC);
        Mma<T>::run(st[kt][0], kf, qf[0][s]);
        Mma<T>::run(st[kt][1], kf, qf[1][s]);
      }

    const bool diag = kv0 + BKV > tq0;
    float tmax[2] = {-INFINITY, -INFINITY};
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
      for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          float v = st[kt][c][r] * sc;
          if (diag && kv0 + kt * 16 + lg * 4 + r > tq0 + c * 16 + l16) v = -INFINITY;
          st[kt][c][r] = v;
          tmax[c] = fmaxf(tmax[c], v);
        }
    float alpha[2];
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const float mnew = fmaxf(mrow[c], group4_max(tmax[c]));
      alpha[c] = exp2f(mrow[c] - mnew);
      mrow[c] = mnew;
    }
    float psum[2] = {0.f, 0.f};
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
      for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float p = exp2f(st[kt][c][r] - mrow[c]);
          st[kt][c][r] = p;
          psum[c] += p;
        }
#pragma unroll
    for (int c = 0; c < 2; ++c) lrow[c] = lrow[c] * alpha[c] + group4_sum(psum[c]);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      oacc[i][0] *= alpha[0];
      oacc[i][1] *= alpha[1];
    }
    constexpr int NPT = CFrag<T>::NPT;
#pragma unroll
    for (int kk = 0; kk < 4 / NPT; ++kk) {
      f32x4 t0[NPT], t1[NPT];
#pragma unroll
      for (int q = 0; q < NPT; ++q) {
        t0[q] = st[kk * NPT + q][0];
        t1[q] = st[kk * NPT + q][1];
      }
      const V pb0 = CFrag<T>::pack(t0), pb1 = CFrag<T>::pack(t1);
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) {
        const V va = CFrag<T>::read(Vt + (dt * 16 + l16) * A::TSTR64, kk * 16 * NPT, lg);
        Mma<T>::run(oacc[dt][0], va, pb0);
        Mma<T>::run(oacc[dt][1], va, pb1);
      }
    }
  }
  if (!active) return;
  const int ldo = H * D;
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    const float inv = 1.0f / lrow[c];
    const int t = tq0 + c * 16 + l16;
    T* dst = o + (row0 + t) * ldo + h * D;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      typename A::T4 w;
#pragma unroll
      for (int r = 0; r < 4; ++r) w[r] = from_f32<T>(oacc[dt][c][r] * inv);
      *reinterpret_cast<typename A::T4*>(dst + dt * 16 + lg * 4) = w;
    }
    if (lg == 0) lse[((size_t)qbk.b * H + h) * Tn + t] = (mrow[c] + log2f(lrow[c])) * kLn2;
  }
}

// --------------------------------------------------------------------------
// delta[b, h, t] = sum_d dO * O
// --------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(256) void attn_delta_kernel(const T* __restrict__ o,
                                                         const T* __restrict__ dout, int Tn,
                                                         int H, size_t total,
                                                         float* __restrict__ delta) {
  const size_t w = blockIdx.x * 4ull + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (w >= total) return;
  const size_t m = w / H;
  const int h = (int)(w % H);
  const size_t off = m * (size_t)(H * D) + h * D;
  float s = to_f32(o[off + lane]) * to_f32(dout[off + lane]) +
            to_f32(o[off + lane + 64]) * to_f32(dout[off + lane + 64]);
  s = wave_sum(s);
  if (lane == 0) {
    const size_t b = m / Tn, t = m % Tn;
    delta[(b * H + h) * Tn + t] = s;
  }
}

// --------------------------------------------------------------------------
// backward, dQ: shaped like the forward (one wavefront per head, 32 rows)
// --------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(kMaxHeadsPerWGdQ * 64) void attn_bwd_dq_kernel(
    const T* __restrict__ qkv, int ldq, const T* __restrict__ dout, const float* __restrict__ lse,
    const float* __restrict__ delta, int Tn, int H, int hpg, T* __restrict__ dqkv, int ldd) {
  typedef AttnTypes<T> A;
  typedef typename A::V V;
  __shared__ __align__(16) T Ks[BKV * A::KSTR];
  __shared__ __align__(16) T Vs[BKV * A::KSTR];
  __shared__ __align__(16) T Kt[D * A::TSTR64];

  const int ngroups = (H + hpg - 1) / hpg;
  const QBlock qbk = qblock_of(blockIdx.x, Tn / BQ, ngroups);
  const int tq0 = qbk.qb * BQ;
  const int tid = threadIdx.x, nthr = blockDim.x;
  const int wave = tid >> 6, lane = tid & 63, l16 = lane & 15, lg = lane >> 4;
  const int h = qbk.hg * hpg + wave;
  const bool active = h < H;
  const size_t row0 = (size_t)qbk.b * Tn;
  const int ldo = H * D;

  V qf[2][A::NS], df[2][A::NS];
  float lse2[2], dl[2];
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    const int t = tq0 + c * 16 + l16;
#pragma unroll
    for (int s = 0; s < A::NS; ++s) {
      qf[c][s] = active ? *reinterpret_cast<const V*>(qkv + (row0 + t) * ldq + h * D + s * A::KB + lg * A::VEC) : V{};
      df[c][s] = active ? *reinterpret_cast<const V*>(dout + (row0 + t) * ldo + h * D + s * A::KB + lg * A::VEC) : V{};
    }
    lse2[c] = active ? lse[((size_t)qbk.b * H + h) * Tn + t] * kLog2e : 0.f;
    dl[c] = active ? delta[((size_t)qbk.b * H + h) * Tn + t] : 0.f;
  }
  f32x4 dq[8][2];
#pragma unroll
  for (int i = 0; i < 8; ++i) dq[i][0] = dq[i][1] = f32x4{0.f, 0.f, 0.f, 0.f};
  const float sc = kLog2e / sqrtf((float)D);
  const T* kbase = qkv + H * D;
  const T* vbase = qkv + (H + 1) * D;

  const int kv_end = tq0 + BQ;
  for (int kv0 = 0; kv0 < kv_end; kv0 += BKV) {
    __syncthreads();
    stage_rows<T, true, true>(kbase + (row0 + kv0) * ldq, ldq, BKV, Ks, Kt, A::TSTR64, tid, nthr);
    stage_rows<T, true, false>(vbase + (row0 + kv0) * ldq, ldq, BKV, Vs, nullptr, 0, tid, nthr);
    __syncthreads();
    if (!active) continue;

    f32x4 st[4][2], dpt[4][2];
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
      st[kt][0] = st[kt][1] = dpt[kt][0] = dpt[kt][1] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < A::NS; ++s)
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) {
        const V kf = *reinterpret_cast<const V*>(Ks + (kt * 16 + l16) * A::KSTR + s * A::KB + lg * A::VEC);
        const V vf = *reinterpret_cast<const V*>(Vs + (kt * 16 + l16) * A::KSTR + s * A::KB + lg * A::VEC);
        Mma<T>::run(st[kt][0], kf, qf[0][s]);
        Mma<T>::run(st[kt][1], kf, qf[1][s]);
        Mma<T>::run(dpt[kt][0], vf, df[0][s]);
        Mma<T>::run(dpt[kt][1], vf, df[1][s]);
      }
    const bool diag = kv0 + BKV > tq0;
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
      for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          float p = exp2f(st[kt][c][r] * sc - lse2[c]);
          if (diag && kv0 + kt * 16 + lg * 4 + r > tq0 + c * 16 + l16) p = 0.f;
          st[kt][c][r] = p * (dpt[kt][c][r] - dl[c]);       // dS
        }
    constexpr int NPT = CFrag<T>::NPT;
#pragma unroll
    for (int kk = 0; kk < 4 / NPT; ++kk) {
      f32x4 t0[NPT], t1[NPT];
#pragma unroll
      for (int q = 0; q < NPT; ++q) {
        t0[q] = st[kk * NPT + q][0];
        t1[q] = st[kk * NPT + q][1];
      }
      const V b0 = CFrag<T>::pack(t0), b1 = CFrag<T>::pack(t1);
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) {
        const V ka = CFrag<T>::read(Kt + (dt * 16 + l16) * A::TSTR64, kk * 16 * NPT, lg);
        Mma<T>::run(dq[dt][0], ka, b0);
        Mma<T>::run(dq[dt][1], ka, b1);
      }
    }
  }
  if (!active) return;
  const float scale = 1.0f / sqrtf((float)D);
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    const int t = tq0 + c * 16 + l16;
    T* dst = dqkv + (row0 + t) * ldd + h * D;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      typename A::T4 w;
#pragma unroll
      for (int r = 0; r < 4; ++r) w[r] = from_f32<T>(dq[dt][c][r] * scale);
      *reinterpret_cast<typename A::T4*>(dst + dt * 16 + lg * 4) = w;
    }
  }
}

// --------------------------------------------------------------------------
// backward, dK and dV: one workgroup per 64-key block, 4 wavefronts x 16 keys,
// looping over every later 32-token query block and every head.
// --------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(256) void attn_bwd_dkv_kernel(
    const T* __restrict__ qkv, int ldq, const T* __restrict__ dout, const float* __restrict__ lse,
    const float* __restrict__ delta, int Tn, int H, T* __restrict__ dqkv, int ldd) {
  typedef AttnTypes<T> A;
  typedef typename A::V V;
  __shared__ __align__(16) T Qs[BQ * A::KSTR];
  __shared__ __align__(16) T Qt[D * A::TSTR32];
  __shared__ __align__(16) T Os[BQ * A::KSTR];
  __shared__ __align__(16) T Ot[D * A::TSTR32];
  __shared__ float lse_s[BQ], dl_s[BQ];

  const int nkb = Tn / BKV;
  const int b = blockIdx.x / nkb;
  const int kblk = blockIdx.x % nkb;               // low key blocks carry the most work: first
  const int kv0 = kblk * BKV;
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, l16 = lane & 15, lg = lane >> 4;
  const size_t row0 = (size_t)b * Tn;
  const int ldo = H * D;
  const int key = kv0 + wave * 16 + l16;           // this lane's key column

  V kf[A::NS], vf[A::NS];
#pragma unroll
  for (int s = 0; s < A::NS; ++s) {
    kf[s] = *reinterpret_cast<const V*>(qkv + (row0 + key) * ldq + H * D + s * A::KB + lg * A::VEC);
    vf[s] = *reinterpret_cast<const V*>(qkv + (row0 + key) * ldq + (H + 1) * D + s * A::KB + lg * A::VEC);
  }
  f32x4 dk[8], dv[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) dk[i] = dv[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  const float sc = kLog2e / sqrtf((float)D);
  constexpr int NPT = CFrag<T>::NPT;

  for (int tq0 = kv0; tq0 < Tn; tq0 += BQ) {
    for (int h = 0; h < H; ++h) {
      __syncthreads();
      stage_rows<T, true, true>(qkv + (row0 + tq0) * ldq + h * D, ldq, BQ, Qs, Qt, A::TSTR32, tid, 256);
      stage_rows<T, true, true>(dout + (row0 + tq0) * ldo + h * D, ldo, BQ, Os, Ot, A::TSTR32, tid, 256);
      if (tid < BQ) lse_s[tid] = lse[((size_t)b * H + h) * Tn + tq0 + tid] * kLog2e;
      else if (tid < 2 * BQ) dl_s[tid - BQ] = delta[((size_t)b * H + h) * Tn + tq0 + tid - BQ];
      __syncthreads();

      // S[row][key] and dP[row][key] for 32 rows (2 tiles) x this wave's 16 keys
      f32x4 sa[2], dpa[2];
      sa[0] = sa[1] = dpa[0] = dpa[1] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < A::NS; ++s)
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          const V qa = *reinterpret_cast<const V*>(Qs + (c * 16 + l16) * A::KSTR + s * A::KB + lg * A::VEC);
          const V da = *reinterpret_cast<const V*>(Os + (c * 16 + l16) * A::KSTR + s * A::KB + lg * A::VEC);
          Mma<T>::run(sa[c], qa, kf[s]);
          Mma<T>::run(dpa[c], da, vf[s]);
        }
      const bool diag = tq0 < kv0 + BKV;
      f32x4 pa[2], dsa[2];
#pragma unroll
      for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int rl = c * 16 + lg * 4 + r;     // local query row
          float p = exp2f(sa[c][r] * sc - lse_s[rl]);
          if (diag && key > tq0 + rl) p = 0.f;
          pa[c][r] = p;
          dsa[c][r] = p * (dpa[c][r] - dl_s[rl]);
        }
      // dV^T[d][key] += dO^T[d][rows] P[rows][key];  dK^T += Q^T dS
#pragma unroll
      for (int kk = 0; kk < 2 / NPT; ++kk) {
        const V pb = CFrag<T>::pack(pa + kk * NPT);
        const V sb = CFrag<T>::pack(dsa + kk * NPT);
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) {
          const V oa = CFrag<T>::read(Ot + (dt * 16 + l16) * A::TSTR32, kk * 16 * NPT, lg);
          const V qa = CFrag<T>::read(Qt + (dt * 16 + l16) * A::TSTR32, kk * 16 * NPT, lg);
          Mma<T>::run(dv[dt], oa, pb);
          Mma<T>::run(dk[dt], qa, sb);
        }
      }
    }
  }
  const float scale = 1.0f / sqrtf((float)D);
  T* dkdst = dqkv + (row0 + key) * ldd + H * D;
  T* dvdst = dqkv + (row0 + key) * ldd + (H + 1) * D;
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) {
    typename A::T4 wk, wv;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      wk[r] = from_f32<T>(dk[dt][r] * scale);
      wv[r] = from_f32<T>(dv[dt][r]);
    }
    *reinterpret_cast<typename A::T4*>(dkdst + dt * 16 + lg * 4) = wk;
    *reinterpret_cast<typename A::T4*>(dvdst + dt * 16 + lg * 4) = wv;
  }
}

inline int heads_per_group(int H, int maxw) {
  const int ng = (H + maxw - 1) / maxw;
  return (H + ng - 1) / ng;
}

}  // namespace

hipError_t attn_fwd(DType t, const void* qkv, int ldq, int B, int T, int H, void* o, float* lse,
                    hipStream_t s) {
  if (T % BKV || H < 1 || H > 16) return hipErrorInvalidValue;
  const int hpg = heads_per_group(H, kMaxHeadsPerWG), ng = (H + hpg - 1) / hpg;
  dim3 grid(B * (T / BQ) * ng), block(64 * hpg);
  if (t == DType::BF16)
    hipLaunchKernelGGL(attn_fwd_kernel<bf16>, grid, block, 0, s, static_cast<const bf16*>(qkv), ldq, T,
                       H, hpg, static_cast<bf16*>(o), lse);
  else
    hipLaunchKernelGGL(attn_fwd_kernel<float>, grid, block, 0, s, static_cast<const float*>(qkv), ldq,
                       T, H, hpg, static_cast<float*>(o), lse);
  return hipGetLastError();
}

hipError_t attn_bwd_delta(DType t, const void* o, const void* dout, int B, int T, int H,
                          float* delta, hipStream_t s) {
  const size_t total = (size_t)B * T * H;
  dim3 grid((unsigned)((total + 3) / 4)), block(256);
  if (t == DType::BF16)
    hipLaunchKernelGGL(attn_delta_kernel<bf16>, grid, block, 0, s, static_cast<const bf16*>(o),
                       static_cast<const bf16*>(dout), T, H, total, delta);
  else
    hipLaunchKernelGGL(attn_delta_kernel<float>, grid, block, 0, s, static_cast<const float*>(o),
                       static_cast<const float*>(dout), T, H, total, delta);
  return hipGetLastError();
}

hipError_t attn_bwd(DType t, const void* qkv, int ldq, const void* dout, const float* lse,
                    const float* delta, int B, int T, int H, void* dqkv, int ldd, hipStream_t s) {
  if (T % BKV || H < 1 || H > 16) return hipErrorInvalidValue;
  const int hpg = heads_per_group(H, kMaxHeadsPerWGdQ), ng = (H + hpg - 1) / hpg;
  dim3 gq(B * (T / BQ) * ng), bq(64 * hpg);
  dim3 gk(B * (T / BKV)), bk(256);
  if (t == DType::BF16) {
    const bf16* q = static_cast<const bf16*>(qkv);
    const bf16* d = static_cast<const bf16*>(dout);
    bf16* g = static_cast<bf16*>(dqkv);
    hipLaunchKernelGGL(attn_bwd_dkv_kernel<bf16>, gk, bk, 0, s, q, ldq, d, lse, delta, T, H, g, ldd);
    hipLaunchKernelGGL(attn_bwd_dq_kernel<bf16>, gq, bq, 0, s, q, ldq, d, lse, delta, T, H, hpg, g, ldd);
  } else {
    const float* q = static_cast<const float*>(qkv);
    const float* d = static_cast<const float*>(dout);
    float* g = static_cast<float*>(dqkv);
    hipLaunchKernelGGL(attn_bwd_dkv_kernel<float>, gk, bk, 0, s, q, ldq, d, lse, delta, T, H, g, ldd);
    hipLaunchKernelGGL(attn_bwd_dq_kernel<float>, gq, bq, 0, s, q, ldq, d, lse, delta, T, H, hpg, g, ldd);
  }
  return hipGetLastError();
}

}  // namespace nc
