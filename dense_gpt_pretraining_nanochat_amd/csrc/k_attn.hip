// Causal multi-query attention on the CDNA4 matrix cores: forward, and a
// backward without atomics in one of two forms. With a dS buffer (the
// training step): delta = <dO, O>, then dK/dV (which also stores the dS it
// forms), then dQ as one product over the stored dS. Without one: a dQ
// kernel that recomputes S and dP (and computes delta) runs first, then dK/dV.
//
// All query heads share one key/value head (followin.io release article,
// architecture list: multi-query attention); the objective is next-token
// prediction, so position t attends to keys u <= t (wmrh.cn tutorial, section
// 2.3). Scale 1/sqrt(128).
//
// Layout: the fused projection buffer holds, per token, H query heads, then
// the key head, then the value head, 128 values each (after rotary + QK-norm).
//
// Every tile is staged in LDS row-major ([row][128], 16-byte coalesced global
// loads and LDS writes). Operands that a product needs with the row index as
// its contraction index are read with the gfx950 LDS transpose read
// (ds_read_b64_tr_b16): in each 16-lane group, source lane 4j+q names row
// k0+j, columns n0+4q..n0+4q+3, and output lane i receives rows k0..k0+3 of
// column n0+i - one matrix-core fragment.
//
// Forward (flash style): a workgroup owns 64 query tokens of two heads, one
// wavefront per (head, 32 tokens). Each K/V tile of 64 keys is staged once
// and read by all four wavefronts; the next tile is prefetched into registers
// while the current one is in use (two LDS buffers, one barrier per tile). A
// wavefront computes S^T = K Q^T so each lane column is one query row: the
// softmax sums stay in the lane and P^T feeds O^T += V^T P^T straight from
// registers. The softmax needs no running maximum (see kScoreMax2).
//
// Backward: dK/dV of a 128-key block are summed over all heads and one chunk
// of up to 2048 later query tokens by one workgroup (16 keys per wavefront,
// accumulators in registers, query blocks visited from the last one down so
// that the key blocks of a batch row running together share the Q/dO tiles
// in L2); the work items are issued longest first (early
// key blocks), which balances them under the causal mask; with one chunk per
// key block (T <= 2048) the workgroup writes dK and dV itself, otherwise a
// second pass adds the chunk partials in a fixed order. dQ comes either from
// the stored dS (a bandwidth-bound product: 128 queries x 2 heads per
// workgroup, K staged once for its eight wavefronts) or from a kernel shaped
// like the forward that recomputes S and dP (32-key tiles). No atomics
// anywhere, so the results are bitwise reproducible.
#include <math.h>

#include <mutex>
#include <type_traits>

#include "common.h"
#include "launch.h"

namespace nc {
namespace {

constexpr int D = 128;
constexpr int BQ = 32;        // query tokens per wavefront (fwd, dQ)
constexpr int FQB = 64;       // query tokens per fwd / dQ workgroup (2 heads x 2 x 32)
constexpr int BQK = 64;       // query tokens per step (dK/dV)
constexpr int BKV = 64;       // keys per tile (fwd)
constexpr int BKVQ = 32;      // keys per tile (dQ)
constexpr int BKW = 128;      // keys per dK/dV workgroup (8 wavefronts x 16)
constexpr int DKW_THREADS = 512;
// Query tokens per dK/dV work item (one fp32 partial per chunk). Measured on
// the depth-20 shape (T = 2048, 10 heads), dK/dV + reduction + dQ per layer:
// 512 -> 1468 us, 1024 -> 1382 us, 2048 (one item per key block) -> 1363 us:
// fewer, longer items cost less partial traffic and fewer workgroup starts,
// and issuing them longest first keeps the tail short.
constexpr int QCH = 2048;
// Forward and dQ: 4-wavefront workgroups compiled for two wavefronts per SIMD
// (<= 256 registers), so two workgroups share a CU.
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

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

// Fragments whose contraction index runs over accumulator rows. A lane of
// group g holds rows 4g..4g+3 of each 16-row accumulator tile; bf16 fragments
// span two tiles (contraction 32: rows 4g..4g+3, then 16+4g..16+4g+3), fp32
// fragments one tile (contraction 16).
//   pack(): the operand built from this lane's own accumulators;
//   read(): the matching operand from a row-major LDS array X[k][mn] (stride in
//           elements), lane (g, i) getting column mn0 + i.
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
  __device__ __forceinline__ static bf16x8 read(const bf16* X, int stride, int k0, int mn0,
                                                int lane) {
    const int g = lane >> 4, s = lane & 15;
    const bf16* p0 = X + (k0 + 4 * g + (s >> 2)) * stride + mn0 + 4 * (s & 3);
    const s16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)p0);
    const s16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p0 + 16 * stride));
    typedef short s16x8 __attribute__((ext_vector_type(8)));
    const s16x8 ab = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
    return __builtin_bit_cast(bf16x8, ab);
  }
};
template <> struct CFrag<float> {
  static constexpr int NPT = 1;
  __device__ __forceinline__ static f32x4 pack(const f32x4* t) { return t[0]; }
  __device__ __forceinline__ static f32x4 read(const float* X, int stride, int k0, int mn0,
                                               int lane) {
    const int g = lane >> 4, i = lane & 15;
    const float* p = X + (k0 + 4 * g) * stride + mn0 + i;
    return f32x4{p[0], p[stride], p[2 * stride], p[3 * stride]};
  }
};

template <typename T>
struct AttnTypes {
  static constexpr int VEC = Vec16<T>::N;
  static constexpr int KB = 4 * VEC;           // contraction per fragment
  static constexpr int NS = D / KB;            // fragments along the head dim
  static constexpr int KSTR = D + VEC;         // LDS row stride, 16-byte pad
  // bf16 tiles: a 32-byte pad. Measured with the bank-conflict counter, it
  // leaves both the 16-byte row reads and the transpose reads conflict-free
  // (with the 16-byte pad, 25-44% of the attention kernels' LDS cycles were
  // conflicts): the LDS serves 32 lanes of a 16-byte read, or all 64 lanes
  // of an 8-byte one, per pass over its banks.
  static constexpr int VSTR = sizeof(T) == 2 ? D + 2 * VEC : D + VEC;
  static constexpr int DC = D / VEC;           // 16-byte chunks per 128-wide row
  typedef typename Vec16<T>::type V;
  typedef T T4 __attribute__((ext_vector_type(4)));
};

// A tile of R rows of 128 values, two sources (e.g. K and V, or Q and dO),
// staged row-major into two LDS arrays. bf16 prefetches into registers (up to
// PF chunks per thread); fp32 stages synchronously.
template <typename T, int R, int PF, int S0 = AttnTypes<T>::KSTR, int S1 = AttnTypes<T>::KSTR>
struct PairStager {
  typedef AttnTypes<T> A;
  static constexpr int CHUNKS = 2 * R * A::DC;
  typename A::V reg[PF];

  __device__ __forceinline__ static const T* src_of(const T* s0, const T* s1, size_t ld, int c) {
    const int which = c / (R * A::DC), r = (c / A::DC) % R, dc = c % A::DC;
    return (which ? s1 : s0) + (size_t)r * ld + dc * A::VEC;
  }
  __device__ __forceinline__ static T* dst_of(T* d0, T* d1, int c) {
    const int which = c / (R * A::DC), r = (c / A::DC) % R, dc = c % A::DC;
    return (which ? d1 + r * S1 : d0 + r * S0) + dc * A::VEC;
  }
  __device__ __forceinline__ void load(const T* s0, const T* s1, size_t ld, int tid, int nthr) {
#pragma unroll
    for (int i = 0; i < PF; ++i) {
      const int c = tid + i * nthr;
      if (c < CHUNKS) reg[i] = *reinterpret_cast<const typename A::V*>(src_of(s0, s1, ld, c));
    }
  }
  __device__ __forceinline__ void store(T* d0, T* d1, int tid, int nthr) const {
#pragma unroll
    for (int i = 0; i < PF; ++i) {
      const int c = tid + i * nthr;
      if (c < CHUNKS) *reinterpret_cast<typename A::V*>(dst_of(d0, d1, c)) = reg[i];
    }
  }
  __device__ __forceinline__ static void copy(const T* s0, const T* s1, size_t ld, T* d0, T* d1,
                                              int tid, int nthr) {
    for (int c = tid; c < CHUNKS; c += nthr)
      *reinterpret_cast<typename A::V*>(dst_of(d0, d1, c)) =
          *reinterpret_cast<const typename A::V*>(src_of(s0, s1, ld, c));
  }
};

// workgroup -> (batch, query block, head group); heavy (late) query blocks first
struct QBlock {
  int b, qb, hg;
};
__device__ __forceinline__ QBlock qblock_of(int bid, int nqb, int ngroups) {
  // the hardware deals workgroups to the 8 XCDs round-robin; remapped, each
  // XCD takes a contiguous range (whole batch rows), so the workgroups running
  // on one XCD share their row's K/V tiles in its L2
  const int nb = gridDim.x;
  if ((nb & 7) == 0) bid = (bid & 7) * (nb >> 3) + (bid >> 3);
  const int per_b = nqb * ngroups;
  QBlock q;
  q.b = bid / per_b;
  const int r = bid % per_b;
  q.qb = nqb - 1 - r / ngroups;
  q.hg = r % ngroups;
  return q;
}

constexpr bool kPrefetch(int esz) { return esz == 2; }

// --------------------------------------------------------------------------
// forward
// --------------------------------------------------------------------------
// Softmax without a running maximum. The query and key head vectors arrive
// RMS-normalised (QK-norm), so |q|, |k| <= sqrt(128) and every scaled score
// q.k / sqrt(128) is at most sqrt(128) = 11.31 (Cauchy-Schwarz). Subtracting
// the fixed bound kScoreMax2 (log2 domain, with margin for bf16 rounding of
// q and k) instead of the row maximum keeps every exponent <= 0 and >= -33,
// so p = 2^(s - bound) neither overflows nor underflows in fp32, and the
// output sum_u p_u v_u / sum_u p_u is the softmax exactly (up to rounding).
// That removes the per-tile maximum, its shuffles and the rescaling of the
// output accumulators; per score the vector work is one FMA, one exp2, one
// add and half a conversion.
constexpr float kScoreMax2 = 17.0f;   // > sqrt(128) * log2(e) = 16.32

template <typename T>
__global__ __launch_bounds__(256, sizeof(T) == 2 ? 2 : 1) void attn_fwd_kernel(
    const T* __restrict__ qkv, int ldq, int Tn, int H, T* __restrict__ o, float* __restrict__ lse) {
  typedef AttnTypes<T> A;
  typedef typename A::V V;
  constexpr int KT = BKV * A::VSTR;            // K tile: row-major, read with 16-byte reads
  constexpr int VT = BKV * A::VSTR;            // V tile: row-major, read with transpose reads
  __shared__ __align__(16) T Ks[2 * KT];
  __shared__ __align__(16) T Vs[2 * VT];

  // workgroup: 64 query tokens x 2 heads; wavefront w: head 2*pair + (w & 1),
  // query tokens tq0 .. tq0 + 31 with tq0 = block start + 32 * (w >> 1)
  const QBlock qbk = qblock_of(blockIdx.x, Tn / FQB, (H + 1) / 2);
  const int tb0 = qbk.qb * FQB;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63, l16 = lane & 15, lg = lane >> 4;
  const int h = 2 * qbk.hg + (wave & 1);
  const int tq0 = tb0 + BQ * (wave >> 1);
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
  float lsum[2] = {0.f, 0.f};                  // this lane's share of the row sums
  const float sc = kLog2e / sqrtf((float)D);

  constexpr bool PFT = kPrefetch(sizeof(T));
  constexpr int NT = 256;                       // threads per workgroup
  typedef PairStager<T, BKV, PFT ? 8 : 1, A::VSTR, A::VSTR> Stager;
  Stager stg;
  const int ntiles = (tb0 + FQB + BKV - 1) / BKV;   // the last tile is the diagonal one
  if (PFT) {
    stg.load(kbase + row0 * ldq, vbase + row0 * ldq, ldq, tid, NT);
    stg.store(Ks, Vs, tid, NT);
  } else {
    Stager::copy(kbase + row0 * ldq, vbase + row0 * ldq, ldq, Ks, Vs, tid, NT);
  }
  __syncthreads();

  // One K/V tile: S^T = K Q^T (lane (lg, l16) holds keys kv0 + 16 kt + 4 lg + r
  // of query c*16 + l16), p = 2^(s*scale - bound), O^T += V^T P^T. Wavefronts
  // without a head (odd H) run on zero queries and store nothing. Only the
  // last tile needs the causal mask.
  auto tile = [&](auto masked, const T* K, const T* Vv, int kv0) {
    constexpr bool MASKED = decltype(masked)::value;
    f32x4 st[4][2];
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) st[kt][0] = st[kt][1] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < A::NS; ++s)
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) {
        const V kf = *reinterpret_cast<const V*>(K + (kt * 16 + l16) * A::VSTR + s * A::KB + lg * A::VEC);
        Mma<T>::run(st[kt][0], kf, qf[0][s]);
        Mma<T>::run(st[kt][1], kf, qf[1][s]);
      }
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
      for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          float p = __builtin_amdgcn_exp2f(fmaf(st[kt][c][r], sc, -kScoreMax2));
          if constexpr (MASKED) {
            if (kv0 + kt * 16 + lg * 4 + r > tq0 + c * 16 + l16) p = 0.f;
          }
          st[kt][c][r] = p;
          lsum[c] += p;
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
        const V va = CFrag<T>::read(Vv, A::VSTR, kk * 16 * NPT, dt * 16, lane);
        Mma<T>::run(oacc[dt][0], va, pb0);
        Mma<T>::run(oacc[dt][1], va, pb1);
      }
    }
  };

  for (int it = 0; it + 1 < ntiles; ++it) {
    const int kv0 = it * BKV;
    T* Kn = Ks + ((it + 1) & 1) * KT;
    T* Vn = Vs + ((it + 1) & 1) * VT;
    if (PFT)
      stg.load(kbase + (row0 + kv0 + BKV) * ldq, vbase + (row0 + kv0 + BKV) * ldq, ldq, tid, NT);
    tile(std::false_type{}, Ks + (it & 1) * KT, Vs + (it & 1) * VT, kv0);
    if (PFT) {
      stg.store(Kn, Vn, tid, NT);
    } else {
      __syncthreads();   // single-buffered fp32 path: wait for readers first
      Stager::copy(kbase + (row0 + kv0 + BKV) * ldq, vbase + (row0 + kv0 + BKV) * ldq, ldq, Kn,
                   Vn, tid, NT);
    }
    __syncthreads();
  }
  {
    const int it = ntiles - 1;
    tile(std::true_type{}, Ks + (it & 1) * KT, Vs + (it & 1) * VT, it * BKV);
  }
  if (!active) return;
  const int ldo = H * D;
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    const float l = group4_sum(lsum[c]);
    const float inv = 1.0f / l;
    const int t = tq0 + c * 16 + l16;
    T* dst = o + (row0 + t) * ldo + h * D;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      typename A::T4 w;
#pragma unroll
      for (int r = 0; r < 4; ++r) w[r] = from_f32<T>(oacc[dt][c][r] * inv);
      *reinterpret_cast<typename A::T4*>(dst + dt * 16 + lg * 4) = w;
    }
    if (lg == 0) lse[((size_t)qbk.b * H + h) * Tn + t] = (kScoreMax2 + log2f(l)) * kLn2;
  }
}

// --------------------------------------------------------------------------
// backward, dQ: shaped like the forward (one wavefront per head, 32 rows)
// --------------------------------------------------------------------------
// It also computes delta[b, h, t] = <dO, O> of its own query rows (each row's
// 128 values sit in the four lanes of one column of the dO fragments; O is
// read in the same layout) and writes it for the dK/dV kernel, which runs
// after it.
template <typename T>
__global__ __launch_bounds__(256, 2) void attn_bwd_dq_kernel(
    const T* __restrict__ qkv, int ldq, const T* __restrict__ o, const T* __restrict__ dout,
    const float* __restrict__ lse, float* __restrict__ delta, int Tn, int H, T* __restrict__ dqkv,
    int ldd) {
  typedef AttnTypes<T> A;
  typedef typename A::V V;
  constexpr int BK = BKVQ;                      // keys per tile
  constexpr int TILE = BK * A::VSTR;
  __shared__ __align__(16) T Ks[2 * TILE];
  __shared__ __align__(16) T Vs[2 * TILE];

  // workgroup: 64 query tokens x 2 heads, as in the forward
  const QBlock qbk = qblock_of(blockIdx.x, Tn / FQB, (H + 1) / 2);
  const int tb0 = qbk.qb * FQB;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63, l16 = lane & 15, lg = lane >> 4;
  const int h = 2 * qbk.hg + (wave & 1);
  const int tq0 = tb0 + BQ * (wave >> 1);
  const bool active = h < H;
  const size_t row0 = (size_t)qbk.b * Tn;
  const int ldo = H * D;

  V qf[2][A::NS], df[2][A::NS];
  float lse2[2], dl[2];
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    const int t = tq0 + c * 16 + l16;
    float pd = 0.f;
#pragma unroll
    for (int s = 0; s < A::NS; ++s) {
      qf[c][s] = active ? *reinterpret_cast<const V*>(qkv + (row0 + t) * ldq + h * D + s * A::KB + lg * A::VEC) : V{};
      df[c][s] = active ? *reinterpret_cast<const V*>(dout + (row0 + t) * ldo + h * D + s * A::KB + lg * A::VEC) : V{};
      const V of = active ? *reinterpret_cast<const V*>(o + (row0 + t) * ldo + h * D + s * A::KB + lg * A::VEC) : V{};
#pragma unroll
      for (int e = 0; e < A::VEC; ++e) pd = fmaf(to_f32(df[c][s][e]), to_f32(of[e]), pd);
    }
    dl[c] = group4_sum(pd);
    lse2[c] = active ? lse[((size_t)qbk.b * H + h) * Tn + t] * kLog2e : 0.f;
    if (active && lg == 0) delta[((size_t)qbk.b * H + h) * Tn + t] = dl[c];
  }
  f32x4 dq[8][2];
#pragma unroll
  for (int i = 0; i < 8; ++i) dq[i][0] = dq[i][1] = f32x4{0.f, 0.f, 0.f, 0.f};
  const float sc = kLog2e / sqrtf((float)D);
  const T* kbase = qkv + H * D;
  const T* vbase = qkv + (H + 1) * D;

  constexpr bool PFT = kPrefetch(sizeof(T));
  constexpr int NT = 256;                       // threads per workgroup
  typedef PairStager<T, BK, PFT ? 4 : 1, A::VSTR, A::VSTR> Stager;
  Stager stg;
  // tiles 0 .. ntiles - 3 lie below every query of the block; the last two
  // (keys tb0 .. tb0 + 63) need the causal mask
  const int ntiles = (tb0 + FQB + BK - 1) / BK;
  if (PFT) {
    stg.load(kbase + row0 * ldq, vbase + row0 * ldq, ldq, tid, NT);
    stg.store(Ks, Vs, tid, NT);
  } else {
    Stager::copy(kbase + row0 * ldq, vbase + row0 * ldq, ldq, Ks, Vs, tid, NT);
  }
  __syncthreads();

  // One K/V tile: S^T and dP^T, dS = P (dP - delta), dQ += dS K. Inactive
  // wavefronts run on zero Q/dO fragments, which gives dS = 0.
  auto tile = [&](auto masked, const T* K, const T* Vv, int kv0) {
    constexpr bool MASKED = decltype(masked)::value;
    f32x4 st[BK / 16][2], dpt[BK / 16][2];
#pragma unroll
    for (int kt = 0; kt < BK / 16; ++kt)
      st[kt][0] = st[kt][1] = dpt[kt][0] = dpt[kt][1] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < A::NS; ++s)
#pragma unroll
      for (int kt = 0; kt < BK / 16; ++kt) {
        const V kf = *reinterpret_cast<const V*>(K + (kt * 16 + l16) * A::VSTR + s * A::KB + lg * A::VEC);
        const V vf = *reinterpret_cast<const V*>(Vv + (kt * 16 + l16) * A::VSTR + s * A::KB + lg * A::VEC);
        Mma<T>::run(st[kt][0], kf, qf[0][s]);
        Mma<T>::run(st[kt][1], kf, qf[1][s]);
        Mma<T>::run(dpt[kt][0], vf, df[0][s]);
        Mma<T>::run(dpt[kt][1], vf, df[1][s]);
      }
#pragma unroll
    for (int kt = 0; kt < BK / 16; ++kt)
#pragma unroll
      for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          float p = __builtin_amdgcn_exp2f(fmaf(st[kt][c][r], sc, -lse2[c]));
          if constexpr (MASKED) {
            if (kv0 + kt * 16 + lg * 4 + r > tq0 + c * 16 + l16) p = 0.f;
          }
          st[kt][c][r] = p * (dpt[kt][c][r] - dl[c]);       // dS
        }
    constexpr int NPT = CFrag<T>::NPT;
#pragma unroll
    for (int kk = 0; kk < BK / 16 / NPT; ++kk) {
      f32x4 t0[NPT], t1[NPT];
#pragma unroll
      for (int q = 0; q < NPT; ++q) {
        t0[q] = st[kk * NPT + q][0];
        t1[q] = st[kk * NPT + q][1];
      }
      const V b0 = CFrag<T>::pack(t0), b1 = CFrag<T>::pack(t1);
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) {
        const V ka = CFrag<T>::read(K, A::VSTR, kk * 16 * NPT, dt * 16, lane);   // K^T
        Mma<T>::run(dq[dt][0], ka, b0);
        Mma<T>::run(dq[dt][1], ka, b1);
      }
    }
  };
  auto next = [&](int it) {                      // stage tile it + 1, then barrier
    const int kv0 = it * BK;
    T* Kn = Ks + ((it + 1) & 1) * TILE;
    T* Vn = Vs + ((it + 1) & 1) * TILE;
    if (PFT) {
      stg.store(Kn, Vn, tid, NT);
    } else {
      __syncthreads();
      Stager::copy(kbase + (row0 + kv0 + BK) * ldq, vbase + (row0 + kv0 + BK) * ldq, ldq, Kn, Vn,
                   tid, NT);
    }
    __syncthreads();
  };

  for (int it = 0; it + 2 < ntiles; ++it) {
    const int kv0 = it * BK;
    if (PFT) stg.load(kbase + (row0 + kv0 + BK) * ldq, vbase + (row0 + kv0 + BK) * ldq, ldq, tid, NT);
    tile(std::false_type{}, Ks + (it & 1) * TILE, Vs + (it & 1) * TILE, kv0);
    next(it);
  }
  {
    const int it = ntiles - 2, kv0 = it * BK;   // keys tb0 .. tb0 + 31
    if (PFT) stg.load(kbase + (row0 + kv0 + BK) * ldq, vbase + (row0 + kv0 + BK) * ldq, ldq, tid, NT);
    tile(std::true_type{}, Ks + (it & 1) * TILE, Vs + (it & 1) * TILE, kv0);
    next(it);
  }
  {
    const int it = ntiles - 1, kv0 = it * BK;   // keys tb0 + 32 .. tb0 + 63: none for the lower half
    if (kv0 < tq0 + BQ) tile(std::true_type{}, Ks + (it & 1) * TILE, Vs + (it & 1) * TILE, kv0);
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
// delta[b, h, t] = <dO, O> of each query row and head: 16 lanes per row of 128,
// 16-byte loads (the dK/dV kernel needs it before any dQ work when dQ is
// formed from the stored dS).
// --------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(256) void attn_delta_kernel(const T* __restrict__ o,
                                                         const T* __restrict__ dout, int Tn,
                                                         int H, size_t total,
                                                         float* __restrict__ delta) {
  typedef AttnTypes<T> A;
  constexpr int PER = D / 16;                  // elements per lane
  const size_t w = blockIdx.x * 16ull + (threadIdx.x >> 4);
  const int sl = threadIdx.x & 15;
  if (w >= total) return;
  const size_t m = w / H;
  const int h = (int)(w % H);
  const size_t off = m * (size_t)(H * D) + h * D + sl * PER;
  float acc = 0.f;
#pragma unroll
  for (int v = 0; v < PER / A::VEC; ++v) {
    const typename A::V a = *reinterpret_cast<const typename A::V*>(o + off + v * A::VEC);
    const typename A::V c = *reinterpret_cast<const typename A::V*>(dout + off + v * A::VEC);
#pragma unroll
    for (int e = 0; e < A::VEC; ++e) acc = fmaf(to_f32(c[e]), to_f32(a[e]), acc);
  }
  acc = lane16_sum(acc);
  if (sl == 0) {
    const size_t bb = m / Tn, t = m % Tn;
    delta[(bb * H + h) * Tn + t] = acc;
  }
}

// Stored dS^T: within each 64-query block of a key row, lane group lg of the
// writing wavefront keeps its 16 values (queries 16c + 4lg + r, c and r < 4)
// as 16-byte chunks lg, 4 + lg, ... (bf16: 8 values per chunk, fp32: 4), so
// query q = 16c + 4lg + r sits at position chunk * E + e with
// idx = 4c + r, chunk = (idx / E) * 4 + lg, e = idx % E. Here c counts 16-query
// tiles from the start of a run of 64-query blocks (block c / 4).
template <typename T>
__device__ __forceinline__ int ds_chunk_pos(int c, int lg, int r) {
  constexpr int E = Vec16<T>::N;
  const int idx = 4 * (c & 3) + r;
  return 64 * (c >> 2) + ((idx / E) * 4 + lg) * E + idx % E;
}

// B operand of dQ^T += K^T dS^T from an LDS copy of stored dS^T rows (keys
// k0.., 64 queries per row in the order above): the same fragment that
// CFrag<T>::read gives for plain rows, query tile c (16 queries) of the block.
template <typename T> struct DsFrag;
template <> struct DsFrag<bf16> {
  __device__ __forceinline__ static bf16x8 read(const bf16* X, int stride, int k0, int c, int lane) {
    // source lane 4j + q names row k0 + j, the four values of queries
    // 16c + 4q .. +3, which are consecutive positions
    const int g = lane >> 4, s = lane & 15;
    const bf16* p0 = X + (k0 + 4 * g + (s >> 2)) * stride + ds_chunk_pos<bf16>(c, s & 3, 0);
    const s16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)p0);
    const s16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p0 + 16 * stride));
    typedef short s16x8 __attribute__((ext_vector_type(8)));
    const s16x8 ab = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
    return __builtin_bit_cast(bf16x8, ab);
  }
};
template <> struct DsFrag<float> {
  __device__ __forceinline__ static f32x4 read(const float* X, int stride, int k0, int c, int lane) {
    const int g = lane >> 4, i = lane & 15;
    const float* p = X + (k0 + 4 * g) * stride + ds_chunk_pos<float>(c, i >> 2, i & 3);
    return f32x4{p[0], p[stride], p[2 * stride], p[3 * stride]};
  }
};

// --------------------------------------------------------------------------
// dQ from the stored dS: dQ^T[d][t] = sum_u K^T[d][u] dS^T[u][t] / sqrt(128),
// one product instead of the three of attn_bwd_dq_kernel (which recomputes S
// and dP). A workgroup owns 128 query tokens of two heads, one wavefront per
// (head, 32 tokens); each 32-key tile stages K [32 x 128] once for the eight
// wavefronts and the two heads' dS^T [32 keys x 128 queries] in LDS
// (registers two tiles ahead), and both operands are read with the LDS
// transpose read (contraction over rows). dS^T was written for every
// (key, query) pair this reads, zero where the causal mask removes it, so no
// mask is applied here; tiles wholly past a wavefront's queries are skipped.
// When T is not a multiple of 128 the last block's upper half lies past T:
// its wavefronts only help stage and store nothing.
// --------------------------------------------------------------------------
constexpr int DQB = 128;      // query tokens per dQ-from-dS workgroup
template <typename T>
__global__ __launch_bounds__(512, 4) void attn_bwd_dq_ds_kernel(const T* __restrict__ qkv, int ldq,
                                                             const T* __restrict__ ds, int Tn,
                                                             int H, T* __restrict__ dqkv,
                                                             int ldd) {
  typedef AttnTypes<T> A;
  typedef typename A::V V;
  constexpr int BK = BKVQ;                      // keys per tile
  constexpr int KT = BK * A::VSTR;              // K tile (elements)
  constexpr int DSTR = DQB + (sizeof(T) == 2 ? 2 * A::VEC : A::VEC);   // dS^T row: 128 queries + pad
  constexpr int DT = BK * DSTR;                 // dS^T tile of one head
  constexpr int KCH = BK * A::DC;               // 16-byte chunks of a K tile
  constexpr int DCH = DQB / A::VEC;             // 16-byte chunks of a dS^T row
  constexpr int CH = KCH + 2 * BK * DCH;        // chunks staged per tile
  constexpr int NT = 512;
  static_assert(CH % NT == 0, "whole chunks per thread");
  constexpr int PF = CH / NT;
  __shared__ __align__(16) T Ks[2 * KT];
  __shared__ __align__(16) T Ds[2 * 2 * DT];   // [buffer][head of the pair]

  const QBlock qbk = qblock_of(blockIdx.x, (Tn + DQB - 1) / DQB, (H + 1) / 2);
  const int tb0 = qbk.qb * DQB;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int hl = wave & 1;
  const int h = 2 * qbk.hg + hl;
  const int tq0 = tb0 + BQ * (wave >> 1);
  const bool active = h < H && tq0 < Tn;
  const size_t row0 = (size_t)qbk.b * Tn;
  const int Tpad = (Tn + BKW - 1) / BKW * BKW, nqb = (Tn + DQB - 1) / DQB;
  // for an odd head count the last pair's second head reads the first's rows (never stored)
  const int h1 = min(2 * qbk.hg + 1, H - 1);
  const T* ds0 = ds + (((size_t)qbk.b * H + 2 * qbk.hg) * nqb + qbk.qb) * Tpad * DQB;
  const T* ds1 = ds + (((size_t)qbk.b * H + h1) * nqb + qbk.qb) * Tpad * DQB;
  const T* kbase = qkv + row0 * ldq + H * D;

  auto src_of = [&](int kv0, int c) -> const T* {
    if (c < KCH) return kbase + (size_t)(kv0 + c / A::DC) * ldq + (c % A::DC) * A::VEC;
    c -= KCH;
    const int j = c / (BK * DCH), r = (c / DCH) % BK, dc = c % DCH;
    // (queries past T, in the last block when T % 128 == 64: never written, never used)
    return (j ? ds1 : ds0) + (size_t)(kv0 + r) * DQB + dc * A::VEC;
  };
  auto dst_of = [&](int buf, int c) -> T* {
    if (c < KCH) return Ks + buf * KT + (c / A::DC) * A::VSTR + (c % A::DC) * A::VEC;
    c -= KCH;
    const int j = c / (BK * DCH), r = (c / DCH) % BK, dc = c % DCH;
    return Ds + (buf * 2 + j) * DT + r * DSTR + dc * A::VEC;
  };
  typedef V Regs[PF];
  auto load = [&](int kv0, Regs& reg) {
#pragma unroll
    for (int i = 0; i < PF; ++i) reg[i] = *reinterpret_cast<const V*>(src_of(kv0, tid + i * NT));
  };
  auto store = [&](int buf, const Regs& reg) {
#pragma unroll
    for (int i = 0; i < PF; ++i) *reinterpret_cast<V*>(dst_of(buf, tid + i * NT)) = reg[i];
  };

  f32x4 dq[8][2];
#pragma unroll
  for (int i = 0; i < 8; ++i) dq[i][0] = dq[i][1] = f32x4{0.f, 0.f, 0.f, 0.f};
  constexpr int NPT = CFrag<T>::NPT;
  const int ntiles = min(tb0 + DQB, Tn) / BK;   // keys 0 .. last query of the block (at least 2 tiles)
  // Tiles go HBM -> registers two tiles ahead of their use (two register
  // sets, alternating) -> LDS one tile ahead (two buffers): one tile of
  // loads in flight per workgroup did not cover the load latency.
  Regs ra, rb;
  load(0, ra);
  store(0, ra);
  __syncthreads();
  load(BK, ra);                                 // tile 1
  if (ntiles > 2) load(2 * BK, rb);             // tile 2
  const int c0 = (tq0 - tb0) / 16;              // the wavefront's first 16-query tile in the block
  // step it computes tile it from buffer it & 1; `nxt` holds tile it + 1
  auto step = [&](int it, Regs& nxt) {
    const int kv0 = it * BK;
    if (active && kv0 < tq0 + BQ) {             // some key of the tile is <= a query of the wavefront
      const T* K = Ks + (it & 1) * KT;
      const T* Dh = Ds + ((it & 1) * 2 + hl) * DT;
#pragma unroll
      for (int kk = 0; kk < BK / 16 / NPT; ++kk) {
        const V b0 = DsFrag<T>::read(Dh, DSTR, kk * 16 * NPT, c0, lane);
        const V b1 = DsFrag<T>::read(Dh, DSTR, kk * 16 * NPT, c0 + 1, lane);
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) {
          const V ka = CFrag<T>::read(K, A::VSTR, kk * 16 * NPT, dt * 16, lane);   // K^T
          Mma<T>::run(dq[dt][0], ka, b0);
          Mma<T>::run(dq[dt][1], ka, b1);
        }
      }
    }
    if (it + 1 < ntiles) {
      // buffer (it + 1) & 1 was last read in step it - 1, before the barrier that ended it
      store((it + 1) & 1, nxt);
      if (it + 3 < ntiles) load((it + 3) * BK, nxt);
      __syncthreads();
    }
  };
  int it = 0;
  for (; it + 1 < ntiles; it += 2) {
    step(it, ra);
    step(it + 1, rb);
  }
  if (it < ntiles) step(it, ra);
  if (!active) return;
  const float scale = 1.0f / sqrtf((float)D);
  const int l16 = lane & 15, lg = lane >> 4;
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
// backward, dK and dV: one workgroup per 128-key block (and query chunk), 8
// wavefronts x 16 keys, looping over the chunk's 64-token query blocks (from
// the last one down) and, inside each, every head.
// --------------------------------------------------------------------------
__host__ __device__ inline int dkv_chunks(int Tn, int kblk) {
  return (Tn - kblk * BKW + QCH - 1) / QCH;
}

// Work item i (per batch) -> (key block, query chunk), key blocks in order.
__device__ inline void dkv_item(int Tn, int i, int* kblk, int* chunk) {
  const int nkb = (Tn + BKW - 1) / BKW;
  int kb = 0;
  for (; kb < nkb; ++kb) {
    const int n = dkv_chunks(Tn, kb);
    if (i < n) break;
    i -= n;
  }
  *kblk = kb;
  *chunk = i;
}

// DIRECT (one query chunk per key block, T <= QCH): dK (scaled by 1/sqrt(D))
// and dV (times rs of its row, when rs is given) go straight into the key and
// value columns of dqkv; otherwise each chunk leaves an fp32 partial for
// attn_dkv_reduce_kernel.
// STORE_DS: the workgroup also writes the dS^T values it forms (its 128 keys x
// its query chunk, every head) in the activation type into ds, laid out
// [b][h][query block of 128][key < Tpad][128 queries] (Tpad = T rounded up to
// 128, so a wavefront whose keys lie past T writes into pad rows instead of
// branching), for the dQ kernel that reads them instead of recomputing S and
// dP: each of its workgroups then reads one contiguous stretch.
template <typename T, bool DIRECT, bool STORE_DS>
__global__ __launch_bounds__(DKW_THREADS) void attn_bwd_dkv_kernel(
    const T* __restrict__ qkv, int ldq, const T* __restrict__ dout, const float* __restrict__ lse,
    const float* __restrict__ delta, int B, int Tn, int H, float* __restrict__ part,
    T* __restrict__ dqkv, int ldd, const float* __restrict__ rs, T* __restrict__ ds) {
  typedef AttnTypes<T> A;
  typedef typename A::V V;
  constexpr int SQ = BQK;                      // query rows per step
  // Q and dO are read both as 16-byte row fragments and with the transpose
  // read: the 32-byte row pad keeps both patterns free of bank conflicts
  constexpr int ST = A::VSTR;
  constexpr int TILE = SQ * ST;
  __shared__ __align__(16) T Qs[2 * TILE];
  __shared__ __align__(16) T Os[2 * TILE];
  __shared__ float stat_s[2][2 * SQ];          // lse (log2 domain), then delta

  // items are numbered item-major, batch-minor: early (long) key blocks start first
  const int b = blockIdx.x % B;
  int kblk, chunk;
  dkv_item(Tn, blockIdx.x / B, &kblk, &chunk);
  const int kv0 = kblk * BKW;
  const int q0 = kv0 + chunk * QCH;                      // first query token of this chunk
  const int q1 = min(Tn, q0 + QCH);
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63, l16 = lane & 15, lg = lane >> 4;
  const size_t row0 = (size_t)b * Tn;
  const int ldo = H * D;
  const int key0 = kv0 + wave * 16;            // this wave's 16 keys: key0 + l16
  // T is a multiple of 64, so a wave's 16 keys are either all inside or all past T
  const bool kact = key0 < Tn;

  V kf[1][A::NS], vf[1][A::NS];
#pragma unroll
  for (int kt = 0; kt < 1; ++kt)
#pragma unroll
    for (int s = 0; s < A::NS; ++s) {
      const size_t r = row0 + key0 + kt * 16 + l16;
      kf[kt][s] = kact ? *reinterpret_cast<const V*>(qkv + r * ldq + H * D + s * A::KB + lg * A::VEC) : V{};
      vf[kt][s] = kact ? *reinterpret_cast<const V*>(qkv + r * ldq + (H + 1) * D + s * A::KB + lg * A::VEC) : V{};
    }
  f32x4 dk[8][1], dv[8][1];
#pragma unroll
  for (int i = 0; i < 8; ++i) dk[i][0] = dv[i][0] = f32x4{0.f, 0.f, 0.f, 0.f};
  const float sc = kLog2e / sqrtf((float)D);
  constexpr int NPT = CFrag<T>::NPT;

  // iteration space: query blocks tq0 = q0, q0+SQ, ... < q1 and heads h
  const int nqb = (q1 - q0) / SQ;
  const int niter = nqb * H;
  constexpr bool PFT = kPrefetch(sizeof(T));
  // Query blocks are visited from the last one down: the workgroups of one
  // batch row (one XCD) that run together then read the same Q/dO tiles at
  // about the same time, and the later ones find them in L2.
  auto qblk = [&](int i) { return q0 + (nqb - 1 - i / H) * SQ; };
  auto qsrc = [&](int i) { return qkv + (row0 + qblk(i)) * ldq + (i % H) * D; };
  auto osrc = [&](int i) { return dout + (row0 + qblk(i)) * ldo + (i % H) * D; };
  // Per-row statistics of step i: threads tid < SQ hold lse, SQ <= tid < 2 SQ
  // delta. Every thread loads an in-range element (of either array), so the
  // load needs no branch; lse goes to the log2 domain only when it is stored.
  // (A load under a branch, or a use right after it, makes the compiler wait
  // for every load in flight, the tile prefetch included.)
  const float* stat_src = (tid & SQ) ? delta : lse;
  auto stat_raw = [&](int i) -> float {
    const int h = i % H, t = qblk(i) + (tid % SQ);
    return stat_src[((size_t)b * H + h) * Tn + t];
  };
  auto stat_put = [&](int buf, float raw) {
    if (tid < 2 * SQ) stat_s[buf][tid] = tid < SQ ? raw * kLog2e : raw;
  };
  // Q and dO rows have different strides: staged chunk by chunk from either source
  for (int c = tid; c < 2 * SQ * A::DC; c += DKW_THREADS) {
    const int which = c / (SQ * A::DC), r = (c / A::DC) % SQ, dc = c % A::DC;
    const T* src = which ? osrc(0) + (size_t)r * ldo : qsrc(0) + (size_t)r * ldq;
    *reinterpret_cast<V*>((which ? Os : Qs) + r * ST + dc * A::VEC) =
        *reinterpret_cast<const V*>(src + dc * A::VEC);
  }
  stat_put(0, stat_raw(0));
  __syncthreads();

  // bf16: Q/dO tiles are prefetched into registers two steps ahead (one step
  // of math does not cover the load latency), alternating between two sets
  constexpr int NPRE = 2 * SQ * A::DC / DKW_THREADS;
  typedef typename A::V PreSet[PFT ? NPRE : 1];
  auto prefetch = [&](int i, PreSet& pre) {
#pragma unroll
    for (int j = 0; j < NPRE; ++j) {
      const int c = tid + j * DKW_THREADS;     // NPRE * threads = 2 * SQ * DC chunks
      const int which = c / (SQ * A::DC), r = (c / A::DC) % SQ, dc = c % A::DC;
      const T* src = which ? osrc(i) + (size_t)r * ldo : qsrc(i) + (size_t)r * ldq;
      pre[j] = *reinterpret_cast<const V*>(src + dc * A::VEC);
    }
  };
  PreSet preA, preB;
  // prefetches past the last step reload the last step's tile (in range, never used)
  if (PFT) prefetch(min(1, niter - 1), preA);

  auto step = [&](const int it, PreSet& pre, PreSet& pre2) {
    const int tq0 = qblk(it);
    const T* Q = Qs + (it & 1) * TILE;
    const T* O = Os + (it & 1) * TILE;
    const float* lse_s = stat_s[it & 1];
    const float* dl_s = stat_s[it & 1] + SQ;
    const bool more = it + 1 < niter;
    // next step's lse / delta, requested now and stored after this step's math
    const float stat_next = stat_raw(more ? it + 1 : it);
    if (PFT) prefetch(min(it + 2, niter - 1), pre2);

    // (a wavefront whose keys lie past T works on zero K/V fragments and
    // stores nothing: no branch here keeps the accumulators in place)
    {
    // S[row][key] and dP[row][key]: 2 row tiles x 2 key tiles
    constexpr int NC = SQ / 16;                // 16-row query tiles per step
    f32x4 sa[NC][1], dpa[NC][1];
#pragma unroll
    for (int c = 0; c < NC; ++c) sa[c][0] = dpa[c][0] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < A::NS; ++s)
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        const V qa = *reinterpret_cast<const V*>(Q + (c * 16 + l16) * ST + s * A::KB + lg * A::VEC);
        const V da = *reinterpret_cast<const V*>(O + (c * 16 + l16) * ST + s * A::KB + lg * A::VEC);
#pragma unroll
        for (int kt = 0; kt < 1; ++kt) {
          Mma<T>::run(sa[c][kt], qa, kf[kt][s]);
          Mma<T>::run(dpa[c][kt], da, vf[kt][s]);
        }
      }
    // only steps that reach the wavefront's keys need the causal mask: a
    // uniform branch picks the unmasked code for all the others
    f32x4 pa[1][NC], dsa[1][NC];   // [kt][c]
    auto softmax = [&](auto masked) {
      constexpr bool MASKED = decltype(masked)::value;
#pragma unroll
      for (int c = 0; c < NC; ++c)
#pragma unroll
        for (int kt = 0; kt < 1; ++kt)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int rl = c * 16 + lg * 4 + r;     // local query row
            float p = __builtin_amdgcn_exp2f(fmaf(sa[c][kt][r], sc, -lse_s[rl]));
            if constexpr (MASKED) {
              if (key0 + kt * 16 + l16 > tq0 + rl) p = 0.f;
            }
            pa[kt][c][r] = p;
            dsa[kt][c][r] = p * (dpa[c][kt][r] - dl_s[rl]);
          }
    };
    if (tq0 < key0 + 16) softmax(std::true_type{});
    else softmax(std::false_type{});
    if constexpr (STORE_DS) {
      // row key0 + l16 of dS^T: the lane holds queries tq0 + 16c + 4lg + r
      // (c, r < 4) and writes them as 16-byte chunks in the order of
      // ds_chunk_pos (each store instruction then covers 64 contiguous bytes
      // of every row it touches)
      const int Tpad = (Tn + BKW - 1) / BKW * BKW, nqb = (Tn + DQB - 1) / DQB;
      T* drow = ds + ((((size_t)b * H + it % H) * nqb + tq0 / DQB) * Tpad + key0 + l16) * DQB + tq0 % DQB;
      constexpr int E16 = A::VEC;                // values per 16-byte chunk
#pragma unroll
      for (int v = 0; v < 16 / E16; ++v) {
        V w;
#pragma unroll
        for (int e = 0; e < E16; ++e) {
          const int idx = v * E16 + e;           // the lane's 16 values in (c, r) order
          w[e] = from_f32<T>(dsa[0][idx / 4][idx % 4]);
        }
        *reinterpret_cast<V*>(drow + (v * 4 + lg) * E16) = w;
      }
    }
    // dV^T[d][key] += dO^T[d][rows] P[rows][key];  dK^T += Q^T dS
#pragma unroll
    for (int kk = 0; kk < NC / NPT; ++kk)
#pragma unroll
      for (int kt = 0; kt < 1; ++kt) {
        const V pb = CFrag<T>::pack(pa[kt] + kk * NPT);
        const V sb = CFrag<T>::pack(dsa[kt] + kk * NPT);
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) {
          const V oa = CFrag<T>::read(O, ST, kk * 16 * NPT, dt * 16, lane);
          const V qa = CFrag<T>::read(Q, ST, kk * 16 * NPT, dt * 16, lane);
          Mma<T>::run(dv[dt][kt], oa, pb);
          Mma<T>::run(dk[dt][kt], qa, sb);
        }
      }
    }

    T* Qn = Qs + ((it + 1) & 1) * TILE;
    T* On = Os + ((it + 1) & 1) * TILE;
    if (PFT) {
      // unconditional: after the last step the other buffer is no longer read
      // (its readers finished before the previous barrier)
#pragma unroll
      for (int i = 0; i < NPRE; ++i) {
        const int c = tid + i * DKW_THREADS;
        const int which = c / (SQ * A::DC), r = (c / A::DC) % SQ, dc = c % A::DC;
        *reinterpret_cast<V*>((which ? On : Qn) + r * ST + dc * A::VEC) = pre[i];
      }
      stat_put((it + 1) & 1, stat_next);
    } else if (more) {
      __syncthreads();
      for (int c = tid; c < 2 * SQ * A::DC; c += DKW_THREADS) {
        const int which = c / (SQ * A::DC), r = (c / A::DC) % SQ, dc = c % A::DC;
        const T* src = which ? osrc(it + 1) + (size_t)r * ldo : qsrc(it + 1) + (size_t)r * ldq;
        *reinterpret_cast<V*>((which ? On : Qn) + r * ST + dc * A::VEC) =
            *reinterpret_cast<const V*>(src + dc * A::VEC);
      }
      stat_put((it + 1) & 1, stat_next);
    }
    __syncthreads();
  };
  // two steps per iteration (the prefetch register sets alternate), the odd
  // last step after the loop: no branch inside the loop body, so the compiler
  // tracks the loads in flight across the back edge exactly
  int it = 0;
  for (; it + 1 < niter; it += 2) {
    step(it, preA, preB);
    step(it + 1, preB, preA);
  }
  if (it < niter) step(it, preA, preB);
  if (!kact) return;
  if constexpr (DIRECT) {
    const float scale = 1.0f / sqrtf((float)D);
    typedef T T4 __attribute__((ext_vector_type(4)));
    T* dst = dqkv + (row0 + key0 + l16) * ldd + H * D;
    const float vs = rs ? rs[row0 + key0 + l16] : 1.0f;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      T4 wk, wv;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        wk[r] = from_f32<T>(dk[dt][0][r] * scale);
        wv[r] = from_f32<T>(dv[dt][0][r] * vs);
      }
      *reinterpret_cast<T4*>(dst + dt * 16 + lg * 4) = wk;
      *reinterpret_cast<T4*>(dst + D + dt * 16 + lg * 4) = wv;
    }
    return;
  }
  // fp32 partial sums of this query chunk: part[chunk][token][0..127 dK, 128..255 dV]
  const size_t M = (size_t)B * Tn;
#pragma unroll
  for (int kt = 0; kt < 1; ++kt) {
    float* dst = part + ((size_t)chunk * M + row0 + key0 + kt * 16 + l16) * (2 * D);
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      *reinterpret_cast<f32x4*>(dst + dt * 16 + lg * 4) = dk[dt][kt];
      *reinterpret_cast<f32x4*>(dst + D + dt * 16 + lg * 4) = dv[dt][kt];
    }
  }
}

// dK (scaled by 1/sqrt(D)) and dV (times rs of its row, when given) of each
// key: the sum of its chunk partials in chunk order, written into the key and
// value columns of dqkv.
template <typename T>
__global__ __launch_bounds__(256) void attn_dkv_reduce_kernel(const float* __restrict__ part,
                                                              int B, int Tn, int H,
                                                              T* __restrict__ dqkv, int ldd,
                                                              const float* __restrict__ rs) {
  const size_t M = (size_t)B * Tn;
  const size_t row = blockIdx.x * 4ull + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (row >= M) return;
  const int lane = threadIdx.x & 63;
  const int t = (int)(row % Tn);
  const int nch = dkv_chunks(Tn, t / BKW);
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int c = 0; c < nch; ++c)
    acc += *reinterpret_cast<const f32x4*>(part + ((size_t)c * M + row) * (2 * D) + lane * 4);
  const float scale = lane < 32 ? 1.0f / sqrtf((float)D) : (rs ? rs[row] : 1.0f);
  typedef T T4 __attribute__((ext_vector_type(4)));
  T4 w = {from_f32<T>(acc[0] * scale), from_f32<T>(acc[1] * scale), from_f32<T>(acc[2] * scale),
          from_f32<T>(acc[3] * scale)};
  *reinterpret_cast<T4*>(dqkv + row * ldd + H * D + lane * 4) = w;
}

}  // namespace

hipError_t attn_fwd(DType t, const void* qkv, int ldq, int B, int T, int H, void* o, float* lse,
                    hipStream_t s) {
  if (T % BKV || H < 1 || H > 16) return hipErrorInvalidValue;
  dim3 grid(B * (T / FQB) * ((H + 1) / 2)), block(256);
  if (t == DType::BF16)
    hipLaunchKernelGGL(attn_fwd_kernel<bf16>, grid, block, 0, s, static_cast<const bf16*>(qkv), ldq, T,
                       H, static_cast<bf16*>(o), lse);
  else
    hipLaunchKernelGGL(attn_fwd_kernel<float>, grid, block, 0, s, static_cast<const float*>(qkv), ldq,
                       T, H, static_cast<float*>(o), lse);
  return hipGetLastError();
}

size_t attn_bwd_scratch_floats(int B, int T) {
  const int nch = dkv_chunks(T, 0);
  return nch > 1 ? (size_t)nch * B * T * 2 * D : 0;   // one chunk: dK/dV written directly
}

size_t attn_bwd_ds_elems(int B, int T, int H) {
  return (size_t)B * H * ((T + DQB - 1) / DQB) * ((T + BKW - 1) / BKW * BKW) * DQB;
}

namespace {
template <typename T>
hipError_t attn_bwd_t(const T* q, int ldq, const T* o, const T* d, const float* lse, float* delta, int B, int T_,
                      int H, T* g, int ldd, float* scratch, const float* rs, T* ds, hipStream_t s) {
  dim3 gq(B * (T_ / FQB) * ((H + 1) / 2)), bq(256);
  int items = 0;
  for (int kb = 0; kb < (T_ + BKW - 1) / BKW; ++kb) items += dkv_chunks(T_, kb);
  dim3 gk(B * items), bk(DKW_THREADS);
  const bool direct = dkv_chunks(T_, 0) == 1;     // every key block in one work item
  const size_t M = (size_t)B * T_;
  dim3 gr((unsigned)((M + 3) / 4)), br(256);
  if (ds) {
    // delta first, then dK/dV (which also stores dS^T), then dQ from dS
    const size_t total = M * H;
    hipLaunchKernelGGL(attn_delta_kernel<T>, dim3((unsigned)((total + 15) / 16)), dim3(256), 0, s, o, d, T_, H,
                       total, delta);
    if (direct) {
      hipLaunchKernelGGL((attn_bwd_dkv_kernel<T, true, true>), gk, bk, 0, s, q, ldq, d, lse, delta, B, T_, H,
                         scratch, g, ldd, rs, ds);
    } else {
      hipLaunchKernelGGL((attn_bwd_dkv_kernel<T, false, true>), gk, bk, 0, s, q, ldq, d, lse, delta, B, T_, H,
                         scratch, g, ldd, rs, ds);
      hipLaunchKernelGGL(attn_dkv_reduce_kernel<T>, gr, br, 0, s, scratch, B, T_, H, g, ldd, rs);
    }
    dim3 gd(B * ((T_ + DQB - 1) / DQB) * ((H + 1) / 2)), bd(512);
    hipLaunchKernelGGL(attn_bwd_dq_ds_kernel<T>, gd, bd, 0, s, q, ldq, static_cast<const T*>(ds), T_, H, g, ldd);
    return hipGetLastError();
  }
  // dQ first: it writes the delta rows that dK/dV reads
  hipLaunchKernelGGL(attn_bwd_dq_kernel<T>, gq, bq, 0, s, q, ldq, o, d, lse, delta, T_, H, g, ldd);
  if (direct) {
    hipLaunchKernelGGL((attn_bwd_dkv_kernel<T, true, false>), gk, bk, 0, s, q, ldq, d, lse, delta, B, T_, H,
                       scratch, g, ldd, rs, static_cast<T*>(nullptr));
  } else {
    hipLaunchKernelGGL((attn_bwd_dkv_kernel<T, false, false>), gk, bk, 0, s, q, ldq, d, lse, delta, B, T_, H,
                       scratch, g, ldd, rs, static_cast<T*>(nullptr));
    hipLaunchKernelGGL(attn_dkv_reduce_kernel<T>, gr, br, 0, s, scratch, B, T_, H, g, ldd, rs);
  }
  return hipGetLastError();
}
}  // namespace

hipError_t attn_bwd(DType t, const void* qkv, int ldq, const void* o, const void* dout, const float* lse,
                    float* delta, int B, int T, int H, void* dqkv, int ldd, float* scratch,
                    hipStream_t s, const float* rs, void* ds) {
  if (T % BKV || H < 1 || H > 16) return hipErrorInvalidValue;
  if (t == DType::BF16)
    return attn_bwd_t<bf16>(static_cast<const bf16*>(qkv), ldq, static_cast<const bf16*>(o),
                            static_cast<const bf16*>(dout), lse, delta, B, T, H, static_cast<bf16*>(dqkv), ldd,
                            scratch, rs, static_cast<bf16*>(ds), s);
  return attn_bwd_t<float>(static_cast<const float*>(qkv), ldq, static_cast<const float*>(o),
                           static_cast<const float*>(dout), lse, delta, B, T, H, static_cast<float*>(dqkv), ldd,
                           scratch, rs, static_cast<float*>(ds), s);
}

// ---------------------------------------------------------------------------
// Fixed scratch for callers that cannot allocate device memory (code under
// graph capture, serving loops): the delta rows and the dK/dV chunk partials
// of one attention backward live in this file-scope array instead of a
// caller-provided buffer. Each device holds its own copy for the life of the
// process; in host code `scratch` only names the symbol, so its device
// address is looked up once per device (with that device current) and that
// address is what the kernels receive.
static __device__ __align__(256) char scratch[kAttnFixedScratchBytes];

hipError_t attn_fixed_scratch(void** ptr) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return hipSuccess;
}

}  // namespace nc
