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
// H heads against them (bf16: on the matrix cores; fp32: on the vector
// units). Scores are bounded by sqrt(128) (QK-norm), so the softmax is
// shifted by the same fixed bound as in training and the chunk partials
// sum_u p v and sum_u p simply add; they are combined in chunk order
// (bitwise reproducible).
//
// The linear layers of a decoding step have one row per sequence; the
// few-row product below streams each weight matrix once with many small
// workgroups, folds the block norms in, and writes what the next product
// needs to fold its own norm (the embedding kernel starts that chain).
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
  constexpr int KR = 80;                       // LDS row: 64 keys + 32-byte pad (conflict-free)
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
// stream over W, so a workgroup owns just 16 output columns and one of S
// slices of K (many workgroups, short dependency chains). Its 8 wavefronts
// take interleaved 32-wide k steps of the slice, so together they read each
// W row front to back, and multiply with v_mfma_f32_16x16x32_bf16 (16 W rows
// as the row operand, 16 rows of X as the column operand); loads of the next
// batch of steps are in flight while the current one is multiplied. The
// wavefronts' tiles are added through LDS in wavefront order; with S > 1 each
// slice stores its tile and the last slice of a column block to arrive (an
// arrival counter) adds the S tiles in slice order. Results are therefore
// bitwise reproducible.
//
// The RMS norm of X's rows can be folded in: the producer of the rows left
// per-16-column sums of squares, the norm is applied to the fp32 accumulator
// (Y = rinv * sum_k W x, with x rounded to bf16 unscaled).
constexpr int kSkWaves = 8;
constexpr int kSkU = 4;            // k steps per wavefront per batch
constexpr int kSsqPer = 8;         // 16 x 8 = 128 column blocks: rows up to 2048 wide

template <int MT, int NT, SkEpi EPI, bool NORM>
__global__ __launch_bounds__(512, 2) void skinny_kernel(SkArgs g) {
  constexpr int U = NT == 1 ? kSkU : 2;        // k steps per wavefront per batch
  constexpr int TILES = NT * MT;               // 16 x 16 output tiles per wavefront
  __shared__ __align__(16) float red[kSkWaves * TILES * 256];
  __shared__ float ssq_red[16][32];
  __shared__ float rinv_s[32];
  __shared__ int last_s;
  // wave-uniform in a scalar register, so the step guards below are scalar branches
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15, lg = lane >> 4;
  const int nb = blockIdx.x, sk = blockIdx.y, S = gridDim.y;
  const int n0 = nb * 16 * NT;
  const int nsteps = g.K >> 5;
  const int sb = (int)((long)sk * nsteps / S), se = (int)((long)(sk + 1) * nsteps / S);
  const bf16* __restrict__ W = static_cast<const bf16*>(g.W);
  const bf16* __restrict__ X = static_cast<const bf16*>(g.X);

  float sq[kSsqPer];
  if constexpr (NORM) {
    const int m = tid & 31, grp = tid >> 5;
#pragma unroll
    for (int j = 0; j < kSsqPer; ++j) {
      const int blk = grp + 16 * j;
      sq[j] = (blk < g.nssq && m < g.M) ? g.ssq_in[blk * 32 + m] : 0.f;
    }
  }

  // The residual tile this thread adds to (AddF32) is read now, alongside the
  // first operand loads, so its latency is not paid again in the epilogue;
  // this workgroup is the only writer of these elements.
  f32x4 cres = {0.f, 0.f, 0.f, 0.f};
  if constexpr (EPI == SkEpi::AddF32) {
    if (tid < TILES * 64) {
      const int ln = tid & 63, tile = tid >> 6, nt = tile / MT, mt = tile % MT;
      const int m = 16 * mt + (ln & 15), n = n0 + 16 * nt + 4 * (ln >> 4);
      if (m < g.M) cres = *reinterpret_cast<const f32x4*>(static_cast<const float*>(g.C) + (size_t)m * g.ldc + n);
    }
  }
  const bf16* wrow = W + (size_t)(n0 + l16) * g.ldw + 8 * lg;
  const size_t wtile = (size_t)16 * g.ldw;     // next 16 W rows
  f32x4 acc[NT][MT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[nt][mt] = f32x4{0.f, 0.f, 0.f, 0.f};
  auto load = [&](int s0, bf16x8 (&a)[U][NT], bf16x8 (&x)[U][MT]) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int s = s0 + kSkWaves * u;
      if (s < se) {
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
          a[u][nt] = *reinterpret_cast<const bf16x8*>(wrow + nt * wtile + 32 * s);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          const int m = 16 * mt + l16;
          x[u][mt] = m < g.M ? *reinterpret_cast<const bf16x8*>(X + (size_t)m * g.ldx + 32 * s + 8 * lg)
                             : bf16x8{};
        }
      } else {
        // never multiplied, but kept zero: a matrix instruction the compiler
        // places under an EXEC mask still runs on every lane
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) a[u][nt] = bf16x8{};
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) x[u][mt] = bf16x8{};
      }
    }
  };
  auto mma = [&](int s0, const bf16x8 (&a)[U][NT], const bf16x8 (&x)[U][MT]) {
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (s0 + kSkWaves * u < se)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
#pragma unroll
          for (int mt = 0; mt < MT; ++mt)
            acc[nt][mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[u][nt], x[u][mt], acc[nt][mt], 0, 0, 0);
  };
  constexpr int kBatch = kSkWaves * U;      // k steps of the workgroup per batch
  bf16x8 a0[U][NT], x0[U][MT], a1[U][NT], x1[U][MT];
  int s0 = sb + wave;
  load(s0, a0, x0);
  for (; s0 < se; s0 += 2 * kBatch) {
    load(s0 + kBatch, a1, x1);
    mma(s0, a0, x0);
    load(s0 + 2 * kBatch, a0, x0);
    mma(s0 + kBatch, a1, x1);
  }
#pragma unroll
  for (int nt = 0; nt < NT; ++nt)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
      *reinterpret_cast<f32x4*>(red + ((wave * TILES + nt * MT + mt) * 64 + lane) * 4) = acc[nt][mt];
  if constexpr (NORM) {
    float t = 0.f;
#pragma unroll
    for (int j = 0; j < kSsqPer; ++j) t += sq[j];
    ssq_red[tid >> 5][tid & 31] = t;
  }
  __syncthreads();
  if constexpr (NORM) {
    if (tid < 32) {
      float t = 0.f;
      for (int grp = 0; grp < 16; ++grp) t += ssq_red[grp][tid];
      rinv_s[tid] = 1.0f / sqrtf(t / g.K + g.eps);
    }
  }
  // thread e < TILES * 64: tile (nt, mt) = e / 64, lane ln = e % 64 holds
  // C[16 mt + (ln & 15)][n0 + 16 nt + 4 (ln >> 4) + r]
  const int e = tid;
  f32x4 v = {0.f, 0.f, 0.f, 0.f};
  if (e < TILES * 64) {
#pragma unroll
    for (int w = 0; w < kSkWaves; ++w) v += *reinterpret_cast<const f32x4*>(red + (w * TILES * 64 + e) * 4);
  }
  if (S > 1) {
    // Slices meet through device-coherent (agent-scope) stores and loads of
    // the partial tiles: a store is acknowledged once it is visible to every
    // XCD, so waiting for the acknowledgements before counting in orders the
    // tile before the count, without a whole-L2 write-back.
    float* slot = g.part + ((size_t)nb * S + sk) * (TILES * 256);
    if (e < TILES * 64) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        __hip_atomic_store(slot + e * 4 + i, v[i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): every store of this thread acknowledged
    __syncthreads();
    if (tid == 0)
      last_s = __hip_atomic_fetch_add(g.cnt + nb, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
               (uint32_t)(S - 1);
    __syncthreads();
    if (!last_s) return;
    if (e < TILES * 64) {
      v = f32x4{0.f, 0.f, 0.f, 0.f};
      for (int k = 0; k < S; ++k) {
        const float* src = g.part + ((size_t)nb * S + k) * (TILES * 256) + e * 4;
#pragma unroll
        for (int i = 0; i < 4; ++i)
          v[i] += __hip_atomic_load(src + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
    if (tid == 0) __hip_atomic_store(g.cnt + nb, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __syncthreads();
  if (e >= TILES * 64) return;
  const int ln = e & 63, tile = e >> 6, nt = tile / MT, mt = tile % MT;
  const int m = 16 * mt + (ln & 15), n = n0 + 16 * nt + 4 * (ln >> 4);
  const bool row = m < g.M;
  if constexpr (NORM) v *= rinv_s[m];
  const size_t off = (size_t)m * g.ldc + n;
  if constexpr (EPI == SkEpi::StoreT) {
    if (row)
      *reinterpret_cast<bf16x4*>(static_cast<bf16*>(g.C) + off) =
          bf16x4{(bf16)v[0], (bf16)v[1], (bf16)v[2], (bf16)v[3]};
  } else if constexpr (EPI == SkEpi::Relu2) {
    bf16x4 w;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float r = fmaxf(v[i], 0.f);
      w[i] = (bf16)(r * r);
    }
    if (row) *reinterpret_cast<bf16x4*>(static_cast<bf16*>(g.C) + off) = w;
  } else if constexpr (EPI == SkEpi::AddF32) {
    f32x4 c = v;
    if (row) {
      f32x4* cp = reinterpret_cast<f32x4*>(static_cast<float*>(g.C) + off);
      c = cres + v;
      *cp = c;
      if (g.xb)
        *reinterpret_cast<bf16x4*>(static_cast<bf16*>(g.xb) + off) =
            bf16x4{(bf16)c[0], (bf16)c[1], (bf16)c[2], (bf16)c[3]};
    }
    if (g.ssq_out) {
      // the 16 columns of this block for row m sit in lanes ln, ln ^ 16, ln ^ 32, ln ^ 48
      float q = row ? c[0] * c[0] + c[1] * c[1] + c[2] * c[2] + c[3] * c[3] : 0.f;
      q += __shfl_xor(q, 16, 64);
      q += __shfl_xor(q, 32, 64);
      if (row && (ln >> 4) == 0) g.ssq_out[(nb * NT + nt) * 32 + m] = q;
    }
  } else {
    const float inv = 1.0f / g.cap;
    f32x4 z;
#pragma unroll
    for (int i = 0; i < 4; ++i) z[i] = g.cap * tanhf(v[i] * inv);
    if (row) *reinterpret_cast<f32x4*>(static_cast<float*>(g.C) + off) = z;
  }
}

// One workgroup per sequence: x = n(E[tok]), its bf16 copy and the
// per-16-column sums of squares the next product folds its norm from.
__global__ __launch_bounds__(256) void decode_embed_kernel(const bf16* __restrict__ E,
                                                           const int32_t* __restrict__ tok, int d, int V,
                                                           float eps, float* __restrict__ x,
                                                           bf16* __restrict__ xb, float* __restrict__ ssq,
                                                           uint32_t* status) {
  __shared__ float wsum[4];
  const int m = blockIdx.x, tid = threadIdx.x, lane = tid & 63;
  int id = tok[m];
  if (id < 0 || id >= V) {
    if (tid == 0) atomicOr(status, kStatusTokenRange);
    id = id < 0 ? 0 : V - 1;
  }
  const int c = 8 * tid;                 // this thread's 8 columns
  float v[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  float ss = 0.f;
  if (c < d) {
    const bf16x8 e8 = *reinterpret_cast<const bf16x8*>(E + (size_t)id * d + c);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      v[i] = (float)e8[i];
      ss += v[i] * v[i];
    }
  }
  ss = wave_sum(ss);
  if (lane == 0) wsum[tid >> 6] = ss;
  __syncthreads();
  const float r = 1.0f / sqrtf((wsum[0] + wsum[1] + wsum[2] + wsum[3]) / d + eps);
  float q = 0.f;
  if (c < d) {
    float y[8];
    bf16x8 o;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      y[i] = v[i] * r;
      o[i] = (bf16)y[i];
      q += y[i] * y[i];
    }
    const f32x4 lo = {y[0], y[1], y[2], y[3]}, hi = {y[4], y[5], y[6], y[7]};
    *reinterpret_cast<f32x4*>(x + (size_t)m * d + c) = lo;
    *reinterpret_cast<f32x4*>(x + (size_t)m * d + c + 4) = hi;
    *reinterpret_cast<bf16x8*>(xb + (size_t)m * d + c) = o;
  }
  q += __shfl_xor(q, 1, 64);             // threads 2j, 2j + 1 hold columns 16j .. 16j + 15
  if (c < d && (tid & 1) == 0) ssq[(tid >> 1) * 32 + m] = q;
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

// Measured on MI355X at the decoding shapes (32 rows, bf16): a slice costs
// one more round trip through memory for its partial tile, which outweighs
// the extra parallelism until a workgroup would stream more than 2048 k
// values (two batches per wavefront); 16-column blocks alone give 80-4096
// workgroups.
int skinny_splits(int N, int K) {
  (void)N;
  const int nsteps = K / 32;
  return (nsteps + 2 * kSkWaves * kSkU - 1) / (2 * kSkWaves * kSkU);
}

size_t skinny_part_bytes(int M, int N, int K, int splits) {
  const int S = splits > 0 ? splits : skinny_splits(N, K);
  const int MT = M <= 16 ? 1 : 2;
  return S > 1 ? (size_t)(N / 16) * S * MT * 256 * sizeof(float) : 0;
}

// Wider workgroups re-read X less per column; measured at the decoding shapes
// (32 rows, weights streamed once per step): 4 tiles for the lm_head, 2 for the
// MLP up-projection, 1 for the narrow products, whose workgroup count it would
// halve.
int skinny_ntile(int N, int K) {
  (void)K;
  if (N % 64 == 0 && N / 64 >= 512) return 4;
  if (N % 32 == 0 && N >= 4096) return 2;
  return 1;
}

hipError_t skinny_gemm(const SkArgs& a, SkEpi epi, hipStream_t s) {
  if (a.M < 1 || a.M > kSkinnyMaxRows || a.N < 16 || a.N % 16 || a.K < 32 || a.K % 32 || a.ldw % 8 ||
      a.ldx % 8 || a.ldc % 4 || a.ldw < a.K || a.ldx < a.K || a.ldc < a.N)
    return hipErrorInvalidValue;
  if (a.ssq_in && (a.nssq < 1 || a.nssq > 16 * kSsqPer)) return hipErrorInvalidValue;
  if ((a.xb || a.ssq_out) && epi != SkEpi::AddF32) return hipErrorInvalidValue;
  const int S = a.splits > 0 ? a.splits : skinny_splits(a.N, a.K);
  if (S > a.K / 32 || (S > 1 && (!a.part || !a.cnt))) return hipErrorInvalidValue;
  const int NT = a.ntile > 0 ? a.ntile : skinny_ntile(a.N, a.K);
  if ((NT != 1 && NT != 2 && NT != 4) || a.N % (16 * NT)) return hipErrorInvalidValue;
  const dim3 grid(a.N / (16 * NT), S), block(512);
  const bool norm = a.ssq_in != nullptr;
#define NC_SKINNY(MT, NTV, E)                                                      \
  do {                                                                             \
    if (norm)                                                                      \
      hipLaunchKernelGGL((skinny_kernel<MT, NTV, E, true>), grid, block, 0, s, a);   \
    else                                                                           \
      hipLaunchKernelGGL((skinny_kernel<MT, NTV, E, false>), grid, block, 0, s, a);  \
  } while (0)
#define NC_SKINNY_EPI(MT, NTV)                                             \
  switch (epi) {                                                           \
    case SkEpi::StoreT: NC_SKINNY(MT, NTV, SkEpi::StoreT); break;          \
    case SkEpi::AddF32: NC_SKINNY(MT, NTV, SkEpi::AddF32); break;          \
    case SkEpi::Relu2: NC_SKINNY(MT, NTV, SkEpi::Relu2); break;            \
    case SkEpi::SoftcapF32: NC_SKINNY(MT, NTV, SkEpi::SoftcapF32); break;  \
  }
#define NC_SKINNY_NT(MT)          \
  if (NT == 1) {                  \
    NC_SKINNY_EPI(MT, 1)          \
  } else if (NT == 2) {           \
    NC_SKINNY_EPI(MT, 2)          \
  } else {                        \
    NC_SKINNY_EPI(MT, 4)          \
  }
  if (a.M <= 16) {
    NC_SKINNY_NT(1)
  } else {
    NC_SKINNY_NT(2)
  }
#undef NC_SKINNY_NT
#undef NC_SKINNY_EPI
#undef NC_SKINNY
  return hipGetLastError();
}

hipError_t decode_embed(const void* E, const int32_t* tok, int M, int d, int V, float eps, float* x,
                        void* xb, float* ssq, uint32_t* status, hipStream_t s) {
  if (M < 1 || M > kSkinnyMaxRows || d % 16 || d > 2048) return hipErrorInvalidValue;
  hipLaunchKernelGGL(decode_embed_kernel, dim3(M), dim3(256), 0, s, static_cast<const bf16*>(E), tok, d,
                     V, eps, x, static_cast<bf16*>(xb), ssq, status);
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
