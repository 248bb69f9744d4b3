// Dense contractions of the training step on the CDNA4 matrix cores.
//
// One kernel template covers the three operand orders the step needs:
//   forward  Y[tok, out]  = X[tok, in] . W[out, in]^T       (both K-contiguous)
//   dgrad    dX[tok, in]  = dY[tok, out] . W[out, in]        (B is K-strided)
//   wgrad    dW[out, in]  = dY[tok, out]^T . X[tok, in]      (both K-strided)
// The linear layers are bias-free (followin.io release article, architecture
// list), so a contraction plus an epilogue is the whole layer. Epilogues fuse
// the residual add, the relu^2 activation of the MLP (same list) and its
// derivative, so no separate elementwise pass touches HBM.
//
// Tiling: 128x128 output tile per 256-thread workgroup (4 wavefronts in a 2x2
// grid, 64x64 per wavefront = 4x4 MFMA tiles of 16x16). Each K step stages a
// 128-byte-wide slab of A and B in LDS (double-buffered, one barrier per step,
// next slab prefetched into registers while the matrix cores work). bf16 uses
// v_mfma_f32_16x16x32_bf16, fp32 uses four v_mfma_f32_16x16x4_f32 per 16-byte
// fragment (true fp32 products, fp32 accumulation in both cases).
// K-strided operands are transposed in registers on their way into LDS, so
// the matrix-core reads are always 16-byte, K-contiguous LDS reads.
// Workgroup ids are remapped so each XCD (8 per chip, own L2) walks a
// contiguous, row-grouped range of output tiles.
#include "common.h"
#include "launch.h"

namespace nc {
namespace {

constexpr int kThreads = 256;

template <typename T> struct Mma;
template <> struct Mma<bf16> {
  __device__ __forceinline__ static void run(f32x4& acc, const bf16x8& a, const bf16x8& b) {
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc, 0, 0, 0);
  }
};
template <> struct Mma<float> {
  // lane group g of a 16-byte fragment holds k = 4g..4g+3; MFMA s takes k = 4g+s
  __device__ __forceinline__ static void run(f32x4& acc, const f32x4& a, const f32x4& b) {
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[0], b[0], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[1], b[1], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[2], b[2], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[3], b[3], acc, 0, 0, 0);
  }
};

// Global -> registers -> LDS for one operand slab of R rows x BK k-values.
// LDS layout is [row][k] with a 16-byte pad per row.
template <typename T, bool KC, int R>
struct SlabLoader {
  static constexpr int VEC = Vec16<T>::N;
  static constexpr int BK = 128 / sizeof(T);
  static constexpr int LDSK = BK + VEC;
  static constexpr int NL = R / 32;            // 16-byte loads per thread
  typedef typename Vec16<T>::type V;
  typedef T V4 __attribute__((ext_vector_type(4)));
  static_assert(KC || R % 128 == 0, "strided slabs need R % 128 == 0");
  V reg[NL];

  __device__ __forceinline__ void load(const T* __restrict__ p, int ld, int rows, int r0, int k0,
                                       int tid) {
    if constexpr (KC) {
#pragma unroll
      for (int i = 0; i < NL; ++i) {
        const int c = tid + kThreads * i;
        const int row = c >> 3, col = (c & 7) * VEC;
        const int gr = r0 + row;
        if (gr < rows) reg[i] = *reinterpret_cast<const V*>(p + (size_t)gr * ld + k0 + col);
        else reg[i] = V{};
      }
    } else {
      constexpr int RC = R / VEC;              // 16-byte chunks along the row dim
#pragma unroll
      for (int u = 0; u < NL / 4; ++u) {
        const int unit = tid + kThreads * u;
        const int rc = unit % RC, kg = unit / RC;
        const int gr = r0 + rc * VEC;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int k = k0 + kg * 4 + j;
          if (gr < rows) reg[u * 4 + j] = *reinterpret_cast<const V*>(p + (size_t)k * ld + gr);
          else reg[u * 4 + j] = V{};
        }
      }
    }
  }

  __device__ __forceinline__ void store(T* lds, int tid) const {
    if constexpr (KC) {
#pragma unroll
      for (int i = 0; i < NL; ++i) {
        const int c = tid + kThreads * i;
        const int row = c >> 3, col = (c & 7) * VEC;
        *reinterpret_cast<V*>(lds + row * LDSK + col) = reg[i];
      }
    } else {
      constexpr int RC = R / VEC;
#pragma unroll
      for (int u = 0; u < NL / 4; ++u) {
        const int unit = tid + kThreads * u;
        const int rc = unit % RC, kg = unit / RC;
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
          V4 w = {reg[u * 4 + 0][e], reg[u * 4 + 1][e], reg[u * 4 + 2][e], reg[u * 4 + 3][e]};
          *reinterpret_cast<V4*>(lds + (rc * VEC + e) * LDSK + kg * 4) = w;
        }
      }
    }
  }
};

template <typename T, bool AK, bool BKC, Epi EPI, int BM, int BN, int WM, int WN>
__global__ __launch_bounds__(kThreads) void gemm_kernel(GemmArgs g) {
  constexpr int VEC = Vec16<T>::N;
  constexpr int KB = 4 * VEC;                 // k per matrix-core fragment
  constexpr int BK = 128 / sizeof(T);         // k per LDS slab
  constexpr int LDSK = BK + VEC;
  constexpr int TM = BM / WM, TN = BN / WN;
  constexpr int FM = TM / 16, FN = TN / 16;
  typedef typename Vec16<T>::type V;
  static_assert(WM * WN * kWave == kThreads, "4 wavefronts");

  __shared__ __align__(16) T smem[2 * (BM + BN) * LDSK];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, lg = lane >> 4;
  const int wm = wave % WM, wn = wave / WM;

  // ---- tile scheduling --------------------------------------------------
  const int tiles_m = (g.M + BM - 1) / BM, tiles_n = (g.N + BN - 1) / BN;
  const int ntiles = tiles_m * tiles_n;
  const int total = ntiles * g.splits;
  int bid = blockIdx.x;
  const int nb = gridDim.x;                  // a multiple of 8
  bid = (bid & 7) * (nb >> 3) + (bid >> 3);  // contiguous logical range per XCD
  if (bid >= total) return;
  const int split = bid / ntiles;
  int t = bid - split * ntiles;
  constexpr int GROUP = 8;
  const int per_group = GROUP * tiles_n;
  const int first_m = (t / per_group) * GROUP;
  const int gsize = min(tiles_m - first_m, GROUP);
  const int tm = first_m + (t % per_group) % gsize;
  const int tn = (t % per_group) / gsize;
  const int m0 = tm * BM, n0 = tn * BN;

  const int kps = g.K / g.splits;
  const int kbeg = split * kps;
  const int nk = kps / BK;

  const T* __restrict__ A = static_cast<const T*>(g.A);
  const T* __restrict__ B = static_cast<const T*>(g.B);

  SlabLoader<T, AK, BM> la;
  SlabLoader<T, BKC, BN> lb;
  T* As0 = smem;
  T* Bs0 = smem + BM * LDSK;
  T* As1 = smem + (BM + BN) * LDSK;
  T* Bs1 = As1 + BM * LDSK;

  f32x4 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  la.load(A, g.lda, g.M, m0, kbeg, tid);
  lb.load(B, g.ldb, g.N, n0, kbeg, tid);
  la.store(As0, tid);
  lb.store(Bs0, tid);
  __syncthreads();

  for (int it = 0; it < nk; ++it) {
    const bool odd = it & 1;
    const T* As = odd ? As1 : As0;
    const T* Bs = odd ? Bs1 : Bs0;
    const bool more = it + 1 < nk;
    if (more) {
      la.load(A, g.lda, g.M, m0, kbeg + (it + 1) * BK, tid);
      lb.load(B, g.ldb, g.N, n0, kbeg + (it + 1) * BK, tid);
    }
#pragma unroll
    for (int kb = 0; kb < BK / KB; ++kb) {
      V af[FM], bfr[FN];
#pragma unroll
      for (int i = 0; i < FM; ++i)
        af[i] = *reinterpret_cast<const V*>(As + (wm * TM + i * 16 + l16) * LDSK + kb * KB + lg * VEC);
#pragma unroll
      for (int j = 0; j < FN; ++j)
        bfr[j] = *reinterpret_cast<const V*>(Bs + (wn * TN + j * 16 + l16) * LDSK + kb * KB + lg * VEC);
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) Mma<T>::run(acc[i][j], bfr[j], af[i]);
    }
    if (more) {
      la.store(odd ? As0 : As1, tid);
      lb.store(odd ? Bs0 : Bs1, tid);
    }
    __syncthreads();
  }

  // ---- epilogue: lane holds C[m][n..n+3] of each 16x16 tile ----------------
#pragma unroll
  for (int i = 0; i < FM; ++i) {
    const int m = m0 + wm * TM + i * 16 + l16;
    if (m >= g.M) continue;
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int n = n0 + wn * TN + j * 16 + lg * 4;
      if (n >= g.N) continue;
      const f32x4 v = acc[i][j];
      const size_t off = (size_t)m * g.ldc + n;
      typedef T T4 __attribute__((ext_vector_type(4)));
      if constexpr (EPI == Epi::StoreT) {
        T4 w = {from_f32<T>(v[0]), from_f32<T>(v[1]), from_f32<T>(v[2]), from_f32<T>(v[3])};
        *reinterpret_cast<T4*>(static_cast<T*>(g.C) + off) = w;
      } else if constexpr (EPI == Epi::StoreF32) {
        *reinterpret_cast<f32x4*>(static_cast<float*>(g.C) + off) = v;
      } else if constexpr (EPI == Epi::AddF32) {
        f32x4* p = reinterpret_cast<f32x4*>(static_cast<float*>(g.C) + off);
        *p = *p + v;
      } else if constexpr (EPI == Epi::PartialF32) {
        float* base = static_cast<float*>(g.C) + (size_t)split * g.M * g.ldc;
        *reinterpret_cast<f32x4*>(base + off) = v;
      } else if constexpr (EPI == Epi::Relu2) {
        T4 u, a;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          u[r] = from_f32<T>(v[r]);
          const float uf = fmaxf(to_f32(u[r]), 0.f);
          a[r] = from_f32<T>(uf * uf);
        }
        *reinterpret_cast<T4*>(static_cast<T*>(g.C) + off) = u;
        *reinterpret_cast<T4*>(static_cast<T*>(g.C2) + (size_t)m * g.ldc2 + n) = a;
      } else if constexpr (EPI == Epi::Relu2Bwd) {
        const T4 u = *reinterpret_cast<const T4*>(static_cast<const T*>(g.C2) + (size_t)m * g.ldc2 + n);
        T4 w;
#pragma unroll
        for (int r = 0; r < 4; ++r) w[r] = from_f32<T>(v[r] * 2.f * fmaxf(to_f32(u[r]), 0.f));
        *reinterpret_cast<T4*>(static_cast<T*>(g.C) + off) = w;
      }
    }
  }
}

__global__ void splitk_reduce_kernel(const float* __restrict__ part, int splits, size_t n4,
                                     size_t n, float* __restrict__ dst, bool accumulate) {
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n4;
       i += (size_t)gridDim.x * blockDim.x) {
    f32x4 s = accumulate ? reinterpret_cast<const f32x4*>(dst)[i] : f32x4{0.f, 0.f, 0.f, 0.f};
    for (int k = 0; k < splits; ++k) s += reinterpret_cast<const f32x4*>(part + (size_t)k * n)[i];
    reinterpret_cast<f32x4*>(dst)[i] = s;
  }
}

template <typename T, bool AK, bool BKC, Epi EPI>
hipError_t launch(const GemmArgs& g, hipStream_t s) {
  constexpr int BM = 128, BN = 128;
  const int tiles = ((g.M + BM - 1) / BM) * ((g.N + BN - 1) / BN) * g.splits;
  const int grid = (tiles + 7) / 8 * 8;
  hipLaunchKernelGGL((gemm_kernel<T, AK, BKC, EPI, BM, BN, 2, 2>), dim3(grid), dim3(kThreads), 0, s, g);
  return hipGetLastError();
}

template <typename T>
hipError_t dispatch(bool ak, bool bk, Epi epi, const GemmArgs& g, hipStream_t s) {
  if (ak && bk) {
    switch (epi) {
      case Epi::StoreT: return launch<T, true, true, Epi::StoreT>(g, s);
      case Epi::StoreF32: return launch<T, true, true, Epi::StoreF32>(g, s);
      case Epi::AddF32: return launch<T, true, true, Epi::AddF32>(g, s);
      case Epi::Relu2: return launch<T, true, true, Epi::Relu2>(g, s);
      default: break;
    }
  } else if (ak && !bk) {
    switch (epi) {
      case Epi::StoreT: return launch<T, true, false, Epi::StoreT>(g, s);
      case Epi::StoreF32: return launch<T, true, false, Epi::StoreF32>(g, s);
      case Epi::Relu2Bwd: return launch<T, true, false, Epi::Relu2Bwd>(g, s);
      default: break;
    }
  } else if (!ak && !bk) {
    switch (epi) {
      case Epi::StoreF32: return launch<T, false, false, Epi::StoreF32>(g, s);
      case Epi::AddF32: return launch<T, false, false, Epi::AddF32>(g, s);
      case Epi::PartialF32: return launch<T, false, false, Epi::PartialF32>(g, s);
      default: break;
    }
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t gemm(DType t, bool a_kcontig, bool b_kcontig, Epi epi, const GemmArgs& g,
                hipStream_t stream) {
  const int bk = t == DType::BF16 ? 64 : 32;
  if (g.M <= 0 || g.N <= 0 || g.K <= 0 || g.splits <= 0) return hipErrorInvalidValue;
  if (g.M % 16 || g.N % 16 || g.K % (bk * g.splits)) return hipErrorInvalidValue;
  if (epi != Epi::PartialF32 && g.splits != 1) return hipErrorInvalidValue;
  return t == DType::BF16 ? dispatch<bf16>(a_kcontig, b_kcontig, epi, g, stream)
                          : dispatch<float>(a_kcontig, b_kcontig, epi, g, stream);
}

hipError_t splitk_reduce(const float* part, int splits, size_t n, float* dst, bool accumulate,
                         hipStream_t stream) {
  if (n % 4) return hipErrorInvalidValue;
  const size_t n4 = n / 4;
  const int block = 256;
  const size_t want = (n4 + block - 1) / block;
  const int grid = (int)(want < 4096 ? want : 4096);
  hipLaunchKernelGGL(splitk_reduce_kernel, dim3(grid > 0 ? grid : 1), dim3(block), 0, stream,
                     part, splits, n4, n, dst, accumulate);
  return hipGetLastError();
}

}  // namespace nc
