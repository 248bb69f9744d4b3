// Dense contractions of the training step on the CDNA4 matrix cores.
//
// One kernel template covers the three operand orders the step needs:
//   forward  Y[tok, out]  = X[tok, in] . W[out, in]^T       (both K-contiguous)
//   dgrad    dX[tok, in]  = dY[tok, out] . W[out, in]        (B is K-strided)
//   wgrad    dW[out, in]  = dY[tok, out]^T . X[tok, in]      (both K-strided)
// The linear layers are bias-free (followin.io release article, architecture
// list), so a contraction plus an epilogue is the whole layer. Epilogues fuse
// the residual add, the relu^2 activation of the MLP (same list) and its
// derivative, so no separate elementwise pass touches HBM. The parameter-free
// RMSNorm in front of the attention, the MLP and the lm_head (same list) is
// folded into the products around it: the residual-add epilogue (AddF32Xs)
// also writes the new residual row in the activation type and its sums of
// squares per 64 columns, and the product that consumes the normalised row
// takes that unnormalised copy as its A operand and multiplies each output
// row by the norm's 1/rms (rs) before its epilogue operation - the norm is a
// per-row scale, which commutes with the contraction over the row.
//
// Two kernels. Large bf16 products (at least 256 output tiles) take
// gemm_bf16_kernel: a 256x256 output tile per 512-thread workgroup (one per
// CU), v_mfma_f32_32x32x16_bf16, operand slabs loaded straight from global
// memory into a 4-stage LDS ring, and a ping-pong main loop (described at the
// kernel). Everything else, and every fp32 product, takes gemm_kernel: a
// 128x128 tile per 256 threads (2x2 wavefronts of 64x64), each 128-byte-wide
// K slab of A and B staged through registers into LDS (double-buffered, one
// barrier per slab, the next slab loaded while the matrix cores work), with
// v_mfma_f32_16x16x32_bf16 or, for fp32, four v_mfma_f32_16x16x4_f32 per
// 16-byte fragment (true fp32 products; fp32 accumulation in every case).
// In gemm_kernel, K-strided operands are transposed in registers on their way
// into LDS, so its matrix-core reads are always 16-byte, K-contiguous reads.
// Workgroup ids are remapped so each XCD (8 per chip, own L2) walks a
// contiguous, row-grouped range of output tiles.
#include <atomic>
#include <type_traits>

#include "common.h"
#include "launch.h"

namespace nc {
namespace {

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

// Global -> registers -> LDS for one operand slab of R rows x BK k-values,
// loaded by NTHR threads. LDS layout is [row][k] with a 16-byte pad per row.
template <typename T, bool KC, int R, int NTHR>
struct SlabLoader {
  static constexpr int VEC = Vec16<T>::N;
  static constexpr int BK = 128 / sizeof(T);
  static constexpr int LDSK = BK + VEC;
  static constexpr int NL = R * 8 / NTHR;      // 16-byte loads per thread
  typedef typename Vec16<T>::type V;
  typedef T V4 __attribute__((ext_vector_type(4)));
  static_assert(NL >= 1 && (KC || NL % 4 == 0), "slab does not split evenly over the threads");
  V reg[NL];

  __device__ __forceinline__ void load(const T* __restrict__ p, int ld, int rows, int r0, int k0,
                                       int tid) {
    if constexpr (KC) {
#pragma unroll
      for (int i = 0; i < NL; ++i) {
        const int c = tid + NTHR * i;
        const int row = c >> 3, col = (c & 7) * VEC;
        const int gr = r0 + row;
        if (gr < rows) reg[i] = *reinterpret_cast<const V*>(p + (size_t)gr * ld + k0 + col);
        else reg[i] = V{};
      }
    } else {
      constexpr int RC = R / VEC;              // 16-byte chunks along the row dim
#pragma unroll
      for (int u = 0; u < NL / 4; ++u) {
        const int unit = tid + NTHR * u;
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
        const int c = tid + NTHR * i;
        const int row = c >> 3, col = (c & 7) * VEC;
        *reinterpret_cast<V*>(lds + row * LDSK + col) = reg[i];
      }
    } else {
      constexpr int RC = R / VEC;
#pragma unroll
      for (int u = 0; u < NL / 4; ++u) {
        const int unit = tid + NTHR * u;
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

// C[m][n..n+3] = v under epilogue EPI
template <typename T, Epi EPI>
__device__ __forceinline__ void epilogue4(const GemmArgs& g, int split, int m, int n, f32x4 v) {
  const size_t off = (size_t)m * g.ldc + n;
  typedef T T4 __attribute__((ext_vector_type(4)));
  if constexpr (EPI == Epi::StoreT) {
    T4 w = {from_f32<T>(v[0]), from_f32<T>(v[1]), from_f32<T>(v[2]), from_f32<T>(v[3])};
    __builtin_nontemporal_store(w, reinterpret_cast<T4*>(static_cast<T*>(g.C) + off));
  } else if constexpr (EPI == Epi::StoreF32) {
    __builtin_nontemporal_store(v, reinterpret_cast<f32x4*>(static_cast<float*>(g.C) + off));
  } else if constexpr (EPI == Epi::AddF32) {
    f32x4* p = reinterpret_cast<f32x4*>(static_cast<float*>(g.C) + off);
    *p = *p + v;
  } else if constexpr (EPI == Epi::PartialF32) {
    float* base = static_cast<float*>(g.C) + (size_t)split * g.M * g.ldc;
    *reinterpret_cast<f32x4*>(base + off) = v;
  } else if constexpr (EPI == Epi::Relu2) {
    T4 a;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float uf = fmaxf(v[r], 0.f);
      a[r] = from_f32<T>(uf * uf);
    }
    __builtin_nontemporal_store(a, reinterpret_cast<T4*>(static_cast<T*>(g.C) + off));
  } else if constexpr (EPI == Epi::Relu2Bwd) {
    // d relu(u)^2 / du = 2 relu(u) = 2 sqrt(a), a = relu(u)^2 as stored by Relu2
    const T4 a = *reinterpret_cast<const T4*>(static_cast<const T*>(g.C2) + (size_t)m * g.ldc2 + n);
    T4 w;
#pragma unroll
    for (int r = 0; r < 4; ++r) w[r] = from_f32<T>(v[r] * 2.f * sqrtf(to_f32(a[r])));
    *reinterpret_cast<T4*>(static_cast<T*>(g.C) + off) = w;
  } else if constexpr (EPI == Epi::AxpbyT || EPI == Epi::AxpbyF32) {
    const T4 x = *reinterpret_cast<const T4*>(static_cast<const T*>(g.C2) + (size_t)m * g.ldc2 + n);
    f32x4 y;
#pragma unroll
    for (int r = 0; r < 4; ++r) y[r] = fmaf(g.alpha, v[r], g.beta * to_f32(x[r]));
    if constexpr (EPI == Epi::AxpbyT) {
      T4 w;
#pragma unroll
      for (int r = 0; r < 4; ++r) w[r] = from_f32<T>(y[r]);
      *reinterpret_cast<T4*>(static_cast<T*>(g.C) + off) = w;
    } else {
      *reinterpret_cast<f32x4*>(static_cast<float*>(g.C) + off) = y;
    }
  }
}

// Arguments of batch item b: A, B and C2 advance by sa / sb / sc2 elements of
// T, C by sc elements of its own type (T or fp32, by epilogue).
template <typename T, Epi EPI>
__device__ __forceinline__ GemmArgs batch_item(const GemmArgs& g0, int b) {
  GemmArgs g = g0;
  if (b == 0) return g;
  constexpr size_t csz = (EPI == Epi::StoreT || EPI == Epi::Relu2 || EPI == Epi::Relu2Bwd ||
                          EPI == Epi::AxpbyT)
                             ? sizeof(T) : sizeof(float);
  g.A = static_cast<const char*>(g0.A) + (size_t)b * g0.sa * sizeof(T);
  g.B = static_cast<const char*>(g0.B) + (size_t)b * g0.sb * sizeof(T);
  g.C = static_cast<char*>(g0.C) + (size_t)b * g0.sc * csz;
  if (g0.C2) g.C2 = static_cast<char*>(g0.C2) + (size_t)b * g0.sc2 * sizeof(T);
  return g;
}

template <typename T, bool AK, bool BKC, Epi EPI, int BM, int BN, int WM, int WN>
__global__ __launch_bounds__(WM * WN * 64) void gemm_kernel(GemmArgs g0) {
  constexpr int NTHR = WM * WN * 64;
  constexpr int VEC = Vec16<T>::N;
  constexpr int KB = 4 * VEC;                 // k per matrix-core fragment
  constexpr int BK = 128 / sizeof(T);         // k per LDS slab
  constexpr int LDSK = BK + VEC;
  constexpr int TM = BM / WM, TN = BN / WN;
  constexpr int FM = TM / 16, FN = TN / 16;
  typedef typename Vec16<T>::type V;

  __shared__ __align__(16) T smem[2 * (BM + BN) * LDSK];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, lg = lane >> 4;
  const int wm = wave % WM, wn = wave / WM;

  // ---- tile scheduling --------------------------------------------------
  const int tiles_m = (g0.M + BM - 1) / BM, tiles_n = (g0.N + BN - 1) / BN;
  const int ntiles = tiles_m * tiles_n;
  const int per_item = ntiles * g0.splits;
  const int total = per_item * (g0.batch > 1 ? g0.batch : 1);
  int bid = blockIdx.x;
  const int nb = gridDim.x;                  // a multiple of 8
  bid = (bid & 7) * (nb >> 3) + (bid >> 3);  // contiguous logical range per XCD
  if (bid >= total) return;
  const int item = bid / per_item;
  bid -= item * per_item;
  const GemmArgs g = batch_item<T, EPI>(g0, item);
  const int split = bid / ntiles;
  int t = bid - split * ntiles;
  constexpr int GROUP = 8;
  const int per_group = GROUP * tiles_n;
  const int first_m = (t / per_group) * GROUP;
  const int gsize = min(tiles_m - first_m, GROUP);
  const int tm = first_m + (t % per_group) % gsize;
  const int tn = (t % per_group) / gsize;
  const int m0 = tm * BM, n0 = tn * BN;

  // split `split` takes k slabs [split * ns / splits, (split + 1) * ns / splits)
  const int ns = g.K / BK;
  const int sb = (int)((long)split * ns / g.splits), se = (int)((long)(split + 1) * ns / g.splits);
  const int kbeg = sb * BK;
  const int nk = se - sb;

  const T* __restrict__ A = static_cast<const T*>(g.A);
  const T* __restrict__ B = static_cast<const T*>(g.B);

  SlabLoader<T, AK, BM, NTHR> la;
  SlabLoader<T, BKC, BN, NTHR> lb;
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
  constexpr bool SCALED = EPI == Epi::StoreT || EPI == Epi::Relu2 || EPI == Epi::Relu2Bwd;
  static_assert(EPI != Epi::AddF32Xs || TN == 64, "AddF32Xs: one 64-column group per wavefront");
#pragma unroll
  for (int i = 0; i < FM; ++i) {
    const int m = m0 + wm * TM + i * 16 + l16;
    // lanes l16 + 16 lg hold the same row: they skip (or not) together
    if (m >= g.M) continue;
    const float rsm = (SCALED && g.rs) ? g.rs[m] : 1.0f;
    float ss = 0.f;
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int n = n0 + wn * TN + j * 16 + lg * 4;
      if (n >= g.N) continue;
      if constexpr (EPI == Epi::AddF32Xs) {
        const size_t off = (size_t)m * g.ldc + n;
        f32x4* p = reinterpret_cast<f32x4*>(static_cast<float*>(g.C) + off);
        const f32x4 y = *p + acc[i][j];
        *p = y;
        typedef T T4 __attribute__((ext_vector_type(4)));
        const T4 w = {from_f32<T>(y[0]), from_f32<T>(y[1]), from_f32<T>(y[2]), from_f32<T>(y[3])};
        *reinterpret_cast<T4*>(static_cast<T*>(g.xc) + off) = w;
        ss += y[0] * y[0] + y[1] * y[1] + y[2] * y[2] + y[3] * y[3];
      } else if constexpr (SCALED) {
        epilogue4<T, EPI>(g, split, m, n, acc[i][j] * rsm);
      } else {
        epilogue4<T, EPI>(g, split, m, n, acc[i][j]);
      }
    }
    if constexpr (EPI == Epi::AddF32Xs) {
      // the wavefront's 64 columns of row m (N % 64 == 0: all inside or all outside)
      ss = group4_sum(ss);
      const int n64 = n0 + wn * TN;
      if (lg == 0 && n64 < g.N) g.ssq[(size_t)m * (g.N / 64) + n64 / 64] = ss;
    }
  }
}

// ---------------------------------------------------------------------------
// bf16 main-line contraction kernel, any operand order.
// 256x256 tile, 8 wavefronts (2 x 4), 128x64 per wavefront computed with
// v_mfma_f32_32x32x16_bf16 (4 x 2 tiles of 32x32, 128 fp32 accumulators).
//
// Operand slabs of 32 k values go from global memory straight into LDS
// (buffer_load_dwordx4 ... lds: no staging registers, no LDS store instructions)
// through a ring of four stages, three slabs ahead of the matrix cores. Each
// slab is laid out as it sits in memory, with 16-byte chunks XOR-swizzled so
// that both read shapes are bank-conflict free:
//   K-contiguous operand: [256 rows][32 k] (64-byte rows); chunk c of row r is
//     stored at slot c ^ ((r >> 2) & 3). Fragments: ds_read_b128 (lane l: row
//     l%32, k = 8*(l/32)..+7 of the 16-wide step).
//   K-strided operand:    [32 k][256 rows] (512-byte rows); chunk c of k row
//     kr is stored at slot c ^ 4*(kr & 3). Fragments: two LDS transpose reads
//     (ds_read_b64_tr_b16): in each 16-lane group, source lane 4j+q names k
//     row kb+j, columns c0+4q..+3, and output lane i receives k rows
//     kb..kb+3 of column c0+i - the same fragment layout, no transpose pass.
// Each lane's global source is chosen so that its fixed LDS destination
// (instruction base + 16 * lane) receives the swizzled chunk. The main loop
// runs the two wavefronts of each SIMD in ping-pong (one issues its MFMAs
// while the other reads fragments and issues loads, roles swapping at every
// barrier); waits on the direct loads are explicit (vmcnt), and a ring slot
// is refilled only after every wavefront has passed the barrier that follows
// its last read of that slot. Indices past the matrix edge are clamped, which
// only feeds output rows/columns that the epilogue never stores. Final
// outputs are written with non-temporal stores (written once, read by a
// later kernel), so they do not push operand slabs out of L2; split-K
// partials, read back at once by the reduction, are stored normally.
// MFMA 32x32 output layout: lane l, value r holds row 8*(r/4) + 4*(l/32) + r%4,
// column l%32 of the (B-rows x A-rows) product, i.e. C[m = l%32][n = ...].
// ---------------------------------------------------------------------------
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef __attribute__((address_space(3))) void lds_void;

constexpr int kBK = 32;                        // k values per slab
constexpr int kStages = 4;                     // slabs in the LDS ring
constexpr int kSlab = 256 * kBK;               // elements per operand slab (both layouts)

// s_waitcnt immediates (gfx9 encoding: vmcnt in bits 3:0, expcnt 6:4,
// lgkmcnt 11:8): wait until at most n vector-memory ops (and no LDS ops) of
// this wavefront are outstanding.
#define NC_WAIT_VM_LGKM0(n) __builtin_amdgcn_s_waitcnt(0x3070 | (n))

// Transposed LDS read through a restrict-qualified pointer. Once inlined, the
// read carries alias-scope information, so the compiler's wait insertion does
// not treat it as possibly reading the in-flight direct loads (which would put
// a full vmcnt(0) drain in front of it). Ordering against those loads comes
// from the explicit waits and barrier of each ring stage.
__device__ __forceinline__ s16x4 lds_read_tr16(lds_s16x4* __restrict__ p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(p);
}

// 16-byte chunk swizzles: K-contiguous slab (chunk slot of row `row`) and
// K-strided slab (chunk offset of k row `kr`, in 8-element chunks).
__device__ __forceinline__ int kc_swz(int row) { return (row >> 2) & 3; }
__device__ __forceinline__ int ks_swz(int kr) { return 4 * (kr & 3); }

// Direct global->LDS staging of one 256 x 32 operand slab: wavefront w moves
// 2 KB with two 1 KB buffer loads (buffer_load_dwordx4 ... lds). The buffer
// descriptor's base is this tile's first row (K-contiguous) or column
// (K-strided) at the slab's first k, rebuilt per slab in scalar registers, so
// the per-lane offsets stay 32-bit whatever the matrix size; measured 3-8 %
// faster per contraction than the flat-address form (global_load_lds).
template <bool KC>
struct DmaOperand {
  const char* base;                            // this tile's first row (column) at k = kbeg, bytes
  size_t kstep;                                // bytes of one slab along k
  unsigned voff[2];                            // per lane, byte offset inside the slab (< 2^32:
                                               // 256 rows or 32 k rows of at most 65,536 columns)
  int dst[2];                                  // instruction base in the slab (elements)
  __device__ __forceinline__ void init(const bf16* A, int ld, int rows, int r0, int kbeg,
                                       int wave, int lane) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      if constexpr (KC) {
        const int R0 = 32 * wave + 16 * j, R = R0 + lane / 4;
        const int c = (lane % 4) ^ kc_swz(R);
        voff[j] = (unsigned)(((size_t)(min(r0 + R, rows - 1) - r0) * ld + c * 8) * 2);
        dst[j] = R0 * kBK;
      } else {
        const int K0 = 4 * wave + 2 * j, kr = K0 + lane / 32;
        const int c = (lane % 32) ^ ks_swz(kr);
        voff[j] = (unsigned)(((size_t)kr * ld + (min(r0 + c * 8, rows - 8) - r0)) * 2);
        dst[j] = K0 * 256;
      }
    }
    base = KC ? (const char*)(A + (size_t)r0 * ld + kbeg) : (const char*)(A + (size_t)kbeg * ld + r0);
    kstep = KC ? kBK * 2 : (size_t)kBK * ld * 2;
  }
  __device__ __forceinline__ void issue(bf16* slab, int st) const {
    // raw buffer (stride 0), range check at 2^31 - 1 bytes (never reached: every
    // offset is inside the matrix), dword 3 = the gfx9 raw-buffer format word
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(base + (size_t)st * kstep), (short)0, 0x7fffffff, 0x00020000);
#pragma unroll
    for (int j = 0; j < 2; ++j)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)(slab + dst[j]), 16, voff[j], 0, 0, 0);
  }
  // fragment of 32 rows starting at row `r` for k step `ks` (0 or 1)
  __device__ __forceinline__ static bf16x8 frag(const bf16* S, int r, int ks, int lane) {
    if constexpr (KC) {
      const int row = r + (lane & 31), c = (2 * ks + (lane >> 5)) ^ kc_swz(row);
      return *reinterpret_cast<const bf16x8*>(S + row * kBK + c * 8);
    } else {
      const int q = lane >> 4, sl = lane & 15;
      const int kr = ks * 16 + (q >> 1) * 8 + (sl >> 2);
      const int col = (r + (q & 1) * 16 + 4 * (sl & 3)) ^ (8 * ks_swz(kr));
      const s16x4 a = lds_read_tr16((lds_s16x4*)(S + kr * 256 + col));
      // k row kr + 4 has the same (kr & 3): same swizzle
      const s16x4 b = lds_read_tr16((lds_s16x4*)(S + (kr + 4) * 256 + col));
      const s16x8 ab = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
      return __builtin_bit_cast(bf16x8, ab);
    }
  }
};

// Extra epilogue operand (the fp32 residual for AddF32, the saved activation
// for Relu2Bwd), read ahead of use: 4 consecutive values per chunk.
template <Epi EPI> struct EpiIn { typedef f32x4 type; };
template <> struct EpiIn<Epi::Relu2Bwd> { typedef bf16x4 type; };
template <> struct EpiIn<Epi::AxpbyT> { typedef bf16x4 type; };
template <> struct EpiIn<Epi::AxpbyF32> { typedef bf16x4 type; };

template <Epi EPI>
__device__ __forceinline__ void epilogue4_in(const GemmArgs& g, int split, int m, int n, f32x4 v,
                                             typename EpiIn<EPI>::type in) {
  const size_t off = (size_t)m * g.ldc + n;
  if constexpr (EPI == Epi::AddF32) {
    __builtin_nontemporal_store(in + v, reinterpret_cast<f32x4*>(static_cast<float*>(g.C) + off));
  } else if constexpr (EPI == Epi::Relu2Bwd) {
    bf16x4 w;
#pragma unroll
    for (int r = 0; r < 4; ++r) w[r] = from_f32<bf16>(v[r] * 2.f * sqrtf(to_f32(in[r])));
    __builtin_nontemporal_store(w, reinterpret_cast<bf16x4*>(static_cast<bf16*>(g.C) + off));
  } else if constexpr (EPI == Epi::AxpbyT || EPI == Epi::AxpbyF32) {
    f32x4 y;
#pragma unroll
    for (int r = 0; r < 4; ++r) y[r] = fmaf(g.alpha, v[r], g.beta * to_f32(in[r]));
    if constexpr (EPI == Epi::AxpbyT) {
      bf16x4 w;
#pragma unroll
      for (int r = 0; r < 4; ++r) w[r] = from_f32<bf16>(y[r]);
      *reinterpret_cast<bf16x4*>(static_cast<bf16*>(g.C) + off) = w;
    } else {
      *reinterpret_cast<f32x4*>(static_cast<float*>(g.C) + off) = y;
    }
  } else {
    epilogue4<bf16, EPI>(g, split, m, n, v);
  }
}

// Staging of one wavefront's 32 x 64 fp32 accumulator block for the epilogue:
// row r, 16-byte chunk c (0..15) at chunk slot c ^ ((r >> 1) & 15) of a 256-byte
// row, so the column writes (32 rows, one chunk) and the row reads (2 or 4 rows,
// consecutive chunks) both touch 32 distinct 16-byte bank groups per 32 lanes.
// The accesses go through restrict-qualified pointers: like the transposed ring
// reads, they then carry alias-scope information, and the compiler's wait
// insertion does not make them wait for the direct loads of the next tile that
// are in flight into other ring slots.
__device__ __forceinline__ int stg_off(int r, int c) { return r * 64 + ((c ^ ((r >> 1) & 15)) << 2); }
__device__ __forceinline__ void stg_put(float* __restrict__ p, f32x4 v) {
  *reinterpret_cast<f32x4*>(p) = v;
}
__device__ __forceinline__ f32x4 stg_get(const float* __restrict__ p) {
  return *reinterpret_cast<const f32x4*>(p);
}

// bf16 staging of a 32 x 64 block (128-byte rows, 16-byte chunk c of row r at
// chunk slot c ^ ((r >> 2) & 7)): 8-byte column writes and 16-byte row reads
// both conflict-free.
__device__ __forceinline__ int stg16_off(int r, int c) { return r * 64 + ((c ^ ((r >> 2) & 7)) << 3); }
__device__ __forceinline__ void stg_put8(bf16* __restrict__ p, bf16x4 v) {
  *reinterpret_cast<bf16x4*>(p) = v;
}
__device__ __forceinline__ bf16x8 stg_get16(const bf16* __restrict__ p) {
  return *reinterpret_cast<const bf16x8*>(p);
}

// s_waitcnt immediate for "at most n (0..63) vector-memory ops outstanding, no
// LDS ops outstanding" (gfx9: vmcnt bits 3:0 and 15:14, expcnt 6:4 left at 7).
#define NC_WAIT_VM_LGKM0_WIDE(n) __builtin_amdgcn_s_waitcnt(0x0070 | ((n) & 15) | (((n) >> 4) << 14))
// only LDS ops: vmcnt at its maximum
#define NC_WAIT_LGKM0() __builtin_amdgcn_s_waitcnt(0xC07F)

template <Epi EPI, bool AK, bool BKC>
__global__ __launch_bounds__(512) void gemm_bf16_kernel(GemmArgs g0) {
  constexpr int BM = 256, BN = 256;
  constexpr int WM = 2, WN = 4, TM = BM / WM, TN = BN / WN;   // 128 x 64 per wave
  constexpr int FM = TM / 32, FN = TN / 32;                   // 4 x 2 MFMA tiles
  constexpr int STAGE = 2 * kSlab;                            // A slab then B slab
  __shared__ __align__(16) bf16 smem[kStages * STAGE];

  const int tid = threadIdx.x;
  // wavefront index made scalar: the slab offsets, LDS bases (M0) and tile
  // coordinates that depend on it are then scalar arithmetic
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, lh = lane >> 5;
  const int wm = wave % WM, wn = wave / WM;

  const int tiles_m = (g0.M + BM - 1) / BM, tiles_n = (g0.N + BN - 1) / BN;
  const int ntiles = tiles_m * tiles_n;
  const int per_item = ntiles * g0.splits;
  const int total = per_item * (g0.batch > 1 ? g0.batch : 1);
  // Tile slots: total rounded up to a multiple of 8, dealt to the 8 XCDs in
  // contiguous ranges of R (the hardware hands workgroups to the XCDs
  // round-robin, so workgroup p runs on XCD p % 8). With one workgroup per
  // slot (gridDim = 8R) each workgroup takes one tile; with fewer (a
  // persistent launch, one workgroup per compute unit) workgroup p walks
  // slots p/8, p/8 + J, p/8 + 2J, ... of its XCD's range (J = gridDim / 8),
  // the order in which a one-tile-per-workgroup launch would run them.
  const int R = ((total + 7) >> 3);
  const int J = gridDim.x >> 3;
  const int xcd = blockIdx.x & 7;
  int slot = blockIdx.x >> 3;
  auto tile_of = [&](int sl) { return xcd * R + sl; };
  if (slot >= R || tile_of(slot) >= total) return;
  // row tiles per group of the XCD's walk (measured per shape, in the step):
  // 4 for the narrow (<= 5 column tiles) unsplit products; 6 for the narrow
  // split-K products (6 x 5 tiles: a whole group is resident on the XCD's 32
  // compute units, so each A panel and each slice of B is fetched once per
  // group; the weight gradients 3-4 % and the lm_head input gradient 8 %
  // faster than with 8) and for the vocabulary-wide lm_head output (six
  // 640 KB A panels stay in a 4 MB L2 while the B panels stream); 8 otherwise
  const int GROUP = (tiles_n <= 5 && g0.splits == 1) ? 4 : ((tiles_n >= 64 || tiles_n <= 5) ? 6 : 8);
  const int per_group = GROUP * tiles_n;
  // split-K: split `split` takes the 64-wide k slabs [split * ns / splits, (split + 1) * ns / splits)
  const int ns = g0.K / 64;
  struct TileAt {
    int item, split, m0, n0, kbeg, nk;
  };
  auto locate = [&](int bid) {
    TileAt a;
    a.item = bid / per_item;
    bid -= a.item * per_item;
    a.split = bid / ntiles;
    const int t = bid - a.split * ntiles;
    const int first_m = (t / per_group) * GROUP;
    const int gsize = min(tiles_m - first_m, GROUP);
    a.m0 = (first_m + (t % per_group) % gsize) * BM;
    a.n0 = ((t % per_group) / gsize) * BN;
    const int sb = (int)((long)a.split * ns / g0.splits), se = (int)((long)(a.split + 1) * ns / g0.splits);
    a.kbeg = sb * 64;
    a.nk = 2 * (se - sb);                                      // 32-wide stages
    return a;
  };
  TileAt cur = locate(tile_of(slot));
  GemmArgs g = batch_item<bf16, EPI>(g0, cur.item);

  DmaOperand<AK> da;
  DmaOperand<BKC> db;
  da.init(static_cast<const bf16*>(g.A), g.lda, g.M, cur.m0, cur.kbeg, wave, lane);
  db.init(static_cast<const bf16*>(g.B), g.ldb, g.N, cur.n0, cur.kbeg, wave, lane);
  // ring slot of stage s of the current tile: (base + s) % kStages
  int base = 0;
  auto issue = [&](int st) {
    bf16* S = smem + ((base + st) & (kStages - 1)) * STAGE;
    da.issue(S, st);
    db.issue(S + kSlab, st);
  };
  f32x16 acc[FM][FN];

  const int ar = wm * TM, br = wn * TN;
  auto read_step = [&](const bf16* S, int ks, bf16x8 (&fa)[FM], bf16x8 (&fb)[FN]) {
#pragma unroll
    for (int i = 0; i < FM; ++i) fa[i] = DmaOperand<AK>::frag(S, ar + i * 32, ks, lane);
#pragma unroll
    for (int j = 0; j < FN; ++j) fb[j] = DmaOperand<BKC>::frag(S + kSlab, br + j * 32, ks, lane);
  };
  auto mfma_step = [&](const bf16x8 (&fa)[FM], const bf16x8 (&fb)[FN]) {
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[j], fa[i], acc[i][j], 0, 0, 0);
  };
  // Wait until at most `after` stages of this wavefront's direct loads are in
  // flight (4 loads per stage) and all of its LDS reads have returned.
  auto wait_after = [&](int after) {
    if (after >= 2) NC_WAIT_VM_LGKM0(8);
    else if (after == 1) NC_WAIT_VM_LGKM0(4);
    else NC_WAIT_VM_LGKM0(0);
  };
  // Workgroup barrier that the scheduler moves nothing across.
  auto barrier = [&]() {
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
  };

  // Epilogue shape: the lane holds C[m][n..n+3] for m = 32i + l32,
  // n = 32j + 8q + 4*lh; each wavefront stages one 32 x 64 fp32 block at a
  // time and reads it back as row segments (256 contiguous bytes per row).
  // An epilogue that reads memory (the residual for AddF32, the saved
  // activation for Relu2Bwd) keeps one register per staged chunk and refills
  // it with the next 32-row block's chunk as soon as it has been used.
  constexpr int CPR = TN / 4;                                  // 16-byte chunks per row
  constexpr int CH = 32 * CPR / 64;                            // chunks per lane per block
  constexpr bool READS = EPI == Epi::AddF32 || EPI == Epi::AddF32Xs || EPI == Epi::Relu2Bwd ||
                        EPI == Epi::AxpbyT || EPI == Epi::AxpbyF32;
  constexpr bool SCALED = EPI == Epi::StoreT || EPI == Epi::Relu2 || EPI == Epi::Relu2Bwd;
  constexpr bool READS_C2 = EPI == Epi::Relu2Bwd || EPI == Epi::AxpbyT || EPI == Epi::AxpbyF32;
  constexpr bool WIDE = !READS && (EPI == Epi::StoreT || EPI == Epi::Relu2);
  constexpr int CPR8 = TN / 8, CH8 = 32 * CPR8 / 64;
  // Vector-memory instructions one wavefront's epilogue issues for a whole
  // tile (every row and column inside the matrix): its stores, plus the
  // operand loads of the epilogues that read memory (AddF32Xs: the residual
  // load, its store and the copy's store; its sum-of-squares stores and the
  // row-scale loads are left out: counting fewer operations than are issued
  // only makes a wait wait longer).
  constexpr int EPI_VMEM =
      WIDE ? FM * CH8 : (EPI == Epi::AddF32Xs ? 3 * FM * CH : (READS ? 2 * FM * CH : FM * CH));
  // wait counts with the epilogue's operations behind one or two stages
  // (capped at the counter's 63: a smaller count only waits longer)
  constexpr int W_E0 = EPI_VMEM < 63 ? EPI_VMEM : 63;
  constexpr int W_E4 = EPI_VMEM + 4 < 63 ? EPI_VMEM + 4 : 63;
  constexpr int W_E8 = EPI_VMEM + 8 < 63 ? EPI_VMEM + 8 : 63;
  typedef typename EpiIn<EPI>::type In;

  // Ping-pong schedule. Each stage is one memory phase (read all fragments of
  // the stage, issue this wavefront's direct loads three stages ahead, wait)
  // and one compute phase (its 16 MFMAs), each closed by a barrier.
  // Wavefronts 4..7 run one phase behind 0..3; wavefronts w and w + 4 share a
  // SIMD, so on every SIMD one wavefront issues MFMAs while the other moves
  // data. Every wavefront passes the same number of barriers (the leading
  // group adds one at the end, the lagging one at the start).
  // Ring safety: the loads of stage s + 3 go into the slot of stage s - 1,
  // which the leading group read two phases earlier and the lagging group in
  // the phase just closed (its reads had returned before that barrier). A
  // stage's loads from both groups have landed before the barrier that opens
  // the leading group's memory phase for it, since each wavefront waits for
  // its own share of stage s + 1 in its memory phase for stage s.
  //
  // Persistent launch: after the last stage of a tile (every ring read done),
  // the first two stages of the next tile are requested into the next two
  // slots, then the epilogue runs, staging through the other two slots while
  // those loads are in flight. The epilogue's own loads and stores are issued
  // after them; gfx9 counts loads and stores in one in-order counter, so the
  // first two waits of the next tile allow the epilogue's EPI_VMEM operations
  // to remain outstanding (when the tile was whole, so that every one of them
  // was issued; otherwise they wait for everything). A barrier after the
  // epilogue frees the staging slots before the next tile's third stage is
  // requested into them.
  const bool lag = __builtin_amdgcn_readfirstlane(wave) >= 4;
  const bool whole = (g0.M % BM) == 0 && (g0.N % BN) == 0;
  int nk = cur.nk;
#pragma unroll
  for (int st = 0; st < kStages - 1; ++st)
    if (st < nk) issue(st);
  // The empty asm makes the epilogue's arguments live in scalar registers
  // here, so their loads are not scheduled into the loop.
  asm volatile("" ::"s"(g.C), "s"(g.C2), "s"(g.ldc), "s"(g.ldc2));
  wait_after(min(kStages - 2, nk - 1));
  bool carried = false;                                        // epilogue ops queued behind stages 0, 1
  for (;;) {
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
    barrier();
    if (lag) barrier();
    bf16x8 fa0[FM], fb0[FN], fa1[FM], fb1[FN];
    for (int s = 0; s < nk; ++s) {
      const bf16* S = smem + ((base + s) & (kStages - 1)) * STAGE;
      read_step(S, 0, fa0, fb0);
      read_step(S, 1, fa1, fb1);
      if (s + kStages - 1 < nk) issue(s + kStages - 1);
      const int after = min(s + kStages - 1, nk - 1) - (s + 1);
      if (s == 0 && carried) {
        // stage 1 then the previous epilogue's operations, then stages 2 and 3
        if (after >= 2) NC_WAIT_VM_LGKM0_WIDE(W_E8);
        else NC_WAIT_VM_LGKM0_WIDE(W_E0);
      } else {
        wait_after(after);
      }
      barrier();
      mfma_step(fa0, fb0);
      mfma_step(fa1, fb1);
      barrier();
    }
    if (!lag) barrier();

    // row scales of this tile's rows (the lane's accumulator rows), requested
    // before the next tile's loads so that waiting for them never waits for those
    float rsv[FM];
#pragma unroll
    for (int i = 0; i < FM; ++i) rsv[i] = 1.0f;
    if constexpr (SCALED) {
      if (g0.rs) {
#pragma unroll
        for (int i = 0; i < FM; ++i) rsv[i] = g0.rs[min(cur.m0 + wm * TM + i * 32 + l32, g0.M - 1)];
      }
    }

    // next tile of this workgroup, if any: its first two stages go out now
    slot += J;
    const bool more = slot < R && tile_of(slot) < total;
    const TileAt me = cur;
    const int tbase = base;
    if (more) {
      cur = locate(tile_of(slot));
      const GemmArgs gn = batch_item<bf16, EPI>(g0, cur.item);
      da.init(static_cast<const bf16*>(gn.A), gn.lda, gn.M, cur.m0, cur.kbeg, wave, lane);
      db.init(static_cast<const bf16*>(gn.B), gn.ldb, gn.N, cur.n0, cur.kbeg, wave, lane);
      base = tbase + nk;
      issue(0);
      if (cur.nk > 1) issue(1);
    }
    // nothing of the epilogue below moves above these loads
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);

    // ---- epilogue of tile `me` ----
    const GemmArgs ge = batch_item<bf16, EPI>(g0, me.item);
    const int m0 = me.m0, n0 = me.n0;
    In pre[CH];
    auto fetch1 = [&](int i, int u) -> In {
      const int c = lane + 64 * u;
      const int m = min(m0 + wm * TM + i * 32 + c / CPR, ge.M - 1);
      const int n = min(n0 + wn * TN + (c % CPR) * 4, ge.N - 4);
      // read once, right before the output replaces it: non-temporal, like the stores
      if constexpr (READS_C2)
        return __builtin_nontemporal_load(
            reinterpret_cast<const bf16x4*>(static_cast<const bf16*>(ge.C2) + (size_t)m * ge.ldc2 + n));
      else
        return __builtin_nontemporal_load(
            reinterpret_cast<const f32x4*>(static_cast<const float*>(ge.C) + (size_t)m * ge.ldc + n));
    };
    if constexpr (READS) {
#pragma unroll
      for (int u = 0; u < CH; ++u) pre[u] = fetch1(0, u);
    }
    // staging: waves 0-3 in the slot two past the next tile's first stage,
    // waves 4-7 in the one after (neither receives a load before the barrier
    // that ends this epilogue)
    float* wl = reinterpret_cast<float*>(smem + ((tbase + nk + 2 + (wave >> 2)) & (kStages - 1)) * STAGE) +
                (wave & 3) * 32 * 64;
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      if constexpr (WIDE) {
        // bf16 outputs with no extra operand: the values are rounded (after
        // relu^2) in registers and staged as bf16, half the LDS traffic of
        // fp32 staging; read back 8 values (16 bytes) per lane and store
        bf16* wb = reinterpret_cast<bf16*>(wl);
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            bf16x4 w;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              float a = acc[i][j][4 * q + e] * rsv[i];
              if constexpr (EPI == Epi::Relu2) {
                a = fmaxf(a, 0.f);
                a *= a;
              }
              w[e] = from_f32<bf16>(a);
            }
            stg_put8(wb + stg16_off(l32, 4 * j + q) + 4 * lh, w);
          }
#pragma unroll
        for (int u = 0; u < CH8; ++u) {
          const int c = lane + 64 * u;
          const int r = c / CPR8, cc = c % CPR8;
          const int m = m0 + wm * TM + i * 32 + r, n = n0 + wn * TN + cc * 8;
          const bf16x8 w = stg_get16(wb + stg16_off(r, cc));
          if (m < ge.M && n < ge.N)
            __builtin_nontemporal_store(
                w, reinterpret_cast<bf16x8*>(static_cast<bf16*>(ge.C) + (size_t)m * ge.ldc + n));
        }
      } else {
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            f32x4 v = {acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]};
            if constexpr (SCALED) v *= rsv[i];
            stg_put(wl + stg_off(l32, 8 * j + 2 * q + lh), v);
          }
#pragma unroll
        for (int u = 0; u < CH; ++u) {
          const int c = lane + 64 * u;
          const int r = c / CPR, cc = c % CPR;
          const int m = m0 + wm * TM + i * 32 + r, n = n0 + wn * TN + cc * 4;
          const f32x4 v = stg_get(wl + stg_off(r, cc));
          if constexpr (READS) {
            const In x = pre[u];
            // x is waited for here on every path, also where the store below
            // is skipped: otherwise its load could still be in flight when
            // the next tile reuses the register, and the compiler would wait
            // for everything outstanding there, the next tile's loads included
            asm volatile("" ::"v"(x));
            if (i + 1 < FM) pre[u] = fetch1(i + 1, u);
            if constexpr (EPI == Epi::AddF32Xs) {
              // new residual row segment, its bf16 copy, and the sum of its
              // squares over the wavefront's 64 columns: the 16 lanes of a
              // DPP row hold one row's 16 chunks
              const f32x4 y = x + v;
              const float ss = row16_sum(y[0] * y[0] + y[1] * y[1] + y[2] * y[2] + y[3] * y[3]);
              if (m < ge.M && n < ge.N) {
                const size_t off = (size_t)m * ge.ldc + n;
                __builtin_nontemporal_store(y, reinterpret_cast<f32x4*>(static_cast<float*>(ge.C) + off));
                const bf16x4 w = {from_f32<bf16>(y[0]), from_f32<bf16>(y[1]), from_f32<bf16>(y[2]),
                                  from_f32<bf16>(y[3])};
                __builtin_nontemporal_store(w, reinterpret_cast<bf16x4*>(static_cast<bf16*>(ge.xc) + off));
                if (cc == 0) ge.ssq[(size_t)m * (ge.N / 64) + (n0 + wn * TN) / 64] = ss;
              }
            } else {
              if (m < ge.M && n < ge.N) epilogue4_in<EPI>(ge, me.split, m, n, v, x);
            }
          } else {
            if (m < ge.M && n < ge.N) epilogue4<bf16, EPI>(ge, me.split, m, n, v);
          }
        }
      }
    }
    if (!more) break;

    // every wavefront's staging reads have returned: the staging slots are free
    NC_WAIT_LGKM0();
    barrier();
    nk = cur.nk;
    if (nk > 2) issue(2);
    carried = whole;
    if (carried) {
      // stage 0, then stage 1, this epilogue's operations and stage 2
      if (nk > 2) NC_WAIT_VM_LGKM0_WIDE(W_E8);
      else NC_WAIT_VM_LGKM0_WIDE(W_E4);
    } else {
      NC_WAIT_VM_LGKM0(0);
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

// dst[i] (type T) = sum_s part[s * n + i] in split order
template <typename T>
__global__ void splitk_reduce_t_kernel(const float* __restrict__ part, int splits, size_t n4,
                                       size_t n, T* __restrict__ dst) {
  typedef T T4 __attribute__((ext_vector_type(4)));
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n4;
       i += (size_t)gridDim.x * blockDim.x) {
    f32x4 s = reinterpret_cast<const f32x4*>(part)[i];
    for (int k = 1; k < splits; ++k) s += reinterpret_cast<const f32x4*>(part + (size_t)k * n)[i];
    T4 w = {from_f32<T>(s[0]), from_f32<T>(s[1]), from_f32<T>(s[2]), from_f32<T>(s[3])};
    reinterpret_cast<T4*>(dst)[i] = w;
  }
}

template <typename T, bool AK, bool BKC, Epi EPI, int BM, int BN, int WM, int WN>
hipError_t launch_tiles(const GemmArgs& g, hipStream_t s) {
  const int tiles = ((g.M + BM - 1) / BM) * ((g.N + BN - 1) / BN) * g.splits *
                    (g.batch > 1 ? g.batch : 1);
  const int grid = (tiles + 7) / 8 * 8;
  hipLaunchKernelGGL((gemm_kernel<T, AK, BKC, EPI, BM, BN, WM, WN>), dim3(grid), dim3(WM * WN * 64), 0,
                     s, g);
  return hipGetLastError();
}

// Large bf16 products take the 256x256 tile when it still gives at least one
// tile per CU; everything else (and fp32) the 128x128 tile.
// The 256x256 kernel addresses each operand slab through a buffer descriptor
// with 32-bit per-lane offsets, range-checked at 2^31 - 1 bytes: a K-contiguous
// slab spans 256 rows of its operand's stride, so both strides must stay
// below 2^22 elements (2^31 bytes / (256 rows * 2 bytes)). Larger strides take
// the 128x128 kernel, which uses full-width addresses.
std::atomic<bool> g_gemm_persist{true};

bool strides_fit_256(const GemmArgs& g) { return g.lda < (1 << 22) && g.ldb < (1 << 22); }

int choose_tile(bool bf16, const GemmArgs& g) {
  if (!bf16 || g.tile == 128) return 128;
  if (g.tile == 256) return 256;
  if (!strides_fit_256(g)) return 128;
  const long big_tiles = (long)((g.M + 255) / 256) * ((g.N + 255) / 256) * g.splits *
                        (g.batch > 1 ? g.batch : 1);
  return (g.M >= 256 && g.N >= 256 && big_tiles >= 256) ? 256 : 128;
}

template <typename T, bool AK, bool BKC, Epi EPI>
hipError_t launch(const GemmArgs& g, hipStream_t s) {
  if constexpr (std::is_same<T, bf16>::value) {
    if (choose_tile(true, g) == 256) {
      const int tiles = ((g.M + 255) / 256) * ((g.N + 255) / 256) * g.splits *
                        (g.batch > 1 ? g.batch : 1);
      int grid = (tiles + 7) / 8 * 8;
      // Whole-tile products with more tiles than compute units run persistent:
      // one workgroup per compute unit walking its XCD's tiles, each next
      // tile's first loads overlapping the current tile's epilogue.
      const int persist = device_cus() / 8 * 8;
      if (g_gemm_persist.load(std::memory_order_relaxed) && g.splits == 1 && g.M % 256 == 0 &&
          g.N % 256 == 0 && persist >= 8 && grid > persist)
        grid = persist;
      hipLaunchKernelGGL((gemm_bf16_kernel<EPI, AK, BKC>), dim3(grid), dim3(512), 0, s, g);
      return hipGetLastError();
    }
  }
  return launch_tiles<T, AK, BKC, EPI, 128, 128, 2, 2>(g, s);
}

template <typename T, bool AK, bool BKC>
hipError_t dispatch_epi(Epi epi, const GemmArgs& g, hipStream_t s) {
  switch (epi) {
    case Epi::StoreT: return launch<T, AK, BKC, Epi::StoreT>(g, s);
    case Epi::StoreF32: return launch<T, AK, BKC, Epi::StoreF32>(g, s);
    case Epi::AddF32: return launch<T, AK, BKC, Epi::AddF32>(g, s);
    case Epi::Relu2: return launch<T, AK, BKC, Epi::Relu2>(g, s);
    case Epi::Relu2Bwd: return launch<T, AK, BKC, Epi::Relu2Bwd>(g, s);
    case Epi::PartialF32: return launch<T, AK, BKC, Epi::PartialF32>(g, s);
    case Epi::AxpbyT: return launch<T, AK, BKC, Epi::AxpbyT>(g, s);
    case Epi::AxpbyF32: return launch<T, AK, BKC, Epi::AxpbyF32>(g, s);
    case Epi::AddF32Xs: return launch<T, AK, BKC, Epi::AddF32Xs>(g, s);
  }
  return hipErrorInvalidValue;
}

template <typename T>
hipError_t dispatch(bool ak, bool bk, Epi epi, const GemmArgs& g, hipStream_t s) {
  if (ak && bk) return dispatch_epi<T, true, true>(epi, g, s);
  if (ak && !bk) return dispatch_epi<T, true, false>(epi, g, s);
  if (!ak && !bk) return dispatch_epi<T, false, false>(epi, g, s);
  return dispatch_epi<T, false, true>(epi, g, s);
}

}  // namespace

hipError_t gemm(DType t, bool a_kcontig, bool b_kcontig, Epi epi, const GemmArgs& g,
                hipStream_t stream) {
  const int bk = t == DType::BF16 ? 64 : 32;
  if (g.M <= 0 || g.N <= 0 || g.K <= 0 || g.splits <= 0) return hipErrorInvalidValue;
  if (g.M % 16 || g.N % 16 || g.K % bk || g.K / bk < g.splits) return hipErrorInvalidValue;
  if (epi != Epi::PartialF32 && g.splits != 1) return hipErrorInvalidValue;
  if (g.batch < 0 || (g.batch > 1 && epi == Epi::PartialF32)) return hipErrorInvalidValue;
  if ((epi == Epi::Relu2Bwd || epi == Epi::AxpbyT || epi == Epi::AxpbyF32) && !g.C2)
    return hipErrorInvalidValue;
  if (epi == Epi::AddF32Xs && (!g.xc || !g.ssq || g.N % 64 || g.batch > 1)) return hipErrorInvalidValue;
  if (g.rs && (g.batch > 1 || !(epi == Epi::StoreT || epi == Epi::Relu2 || epi == Epi::Relu2Bwd)))
    return hipErrorInvalidValue;
  if (t == DType::BF16 && g.tile == 256 && !strides_fit_256(g)) return hipErrorInvalidValue;
  if ((long)((g.M + 127) / 128) * ((g.N + 127) / 128) * g.splits * (g.batch > 1 ? g.batch : 1) >
      (1L << 30))
    return hipErrorInvalidValue;
  return t == DType::BF16 ? dispatch<bf16>(a_kcontig, b_kcontig, epi, g, stream)
                          : dispatch<float>(a_kcontig, b_kcontig, epi, g, stream);
}

void gemm_set_persistent(bool on) { g_gemm_persist.store(on); }

int gemm_tile(DType t, bool a_kcontig, bool b_kcontig, const GemmArgs& g) {
  (void)a_kcontig;
  (void)b_kcontig;
  return choose_tile(t == DType::BF16, g);
}

int device_cus() {
  static int cache[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 256;
  if (dev < 64 && cache[dev] > 0) return cache[dev];
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
    n = 256;
  if (dev < 64) cache[dev] = n;
  return n;
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

hipError_t splitk_reduce_t(DType t, const float* part, int splits, size_t n, void* dst,
                           hipStream_t stream) {
  if (n % 4 || splits < 1) return hipErrorInvalidValue;
  const size_t n4 = n / 4;
  const int block = 256;
  const size_t want = (n4 + block - 1) / block;
  const int grid = (int)(want < 4096 ? want : 4096);
  if (t == DType::BF16)
    hipLaunchKernelGGL(splitk_reduce_t_kernel<bf16>, dim3(grid > 0 ? grid : 1), dim3(block), 0,
                       stream, part, splits, n4, n, static_cast<bf16*>(dst));
  else
    hipLaunchKernelGGL(splitk_reduce_t_kernel<float>, dim3(grid > 0 ? grid : 1), dim3(block), 0,
                       stream, part, splits, n4, n, static_cast<float*>(dst));
  return hipGetLastError();
}

}  // namespace nc
