// Host-side launch interface of the HIP kernels. Every function enqueues work
// on `stream` and returns hipSuccess or the launch error; none allocates.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace nc {

enum class DType { F32 = 0, BF16 = 1 };

// ---- GEMM: C[M,N] (op)= sum_k A(m,k) * B(n,k) ---------------------------
// A(m,k) = a_kcontig ? A[m*lda + k] : A[k*lda + m]   (likewise for B)
enum class Epi {
  StoreT,      // C (element type T) = acc
  StoreF32,    // C (float) = acc
  AddF32,      // C (float) += acc
  Relu2,       // C (T) = a = relu(acc)^2
  Relu2Bwd,    // C (T) = acc * 2 * sqrt(C2[m,n])       (C2 holds a = relu(u)^2, type T)
  PartialF32,  // C (float) + split*M*ldc = acc over this split's K range
  AxpbyT,      // C (T) = alpha * acc + beta * C2[m,n] (C2 of type T)
  AxpbyF32,    // C (float) = alpha * acc + beta * C2[m,n] (C2 of type T)
  AddF32Xs,    // C (float) += acc; xc (T) = the new C; ssq[m * (N/64) + n/64] = sum of the new
               // C[m, :]^2 over each 64-column group (N % 64 == 0)
};
struct GemmArgs {
  const void* A;
  const void* B;
  void* C;
  void* C2;
  int M, N, K;
  int lda, ldb, ldc, ldc2;
  int splits;        // K slices (PartialF32 only); K % (splits * 64) == 0
  int tile;          // output tile edge: 0 = choose, 128 or 256 (256: bf16 only)
  int batch;         // independent products of this shape (0 or 1: one)
  int64_t sa, sb, sc, sc2;  // element strides between batch items of A, B, C and C2
  float alpha, beta;        // Axpby epilogues
  void* xc;                 // AddF32Xs: copy of the new C rows in T (ld ldc)
  float* ssq;               // AddF32Xs: [M][N/64] sums of squares of the new C rows
  // StoreT, Relu2, Relu2Bwd: acc of row m is multiplied by rs[m] before the
  // epilogue's operation (an RMSNorm's row scale folded into the product whose
  // A operand is the unnormalised row); null: no scale. Unbatched only.
  const float* rs;
};
// compute units of the current device (256 when it cannot be queried)
int device_cus();
hipError_t gemm(DType t, bool a_kcontig, bool b_kcontig, Epi epi, const GemmArgs& g,
                hipStream_t stream);
// Schedule of the 256-tile kernel for whole-tile unsplit products with more
// tiles than compute units: persistent (default; one workgroup per compute
// unit, the next tile's first loads overlapping each epilogue) or one
// workgroup per tile. Results are bitwise identical either way.
void gemm_set_persistent(bool on);
// Tile edge the kernel will use for these arguments (128 or 256).
int gemm_tile(DType t, bool a_kcontig, bool b_kcontig, const GemmArgs& g);
// out[c][r] = in[r][c] for an R x C matrix of T (row strides ld_in, ld_out)
hipError_t transpose(DType t, const void* in, int R, int C, int ld_in, void* out, int ld_out,
                     hipStream_t s);
// dst[i] (=|+=) sum_s part[s*n + i], s = 0..splits-1, in a fixed order.
hipError_t splitk_reduce(const float* part, int splits, size_t n, float* dst, bool accumulate,
                         hipStream_t stream);
// dst[i] (type of t) = sum_s part[s*n + i], s = 0..splits-1, in a fixed order.
hipError_t splitk_reduce_t(DType t, const float* part, int splits, size_t n, void* dst,
                           hipStream_t stream);

// ---- norms and embedding --------------------------------------------------
// x[m,:] = n(E[tok[m],:]) (fp32), rinv[m]; ids outside [0,V) are clamped and flagged.
// Optionally xb[m,:] = T(x[m,:]) and rinv_x[m] = 1/sqrt(mean(x[m,:]^2) + eps) (the next
// norm's row scale), when both are non-null.
hipError_t embed_norm_fwd(DType t, const void* E, const int32_t* tok, int M, int d, int V,
                          float eps, float* x, float* rinv, uint32_t* status, hipStream_t s,
                          void* xb = nullptr, float* rinv_x = nullptr);
// rinv[m] = 1 / sqrt(sum_p ssq[m * P + p] / d + eps), p = 0..P-1 in order
hipError_t ssq_rinv(const float* ssq, int M, int P, int d, float eps, float* rinv, hipStream_t s);
// y[m,:] = n(x[m,:]) as T, rinv[m]
hipError_t rmsnorm_fwd(DType t, const float* x, int M, int d, float eps, void* y, float* rinv,
                       hipStream_t s);
// dx[m,:] (=|+=) rinv*(dy - y*mean(dy*y)); dy and y of type T; optionally g = T(dx).
// prescaled: y is the unnormalised input v and dy the gradient already multiplied by
// rinv, so dx (=|+=) dy - rinv^2 * v * mean(dy * v) (the same gradient).
hipError_t rmsnorm_bwd(DType t, const void* dy, const void* y, const float* rinv, int M, int d,
                       float* dx, bool accumulate, void* g, hipStream_t s, bool prescaled = false);
// embedding-norm backward + deterministic scatter into dE (fp32, every row written)
struct EmbedBwdScratch {
  int32_t* counts;       // [V + 1]
  int32_t* offsets;      // [V + 1]
  int32_t* cursor;       // [V]
  int32_t* list;         // [M]
  int32_t* item_off;     // [V + 1]
  int32_t* part_off;     // [V + 1]
  int32_t* item_bucket;  // [embed_bwd_max_pieces(M, V)]
  int32_t* scan_blocks;  // [embed_bwd_scan_blocks(V)]
  float* part;           // [embed_bwd_max_parts(M), d]
};
// int32 entries of the id scan's per-block sums
uint64_t embed_bwd_scan_blocks(int V);
uint64_t embed_bwd_max_pieces(int64_t M, int V);
uint64_t embed_bwd_max_parts(int64_t M);
hipError_t embed_bwd(DType t, const void* E, const int32_t* tok, const float* rinv0,
                     const float* dx, int M, int d, int V, EmbedBwdScratch ws, float* dE,
                     bool accumulate, hipStream_t s);

// ---- rotary + QK-norm -------------------------------------------------------
// [T, half] cos, then sin, of positions t0 .. t0 + T - 1
hipError_t rope_table(int T, int half, double base, float* cs, hipStream_t s, int t0 = 0);
// in place on qkv[M, ldq]: H query heads at cols [0, H*128), the key head at [H*128, H*128+128).
// rinv_qk may be null. With a cache ([M/T][max_seq][256]), the rotated, normalised key and the
// value of row m also go to position pos0 + m % T of sequence m / T.
hipError_t rope_qknorm_fwd(DType t, void* qkv, int ldq, int M, int T, int H, const float* cs,
                           float eps, float* rinv_qk, hipStream_t s, void* cache = nullptr,
                           int max_seq = 0, int pos0 = 0);
// rs (may be null): the query and key gradients of row m are multiplied by rs[m]
hipError_t rope_qknorm_bwd(DType t, void* dqkv, int ldd, const void* qkv, int ldq, int M, int T,
                           int H, const float* cs, const float* rinv_qk, hipStream_t s,
                           const float* rs = nullptr);

// ---- attention -------------------------------------------------------------
// qkv: [B*T, ldq] with q heads, then k, then v (each 128 wide); o: [B*T, H*128]; lse: [B, H, T]
hipError_t attn_fwd(DType t, const void* qkv, int ldq, int B, int T, int H, void* o, float* lse,
                    hipStream_t s);
// writes dq into dqkv[:, 0:H*128], dk and dv into the next two 128-col blocks,
// and delta[b,h,t] = <dO, O> (o: the forward's output, [B*T, H*128]);
// scratch holds attn_bwd_scratch_floats(B, T) floats of partial dK/dV sums
// (none, and scratch may be null, when T <= 2048: dK/dV are written directly)
size_t attn_bwd_scratch_floats(int B, int T);
// rs (may be null): dV of key row m is multiplied by rs[m] (the row scale of the
// RMSNorm folded into the QKV product; rope_qknorm_bwd applies it to dQ and dK).
// ds (may be null): attn_bwd_ds_elems(B, T, H) elements of T; when given, delta is
// computed first, the dK/dV kernel stores the dS it forms there and dQ is one
// product over it (instead of a dQ kernel that recomputes S and dP).
size_t attn_bwd_ds_elems(int B, int T, int H);
hipError_t attn_bwd(DType t, const void* qkv, int ldq, const void* o, const void* dout, const float* lse,
                    float* delta, int B, int T, int H, void* dqkv, int ldd, float* scratch,
                    hipStream_t s, const float* rs = nullptr, void* ds = nullptr);
// Device address (current device) of the library's fixed attention-backward
// scratch array of kAttnFixedScratchBytes, for the entry point that allocates
// nothing; looked up once per device.
constexpr size_t kAttnFixedScratchBytes = (size_t)32 << 20;
hipError_t attn_fixed_scratch(void** ptr);

// ---- cross-entropy -----------------------------------------------------------
// rows of logits [R, V] (T): per-row loss (fp32) and dlogits (T) = (softmax(z)-onehot)*(1-(z/c)^2)*w;
// dlogits may equal logits (the gradient then replaces them); rs (may be null): the
// gradient of row r is also multiplied by rs[r]
hipError_t softcap_ce(DType t, const void* logits, const int32_t* tgt, int R, int V, float cap,
                      float w, float* loss_rows, void* dlogits, uint32_t* status, hipStream_t s,
                      const float* rs = nullptr);
hipError_t loss_mean(const float* loss_rows, int M, float* out, uint32_t* status, hipStream_t s);
// out[0] = sum of loss_rows[i] over i with token_bytes[targets[i]] > 0, out[1] = sum of those
// lengths, out[2] = out[0] / (ln 2 * out[1]) (NaN when out[1] = 0); fp64, fixed order
hipError_t bits_per_byte(const float* loss_rows, const int32_t* targets, int M, const int32_t* token_bytes,
                         int V, double* out, hipStream_t s);

// ---- inference: KV cache, decode attention ---------------------------------------
// Cache of one layer: [B][max_seq][256] of T (k-hat then v, 128 each).
// Attention of one new query row per batch row b (q-hat in qkv row b) over
// cache positions 0..pos: chunks of 64 keys give fp32 partial sum_u p v and
// sum_u p (p shifted by the fixed score bound), combined in chunk order into
// o[b, H*128] (T). part holds B * ceil((pos+1)/64) * H * 129 floats.
hipError_t decode_attn(DType t, const void* qkv, int ldq, int B, int H, const void* cache,
                       int max_seq, int pos, float* part, void* o, int ldo, hipStream_t s);
// bf16 products with few rows: C[m, n] (epi) sum_k X[m, k] W[n, k] for m < M <=
// kSkinnyMaxRows; W [N, K] and X [M, K] row-major bf16 (K-contiguous), N % 16 == 0,
// K % 32 == 0, leading dimensions multiples of 8 (W, X) and 4 (C).
enum class SkEpi {
  StoreT,      // C (bf16) = acc
  AddF32,      // C (float) += acc; optionally xb (bf16) = C and ssq_out = per-16-column sums of C^2
  Relu2,       // C (bf16) = relu(acc)^2
  SoftcapF32,  // C (float) = cap * tanh(acc / cap)
};
constexpr int kSkinnyMaxRows = 32;
struct SkArgs {
  const void* W;
  int ldw;
  const void* X;          // bf16 [M, K]
  int ldx;
  void* C;
  int ldc;
  int M, N, K;
  // RMS norm of the rows of X folded in (acc scaled by 1/sqrt(ss/K + eps)), ss summed from
  // ssq_in[j * 32 + m], j < nssq (null: no norm)
  const float* ssq_in;
  int nssq;
  float eps;
  void* xb;               // AddF32 only: bf16 copy of the new C rows, ld ldc (null: none)
  float* ssq_out;         // AddF32 only: [N/16][32] sums of squares of the new C rows (null: none)
  float cap;
  float* part;            // split partials: skinny_part_bytes
  uint32_t* cnt;          // N/16 arrival counters, zero on entry (left zero)
  int splits;             // k slices; 0 = skinny_splits(N, K)
  int ntile;              // 16-column tiles per workgroup (1, 2 or 4); 0 = skinny_ntile(N, K)
};
// k splits the product uses, and the partial-tile scratch they need
int skinny_splits(int N, int K);
size_t skinny_part_bytes(int M, int N, int K, int splits = 0);
int skinny_ntile(int N, int K);
hipError_t skinny_gemm(const SkArgs& a, SkEpi epi, hipStream_t s);
// x[m] = n(E[tok[m]]) (fp32), xb[m] = bf16 copy, ssq[j * 32 + m] = sum of x[m]^2 over columns
// 16j..16j+15; one row per sequence (M <= 32), d <= 2048
hipError_t decode_embed(const void* E, const int32_t* tok, int M, int d, int V, float eps, float* x,
                        void* xb, float* ssq, uint32_t* status, hipStream_t s);
// dst[r, :] = src[(r + 1) * stride - 1, :] for r < rows, 0 for rows <= r < rows_pad (T, width d)
hipError_t gather_last_rows(DType t, const void* src, int stride, int rows, int rows_pad, int d,
                            void* dst, hipStream_t s);
// out[r, v] = c * tanh(in[r, v] / c), fp32, r < rows
hipError_t softcap_rows(const float* in, int rows, int V, float cap, float* out, hipStream_t s);
// ---- optimizer step -------------------------------------------------------------
constexpr int kOptMaxRanges = 160;        // tensors of one parameter buffer, at most
constexpr int kNormBlocksPerRange = 64;   // fixed grid: the norm is bitwise reproducible
constexpr int kMuonParts = 256;           // blocks (and fp64 partials) of the momentum kernel
struct OptRanges {                        // element ranges of a flat fp32 buffer
  uint64_t off[kOptMaxRanges];
  uint64_t cnt[kOptMaxRanges];
  int n;
};
struct AdamWArgs {
  float lr, beta1, beta2, eps;
  float decay;                            // 1 - lr * weight_decay
  float bc1, bc2;                         // 1 / (1 - beta^step)
};
// norm_scale[0] = ||grads over the ranges||_2, norm_scale[1] = min(1, max_norm / (norm + 1e-6))
// (1 when max_norm <= 0); partial holds n * kNormBlocksPerRange doubles
hipError_t grad_norm(const float* grads, const OptRanges& rg, double* partial, float max_norm,
                     float* norm_scale, hipStream_t s);
// AdamW on n elements; the gradient is scaled by norm_scale[1]
hipError_t adamw(DType t, void* p, const float* g, float* m, float* v, size_t n, const AdamWArgs& a,
                 const float* norm_scale, hipStream_t s);
// For `items` matrices of n elements (g and buf at stride gs, u packed):
// buf = mu buf + s g, u = s g + mu buf (s = norm_scale[1]); kMuonParts fp64
// partials of ||u||^2 per item. n and gs are multiples of 4.
hipError_t muon_momentum(const float* g, float* buf, size_t gs, float* u, size_t n, int items,
                         float mu, const float* norm_scale, double* partial, hipStream_t s);
// x (T) = u / (||u||_F + 1e-7), per item (u, x packed)
hipError_t muon_normalize(DType t, const float* u, size_t n, int items, const double* partial,
                          void* x, hipStream_t s);
// p (T) = p * decay - coef * x (fp32), per item (p at stride ps, x packed)
hipError_t muon_update(DType t, void* p, size_t ps, const float* x, size_t n, int items, float decay,
                       float coef, hipStream_t s);
// ---- init and utilities -----------------------------------------------------
struct InitSeg {
  size_t begin, end;   // element range [begin, end)
  double std;
};
hipError_t init_params(DType t, uint64_t seed, const InitSeg* segs, int nseg, size_t total,
                       void* params, hipStream_t s);
hipError_t fill_zero(void* p, size_t bytes, hipStream_t s);

}  // namespace nc
