// Host side of the library: config validation, the flat parameter layout, the
// workspace plan and the kernel sequence of one training step. Stateless:
// every buffer belongs to the caller and every launch goes on the caller's
// stream. See include/nanochat.h for the contract of each entry point.
#include "../../include/nanochat.h"

#include <math.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <string>
#include <vector>

#include "launch.h"

using nc::DType;
using nc::Epi;

namespace {

thread_local int g_last_hip = 0;
constexpr uint64_t kAlign = 256;

inline uint64_t align_up(uint64_t v, uint64_t a) { return (v + a - 1) / a * a; }

struct Dims {
  int L, d, H, F, Q, V, T, B;
  int64_t M;
  size_t esz;   // bytes per element of dtype
  DType dt;
};

int validate(const nc_config* c) {
  if (!c) return NC_ERR_NULL;
  if (c->n_kv_head != 1 || c->head_dim != 128) return NC_ERR_UNSUPPORTED;
  // width 64*depth must hold whole 128-dim heads: depth even, H = depth/2 <= 16
  if (c->depth < 2 || c->depth > 32 || c->depth % 2) return NC_ERR_INVALID_CONFIG;
  if (c->vocab_size < 128 || c->vocab_size > 65536 || c->vocab_size % 128) return NC_ERR_INVALID_CONFIG;
  if (c->seq_len < 64 || c->seq_len % 64) return NC_ERR_INVALID_CONFIG;
  if (c->batch < 1) return NC_ERR_INVALID_CONFIG;
  if ((int64_t)c->batch * c->seq_len > (int64_t)1 << 30) return NC_ERR_INVALID_CONFIG;
  if (!(c->softcap > 0.f) || !(c->rope_base > 1.f) || !(c->rms_eps >= 0.f) || !(c->init_std > 0.f))
    return NC_ERR_INVALID_CONFIG;
  if (c->dtype != NC_F32 && c->dtype != NC_BF16) return NC_ERR_INVALID_CONFIG;
  return NC_OK;
}

Dims dims_of(const nc_config* c) {
  Dims D;
  D.L = c->depth;
  D.d = 64 * c->depth;
  D.H = D.d / 128;
  D.F = 4 * D.d;
  D.Q = D.d + 256;
  D.V = c->vocab_size;
  D.T = c->seq_len;
  D.B = c->batch;
  D.M = (int64_t)c->batch * c->seq_len;
  D.dt = c->dtype == NC_BF16 ? DType::BF16 : DType::F32;
  D.esz = c->dtype == NC_BF16 ? 2 : 4;
  return D;
}

struct Tensor {
  const char* kind;
  int layer;
  int64_t rows, cols;
  uint64_t offset;
};

std::vector<Tensor> layout_of(const Dims& D) {
  std::vector<Tensor> t;
  uint64_t off = 0;
  auto add = [&](const char* k, int l, int64_t r, int64_t c) {
    t.push_back({k, l, r, c, off});
    off = align_up(off + (uint64_t)(r * c), 128);
  };
  add("E", -1, D.V, D.d);
  for (int l = 0; l < D.L; ++l) {
    add("Wqkv", l, D.Q, D.d);
    add("Wo", l, D.d, D.d);
    add("Wfc", l, D.F, D.d);
    add("Wpr", l, D.d, D.F);
  }
  add("U", -1, D.V, D.d);
  return t;
}

uint64_t param_elems(const Dims& D) {
  const auto t = layout_of(D);
  return align_up(t.back().offset + (uint64_t)(t.back().rows * t.back().cols), 128);
}

// Rows of the lm_head / loss processed at once. A chunk's logits (activation
// type; the cross-entropy kernel overwrites them with their gradient) are the
// only [rows, V] buffer in the workspace, so its size does not grow with the
// batch: 32,768 rows x 65,536 ids x 2 bytes = 4.3 GB in bf16 mode. Measured
// at depth 20 (65,536 tokens): 16,384-row chunks make the step 1.5 ms slower
// (the chunk's input-gradient product needs a 4-way split to fill the chip),
// 32,768 rows cost 1.6 ms against one chunk of the whole batch.
constexpr int64_t kLmChunkRowsDefault = 32768;
std::atomic<int64_t> g_lm_chunk_rows{kLmChunkRowsDefault};
int64_t chunk_rows(const Dims& D) { return std::min<int64_t>(D.M, g_lm_chunk_rows.load()); }

// K slices for the lm_head input gradient dxf[mc, d] = dlogits . U (contraction
// over the vocabulary): a chunk of a few thousand rows has too few output tiles
// to fill the chip, so the product is split until there are about four tiles
// per compute unit (fixed-order fp32 reduction into the activation type).
int dgrad_splits(DType dt, int64_t rows, int N, int K) {
  nc::GemmArgs g{};
  g.M = (int)rows;
  g.N = N;
  g.K = K;
  g.lda = K;
  g.ldb = N;
  g.splits = 1;
  const int tile = nc::gemm_tile(dt, true, false, g);
  const int64_t tiles = ((rows + tile - 1) / tile) * ((N + tile - 1) / tile);
  const int bk = dt == DType::BF16 ? 64 : 32;
  int s = 1;
  while (tiles * s < 4 * (int64_t)nc::device_cus() && s < 8 && K / bk >= 2 * s) s *= 2;
  return s;
}

// Split-K plan for a weight gradient dW[N1, N2] = X1^T X2 contracted over K
// token rows (both operands read K-strided). Each split takes a contiguous run
// of whole 64-wide k slabs (runs differ by at most one slab). The split count
// minimises an estimate of rounds-of-workgroups x slabs-per-workgroup plus the
// fp32 partial traffic, so the last round of workgroups is not left mostly idle.
struct WgradPlan {
  int tile;
  int splits;
  uint64_t partial_floats;
};
WgradPlan wgrad_plan(DType dt, int64_t N1, int64_t N2, int64_t K) {
  WgradPlan p;
  p.tile = (dt == DType::BF16 && N1 >= 256 && N2 >= 256) ? 256 : 128;
  const int64_t tiles = ((N1 + p.tile - 1) / p.tile) * ((N2 + p.tile - 1) / p.tile);
  const int64_t ns = K / (dt == DType::BF16 ? 64 : 32);
  const int64_t slots = (int64_t)nc::device_cus() * (p.tile == 256 ? 1 : 2);
  const double slab_us = p.tile == 256 ? 2.2 : 0.6;           // one k slab of one tile
  const double bytes_per_us = 5.0e6;                          // partial write + reduce read
  int best = 1;
  double best_cost = 1e300;
  for (int s = 1; s <= 32 && s <= ns; ++s) {
    const int64_t rounds = (tiles * s + slots - 1) / slots;
    double cost = (double)rounds * (double)((ns + s - 1) / s) * slab_us;
    if (s > 1) cost += (double)s * N1 * N2 * 8.0 / bytes_per_us + 4.0;
    if (cost < best_cost) {
      best_cost = cost;
      best = s;
    }
  }
  p.splits = best;
  p.partial_floats = best > 1 ? (uint64_t)best * N1 * N2 : 0;
  return p;
}

struct LayerActs {
  uint64_t h, rinv1, qkv, rqk, o, lse, h2, rinv2, a;
};

// A named piece of the workspace (offset and size in bytes).
struct Piece {
  std::string name;
  uint64_t offset, bytes;
};

struct Plan {
  std::vector<Piece> pieces;
  uint64_t status, cs, x, rinv0, xf, rinvf, ssq, loss_rows, logits;
  std::vector<LayerActs> acts;
  // backward only
  uint64_t dx, g, dh, dbig, dout, delta, partial, attn_part, attn_ds, counts, offsets, cursor, list;
  uint64_t item_off, part_off, item_bucket, scan_blocks;
  uint64_t total;
};

// Every piece is followed by a guard of kGuard bytes that no kernel writes, so
// a test can fill the workspace with a pattern and find any write outside the
// pieces after a call.
constexpr uint64_t kGuard = 256;

Plan plan_of(const Dims& D, bool bwd, bool record = false) {
  Plan p{};
  uint64_t off = 0;
  std::string prefix;
  auto take_named = [&](const char* name, uint64_t bytes) {
    const uint64_t o = off;
    if (record) {
      if (!prefix.empty()) p.pieces.push_back({prefix + name, o, bytes});
      else p.pieces.push_back({name, o, bytes});
    }
    off = align_up(off + std::max<uint64_t>(bytes, 1), kAlign) + kGuard;
    return o;
  };
  const uint64_t M = D.M, e = D.esz;
  const uint64_t Mc = chunk_rows(D);
  p.status = take_named("status", 256);
  p.cs = take_named("rope_table", (uint64_t)D.T * 64 * 2 * 4);
  p.x = take_named("x", M * D.d * 4);
  p.rinv0 = take_named("rinv0", M * 4);
  p.xf = take_named("xf", M * D.d * e);
  p.rinvf = take_named("rinvf", M * 4);
  p.ssq = take_named("ssq", M * (D.d / 64) * 4);              // per-64-column sums of squares
  p.loss_rows = take_named("loss_rows", M * 4);
  p.logits = take_named("logits", Mc * D.V * e);                // the logit gradient replaces them
  const int nsets = bwd ? D.L : 1;
  for (int l = 0; l < nsets; ++l) {
    LayerActs a;
    prefix = "h" + std::to_string(l) + ".";
    a.h = take_named("h", M * D.d * e);
    a.rinv1 = take_named("rinv1", M * 4);
    a.qkv = take_named("qkv", M * D.Q * e);
    a.rqk = take_named("rqk", M * (D.H + 1) * 4);
    a.o = take_named("o", M * D.d * e);
    a.lse = take_named("lse", M * D.H * 4);
    a.h2 = take_named("h2", M * D.d * e);
    a.rinv2 = take_named("rinv2", M * 4);
    a.a = take_named("a", M * D.F * e);
    p.acts.push_back(a);
  }
  prefix.clear();
  if (bwd) {
    p.dx = take_named("dx", M * D.d * 4);
    p.g = take_named("g", M * D.d * e);
    p.dh = take_named("dh", M * D.d * 4);        // T-typed input gradients; fp32 partial sums for dE
    p.dbig = take_named("dbig", M * std::max(D.F, D.Q) * e);
    p.dout = take_named("dout", M * D.d * e);
    p.delta = take_named("delta", M * D.H * 4);
    uint64_t part = 0;
    const int64_t shapes[4][2] = {{D.Q, D.d}, {D.d, D.d}, {D.F, D.d}, {D.d, D.F}};
    for (auto& sh : shapes) part = std::max(part, wgrad_plan(D.dt, sh[0], sh[1], D.M).partial_floats);
    const int sx = dgrad_splits(D.dt, Mc, D.d, D.V);
    if (sx > 1) part = std::max<uint64_t>(part, (uint64_t)sx * Mc * D.d);
    p.partial = take_named("partial", part * 4);
    p.attn_part = take_named("attn_part", nc::attn_bwd_scratch_floats(D.B, D.T) * 4);
    // dS^T of one layer's attention backward: the logits chunk is free by then
    // (the lm_head and loss finish before the blocks' backward), so it holds
    // dS^T when large enough (every workload here), otherwise a piece of its own
    const uint64_t ds_bytes = nc::attn_bwd_ds_elems(D.B, D.T, D.H) * e;
    p.attn_ds = ds_bytes <= Mc * D.V * e ? p.logits : take_named("attn_ds", ds_bytes);
    p.counts = take_named("counts", (uint64_t)(D.V + 1) * 4);
    p.offsets = take_named("offsets", (uint64_t)(D.V + 1) * 4);
    p.cursor = take_named("cursor", (uint64_t)D.V * 4);
    p.list = take_named("list", M * 4);
    p.item_off = take_named("item_off", (uint64_t)(D.V + 1) * 4);
    p.part_off = take_named("part_off", (uint64_t)(D.V + 1) * 4);
    p.item_bucket = take_named("item_bucket", nc::embed_bwd_max_pieces(M, D.V) * 4);
    p.scan_blocks = take_named("scan_blocks", nc::embed_bwd_scan_blocks(D.V) * 4);
  }
  p.total = off;
  return p;
}

bool misaligned(const void* p) { return ((uintptr_t)p) % kAlign != 0; }

#define HIPCHECK(expr)                          \
  do {                                          \
    hipError_t _e = (expr);                     \
    if (_e != hipSuccess) {                     \
      g_last_hip = (int)_e;                     \
      return NC_ERR_HIP;                        \
    }                                           \
  } while (0)

template <typename P>
P* at(void* base, uint64_t off) {
  return reinterpret_cast<P*>(static_cast<char*>(base) + off);
}

// dW[N1,N2] = X1^T X2 over M rows (X1 [M, N1], X2 [M, N2]), both operands read
// K-strided, split over K with a fixed-order fp32 reduction.
hipError_t wgrad(DType dt, const void* X1, const void* X2, float* dW, float* partial, int64_t M,
                 int N1, int N2, const WgradPlan& p, hipStream_t s, bool accumulate = false) {
  nc::GemmArgs g{};
  g.A = X1;
  g.B = X2;
  g.M = N1;
  g.N = N2;
  g.K = (int)M;
  g.lda = N1;
  g.ldb = N2;
  g.ldc = N2;
  g.splits = p.splits;
  g.tile = p.tile;
  if (p.splits == 1) {
    g.C = dW;
    return nc::gemm(dt, false, false, accumulate ? Epi::AddF32 : Epi::StoreF32, g, s);
  }
  g.C = partial;
  hipError_t e = nc::gemm(dt, false, false, Epi::PartialF32, g, s);
  if (e != hipSuccess) return e;
  return nc::splitk_reduce(partial, p.splits, (size_t)N1 * N2, dW, accumulate, s);
}

// rs: row scale of a folded RMSNorm (StoreT / Relu2 / Relu2Bwd); xc, ssq: the
// copy and the sums of squares an AddF32Xs product writes for the next norm
hipError_t gemm_simple(DType dt, bool ak, bool bk, Epi epi, const void* A, const void* B, void* C,
                       void* C2, int64_t M, int N, int K, int lda, int ldb, int ldc, int ldc2,
                       hipStream_t s, const float* rs = nullptr, void* xc = nullptr,
                       float* ssq = nullptr) {
  nc::GemmArgs g{};
  g.rs = rs;
  g.xc = xc;
  g.ssq = ssq;
  g.A = A;
  g.B = B;
  g.C = C;
  g.C2 = C2;
  g.M = (int)M;
  g.N = N;
  g.K = K;
  g.lda = lda;
  g.ldb = ldb;
  g.ldc = ldc;
  g.ldc2 = ldc2;
  g.splits = 1;
  return nc::gemm(dt, ak, bk, epi, g, s);
}

int run_step(const nc_config* cfg, const void* params, const int32_t* tokens,
             const int32_t* targets, float* grads, void* ws, uint64_t ws_bytes, float* loss_dev,
             void* stream, bool bwd, bool accumulate = false) {
  int rc = validate(cfg);
  if (rc) return rc;
  if (!params || !tokens || !targets || !ws || !loss_dev || (bwd && !grads)) return NC_ERR_NULL;
  if (misaligned(params) || misaligned(tokens) || misaligned(targets) || misaligned(ws) ||
      misaligned(loss_dev) || (bwd && misaligned(grads)))
    return NC_ERR_ALIGN;
  const Dims D = dims_of(cfg);
  const Plan P = plan_of(D, bwd);
  if (ws_bytes < P.total) return NC_ERR_WORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const DType dt = D.dt;
  const size_t e = D.esz;
  const auto lay = layout_of(D);
  auto W = [&](int idx) { return static_cast<const char*>(params) + lay[idx].offset * e; };
  auto G = [&](int idx) { return grads + lay[idx].offset; };
  const int iE = 0, iU = 1 + 4 * D.L;
  const int64_t M = D.M;
  const float eps = cfg->rms_eps;

  uint32_t* status = at<uint32_t>(ws, P.status);
  float* cs = at<float>(ws, P.cs);
  float* x = at<float>(ws, P.x);
  float* rinv0 = at<float>(ws, P.rinv0);
  void* xf = at<char>(ws, P.xf);
  float* rinvf = at<float>(ws, P.rinvf);
  float* loss_rows = at<float>(ws, P.loss_rows);
  void* logits = at<char>(ws, P.logits);
  void* dlog = logits;                           // the gradient overwrites the logits

  HIPCHECK(nc::fill_zero(status, 256, s));
  HIPCHECK(nc::rope_table(D.T, 64, (double)cfg->rope_base, cs, s));
  // The RMSNorms in front of the attention, the MLP and the lm_head are folded
  // into the products around them: the product that feeds the residual stream
  // also writes the new residual in the activation type (h, h2, xf hold these
  // unnormalised copies) and its per-64-column sums of squares, one small pass
  // turns those into 1/rms per row, and the consuming product scales its
  // output rows by it. The embedding kernel does the first block's norm itself.
  float* ssq = at<float>(ws, P.ssq);
  HIPCHECK(nc::embed_norm_fwd(dt, W(iE), tokens, (int)M, D.d, D.V, eps, x, rinv0, status, s,
                              at<char>(ws, P.acts[0].h), at<float>(ws, P.acts[0].rinv1)));

  // ---------------- forward through the blocks ----------------
  for (int l = 0; l < D.L; ++l) {
    const LayerActs& A = P.acts[bwd ? l : 0];
    void* h = at<char>(ws, A.h);
    void* qkv = at<char>(ws, A.qkv);
    void* o = at<char>(ws, A.o);
    void* h2 = at<char>(ws, A.h2);
    void* a = at<char>(ws, A.a);
    const float* rinv1 = at<float>(ws, A.rinv1);
    float* rinv2 = at<float>(ws, A.rinv2);
    // where this block's output residual (the next norm's input) goes
    const bool last = l + 1 == D.L;
    const LayerActs& An = P.acts[bwd && !last ? l + 1 : 0];
    void* xnext = last ? xf : at<char>(ws, An.h);
    float* rnext = last ? rinvf : at<float>(ws, An.rinv1);
    const int base = 1 + 4 * l;
    HIPCHECK(gemm_simple(dt, true, true, Epi::StoreT, h, W(base + 0), qkv, nullptr, M, D.Q, D.d,
                         D.d, D.d, D.Q, 0, s, rinv1));
    HIPCHECK(nc::rope_qknorm_fwd(dt, qkv, D.Q, (int)M, D.T, D.H, cs, eps, at<float>(ws, A.rqk), s));
    HIPCHECK(nc::attn_fwd(dt, qkv, D.Q, D.B, D.T, D.H, o, at<float>(ws, A.lse), s));
    HIPCHECK(gemm_simple(dt, true, true, Epi::AddF32Xs, o, W(base + 1), x, nullptr, M, D.d, D.d,
                         D.d, D.d, D.d, 0, s, nullptr, h2, ssq));
    HIPCHECK(nc::ssq_rinv(ssq, (int)M, D.d / 64, D.d, eps, rinv2, s));
    HIPCHECK(gemm_simple(dt, true, true, Epi::Relu2, h2, W(base + 2), a, nullptr, M, D.F, D.d,
                         D.d, D.d, D.F, 0, s, rinv2));
    HIPCHECK(gemm_simple(dt, true, true, Epi::AddF32Xs, a, W(base + 3), x, nullptr, M, D.d, D.F,
                         D.F, D.F, D.d, 0, s, nullptr, xnext, ssq));
    HIPCHECK(nc::ssq_rinv(ssq, (int)M, D.d / 64, D.d, eps, rnext, s));
  }

  // ---------------- lm_head + softcap cross-entropy, by row chunks ----------------
  const int64_t Mc = chunk_rows(D);
  void* dxf = bwd ? at<char>(ws, P.dh) : nullptr;
  float* partial_x = bwd ? at<float>(ws, P.partial) : nullptr;
  const float w = 1.0f / (float)M;
  for (int64_t r0 = 0; r0 < M; r0 += Mc) {
    const int64_t mc = std::min<int64_t>(Mc, M - r0);
    const char* xfc = static_cast<const char*>(xf) + r0 * D.d * e;
    HIPCHECK(gemm_simple(dt, true, true, Epi::StoreT, xfc, W(iU), logits, nullptr, mc, D.V,
                         D.d, D.d, D.d, D.V, 0, s, rinvf + r0));
    // the logit gradient carries the final norm's row scale, so dxf and dU
    // below come out right from the unnormalised xf
    HIPCHECK(nc::softcap_ce(dt, logits, targets + r0, (int)mc, D.V, cfg->softcap, w,
                            loss_rows + r0, bwd ? dlog : nullptr, status, s, rinvf + r0));
    if (bwd) {
      // dxf = dlog . U (U read K-strided: contraction over its rows), split
      // over the vocabulary when the chunk alone would not fill the chip
      char* dxfc = static_cast<char*>(dxf) + r0 * D.d * e;
      const int sx = dgrad_splits(dt, mc, D.d, D.V);
      if (sx == 1) {
        HIPCHECK(gemm_simple(dt, true, false, Epi::StoreT, dlog, W(iU), dxfc, nullptr, mc, D.d,
                             D.V, D.V, D.d, D.d, 0, s));
      } else {
        nc::GemmArgs g{};
        g.A = dlog;
        g.B = W(iU);
        g.C = partial_x;
        g.M = (int)mc;
        g.N = D.d;
        g.K = D.V;
        g.lda = D.V;
        g.ldb = D.d;
        g.ldc = D.d;
        g.splits = sx;
        HIPCHECK(nc::gemm(dt, true, false, Epi::PartialF32, g, s));
        HIPCHECK(nc::splitk_reduce_t(dt, partial_x, sx, (size_t)mc * D.d, dxfc, s));
      }
      // dU (+)= dlog^T . xf_chunk: both operands contracted over their rows
      HIPCHECK(gemm_simple(dt, false, false, (r0 == 0 && !accumulate) ? Epi::StoreF32 : Epi::AddF32, dlog, xfc,
                           G(iU), nullptr, D.V, D.d, (int)mc, D.V, D.d, D.d, 0, s));
    }
  }
  HIPCHECK(nc::loss_mean(loss_rows, (int)M, loss_dev, status, s));
  if (!bwd) return NC_OK;

  // ---------------- backward ----------------
  float* dx = at<float>(ws, P.dx);
  void* g = at<char>(ws, P.g);
  void* dbig = at<char>(ws, P.dbig);
  void* dout = at<char>(ws, P.dout);
  float* delta = at<float>(ws, P.delta);
  float* partial = at<float>(ws, P.partial);
  HIPCHECK(nc::rmsnorm_bwd(dt, dxf, xf, rinvf, (int)M, D.d, dx, false, g, s, true));
  const WgradPlan pQ = wgrad_plan(dt, D.Q, D.d, M), pO = wgrad_plan(dt, D.d, D.d, M);
  const WgradPlan pFC = wgrad_plan(dt, D.F, D.d, M), pPR = wgrad_plan(dt, D.d, D.F, M);
  void* dh = at<char>(ws, P.dh);
  const int Mi = (int)M;
  for (int l = D.L - 1; l >= 0; --l) {
    const LayerActs& A = P.acts[l];
    const int base = 1 + 4 * l;
    void* h = at<char>(ws, A.h);
    void* qkv = at<char>(ws, A.qkv);
    void* o = at<char>(ws, A.o);
    void* h2 = at<char>(ws, A.h2);
    void* a = at<char>(ws, A.a);
    // MLP: x_out = x_mid + relu(h2 Wfc^T)^2 Wpr^T
    HIPCHECK(wgrad(dt, g, a, G(base + 3), partial, M, D.d, D.F, pPR, s, accumulate));
    // d(pre-activation) times the MLP norm's row scale: with h2 unnormalised,
    // the weight gradient and the norm input gradient below then come out right
    HIPCHECK(gemm_simple(dt, true, false, Epi::Relu2Bwd, g, W(base + 3), dbig, a, M, D.F, D.d,
                         D.d, D.F, D.F, D.F, s, at<float>(ws, A.rinv2)));
    HIPCHECK(wgrad(dt, dbig, h2, G(base + 2), partial, M, D.F, D.d, pFC, s, accumulate));
    HIPCHECK(gemm_simple(dt, true, false, Epi::StoreT, dbig, W(base + 2), dh, nullptr, M, D.d,
                         D.F, D.F, D.d, D.d, 0, s));
    HIPCHECK(nc::rmsnorm_bwd(dt, dh, h2, at<float>(ws, A.rinv2), Mi, D.d, dx, true, g, s, true));
    // attention: x_mid = x_in + o Wo^T
    HIPCHECK(wgrad(dt, g, o, G(base + 1), partial, M, D.d, D.d, pO, s, accumulate));
    HIPCHECK(gemm_simple(dt, true, false, Epi::StoreT, g, W(base + 1), dout, nullptr, M, D.d, D.d,
                         D.d, D.d, D.d, 0, s));
    // every gradient of qkv carries the attention norm's row scale (h is unnormalised)
    HIPCHECK(nc::attn_bwd(dt, qkv, D.Q, o, dout, at<float>(ws, A.lse), delta, D.B, D.T, D.H, dbig,
                          D.Q, at<float>(ws, P.attn_part), s, at<float>(ws, A.rinv1),
                          at<char>(ws, P.attn_ds)));
    HIPCHECK(nc::rope_qknorm_bwd(dt, dbig, D.Q, qkv, D.Q, Mi, D.T, D.H, cs,
                                 at<float>(ws, A.rqk), s, at<float>(ws, A.rinv1)));
    HIPCHECK(wgrad(dt, dbig, h, G(base + 0), partial, M, D.Q, D.d, pQ, s, accumulate));
    HIPCHECK(gemm_simple(dt, true, false, Epi::StoreT, dbig, W(base + 0), dh, nullptr, M, D.d,
                         D.Q, D.Q, D.d, D.d, 0, s));
    HIPCHECK(nc::rmsnorm_bwd(dt, dh, h, at<float>(ws, A.rinv1), Mi, D.d, dx, true, g, s, true));
  }
  nc::EmbedBwdScratch es;
  es.counts = at<int32_t>(ws, P.counts);
  es.offsets = at<int32_t>(ws, P.offsets);
  es.cursor = at<int32_t>(ws, P.cursor);
  es.list = at<int32_t>(ws, P.list);
  es.item_off = at<int32_t>(ws, P.item_off);
  es.part_off = at<int32_t>(ws, P.part_off);
  es.item_bucket = at<int32_t>(ws, P.item_bucket);
  es.scan_blocks = at<int32_t>(ws, P.scan_blocks);
  es.part = static_cast<float*>(dh);     // embed_bwd_max_parts(M) * d floats <= M * d
  HIPCHECK(nc::embed_bwd(dt, W(iE), tokens, rinv0, dx, (int)M, D.d, D.V, es, G(iE), accumulate, s));
  return NC_OK;
}

}  // namespace

extern "C" {

int nc_config_from_depth(int32_t depth, int32_t vocab_size, int32_t seq_len, int32_t batch,
                         int32_t dtype, nc_config* out) {
  if (!out) return NC_ERR_NULL;
  nc_config c;
  c.depth = depth;
  c.vocab_size = vocab_size;
  c.seq_len = seq_len;
  c.batch = batch;
  c.n_kv_head = 1;
  c.head_dim = 128;
  c.softcap = 15.0f;
  c.rope_base = 10000.0f;
  c.rms_eps = 1e-6f;
  c.init_std = 0.02f;
  c.dtype = dtype;
  const int rc = validate(&c);
  if (rc) return rc;
  *out = c;
  return NC_OK;
}

int nc_validate_config(const nc_config* cfg) { return validate(cfg); }

int nc_set_lm_chunk_rows(int32_t rows) {
  if (rows < 0 || rows % 64) return NC_ERR_ARG;
  g_lm_chunk_rows.store(rows == 0 ? kLmChunkRowsDefault : rows);
  return NC_OK;
}

int nc_set_gemm_persistent(int32_t on) {
  if (on != 0 && on != 1) return NC_ERR_ARG;
  nc::gemm_set_persistent(on == 1);
  return NC_OK;
}

int nc_lm_chunk_rows(const nc_config* cfg, int32_t* rows) {
  const int rc = validate(cfg);
  if (rc) return rc;
  if (!rows) return NC_ERR_NULL;
  *rows = (int32_t)chunk_rows(dims_of(cfg));
  return NC_OK;
}

int nc_param_count(const nc_config* cfg, uint64_t* n) {
  const int rc = validate(cfg);
  if (rc) return rc;
  if (!n) return NC_ERR_NULL;
  *n = param_elems(dims_of(cfg));
  return NC_OK;
}

int nc_param_layout(const nc_config* cfg, nc_tensor_info* out, int32_t cap, int32_t* n) {
  const int rc = validate(cfg);
  if (rc) return rc;
  if (!n || (cap > 0 && !out)) return NC_ERR_NULL;
  const auto t = layout_of(dims_of(cfg));
  *n = (int32_t)t.size();
  for (int i = 0; i < (int)t.size() && i < cap; ++i) {
    memset(out[i].name, 0, sizeof(out[i].name));
    if (t[i].layer < 0) snprintf(out[i].name, sizeof(out[i].name), "%s", t[i].kind);
    else snprintf(out[i].name, sizeof(out[i].name), "h%d.%s", t[i].layer, t[i].kind);
    out[i].offset = t[i].offset;
    out[i].rows = t[i].rows;
    out[i].cols = t[i].cols;
  }
  return NC_OK;
}

int nc_workspace_bytes(const nc_config* cfg, int32_t with_backward, uint64_t* bytes) {
  const int rc = validate(cfg);
  if (rc) return rc;
  if (!bytes) return NC_ERR_NULL;
  *bytes = plan_of(dims_of(cfg), with_backward != 0).total;
  return NC_OK;
}

int nc_workspace_pieces(const nc_config* cfg, int32_t with_backward, nc_ws_piece* out, int32_t cap,
                        int32_t* n) {
  const int rc = validate(cfg);
  if (rc) return rc;
  if (!n || (cap > 0 && !out)) return NC_ERR_NULL;
  const Plan P = plan_of(dims_of(cfg), with_backward != 0, true);
  *n = (int32_t)P.pieces.size();
  for (int i = 0; i < (int)P.pieces.size() && i < cap; ++i) {
    memset(out[i].name, 0, sizeof(out[i].name));
    snprintf(out[i].name, sizeof(out[i].name), "%s", P.pieces[i].name.c_str());
    out[i].offset = P.pieces[i].offset;
    out[i].bytes = P.pieces[i].bytes;
  }
  return NC_OK;
}

int nc_token_losses_offset(const nc_config* cfg, int32_t with_backward, uint64_t* byte_offset) {
  const int rc = validate(cfg);
  if (rc) return rc;
  if (!byte_offset) return NC_ERR_NULL;
  *byte_offset = plan_of(dims_of(cfg), with_backward != 0).loss_rows;
  return NC_OK;
}

int nc_init_params(uint64_t seed, const nc_config* cfg, void* params, void* stream) {
  const int rc = validate(cfg);
  if (rc) return rc;
  if (!params) return NC_ERR_NULL;
  if (misaligned(params)) return NC_ERR_ALIGN;
  const Dims D = dims_of(cfg);
  const auto lay = layout_of(D);
  std::vector<nc::InitSeg> segs;
  const double base = (double)cfg->init_std;
  const double proj = 1.0 / sqrt(2.0 * (double)D.L);
  for (const auto& t : lay) {
    const bool is_proj = !strcmp(t.kind, "Wo") || !strcmp(t.kind, "Wpr");
    segs.push_back({t.offset, t.offset + (uint64_t)(t.rows * t.cols), base * (is_proj ? proj : 1.0)});
  }
  HIPCHECK(nc::init_params(D.dt, seed, segs.data(), (int)segs.size(), param_elems(D), params,
                           static_cast<hipStream_t>(stream)));
  return NC_OK;
}

int nc_forward_loss(const nc_config* cfg, const void* params, const int32_t* tokens,
                    const int32_t* targets, void* ws, uint64_t ws_bytes, float* loss_dev,
                    void* stream) {
  return run_step(cfg, params, tokens, targets, nullptr, ws, ws_bytes, loss_dev, stream, false);
}

int nc_eval_bpb(const nc_config* cfg, const void* params, const int32_t* tokens, const int32_t* targets,
                const int32_t* token_bytes, void* ws, uint64_t ws_bytes, float* loss_dev, double* bpb_dev,
                void* stream) {
  int rc = validate(cfg);
  if (rc) return rc;
  if (!token_bytes || !bpb_dev) return NC_ERR_NULL;
  if (misaligned(token_bytes) || misaligned(bpb_dev)) return NC_ERR_ALIGN;
  rc = run_step(cfg, params, tokens, targets, nullptr, ws, ws_bytes, loss_dev, stream, false);
  if (rc) return rc;
  const Dims D = dims_of(cfg);
  const Plan P = plan_of(D, false);
  HIPCHECK(nc::bits_per_byte(at<float>(ws, P.loss_rows), targets, (int)D.M, token_bytes, D.V, bpb_dev,
                             static_cast<hipStream_t>(stream)));
  return NC_OK;
}

int nc_forward_backward(const nc_config* cfg, const void* params, const int32_t* tokens,
                        const int32_t* targets, float* grads, void* ws, uint64_t ws_bytes,
                        float* loss_dev, void* stream) {
  return run_step(cfg, params, tokens, targets, grads, ws, ws_bytes, loss_dev, stream, true);
}

int nc_forward_backward_accumulate(const nc_config* cfg, const void* params, const int32_t* tokens,
                                   const int32_t* targets, float* grads, void* ws,
                                   uint64_t ws_bytes, float* loss_dev, void* stream) {
  return run_step(cfg, params, tokens, targets, grads, ws, ws_bytes, loss_dev, stream, true, true);
}

// ---------------------------------------------------------------- optimizer

namespace {

// Quintic Newton-Schulz coefficients of Muon's public description.
constexpr float kNsA = 3.4445f, kNsB = -4.7750f, kNsC = 2.0315f;

struct OptPlan {
  uint64_t norm_partial, norm_scale, muon_partial;
  uint64_t u, x0, x, a, bt, df, xf;
  uint64_t total;
};

// Muon runs each matrix kind (Wqkv, Wo, Wfc, Wpr) for all layers at once,
// so its buffers hold `depth` matrices of the largest kind.
OptPlan opt_plan_of(const Dims& D) {
  OptPlan P{};
  uint64_t off = 0;
  auto take = [&](uint64_t bytes) {
    const uint64_t o = off;
    off = align_up(off + bytes, kAlign);
    return o;
  };
  const uint64_t big = (uint64_t)D.L * D.F * D.d;    // all layers' Wfc (or Wpr)
  const uint64_t sq = (uint64_t)D.L * D.d * D.d;     // r x r per layer, r = d (every short side)
  P.norm_partial = take(sizeof(double) * nc::kOptMaxRanges * nc::kNormBlocksPerRange);
  P.norm_scale = take(4 * sizeof(float));
  P.muon_partial = take(sizeof(double) * nc::kMuonParts * D.L);
  P.u = take(4 * big);
  P.x0 = take(D.esz * big);
  P.x = take(D.esz * big);
  P.a = take(D.esz * sq);
  P.bt = take(D.esz * sq);
  P.df = take(4 * big);
  P.xf = take(4 * big);
  P.total = off;
  return P;
}

int validate_optim(const nc_optim_config* o) {
  if (!o) return NC_ERR_NULL;
  auto finite_nonneg = [](float v) { return v >= 0.f && v < 1e30f; };
  if (!finite_nonneg(o->lr_adamw) || !finite_nonneg(o->lr_muon)) return NC_ERR_ARG;
  if (!(o->beta1 >= 0.f && o->beta1 < 1.f) || !(o->beta2 >= 0.f && o->beta2 < 1.f)) return NC_ERR_ARG;
  if (!(o->eps > 0.f) || !finite_nonneg(o->wd_adamw) || !finite_nonneg(o->wd_muon)) return NC_ERR_ARG;
  if (!(o->momentum >= 0.f && o->momentum < 1.f)) return NC_ERR_ARG;
  if (!(o->max_grad_norm < 1e30f)) return NC_ERR_ARG;
  if (o->ns_steps < 0 || o->ns_steps > 16 || o->step < 1) return NC_ERR_ARG;
  return NC_OK;
}

// `batch` products of one shape, items at strides sa, sb, sc (elements)
hipError_t gemm_batched(DType dt, bool ak, bool bk, Epi epi, const void* A, const void* B, void* C,
                        int M, int N, int K, int lda, int ldb, int ldc, int batch, int64_t sa,
                        int64_t sb, int64_t sc, hipStream_t s) {
  nc::GemmArgs g{};
  g.A = A;
  g.B = B;
  g.C = C;
  g.M = M;
  g.N = N;
  g.K = K;
  g.lda = lda;
  g.ldb = ldb;
  g.ldc = ldc;
  g.splits = 1;
  g.batch = batch;
  g.sa = sa;
  g.sb = sb;
  g.sc = sc;
  return nc::gemm(dt, ak, bk, epi, g, s);
}

// Batched product with the alpha * acc + beta * C2 epilogue (C2 laid out as C).
hipError_t gemm_axpby(DType dt, bool ak, bool bk, Epi epi, const void* A, const void* B, void* C,
                      const void* C2, int M, int N, int K, int lda, int ldb, int ldc, int batch,
                      int64_t sa, int64_t sb, int64_t sc, float alpha, float beta, hipStream_t s) {
  nc::GemmArgs g{};
  g.A = A;
  g.B = B;
  g.C = C;
  g.C2 = const_cast<void*>(C2);
  g.M = M;
  g.N = N;
  g.K = K;
  g.lda = lda;
  g.ldb = ldb;
  g.ldc = ldc;
  g.ldc2 = ldc;
  g.splits = 1;
  g.batch = batch;
  g.sa = sa;
  g.sb = sb;
  g.sc = sc;
  g.sc2 = sc;
  g.alpha = alpha;
  g.beta = beta;
  return nc::gemm(dt, ak, bk, epi, g, s);
}

// One Muon step on every layer's [R, C] matrix of one kind: params, grads and
// momentum of layer l sit at element offset first + l * stride.
int muon_kind(const Dims& D, const OptPlan& P, void* ows, const nc_optim_config* o, void* params,
              const float* grads, float* m1, uint64_t first, uint64_t stride, int R, int C,
              hipStream_t s) {
  const DType dt = D.dt;
  const int L = D.L;
  const size_t n = (size_t)R * C;
  const bool tall = R > C;
  const int r = tall ? C : R, c = tall ? R : C;   // the iteration runs on X [r, c], r <= c
  const float* norm_scale = at<float>(ows, P.norm_scale);
  double* mpart = at<double>(ows, P.muon_partial);
  float* u = at<float>(ows, P.u);
  float* df = at<float>(ows, P.df);
  float* xf = at<float>(ows, P.xf);
  void* p = static_cast<char*>(params) + first * D.esz;
  const float decay = 1.0f - o->lr_muon * o->wd_muon;
  const float scale = std::sqrt(std::max(1.0f, (float)R / (float)C));
  HIPCHECK(nc::muon_momentum(grads + first, m1 + first, stride, u, n, L, o->momentum, norm_scale,
                             mpart, s));
  if (o->ns_steps == 0) {
    HIPCHECK(nc::muon_normalize(DType::F32, u, n, L, mpart, xf, s));
    HIPCHECK(nc::muon_update(dt, p, stride, xf, n, L, decay, o->lr_muon * scale, s));
    return NC_OK;
  }
  char* x0 = at<char>(ows, P.x0);
  HIPCHECK(nc::muon_normalize(dt, u, n, L, mpart, x0, s));
  char* X = x0;
  if (tall) {
    X = at<char>(ows, P.x);
    for (int l = 0; l < L; ++l)
      HIPCHECK(nc::transpose(dt, x0 + l * n * D.esz, R, C, C, X + l * n * D.esz, R, s));
  }
  void* A = at<char>(ows, P.a);
  void* bt = at<char>(ows, P.bt);
  char* Xn = tall ? x0 : at<char>(ows, P.x);       // the other iterate buffer
  const int64_t rr = (int64_t)r * r, rc = (int64_t)r * c;
  for (int k = 0; k < o->ns_steps; ++k) {
    // A = X X^T;  bt = A A^T + (b/c) A  (= (b A + c A^2) / c, A symmetric)
    HIPCHECK(gemm_batched(dt, true, true, Epi::StoreT, X, X, A, r, r, c, c, c, r, L, rc, rc, rr, s));
    HIPCHECK(gemm_axpby(dt, true, true, Epi::AxpbyT, A, A, bt, A, r, r, r, r, r, r, L, rr, rr, rr, 1.0f,
                        kNsB / kNsC, s));
    // next iterate a X + (b A + c A^2) X = c (bt X) + a X; the last one in fp32 (df)
    const bool last = k + 1 == o->ns_steps;
    HIPCHECK(gemm_axpby(dt, true, false, last ? Epi::AxpbyF32 : Epi::AxpbyT, bt, X,
                        last ? static_cast<void*>(df) : static_cast<void*>(Xn), X, r, c, r, r, c, c, L,
                        rr, rc, rc, kNsC, kNsA, s));
    if (!last) std::swap(X, Xn);
  }
  const float* fin = df;
  if (tall) {
    for (int l = 0; l < L; ++l)
      HIPCHECK(nc::transpose(DType::F32, df + l * n, r, c, c, xf + l * n, r, s));
    fin = xf;
  }
  HIPCHECK(nc::muon_update(dt, p, stride, fin, n, L, decay, o->lr_muon * scale, s));
  return NC_OK;
}

}  // namespace

int nc_optimizer_state_bytes(const nc_config* cfg, uint64_t* bytes) {
  const int rc = validate(cfg);
  if (rc) return rc;
  if (!bytes) return NC_ERR_NULL;
  *bytes = 2 * sizeof(float) * param_elems(dims_of(cfg));
  return NC_OK;
}

int nc_optimizer_workspace_bytes(const nc_config* cfg, uint64_t* bytes) {
  const int rc = validate(cfg);
  if (rc) return rc;
  if (!bytes) return NC_ERR_NULL;
  *bytes = opt_plan_of(dims_of(cfg)).total;
  return NC_OK;
}

int nc_optimizer_step(const nc_config* cfg, const nc_optim_config* optim, void* params,
                      const float* grads, float* state, void* ows, uint64_t ows_bytes,
                      float* grad_norm_dev, void* stream) {
  int rc = validate(cfg);
  if (rc) return rc;
  rc = validate_optim(optim);
  if (rc) return rc;
  if (!params || !grads || !state || !ows || !grad_norm_dev) return NC_ERR_NULL;
  if (misaligned(params) || misaligned(grads) || misaligned(state) || misaligned(ows) ||
      misaligned(grad_norm_dev))
    return NC_ERR_ALIGN;
  const Dims D = dims_of(cfg);
  const OptPlan P = opt_plan_of(D);
  if (ows_bytes < P.total) return NC_ERR_WORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const auto lay = layout_of(D);
  const uint64_t N = param_elems(D);
  if ((int)lay.size() > nc::kOptMaxRanges) return NC_ERR_UNSUPPORTED;
  // global norm and clip factor
  nc::OptRanges rg{};
  rg.n = (int)lay.size();
  for (int i = 0; i < rg.n; ++i) {
    rg.off[i] = lay[i].offset;
    rg.cnt[i] = (uint64_t)(lay[i].rows * lay[i].cols);
  }
  float* norm_scale = at<float>(ows, P.norm_scale);
  HIPCHECK(nc::grad_norm(grads, rg, at<double>(ows, P.norm_partial), optim->max_grad_norm,
                         norm_scale, s));
  HIPCHECK(hipMemcpyAsync(grad_norm_dev, norm_scale, sizeof(float), hipMemcpyDeviceToDevice, s));
  float* m1 = state;          // AdamW first moment, or Muon momentum
  float* m2 = state + N;      // AdamW second moment (E and U only)
  nc::AdamWArgs aa;
  aa.lr = optim->lr_adamw;
  aa.beta1 = optim->beta1;
  aa.beta2 = optim->beta2;
  aa.eps = optim->eps;
  aa.decay = 1.0f - optim->lr_adamw * optim->wd_adamw;
  aa.bc1 = (float)(1.0 / (1.0 - std::pow((double)optim->beta1, (double)optim->step)));
  aa.bc2 = (float)(1.0 / (1.0 - std::pow((double)optim->beta2, (double)optim->step)));
  for (const auto& t : lay) {                            // E and U: AdamW
    if (t.layer >= 0) continue;
    void* p = static_cast<char*>(params) + t.offset * D.esz;
    HIPCHECK(nc::adamw(D.dt, p, grads + t.offset, m1 + t.offset, m2 + t.offset,
                       (size_t)(t.rows * t.cols), aa, norm_scale, s));
  }
  // block matrices: Muon, one kind (same shape in every layer) at a time
  const uint64_t stride = D.L > 1 ? lay[1 + 4].offset - lay[1].offset : 0;
  for (int k = 0; k < 4; ++k) {
    const auto& t = lay[1 + k];
    for (int l = 1; l < D.L; ++l)
      if (lay[1 + 4 * l + k].offset != t.offset + l * stride) return NC_ERR_UNSUPPORTED;
    rc = muon_kind(D, P, ows, optim, params, grads, m1, t.offset, stride, (int)t.rows, (int)t.cols, s);
    if (rc) return rc;
  }
  return NC_OK;
}

// ---------------------------------------------------------------- inference

namespace {

struct InferPlan {
  uint64_t status, skcnt, cs, x, rinv, h, qkv, rqk, o, lse, h2, a, xf, last, logits, part, xb, ssq,
      skpart;
  uint64_t sync_bytes;   // status word and few-row product counters, cleared by every call
  uint64_t total;
};

int pad16(int v) { return (v + 15) / 16 * 16; }

// Rows: the longest prompt (batch x seq_len) or the padded decode batch,
// whichever is larger; the status word comes first, as in the step workspace.
InferPlan infer_plan_of(const Dims& D, int max_seq) {
  InferPlan P{};
  uint64_t off = 0;
  auto take = [&](uint64_t bytes) {
    const uint64_t o = off;
    off = align_up(off + std::max<uint64_t>(bytes, 1), kAlign);
    return o;
  };
  const uint64_t Bp = (uint64_t)pad16(D.B);
  const uint64_t R = std::max<uint64_t>((uint64_t)D.M, Bp), e = D.esz;
  // status word, then the arrival counters of the few-row products (N/16 <= V/16)
  P.sync_bytes = align_up(256 + (uint64_t)(D.V / 16) * 4, kAlign);
  P.status = take(P.sync_bytes);
  P.skcnt = P.status + 256;
  P.cs = take((uint64_t)D.T * 64 * 2 * 4);
  P.x = take(R * D.d * 4);
  P.rinv = take(R * 4);
  P.h = take(R * D.d * e);
  P.qkv = take(R * D.Q * e);
  P.rqk = take(R * (D.H + 1) * 4);
  P.o = take(R * D.d * e);
  P.lse = take((uint64_t)D.B * D.H * D.T * 4);
  P.h2 = take(R * D.d * e);
  P.a = take(R * D.F * e);
  P.xf = take(R * D.d * e);
  P.last = take(Bp * D.d * e);
  P.logits = take(Bp * D.V * 4);
  const uint64_t nch = ((uint64_t)max_seq + 63) / 64;
  P.part = take((uint64_t)D.B * nch * D.H * 129 * 4);
  P.xb = take(Bp * D.d * 2);
  P.ssq = take(128 * 32 * 4);
  uint64_t part = 0;
  if (D.B <= nc::kSkinnyMaxRows) {
    const int shapes[5][2] = {{D.Q, D.d}, {D.d, D.d}, {D.F, D.d}, {D.d, D.F}, {D.V, D.d}};
    for (const auto& nk : shapes)
      part = std::max<uint64_t>(part, nc::skinny_part_bytes(D.B, nk[0], nk[1]));
  }
  P.skpart = take(part);
  P.total = off;
  return P;
}

uint64_t kv_layer_bytes(const Dims& D, int max_seq) {
  return (uint64_t)D.B * max_seq * 256 * D.esz;
}

// Linear layer of the prefill (and the wide-batch / fp32 decoding) path:
// Y = X W^T under an epilogue through the tiled GEMM.
hipError_t infer_linear(DType dt, Epi epi, const void* X, const void* W, void* C, int64_t M, int N, int K,
                        int ldx, int ldc, hipStream_t s) {
  return gemm_simple(dt, true, true, epi, X, W, C, nullptr, M, N, K, ldx, K, ldc, 0, s);
}

bool few_rows(const Dims& D, int64_t M) { return D.dt == DType::BF16 && M <= nc::kSkinnyMaxRows; }

// The blocks over M rows (prefill: the prompt, B x Tseq rows; decode: one row
// per sequence, padded to 16 when the tiled GEMM runs), storing k-hat and v
// of the first kv_rows rows at cache positions pos0 + t. cs holds the rotary
// table of positions pos0 .. pos0 + Tseq - 1.
int infer_blocks(const Dims& D, const nc_config* cfg, const std::vector<Tensor>& lay,
                 const void* params, void* ws, const InferPlan& P, int64_t M, int kv_rows, int Tseq,
                 int pos0, bool prefill, void* kv, int max_seq, hipStream_t s) {
  const DType dt = D.dt;
  const float eps = cfg->rms_eps;
  auto W = [&](int idx) { return static_cast<const char*>(params) + lay[idx].offset * D.esz; };
  float* x = at<float>(ws, P.x);
  float* rinv = at<float>(ws, P.rinv);
  void* h = at<char>(ws, P.h);
  void* qkv = at<char>(ws, P.qkv);
  void* o = at<char>(ws, P.o);
  void* h2 = at<char>(ws, P.h2);
  void* a = at<char>(ws, P.a);
  const float* cs = at<float>(ws, P.cs);
  for (int l = 0; l < D.L; ++l) {
    const int base = 1 + 4 * l;
    void* cache = static_cast<char*>(kv) + (uint64_t)l * kv_layer_bytes(D, max_seq);
    HIPCHECK(nc::rmsnorm_fwd(dt, x, (int)M, D.d, eps, h, rinv, s));
    HIPCHECK(infer_linear(dt, Epi::StoreT, h, W(base + 0), qkv, M, D.Q, D.d, D.d, D.Q, s));
    HIPCHECK(nc::rope_qknorm_fwd(dt, qkv, D.Q, kv_rows, Tseq, D.H, cs, eps, nullptr, s, cache, max_seq,
                                 pos0));
    if (prefill)
      HIPCHECK(nc::attn_fwd(dt, qkv, D.Q, D.B, Tseq, D.H, o, at<float>(ws, P.lse), s));
    else
      HIPCHECK(nc::decode_attn(dt, qkv, D.Q, D.B, D.H, cache, max_seq, pos0, at<float>(ws, P.part), o,
                               D.d, s));
    HIPCHECK(infer_linear(dt, Epi::AddF32, o, W(base + 1), x, M, D.d, D.d, D.d, D.d, s));
    HIPCHECK(nc::rmsnorm_fwd(dt, x, (int)M, D.d, eps, h2, rinv, s));
    HIPCHECK(infer_linear(dt, Epi::Relu2, h2, W(base + 2), a, M, D.F, D.d, D.d, D.F, s));
    HIPCHECK(infer_linear(dt, Epi::AddF32, a, W(base + 3), x, M, D.d, D.F, D.F, D.d, s));
  }
  return NC_OK;
}

// Final norm, then the capped logits of the last row of every `stride` rows.
int infer_logits(const Dims& D, const nc_config* cfg, const std::vector<Tensor>& lay,
                 const void* params, void* ws, const InferPlan& P, int64_t M, int stride,
                 float* logits_out, hipStream_t s) {
  const DType dt = D.dt;
  void* xf = at<char>(ws, P.xf);
  void* last = at<char>(ws, P.last);
  const char* U = static_cast<const char*>(params) + lay[1 + 4 * D.L].offset * D.esz;
  HIPCHECK(nc::rmsnorm_fwd(dt, at<float>(ws, P.x), (int)M, D.d, cfg->rms_eps, xf, at<float>(ws, P.rinv), s));
  if (few_rows(D, D.B)) {
    HIPCHECK(nc::gather_last_rows(dt, xf, stride, D.B, D.B, D.d, last, s));
    nc::SkArgs g{};
    g.W = U;
    g.ldw = D.d;
    g.X = last;
    g.ldx = D.d;
    g.C = logits_out;
    g.ldc = D.V;
    g.M = D.B;
    g.N = D.V;
    g.K = D.d;
    g.cap = cfg->softcap;
    g.part = at<float>(ws, P.skpart);
    g.cnt = at<uint32_t>(ws, P.skcnt);
    HIPCHECK(nc::skinny_gemm(g, nc::SkEpi::SoftcapF32, s));
    return NC_OK;
  }
  const int Bp = pad16(D.B);
  float* lg = at<float>(ws, P.logits);
  HIPCHECK(nc::gather_last_rows(dt, xf, stride, D.B, Bp, D.d, last, s));
  HIPCHECK(gemm_simple(dt, true, true, Epi::StoreF32, last, U, lg, nullptr, Bp, D.V, D.d, D.d, D.d,
                       D.V, 0, s));
  HIPCHECK(nc::softcap_rows(lg, D.B, D.V, cfg->softcap, logits_out, s));
  return NC_OK;
}

// bf16 decoding of up to 32 sequences: every linear layer through the
// few-row product, the block norms folded into the products that read the
// residual stream (its producers leave a bf16 copy and per-16-column sums of
// squares), the cache written by the rotary kernel.
int decode_few_rows(const Dims& D, const nc_config* cfg, const std::vector<Tensor>& lay,
                    const void* params, const int32_t* tokens, int pos, void* kv, int max_seq, void* ws,
                    const InferPlan& P, float* logits, hipStream_t s) {
  const float eps = cfg->rms_eps;
  auto W = [&](int idx) { return static_cast<const char*>(params) + lay[idx].offset * D.esz; };
  float* x = at<float>(ws, P.x);
  void* xb = at<char>(ws, P.xb);
  float* ssq = at<float>(ws, P.ssq);
  void* qkv = at<char>(ws, P.qkv);
  void* o = at<char>(ws, P.o);
  void* a = at<char>(ws, P.a);
  const int nssq = D.d / 16;
  auto lin = [&](int widx, const void* X, int ldx, void* C, int ldc, int N, int K, nc::SkEpi epi,
                 bool norm, bool emit, float cap) {
    nc::SkArgs g{};
    g.W = widx >= 0 ? W(widx) : nullptr;
    g.ldw = K;
    g.X = X;
    g.ldx = ldx;
    g.C = C;
    g.ldc = ldc;
    g.M = D.B;
    g.N = N;
    g.K = K;
    if (norm) {
      g.ssq_in = ssq;
      g.nssq = nssq;
      g.eps = eps;
    }
    if (emit) {
      g.xb = xb;
      g.ssq_out = ssq;
    }
    g.cap = cap;
    g.part = at<float>(ws, P.skpart);
    g.cnt = at<uint32_t>(ws, P.skcnt);
    return nc::skinny_gemm(g, epi, s);
  };
  HIPCHECK(nc::decode_embed(W(0), tokens, D.B, D.d, D.V, eps, x, xb, ssq, at<uint32_t>(ws, P.status), s));
  const float* cs = at<float>(ws, P.cs);
  for (int l = 0; l < D.L; ++l) {
    const int base = 1 + 4 * l;
    void* cache = static_cast<char*>(kv) + (uint64_t)l * kv_layer_bytes(D, max_seq);
    HIPCHECK(lin(base + 0, xb, D.d, qkv, D.Q, D.Q, D.d, nc::SkEpi::StoreT, true, false, 0.f));
    HIPCHECK(nc::rope_qknorm_fwd(D.dt, qkv, D.Q, D.B, 1, D.H, cs, eps, nullptr, s, cache, max_seq, pos));
    HIPCHECK(nc::decode_attn(D.dt, qkv, D.Q, D.B, D.H, cache, max_seq, pos, at<float>(ws, P.part), o, D.d,
                             s));
    HIPCHECK(lin(base + 1, o, D.d, x, D.d, D.d, D.d, nc::SkEpi::AddF32, false, true, 0.f));
    HIPCHECK(lin(base + 2, xb, D.d, a, D.F, D.F, D.d, nc::SkEpi::Relu2, true, false, 0.f));
    HIPCHECK(lin(base + 3, a, D.F, x, D.d, D.d, D.F, nc::SkEpi::AddF32, false, true, 0.f));
  }
  HIPCHECK(lin(1 + 4 * D.L, xb, D.d, logits, D.V, D.V, D.d, nc::SkEpi::SoftcapF32, true, false,
               cfg->softcap));
  return NC_OK;
}

int check_infer_args(const nc_config* cfg, const void* params, const void* tokens, const void* kv,
                     int max_seq, const void* ws, const float* logits) {
  const int rc = validate(cfg);
  if (rc) return rc;
  if (!params || !tokens || !kv || !ws || !logits) return NC_ERR_NULL;
  if (misaligned(params) || misaligned(tokens) || misaligned(kv) || misaligned(ws) ||
      misaligned(logits))
    return NC_ERR_ALIGN;
  if (max_seq < 1 || max_seq > (1 << 24)) return NC_ERR_ARG;
  return NC_OK;
}

}  // namespace

int nc_kv_cache_bytes(const nc_config* cfg, int32_t max_seq, uint64_t* bytes) {
  const int rc = validate(cfg);
  if (rc) return rc;
  if (!bytes) return NC_ERR_NULL;
  if (max_seq < 1 || max_seq > (1 << 24)) return NC_ERR_ARG;
  const Dims D = dims_of(cfg);
  *bytes = (uint64_t)D.L * kv_layer_bytes(D, max_seq);
  return NC_OK;
}

int nc_infer_workspace_bytes(const nc_config* cfg, int32_t max_seq, uint64_t* bytes) {
  const int rc = validate(cfg);
  if (rc) return rc;
  if (!bytes) return NC_ERR_NULL;
  if (max_seq < 1 || max_seq > (1 << 24)) return NC_ERR_ARG;
  *bytes = infer_plan_of(dims_of(cfg), max_seq).total;
  return NC_OK;
}

int nc_prefill(const nc_config* cfg, const void* params, const int32_t* tokens, int32_t T0, void* kv,
               int32_t max_seq, void* ws, uint64_t ws_bytes, float* logits, void* stream) {
  int rc = check_infer_args(cfg, params, tokens, kv, max_seq, ws, logits);
  if (rc) return rc;
  if (T0 < 64 || T0 % 64 || T0 > cfg->seq_len || T0 > max_seq) return NC_ERR_ARG;
  const Dims D = dims_of(cfg);
  const InferPlan P = infer_plan_of(D, max_seq);
  if (ws_bytes < P.total) return NC_ERR_WORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  Dims Dp = D;
  Dp.T = T0;
  Dp.M = (int64_t)D.B * T0;
  const auto lay = layout_of(D);
  const char* E = static_cast<const char*>(params) + lay[0].offset * D.esz;
  uint32_t* status = at<uint32_t>(ws, P.status);
  HIPCHECK(nc::fill_zero(status, P.sync_bytes, s));
  HIPCHECK(nc::rope_table(T0, 64, (double)cfg->rope_base, at<float>(ws, P.cs), s, 0));
  HIPCHECK(nc::embed_norm_fwd(D.dt, E, tokens, (int)Dp.M, D.d, D.V, cfg->rms_eps, at<float>(ws, P.x),
                              at<float>(ws, P.rinv), status, s));
  rc = infer_blocks(Dp, cfg, lay, params, ws, P, Dp.M, (int)Dp.M, T0, 0, true, kv, max_seq, s);
  if (rc) return rc;
  return infer_logits(Dp, cfg, lay, params, ws, P, Dp.M, T0, logits, s);
}

int nc_decode_step(const nc_config* cfg, const void* params, const int32_t* tokens, int32_t pos,
                   void* kv, int32_t max_seq, void* ws, uint64_t ws_bytes, float* logits,
                   void* stream) {
  int rc = check_infer_args(cfg, params, tokens, kv, max_seq, ws, logits);
  if (rc) return rc;
  if (pos < 0 || pos >= max_seq) return NC_ERR_ARG;
  const Dims D = dims_of(cfg);
  if (D.H > 16) return NC_ERR_UNSUPPORTED;
  const InferPlan P = infer_plan_of(D, max_seq);
  if (ws_bytes < P.total) return NC_ERR_WORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const auto lay = layout_of(D);
  const char* E = static_cast<const char*>(params) + lay[0].offset * D.esz;
  uint32_t* status = at<uint32_t>(ws, P.status);
  HIPCHECK(nc::fill_zero(status, P.sync_bytes, s));
  HIPCHECK(nc::rope_table(1, 64, (double)cfg->rope_base, at<float>(ws, P.cs), s, pos));
  if (few_rows(D, D.B))
    return decode_few_rows(D, cfg, lay, params, tokens, pos, kv, max_seq, ws, P, logits, s);
  // the tiled GEMM wants rows in multiples of 16; the rows past the batch stay
  // zero through the blocks (every row is independent)
  const int Mr = pad16(D.B);
  Dims Dd = D;
  Dd.M = Mr;
  HIPCHECK(nc::fill_zero(at<char>(ws, P.x), (size_t)Mr * D.d * 4, s));
  HIPCHECK(nc::fill_zero(at<char>(ws, P.o), (size_t)Mr * D.d * D.esz, s));
  HIPCHECK(nc::embed_norm_fwd(D.dt, E, tokens, D.B, D.d, D.V, cfg->rms_eps, at<float>(ws, P.x),
                              at<float>(ws, P.rinv), status, s));
  rc = infer_blocks(Dd, cfg, lay, params, ws, P, Mr, D.B, 1, pos, false, kv, max_seq, s);
  if (rc) return rc;
  return infer_logits(Dd, cfg, lay, params, ws, P, Mr, 1, logits, s);
}

int nc_read_device_status(const void* ws, uint32_t* flags, void* stream) {
  if (!ws || !flags) return NC_ERR_NULL;
  if (misaligned(ws)) return NC_ERR_ALIGN;
  hipStream_t s = static_cast<hipStream_t>(stream);
  HIPCHECK(hipMemcpyAsync(flags, ws, sizeof(uint32_t), hipMemcpyDeviceToHost, s));
  HIPCHECK(hipStreamSynchronize(s));
  return NC_OK;
}

const char* nc_status_string(int code) {
  switch (code) {
    case NC_OK: return "ok";
    case NC_ERR_INVALID_CONFIG: return "invalid config";
    case NC_ERR_UNSUPPORTED: return "unsupported config (n_kv_head must be 1, head_dim 128)";
    case NC_ERR_NULL: return "null pointer";
    case NC_ERR_ALIGN: return "device pointer not 256-byte aligned";
    case NC_ERR_WORKSPACE: return "workspace too small";
    case NC_ERR_HIP: return "HIP launch or runtime error";
    case NC_ERR_ARG: return "argument out of range";
    default: return "unknown status";
  }
}

int nc_last_hip_error(void) { return g_last_hip; }

// ---------------- single-step entry points ----------------

static bool bad_dtype(int32_t t) { return t != NC_F32 && t != NC_BF16; }
static DType dt_of(int32_t t) { return t == NC_BF16 ? DType::BF16 : DType::F32; }

int nc_op_gemm(int32_t dtype, int32_t a_kcontig, int32_t b_kcontig, int32_t epilogue,
               const void* A, const void* B, void* C, void* C2, int32_t M, int32_t N, int32_t K,
               int32_t lda, int32_t ldb, int32_t ldc, void* stream) {
  if (bad_dtype(dtype) || epilogue < 0 || epilogue > 4) return NC_ERR_ARG;
  if (!A || !B || !C || (epilogue == 4 && !C2)) return NC_ERR_NULL;
  if (M <= 0 || N <= 0 || K <= 0 || M % 16 || N % 16 || K % 64) return NC_ERR_ARG;
  const int vec = dtype == NC_BF16 ? 8 : 4;
  if (lda % vec || ldb % vec || ldc % 4) return NC_ERR_ARG;
  if (lda < (a_kcontig ? K : M) || ldb < (b_kcontig ? K : N) || ldc < N) return NC_ERR_ARG;
  static const Epi map[5] = {Epi::StoreT, Epi::StoreF32, Epi::AddF32, Epi::Relu2, Epi::Relu2Bwd};
  HIPCHECK(gemm_simple(dt_of(dtype), a_kcontig != 0, b_kcontig != 0, map[epilogue], A, B, C, C2, M,
                       N, K, lda, ldb, ldc, ldc, static_cast<hipStream_t>(stream)));
  return NC_OK;
}

int nc_op_few_rows_scratch_bytes(int32_t M, int32_t N, int32_t K, int32_t splits, uint64_t* bytes) {
  if (!bytes) return NC_ERR_NULL;
  if (M < 1 || M > nc::kSkinnyMaxRows || N < 16 || N % 16 || K < 32 || K % 32 || splits < 0 ||
      splits > K / 32)
    return NC_ERR_ARG;
  *bytes = align_up((uint64_t)(N / 16) * 4, kAlign) + nc::skinny_part_bytes(M, N, K, splits);
  return NC_OK;
}

int nc_op_few_rows_gemm(int32_t epilogue, const void* W, int32_t ldw, const void* X, int32_t ldx, void* C,
                        int32_t ldc, int32_t M, int32_t N, int32_t K, float cap, const float* ssq_in,
                        float eps, void* xb, float* ssq_out, int32_t splits, int32_t ntile, void* scratch,
                        uint64_t scratch_bytes, void* stream) {
  if (epilogue < 0 || epilogue > 3 || splits < 0 || splits > K / 32) return NC_ERR_ARG;
  if (ntile != 0 && ntile != 1 && ntile != 2 && ntile != 4) return NC_ERR_ARG;
  if (ntile > 0 && N % (16 * ntile)) return NC_ERR_ARG;
  if (!W || !X || !C || !scratch) return NC_ERR_NULL;
  if (misaligned(scratch)) return NC_ERR_ALIGN;
  if (M < 1 || M > nc::kSkinnyMaxRows || N < 16 || N % 16 || K < 32 || K % 32 || K > 2048 * (ssq_in ? 1 : 64))
    return NC_ERR_ARG;
  if (ldw % 8 || ldx % 8 || ldc % 4 || ldw < K || ldx < K || ldc < N) return NC_ERR_ARG;
  if (epilogue == 3 && !(cap > 0.f)) return NC_ERR_ARG;
  if ((xb || ssq_out) && epilogue != 1) return NC_ERR_ARG;
  uint64_t need = 0;
  nc_op_few_rows_scratch_bytes(M, N, K, splits, &need);
  if (scratch_bytes < need) return NC_ERR_WORKSPACE;
  static const nc::SkEpi map[4] = {nc::SkEpi::StoreT, nc::SkEpi::AddF32, nc::SkEpi::Relu2,
                                   nc::SkEpi::SoftcapF32};
  nc::SkArgs g{};
  g.W = W;
  g.ldw = ldw;
  g.X = X;
  g.ldx = ldx;
  g.C = C;
  g.ldc = ldc;
  g.M = M;
  g.N = N;
  g.K = K;
  g.ssq_in = ssq_in;
  g.nssq = K / 16;
  g.eps = eps;
  g.xb = xb;
  g.ssq_out = ssq_out;
  g.cap = cap;
  g.splits = splits;
  g.ntile = ntile;
  g.cnt = static_cast<uint32_t*>(scratch);
  g.part = reinterpret_cast<float*>(static_cast<char*>(scratch) + align_up((uint64_t)(N / 16) * 4, kAlign));
  HIPCHECK(nc::skinny_gemm(g, map[epilogue], static_cast<hipStream_t>(stream)));
  return NC_OK;
}

int nc_op_decode_attn(int32_t dtype, const void* qkv, int32_t ldq, int32_t B, int32_t H, const void* cache,
                      int32_t max_seq, int32_t pos, float* part, void* o, int32_t ldo, void* stream) {
  if (bad_dtype(dtype)) return NC_ERR_ARG;
  if (!qkv || !cache || !part || !o) return NC_ERR_NULL;
  if (B < 1 || H < 1 || H > 16 || pos < 0 || pos >= max_seq || ldq < H * 128 + 256 || ldo < H * 128 ||
      ldq % 8 || ldo % 8)
    return NC_ERR_ARG;
  HIPCHECK(nc::decode_attn(dt_of(dtype), qkv, ldq, B, H, cache, max_seq, pos, part, o, ldo,
                           static_cast<hipStream_t>(stream)));
  return NC_OK;
}

int nc_op_gemm_axpby(int32_t dtype, int32_t a_kcontig, int32_t b_kcontig, int32_t out_f32, const void* A,
                     const void* B, void* C, const void* C2, int32_t M, int32_t N, int32_t K, int32_t lda,
                     int32_t ldb, int32_t ldc, float alpha, float beta, int32_t batch, int64_t sa,
                     int64_t sb, int64_t sc, int32_t tile, void* stream) {
  if (bad_dtype(dtype)) return NC_ERR_ARG;
  if (!A || !B || !C || !C2) return NC_ERR_NULL;
  if (M <= 0 || N <= 0 || K <= 0 || M % 16 || N % 16 || K % 64 || batch < 1) return NC_ERR_ARG;
  const int vec = dtype == NC_BF16 ? 8 : 4;
  if (lda % vec || ldb % vec || ldc % 4) return NC_ERR_ARG;
  if (lda < (a_kcontig ? K : M) || ldb < (b_kcontig ? K : N) || ldc < N) return NC_ERR_ARG;
  if (sa < 0 || sb < 0 || sc < 0 || (tile != 0 && tile != 128 && tile != 256) ||
      (tile == 256 && dtype != NC_BF16))
    return NC_ERR_ARG;
  nc::GemmArgs g{};
  g.A = A;
  g.B = B;
  g.C = C;
  g.C2 = const_cast<void*>(C2);
  g.M = M;
  g.N = N;
  g.K = K;
  g.lda = lda;
  g.ldb = ldb;
  g.ldc = ldc;
  g.ldc2 = ldc;
  g.splits = 1;
  g.tile = tile;
  g.batch = batch;
  g.sa = sa;
  g.sb = sb;
  g.sc = sc;
  g.sc2 = sc;
  g.alpha = alpha;
  g.beta = beta;
  HIPCHECK(nc::gemm(dt_of(dtype), a_kcontig != 0, b_kcontig != 0, out_f32 ? Epi::AxpbyF32 : Epi::AxpbyT, g,
                    static_cast<hipStream_t>(stream)));
  return NC_OK;
}

int nc_op_wgrad(int32_t dtype, const void* X1, const void* X2, float* dW, float* partial,
                int32_t M, int32_t N1, int32_t N2, int32_t splits, void* stream) {
  if (bad_dtype(dtype)) return NC_ERR_ARG;
  if (!X1 || !X2 || !dW || (splits > 1 && !partial)) return NC_ERR_NULL;
  if (M <= 0 || N1 <= 0 || N2 <= 0 || N1 % 16 || N2 % 16 || splits < 1 || M % 64 ||
      M / 64 < splits)
    return NC_ERR_ARG;
  WgradPlan p = wgrad_plan(dt_of(dtype), N1, N2, M);   // same tile choice as the step
  p.splits = splits;
  HIPCHECK(wgrad(dt_of(dtype), X1, X2, dW, partial, M, N1, N2, p, static_cast<hipStream_t>(stream)));
  return NC_OK;
}

int nc_op_transpose(int32_t dtype, const void* in, int32_t R, int32_t C, int32_t ld_in, void* out,
                    int32_t ld_out, void* stream) {
  if (bad_dtype(dtype)) return NC_ERR_ARG;
  if (!in || !out) return NC_ERR_NULL;
  const int vec = dtype == NC_BF16 ? 8 : 4;
  if (R <= 0 || C <= 0 || R % vec || C % vec || ld_in % vec || ld_out % vec || ld_in < C ||
      ld_out < R)
    return NC_ERR_ARG;
  HIPCHECK(nc::transpose(dt_of(dtype), in, R, C, ld_in, out, ld_out,
                         static_cast<hipStream_t>(stream)));
  return NC_OK;
}

int nc_op_rmsnorm_fwd(int32_t dtype, const float* x, int32_t M, int32_t d, float eps, void* y,
                      float* rinv, void* stream) {
  if (bad_dtype(dtype)) return NC_ERR_ARG;
  if (!x || !y || !rinv) return NC_ERR_NULL;
  if (M <= 0 || d <= 0 || d % 64 || d > 2048) return NC_ERR_ARG;
  HIPCHECK(nc::rmsnorm_fwd(dt_of(dtype), x, M, d, eps, y, rinv, static_cast<hipStream_t>(stream)));
  return NC_OK;
}

int nc_op_rmsnorm_bwd(int32_t dtype, const void* dy, const void* y, const float* rinv, int32_t M,
                      int32_t d, float* dx, int32_t accumulate, void* g, void* stream) {
  if (bad_dtype(dtype)) return NC_ERR_ARG;
  if (!dy || !y || !rinv || !dx) return NC_ERR_NULL;
  if (M <= 0 || d <= 0 || d % 64 || d > 2048) return NC_ERR_ARG;
  HIPCHECK(nc::rmsnorm_bwd(dt_of(dtype), dy, y, rinv, M, d, dx, accumulate != 0, g,
                           static_cast<hipStream_t>(stream)));
  return NC_OK;
}

int nc_op_rope_qknorm_fwd(int32_t dtype, void* qkv, int32_t B, int32_t T, int32_t H, float base,
                          float eps, float* rinv_qk, float* cs, void* stream) {
  if (bad_dtype(dtype)) return NC_ERR_ARG;
  if (!qkv || !rinv_qk || !cs) return NC_ERR_NULL;
  if (B <= 0 || T <= 0 || H < 1 || H > 16) return NC_ERR_ARG;
  hipStream_t s = static_cast<hipStream_t>(stream);
  HIPCHECK(nc::rope_table(T, 64, (double)base, cs, s));
  HIPCHECK(nc::rope_qknorm_fwd(dt_of(dtype), qkv, H * 128 + 256, B * T, T, H, cs, eps, rinv_qk, s));
  return NC_OK;
}

int nc_op_rope_qknorm_bwd(int32_t dtype, void* dqkv, const void* qkv, int32_t B, int32_t T,
                          int32_t H, const float* rinv_qk, const float* cs, void* stream) {
  if (bad_dtype(dtype)) return NC_ERR_ARG;
  if (!dqkv || !qkv || !rinv_qk || !cs) return NC_ERR_NULL;
  if (B <= 0 || T <= 0 || H < 1 || H > 16) return NC_ERR_ARG;
  const int ld = H * 128 + 256;
  HIPCHECK(nc::rope_qknorm_bwd(dt_of(dtype), dqkv, ld, qkv, ld, B * T, T, H, cs, rinv_qk,
                               static_cast<hipStream_t>(stream)));
  return NC_OK;
}

int nc_op_attn_fwd(int32_t dtype, const void* qkv, int32_t B, int32_t T, int32_t H, void* o,
                   float* lse, void* stream) {
  if (bad_dtype(dtype)) return NC_ERR_ARG;
  if (!qkv || !o || !lse) return NC_ERR_NULL;
  if (B <= 0 || T < 64 || T % 64 || H < 1 || H > 16) return NC_ERR_ARG;
  HIPCHECK(nc::attn_fwd(dt_of(dtype), qkv, H * 128 + 256, B, T, H, o, lse,
                        static_cast<hipStream_t>(stream)));
  return NC_OK;
}

uint64_t nc_op_attn_bwd_scratch_bytes(int32_t B, int32_t T) {
  if (B <= 0 || T <= 0) return 0;
  return nc::attn_bwd_scratch_floats(B, T) * 4;
}

int nc_op_attn_bwd(int32_t dtype, const void* qkv, const void* o, const void* dout,
                   const float* lse, float* delta, int32_t B, int32_t T, int32_t H, void* dqkv,
                   float* scratch, void* stream) {
  if (bad_dtype(dtype)) return NC_ERR_ARG;
  if (!qkv || !o || !dout || !lse || !delta || !dqkv) return NC_ERR_NULL;
  if (B <= 0 || T < 64 || T % 64 || H < 1 || H > 16) return NC_ERR_ARG;
  if (!scratch && nc::attn_bwd_scratch_floats(B, T) > 0) return NC_ERR_NULL;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int ld = H * 128 + 256;
  HIPCHECK(nc::attn_bwd(dt_of(dtype), qkv, ld, o, dout, lse, delta, B, T, H, dqkv, ld, scratch, s));
  return NC_OK;
}

uint64_t nc_op_attn_bwd_ds_bytes(int32_t dtype, int32_t B, int32_t T, int32_t H) {
  if (bad_dtype(dtype) || B <= 0 || T < 64 || T % 64 || H < 1 || H > 16) return 0;
  return (uint64_t)nc::attn_bwd_ds_elems(B, T, H) * (dtype == NC_BF16 ? 2 : 4);
}

int nc_op_attn_bwd_stored_ds(int32_t dtype, const void* qkv, const void* o, const void* dout,
                             const float* lse, float* delta, int32_t B, int32_t T, int32_t H, void* dqkv,
                             float* scratch, void* ds, void* stream) {
  if (bad_dtype(dtype)) return NC_ERR_ARG;
  if (!qkv || !o || !dout || !lse || !delta || !dqkv || !ds) return NC_ERR_NULL;
  if (B <= 0 || T < 64 || T % 64 || H < 1 || H > 16) return NC_ERR_ARG;
  if (!scratch && nc::attn_bwd_scratch_floats(B, T) > 0) return NC_ERR_NULL;
  if (misaligned(ds)) return NC_ERR_ALIGN;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int ld = H * 128 + 256;
  HIPCHECK(nc::attn_bwd(dt_of(dtype), qkv, ld, o, dout, lse, delta, B, T, H, dqkv, ld, scratch, s, nullptr, ds));
  return NC_OK;
}

int nc_op_attn_bwd_noalloc(int32_t dtype, const void* qkv, const void* o, const void* dout,
                           const float* lse, int32_t B, int32_t T, int32_t H, void* dqkv,
                           void* stream) {
  if (bad_dtype(dtype)) return NC_ERR_ARG;
  if (!qkv || !o || !dout || !lse || !dqkv) return NC_ERR_NULL;
  if (B <= 0 || T < 64 || T % 64 || H < 1 || H > 16) return NC_ERR_ARG;
  const uint64_t delta_bytes = align_up((uint64_t)B * H * T * 4, kAlign);
  const uint64_t part_bytes = (uint64_t)nc::attn_bwd_scratch_floats(B, T) * 4;
  if (delta_bytes + part_bytes > nc::kAttnFixedScratchBytes) return NC_ERR_WORKSPACE;
  void* base = nullptr;
  HIPCHECK(nc::attn_fixed_scratch(&base));
  float* delta = static_cast<float*>(base);
  float* part = at<float>(base, delta_bytes);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int ld = H * 128 + 256;
  HIPCHECK(nc::attn_bwd(dt_of(dtype), qkv, ld, o, dout, lse, delta, B, T, H, dqkv, ld, part, s));
  return NC_OK;
}

int nc_op_softcap_ce(int32_t dtype, const void* logits, const int32_t* targets, int32_t R,
                     int32_t V, float cap, float w, float* loss_rows, void* dlogits,
                     uint32_t* status, void* stream) {
  if (bad_dtype(dtype)) return NC_ERR_ARG;
  if (!logits || !targets || !loss_rows || !status) return NC_ERR_NULL;
  if (R <= 0 || V <= 0 || V % 4 || V > 65536 || !(cap > 0.f)) return NC_ERR_ARG;
  HIPCHECK(nc::softcap_ce(dt_of(dtype), logits, targets, R, V, cap, w, loss_rows, dlogits, status,
                          static_cast<hipStream_t>(stream)));
  return NC_OK;
}

}  // extern "C"
