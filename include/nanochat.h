/*
 * nanochat.h — C ABI of the MI355X (gfx950) training-step library for
 * nanochat's depth-parameterised dense GPT.
 *
 * What the step computes (pages cited by title and section):
 *   - untied token embedding E[V,d] and lm_head U[V,d]; RMSNorm (no learnable
 *     parameters) after the embedding, before each attention and MLP block,
 *     and before lm_head; bias-free linear layers; rotary position embedding
 *     with QK-norm; causal multi-query attention (all query heads share one
 *     K/V head); relu^2 MLP; tanh logit softcap
 *       (followin.io release article, section "純手寫 8000 行代碼，
 *        “Agent 幫不上忙”", architecture list);
 *   - width = 64 * depth, 128-dim heads, 4x MLP, context 2048 at depth 20
 *       (wmrh.cn tutorial, section 2.2; vnrom.net "nanochat: khung thử
 *        nghiệm…", section "Thiết kế depth-only scaling");
 *   - vocabulary of 65,536 ids (wmrh.cn tutorial, section 2.1);
 *   - next-token cross-entropy, averaged over all B*T positions
 *       (wmrh.cn tutorial, section 2.3);
 *   - bf16 or fp32 parameters and activations, chosen explicitly
 *       (vnrom.net, section "Cấu trúc thư mục và module chính": precision is
 *        set by hand, no autocast). Accumulation is always fp32; the residual
 *        stream and its gradient are fp32 in both modes.
 *
 * Conventions the pages leave open are fixed as: RMSNorm eps = 1e-6; rotary
 * on half-split pairs (j, j+64) with angle t * base^(-2j/128), base 10000,
 * applied before the QK RMSNorm; attention scale 1/sqrt(128); softcap
 * z = c*tanh(l/c), c = 15; natural-log loss.
 *
 * Memory and ownership: the caller owns every device buffer (params, grads,
 * tokens, targets, workspace, loss). The library never allocates or frees
 * device memory and keeps no state between calls; two calls may run
 * concurrently only with distinct workspaces. All device pointers must be
 * 256-byte aligned. `stream` is a hipStream_t (NULL = the default stream);
 * every device-side effect is enqueued on it and the call returns before the
 * work completes.
 *
 * Errors: every function returns NC_OK (0) or a negative NC_ERR_* code. The
 * checks on arguments happen on the host before anything is enqueued; a
 * failed check enqueues nothing. NC_ERR_HIP means a launch failed; the HIP
 * error code is kept per thread (nc_last_hip_error). Problems only visible on
 * the device (a token or target id outside [0, V), which the kernels clamp to
 * stay in bounds, or a non-finite loss) set bits in a status word inside the
 * workspace, read with nc_read_device_status. Nothing throws across the ABI.
 */
#ifndef NANOCHAT_H_
#define NANOCHAT_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- return codes ------------------------------------------------------- */
#define NC_OK 0
#define NC_ERR_INVALID_CONFIG (-1) /* a config field out of range            */
#define NC_ERR_UNSUPPORTED (-2)    /* n_kv_head != 1 or head_dim != 128       */
#define NC_ERR_NULL (-3)           /* a required pointer is NULL              */
#define NC_ERR_ALIGN (-4)          /* a device pointer is not 256-B aligned   */
#define NC_ERR_WORKSPACE (-5)      /* ws_bytes below nc_workspace_bytes       */
#define NC_ERR_HIP (-6)            /* a HIP launch or runtime call failed     */
#define NC_ERR_ARG (-7)            /* another argument is out of range        */

/* ---- device status bits (nc_read_device_status) ------------------------- */
#define NC_STATUS_TOKEN_RANGE 1u    /* a token id was outside [0, V)          */
#define NC_STATUS_TARGET_RANGE 2u   /* a target id was outside [0, V)         */
#define NC_STATUS_NONFINITE_LOSS 4u /* the mean loss is NaN or infinite       */

typedef enum { NC_F32 = 0, NC_BF16 = 1 } nc_dtype;

/* Model and batch shape. Derived sizes: d = 64*depth, H = d/128 query heads,
 * F = 4*d, one K/V head, M = batch*seq_len tokens per call. */
typedef struct {
  int32_t depth;      /* L, even, 2..32 (whole 128-dim heads, H = L/2 <= 16)   */
  int32_t vocab_size; /* V, multiple of 128, 128..65536                        */
  int32_t seq_len;    /* T, multiple of 64, >= 64                              */
  int32_t batch;      /* B >= 1                                                */
  int32_t n_kv_head;  /* must be 1 (multi-query attention)                     */
  int32_t head_dim;   /* must be 128                                           */
  float softcap;      /* c > 0; 15 in every workload                           */
  float rope_base;    /* > 1; 10000                                            */
  float rms_eps;      /* >= 0; 1e-6                                            */
  float init_std;     /* > 0; 0.02 (used by nc_init_params)                    */
  int32_t dtype;      /* nc_dtype of params and activations                    */
} nc_config;

/* One parameter tensor: [rows, cols] row-major ([out, in]: y = x W^T),
 * starting `offset` elements into the flat parameter buffer. */
typedef struct {
  char name[32];
  uint64_t offset;
  int64_t rows, cols;
} nc_tensor_info;

/* Fills *out with the shape implied by depth (width 64*depth, 128-dim heads,
 * one K/V head, softcap 15, rope base 10000, eps 1e-6, init std 0.02) and
 * validates it. Host only. */
int nc_config_from_depth(int32_t depth, int32_t vocab_size, int32_t seq_len, int32_t batch,
                         int32_t dtype, nc_config* out);

/* NC_OK if the config is supported, else the error code. Host only. */
int nc_validate_config(const nc_config* cfg);

/* Element count of the flat parameter buffer (and of the gradient buffer),
 * padding included. Order: E, then per layer Wqkv[d+256, d] (query heads 0..H-1,
 * then the key rows, then the value rows), Wo[d, d], Wfc[4d, d], Wpr[d, 4d],
 * then U. Every tensor starts on a multiple of 128 elements. Host only. */
int nc_param_count(const nc_config* cfg, uint64_t* n_elems);

/* Writes up to `cap` tensor records in buffer order and sets *n to the total
 * number of tensors (4*depth + 2). Host only. */
int nc_param_layout(const nc_config* cfg, nc_tensor_info* out, int32_t cap, int32_t* n);

/* Bytes of workspace a call needs; with_backward selects nc_forward_backward
 * (saves every layer's activations) over nc_forward_loss. Host only. */
int nc_workspace_bytes(const nc_config* cfg, int32_t with_backward, uint64_t* bytes);

/* One piece of the workspace plan: what it holds, where it starts and how
 * many bytes it spans. Every piece is followed by at least 256 bytes that no
 * kernel writes (guard bytes), so a caller or test can fill a workspace with a
 * pattern and check after a call that nothing outside the pieces changed. */
typedef struct {
  char name[32];
  uint64_t offset;
  uint64_t bytes;
} nc_ws_piece;

/* Writes up to `cap` pieces of the workspace plan of nc_forward_backward
 * (with_backward != 0) or nc_forward_loss, in address order, and sets *n to
 * their total number. Host only. */
int nc_workspace_pieces(const nc_config* cfg, int32_t with_backward, nc_ws_piece* out, int32_t cap,
                        int32_t* n);

/* Rows of the lm_head + softcapped cross-entropy chunk. The step runs the
 * vocabulary-wide products and the loss over row chunks of the batch, so the
 * only [rows, vocab_size] buffer in the workspace (the chunk's logits, which
 * the loss kernel overwrites with their gradient) does not grow with the
 * batch. nc_set_lm_chunk_rows sets the chunk for every later call in the
 * process (0 restores the default of 32,768 rows; otherwise a positive
 * multiple of 64, else NC_ERR_ARG); it changes nc_workspace_bytes, so it is
 * meant for tuning and tests, not for use while calls are in flight.
 * nc_lm_chunk_rows reports min(batch*seq_len, chunk) for a config. Host only. */
int nc_set_lm_chunk_rows(int32_t rows);
int nc_lm_chunk_rows(const nc_config* cfg, int32_t* rows);

/* Schedule of the large bf16 contractions (256 x 256 output tiles) whose
 * output is whole tiles, is not split over K, and has more tiles than the
 * device has compute units: on = 1 (the default) runs them persistent, one
 * workgroup per compute unit walking its XCD's tiles, with each next tile's
 * first operand loads in flight during the current tile's epilogue; on = 0
 * runs one workgroup per tile. The tiles, their order per XCD and every
 * result are the same either way (bitwise). Process-wide, for measurement and
 * tests; not for use while calls are in flight. on other than 0 or 1:
 * NC_ERR_ARG. Host only. */
int nc_set_gemm_persistent(int32_t on);

/* Byte offset inside the workspace of the per-token losses (fp32 [B*T],
 * row-major like tokens), valid after a forward call until the next call on
 * the same workspace. Host only. */
int nc_token_losses_offset(const nc_config* cfg, int32_t with_backward, uint64_t* byte_offset);

/* Initialises the flat parameter buffer (nc_param_count elements of dtype):
 * element i of every tensor = std * N(0,1) from a counter-based generator
 * (SplitMix64 outputs 2i, 2i+1 for `seed` through Box-Muller, in float64,
 * rounded to float32 and then to dtype); std = init_std, divided by
 * sqrt(2*depth) for Wo and Wpr; padding = 0. Deterministic in (seed, cfg). */
int nc_init_params(uint64_t seed, const nc_config* cfg, void* params, void* stream);

/* Mean next-token loss (fp32, written to *loss_dev) of tokens -> targets,
 * both int32 [batch, seq_len] on the device. */
int nc_forward_loss(const nc_config* cfg, const void* params, const int32_t* tokens,
                    const int32_t* targets, void* ws, uint64_t ws_bytes, float* loss_dev,
                    void* stream);

/* Bits per byte of a batch (harness page, module list in "Cấu trúc thư mục
 * và module chính": the loss-evaluation module reports bits per byte). Runs
 * the forward pass as nc_forward_loss (same workspace; mean loss to
 * *loss_dev), then, over the positions whose target id has a nonzero byte
 * length in token_bytes (int32 [vocab_size] on the device: the tokenizer's
 * byte length of every id; 0 for special tokens), writes to bpb_dev (3
 * doubles on the device): the summed loss in nats, the summed byte lengths,
 * and their ratio in bits per byte, sum / (ln 2 * bytes) (NaN when no
 * position counts). Sums are fp64 in a fixed order. */
int nc_eval_bpb(const nc_config* cfg, const void* params, const int32_t* tokens, const int32_t* targets,
                const int32_t* token_bytes, void* ws, uint64_t ws_bytes, float* loss_dev, double* bpb_dev,
                void* stream);

/* Forward, loss and backward. grads (fp32, nc_param_count elements, same
 * layout as params) is OVERWRITTEN with d(mean loss)/d(params); padding
 * elements are left untouched. */
int nc_forward_backward(const nc_config* cfg, const void* params, const int32_t* tokens,
                        const int32_t* targets, float* grads, void* ws, uint64_t ws_bytes,
                        float* loss_dev, void* stream);

/* As nc_forward_backward, but ADDS d(mean loss)/d(params) to grads instead of
 * overwriting it, for gradient accumulation over several batches (wmrh.cn
 * tutorial, section 4.1: gradient accumulation). The caller zeroes grads
 * before the first batch and scales as it wants (each call adds the gradient
 * of that batch's mean loss). */
int nc_forward_backward_accumulate(const nc_config* cfg, const void* params,
                                   const int32_t* tokens, const int32_t* targets, float* grads,
                                   void* ws, uint64_t ws_bytes, float* loss_dev, void* stream);

/* ---- inference with a KV cache -------------------------------------------
 * An inference engine with a KV cache and a simple prefill / decode flow
 * (followin.io release article, section "花半天用 100 美元訓練的模型， 打敗了
 * GPT-2"; vnrom.net, section "Cấu trúc thư mục và module chính"). The model is
 * the training step's; the mask is causal, so the logits a decoding step
 * returns for position p equal the full-sequence forward's at p.
 *
 * Cache layout: for layer l, row b, position t, 256 values of dtype (the
 * rotary + QK-normalised key head, then the value head) at element
 * ((l * batch + b) * max_seq + t) * 256. cfg.batch is the number of sequences
 * decoded together and cfg.seq_len the longest prompt nc_prefill accepts.
 * Logits are fp32, softcapped (z = c tanh(l / c)), [batch, vocab_size]. */

/* Bytes of the cache for cfg.batch sequences of up to max_seq positions. */
int nc_kv_cache_bytes(const nc_config* cfg, int32_t max_seq, uint64_t* bytes);

/* Bytes of scratch for nc_prefill (prompts up to cfg.seq_len) and
 * nc_decode_step (caches of max_seq positions); the device status word sits
 * where nc_read_device_status expects it. */
int nc_infer_workspace_bytes(const nc_config* cfg, int32_t max_seq, uint64_t* bytes);

/* Runs the prompt tokens [batch, T0] (int32; T0 a multiple of 64, at most
 * cfg.seq_len and max_seq) through the model, fills cache positions 0..T0-1
 * and writes the logits of position T0-1 of every row. */
int nc_prefill(const nc_config* cfg, const void* params, const int32_t* tokens, int32_t T0, void* kv,
               int32_t max_seq, void* ws, uint64_t ws_bytes, float* logits, void* stream);

/* One decoding step: tokens [batch] (int32) at position pos (0 <= pos <
 * max_seq; positions 0..pos-1 of the cache must hold the sequence so far)
 * are run through the model, their keys and values stored at position pos,
 * and the logits of position pos written. Attention reads cache positions
 * 0..pos. Token ids outside [0, V) are clamped and flagged in the status. */
int nc_decode_step(const nc_config* cfg, const void* params, const int32_t* tokens, int32_t pos,
                   void* kv, int32_t max_seq, void* ws, uint64_t ws_bytes, float* logits,
                   void* stream);

/* ---- optimizer step --------------------------------------------------------
 * Muon for the block matrices (Wqkv, Wo, Wfc, Wpr of every layer) and AdamW
 * for the embedding E and the lm_head U (followin.io release article,
 * paragraph after the architecture list: Muon + AdamW, after modded-nanoGPT;
 * vnrom.net, section "Cấu trúc thư mục và module chính": the optimizer module
 * implements AdamW with Muon), after clipping the gradient by its global norm
 * (wmrh.cn tutorial, section 5.1). The pages do not define the update rules;
 * they follow the public descriptions:
 *   AdamW (decoupled weight decay, Adam's bias correction), per element:
 *     m = b1 m + (1-b1) g;  v = b2 v + (1-b2) g^2
 *     p = p (1 - lr wd) - lr (m / (1-b1^step)) / (sqrt(v / (1-b2^step)) + eps)
 *   Muon, per [R, C] matrix:
 *     buf = mu buf + g;  u = g + mu buf  (Nesterov)
 *     X = u / (||u||_F + 1e-7), transposed when R > C, then ns_steps times
 *     X = a X + (b A + c A^2) X with A = X X^T, (a, b, c) = (3.4445, -4.7750,
 *     2.0315), transposed back
 *     p = p (1 - lr wd) - lr max(1, R/C)^(1/2) X
 *   clipping: g is scaled by min(1, max_norm / (||g||_2 + 1e-6)), the norm
 *   over every parameter's gradient; max_norm <= 0 disables it.
 * In bf16 mode the Newton-Schulz products take bf16 operands (fp32
 * accumulation) and parameters are rounded back to bf16; in fp32 mode
 * everything is fp32. */
typedef struct {
  float lr_adamw;      /* AdamW learning rate (E, U), >= 0                       */
  float beta1, beta2;  /* AdamW moment decay rates, in [0, 1)                    */
  float eps;           /* AdamW denominator guard, > 0                           */
  float wd_adamw;      /* AdamW decoupled weight decay, >= 0                     */
  float lr_muon;       /* Muon learning rate (block matrices), >= 0              */
  float momentum;      /* Muon momentum mu, in [0, 1)                            */
  float wd_muon;       /* Muon decoupled weight decay, >= 0                      */
  float max_grad_norm; /* clip threshold; <= 0 disables clipping                 */
  int32_t ns_steps;    /* Newton-Schulz iterations, 0..16 (5 in the description) */
  int32_t step;        /* 1-based index of this step (AdamW bias correction)     */
} nc_optim_config;

/* Bytes of optimizer state: 2 * nc_param_count fp32 values in the parameter
 * layout. The first half holds AdamW's first moment for E and U and Muon's
 * momentum for the matrices, the second half AdamW's second moment (used for
 * E and U only). The caller zeroes it before the first step. */
int nc_optimizer_state_bytes(const nc_config* cfg, uint64_t* bytes);

/* Bytes of scratch nc_optimizer_step needs (norm partials and the
 * Newton-Schulz buffers of the largest matrix). */
int nc_optimizer_workspace_bytes(const nc_config* cfg, uint64_t* bytes);

/* One optimizer step: updates params (in place, dtype of cfg) and state from
 * grads (fp32, not modified); writes the pre-clip global gradient norm (fp32)
 * to *grad_norm_dev. Hyperparameters out of range give NC_ERR_ARG; ows must
 * hold nc_optimizer_workspace_bytes bytes and may not be shared with a
 * concurrent call. Deterministic: a fixed-order norm reduction and no atomics. */
int nc_optimizer_step(const nc_config* cfg, const nc_optim_config* optim, void* params,
                      const float* grads, float* state, void* ows, uint64_t ows_bytes,
                      float* grad_norm_dev, void* stream);

/* Copies the workspace status word to *flags (synchronises on the stream)
 * and clears nothing; each forward call resets it. */
int nc_read_device_status(const void* ws, uint32_t* flags, void* stream);

/* Human-readable text for a return code. */
const char* nc_status_string(int code);

/* HIP error code of this thread's last NC_ERR_HIP (0 if none). */
int nc_last_hip_error(void);

/* ---- single-step entry points -------------------------------------------
 * Each runs one stage of the step on caller buffers, for per-stage parity
 * tests and per-kernel timing. dtype is nc_dtype; "T" below means its
 * element type (float or bf16). Shapes are row-major. */

/* C[M,N] (op)= sum_k A(m,k) B(n,k), with A(m,k) = A[m*lda+k] when a_kcontig,
 * else A[k*lda+m] (same for B). epilogue: 0 store T, 1 store fp32,
 * 2 add into fp32, 3 relu^2 (C = relu(acc)^2 as T), 4 relu^2 backward
 * (C = acc * 2*sqrt(C2) as T, where C2 holds a = relu(u)^2 as stored by
 * epilogue 3, so 2*sqrt(a) = 2*relu(u)). C2 has row stride ldc.
 * M, N multiples of 16; K a multiple of 64. */
int nc_op_gemm(int32_t dtype, int32_t a_kcontig, int32_t b_kcontig, int32_t epilogue,
               const void* A, const void* B, void* C, void* C2, int32_t M, int32_t N, int32_t K,
               int32_t lda, int32_t ldb, int32_t ldc, void* stream);

/* bf16 product with few rows, as KV-cache decoding runs its linear layers
 * (one row per sequence): C[m,n] (epilogue) r_m sum_k X[m,k] W[n,k] for
 * m < M <= 32. W [N,K] and X [M,K] bf16 row-major (K-contiguous); epilogue
 * 0: C bf16 = acc, 1: C fp32 += acc, 2: C bf16 = relu(acc)^2, 3: C fp32 =
 * cap * tanh(acc / cap). r_m = 1 when ssq_in is NULL, else the RMS norm
 * factor 1/sqrt(ss_m / K + eps) with ss_m = sum_j ssq_in[j*32 + m], j < K/16
 * (K <= 2048). Epilogue 1 may also write xb (bf16 copy of the new C rows,
 * leading dimension ldc) and ssq_out[j*32 + m] (sum of the squares of new C
 * row m over columns 16j..16j+15). N % 16 == 0, K % 32 == 0, ldw and ldx
 * multiples of 8, ldc of 4. splits: slices of K (1..K/32) reduced in slice
 * order, 0 = the count decoding uses; ntile: 16-column tiles per workgroup
 * (1, 2 or 4, dividing N/16), 0 = decoding's choice. scratch:
 * nc_op_few_rows_scratch_bytes bytes,
 * 256-B aligned, its first N/16 words zero on entry (left zero). Results do
 * not depend on timing (fixed-order reductions). */
int nc_op_few_rows_scratch_bytes(int32_t M, int32_t N, int32_t K, int32_t splits, uint64_t* bytes);
int nc_op_few_rows_gemm(int32_t epilogue, const void* W, int32_t ldw, const void* X, int32_t ldx, void* C,
                        int32_t ldc, int32_t M, int32_t N, int32_t K, float cap, const float* ssq_in,
                        float eps, void* xb, float* ssq_out, int32_t splits, int32_t ntile, void* scratch,
                        uint64_t scratch_bytes, void* stream);

/* Decoding attention over a KV cache (layout as nc_kv_cache_bytes
 * describes, one layer): for each of B rows of qkv ([B, ldq], q-hat of H
 * heads first) the attention of its query heads over cache positions 0..pos
 * of that row, written to o [B, ldo] (H*128 per row). part is scratch of
 * B * ceil((pos+1)/64) * H * 129 floats. */
int nc_op_decode_attn(int32_t dtype, const void* qkv, int32_t ldq, int32_t B, int32_t H, const void* cache,
                      int32_t max_seq, int32_t pos, float* part, void* o, int32_t ldo, void* stream);

/* Batched contraction with a linear-combination epilogue, as the Newton-Schulz
 * iteration of the optimizer uses it: for batch item i (operands advance by
 * sa, sb and sc elements; C2 is laid out as C and advances with it)
 * C = alpha * (A B^T) + beta * C2, C2 of type T, C of type T (out_f32 = 0)
 * or fp32 (out_f32 = 1). Operand orders and size rules as nc_op_gemm; tile
 * 0 lets the library choose, 128 or 256 (bf16 only) forces the edge. The
 * 256 edge addresses operands with 32-bit offsets: lda and ldb must be below
 * 2^22 elements, else NC_ERR_HIP (the library's own choice falls back to the
 * 128 edge for such strides). */
int nc_op_gemm_axpby(int32_t dtype, int32_t a_kcontig, int32_t b_kcontig, int32_t out_f32, const void* A,
                     const void* B, void* C, const void* C2, int32_t M, int32_t N, int32_t K, int32_t lda,
                     int32_t ldb, int32_t ldc, float alpha, float beta, int32_t batch, int64_t sa,
                     int64_t sb, int64_t sc, int32_t tile, void* stream);

/* Weight-gradient contraction dW[N1,N2] = X1^T X2 over M rows (X1 [M,N1],
 * X2 [M,N2], type T), split over `splits` K slices with a fixed-order fp32
 * reduction through `partial` (splits*N1*N2 floats; unused when splits = 1).
 * Slice i covers the 64-row slabs [i*S/splits, (i+1)*S/splits), S = M/64 for
 * bf16 (M/32 for fp32); M must be a multiple of 64 and splits <= M/64. */
int nc_op_wgrad(int32_t dtype, const void* X1, const void* X2, float* dW, float* partial,
                int32_t M, int32_t N1, int32_t N2, int32_t splits, void* stream);

/* out[c][r] = in[r][c] for an R x C matrix of T (row strides ld_in, ld_out;
 * R, C and both strides multiples of 16 bytes' worth of elements). */
int nc_op_transpose(int32_t dtype, const void* in, int32_t R, int32_t C, int32_t ld_in, void* out,
                    int32_t ld_out, void* stream);

/* y = n(x) (T), rinv per row; x fp32 [M,d]. */
int nc_op_rmsnorm_fwd(int32_t dtype, const float* x, int32_t M, int32_t d, float eps, void* y,
                      float* rinv, void* stream);
/* dx (=|+=) rinv*(dy - y*mean(dy*y)) with dy and y of type T, dx fp32;
 * g (optional) = T(dx). */
int nc_op_rmsnorm_bwd(int32_t dtype, const void* dy, const void* y, const float* rinv, int32_t M,
                      int32_t d, float* dx, int32_t accumulate, void* g, void* stream);
/* In place on qkv [B*T, d+256]: rotary then RMSNorm on the H query heads and
 * the key head; rinv_qk [B*T, H+1]; cs scratch >= T*128 floats. */
int nc_op_rope_qknorm_fwd(int32_t dtype, void* qkv, int32_t B, int32_t T, int32_t H, float base,
                          float eps, float* rinv_qk, float* cs, void* stream);
/* In place on dqkv (same layout): gradient through the QK-norm then the
 * inverse rotation; v columns untouched. cs must hold the table written by
 * the forward call. */
int nc_op_rope_qknorm_bwd(int32_t dtype, void* dqkv, const void* qkv, int32_t B, int32_t T,
                          int32_t H, const float* rinv_qk, const float* cs, void* stream);
/* o [B*T, H*128] (T), lse [B, H, T] fp32 from qkv [B*T, d+256].
 * Precondition: every query and key head vector has RMS <= 1 (as the rotary
 * + QK-norm step leaves them; RMSNorm output satisfies it for any eps >= 0),
 * so scaled scores are bounded by sqrt(128): the softmax subtracts that fixed
 * bound instead of a running row maximum. Unnormalised inputs with scores
 * above ~60 overflow. */
int nc_op_attn_fwd(int32_t dtype, const void* qkv, int32_t B, int32_t T, int32_t H, void* o,
                   float* lse, void* stream);
/* Bytes of scratch nc_op_attn_bwd needs: fp32 partial dK/dV sums per
 * 2048-token query chunk when T > 2048; 0 when T <= 2048 (each key block's
 * dK/dV are then summed and written by one workgroup) and for invalid sizes.
 * Host only. */
uint64_t nc_op_attn_bwd_scratch_bytes(int32_t B, int32_t T);
/* dqkv [B*T, d+256] (T) from qkv, o, dout [B*T, H*128], lse; delta [B, H, T]
 * fp32 is written with <dO, O> per row and head (scratch to the caller); scratch of nc_op_attn_bwd_scratch_bytes(B, T) bytes (may be
 * NULL when that is 0). */
int nc_op_attn_bwd(int32_t dtype, const void* qkv, const void* o, const void* dout,
                   const float* lse, float* delta, int32_t B, int32_t T, int32_t H, void* dqkv,
                   float* scratch, void* stream);
/* Bytes of the dS buffer nc_op_attn_bwd_stored_ds needs: B*H*ceil(T/128)^2*128*128
 * elements of the dtype; 0 for invalid arguments. Host only. */
uint64_t nc_op_attn_bwd_ds_bytes(int32_t dtype, int32_t B, int32_t T, int32_t H);
/* The same attention backward as nc_op_attn_bwd (same arguments, results equal
 * up to rounding order; followin.io release article, architecture list:
 * multi-query attention; wmrh.cn tutorial 2.3: causal next-token objective),
 * computed the way the training step does it: delta first, then one dK/dV pass
 * that also writes dS^T = (P * (dP - delta))^T in the dtype into ds
 * ([b][h][query block of 128][key][128 queries], keys padded to a multiple of
 * 128; the caller's buffer of nc_op_attn_bwd_ds_bytes bytes, 256-byte aligned,
 * overwritten), then dQ as one
 * product dS.K over it - instead of a dQ pass that recomputes S and dP.
 * NC_ERR_NULL when ds is NULL. */
int nc_op_attn_bwd_stored_ds(int32_t dtype, const void* qkv, const void* o, const void* dout,
                             const float* lse, float* delta, int32_t B, int32_t T, int32_t H, void* dqkv,
                             float* scratch, void* ds, void* stream);
/* nc_op_attn_bwd without any caller scratch, for callers that cannot
 * allocate device memory (code under HIP graph capture, serving loops,
 * harnesses that forbid hipMalloc). Same arguments and results as
 * nc_op_attn_bwd (bitwise: the same kernels) except that delta and the dK/dV
 * chunk partials live in a 32 MiB array inside the library, one per device,
 * held until the process ends; the call allocates nothing. Sizes needing more
 * than that, i.e. 4*B*H*T (rounded up to 256) plus, when T > 2048,
 * 4*B*T*256*ceil(T/2048) bytes above 32 MiB (at T = 2048 and H = 10: B up to
 * 409; at T = 4096 and H = 10: B up to 3), are refused with NC_ERR_WORKSPACE
 * before anything is enqueued. Every call on a
 * device shares that device's array and nothing in it needs clearing (each
 * call writes what it reads); calls that overlap on one device (concurrent
 * streams, threads) race on it and must be serialised by the caller. */
int nc_op_attn_bwd_noalloc(int32_t dtype, const void* qkv, const void* o, const void* dout,
                           const float* lse, int32_t B, int32_t T, int32_t H, void* dqkv,
                           void* stream);
/* Per-row loss and (if dlogits != NULL) w-scaled logit gradient (T) from
 * logits [R, V] of type T; dlogits may equal logits (the gradient then
 * replaces them in place); status: device word for range flags (may not be
 * NULL). */
int nc_op_softcap_ce(int32_t dtype, const void* logits, const int32_t* targets, int32_t R,
                     int32_t V, float cap, float w, float* loss_rows, void* dlogits,
                     uint32_t* status, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* NANOCHAT_H_ */
