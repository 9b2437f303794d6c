/* gpt2.h -- C ABI of the MI355X (gfx950) GPT-2 training-step library, libgpt2_mi355x.so.
 *
 * One GPT-2-style decoder-only training step: token + position embedding gather,
 * pre-LayerNorm blocks (causal multi-head self-attention, GELU MLP, residuals), final
 * LayerNorm, tied lm_head with softmax cross-entropy, full backward, AdamW.
 * The operations follow "llm.c 的中文注解-20240421" (an annotated copy of llm.c's
 * train_gpt2.c; cited below as [llm.c] with its section numbers) and "高能技巧！60 行
 * NumPy 代码实现一个 GPT" (GPT in 60 lines of NumPy; cited as [np60] with its section
 * names).
 *
 * Conventions for every entry point:
 *  - All tensors are fp32, row-major, unless stated. "(B,T,C)" means C is contiguous.
 *  - Pointers documented as "device" must be HIP device (or managed) memory; "host" means
 *    ordinary host memory. Arguments named *_is_device select between the two.
 *  - Work is enqueued on the model's HIP stream (or the stream argument of the per-kernel
 *    entry points); a NULL stream means the null (default) stream. Calls return once the
 *    work is enqueued unless they read a result back to the host, which synchronises that
 *    stream.
 *  - Return value: GPT2_OK (0) or a negative GPT2_ERR_* code. Errors never abort the
 *    process; gpt2_last_error() gives a message for the model's last failure, and
 *    gpt2_last_global_error() for failures with no model (build, per-kernel calls).
 *  - A model is bound to one device and one stream and is not re-entrant: do not call
 *    into the same model from two threads at once.
 */
#ifndef GPT2_MI355X_H
#define GPT2_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct gpt2_model gpt2_model; /* opaque; owns every device buffer of one model */

enum {
  GPT2_OK = 0,
  GPT2_ERR_ARG = -1,   /* invalid argument: null pointer, non-positive or unsupported size */
  GPT2_ERR_SHAPE = -2, /* B,T differ from the shape the activations were sized for */
  GPT2_ERR_TOKEN = -3, /* a token or target outside [0, V) */
  GPT2_ERR_STATE = -4, /* call out of order (backward before a forward with targets, ...) */
  GPT2_ERR_OOM = -5,   /* device allocation failed */
  GPT2_ERR_HIP = -6,   /* a HIP runtime call failed */
  GPT2_ERR_IO = -7     /* a file could not be opened, read or written, or is malformed */
};

/* Arithmetic of the training step.
 * GPT2_DTYPE_FP32: every tensor fp32. Each fp32 product of the GEMMs, of the attention
 *   forward and of the attention dQ is formed as six bf16 MFMA products of an exact
 *   three-way bf16 split of its operands (within 2^-23 of the exact product) with fp32
 *   accumulation; so are the attention dK/dV products for head sizes in (32, 64] (other
 *   head sizes: fp32 MFMA; see gpt2_k_matmul_forward and gpt2_k_attention_forward for the
 *   switches that select fp32 MFMA products throughout).
 * GPT2_DTYPE_BF16: mixed precision, the extension to "fp16 or lower" that the llm.c
 *   overview names as a next step: GEMM operands (a bf16 copy of the weights, refreshed
 *   by every gpt2_set_params and gpt2_adamw_step) and all activation tensors are stored
 *   as bf16 (round to nearest even) and multiplied on bf16 MFMA with fp32 accumulation;
 *   LayerNorm statistics, softmax and cross-entropy reductions, the losses, the residual-
 *   stream gradient, the parameter gradients, the master parameters and the AdamW moments
 *   stay fp32. The ABI is unchanged: parameters, gradients, logits and losses are read
 *   and written as fp32. */
/* GPT2_DTYPE_FP16: the same mixed precision with IEEE fp16 (11 significant bits, largest
 *   finite 65504) in place of bf16, on fp16 MFMA. fp16's narrow exponent range needs loss
 *   scaling: the backward starts from d(mean loss)/d(loss) = S/(B*T) with a power-of-two
 *   loss scale S (2^16 at build), so every activation gradient is S times the true one and
 *   stays clear of fp16 underflow; the parameter gradients accumulate the scaled values in
 *   fp32. gpt2_adamw_step first checks them: if any is infinite or NaN (an fp16 overflow in
 *   the backward), the step leaves parameters and moments unchanged ("skipped") and S is
 *   halved; otherwise it applies AdamW to the gradients divided by S, and after every
 *   growth_interval (2000) steps in a row without an overflow S doubles (at most 2^24).
 *   gpt2_get_grads / gpt2_set_grads exchange unscaled gradients (exact: S is a power of
 *   two). The scaler lives on the device; no step waits for it. */
enum { GPT2_DTYPE_FP32 = 0, GPT2_DTYPE_BF16 = 1, GPT2_DTYPE_FP16 = 2 };

/* ---------------------------------------------------------------------------------------
 * Model lifetime and parameters
 * ------------------------------------------------------------------------------------- */

/* Create a model with L layers, C channels, H heads, vocabulary V and maximum sequence
 * length maxT ([llm.c] 1.20 GPT2Config). Allocates, on the current HIP device, one flat
 * block holding parameters, gradients and the two AdamW moments (4 x num_params fp32),
 * all zero. Activations are allocated as one flat block at the first gpt2_forward, for
 * that call's B and T ([llm.c] 1.23 allocates lazily; 1.19 one allocation).
 * Requires C % H == 0, C % 4 == 0 and (C/H) % 4 == 0 with C/H <= 128, C <= 2048 and
 * V < 2^21; all sizes >= 1.
 * *out receives the handle, or NULL on error. */
int gpt2_build(gpt2_model** out, int L, int C, int H, int V, int maxT);

/* As gpt2_build, plus: dtype (GPT2_DTYPE_FP32, GPT2_DTYPE_BF16 or GPT2_DTYPE_FP16; the
 * 16-bit dtypes also need every parameter tensor to start at a multiple of 8 elements); if maxB > 0 and maxTseq > 0 the
 * activation block is allocated now for exactly B = maxB, T = maxTseq; stream is the
 * hipStream_t the model enqueues all its work on (NULL = the null stream). */
int gpt2_build_ex(gpt2_model** out, int L, int C, int H, int V, int maxT, int dtype,
                  int maxB, int maxTseq, void* stream);

/* Release every device buffer and the handle ([llm.c] 1.27 gpt2_free). NULL is a no-op. */
void gpt2_free(gpt2_model* model);

/* Rebind the model to another hipStream_t (NULL = the null stream), after waiting for the
 * work already enqueued on the current one. */
int gpt2_set_stream(gpt2_model* model, void* stream);

/* Block until all work enqueued on the model's stream has finished. Reports
 * GPT2_ERR_TOKEN if a forward since the last check saw an out-of-range token. */
int gpt2_synchronize(gpt2_model* model);

/* The model's configuration ([llm.c] 1.20 GPT2Config): cfg = {L, C, NH, V, maxT}. */
int gpt2_get_config(const gpt2_model* model, int cfg[5]);

/* Number of fp32 parameters: the sum of the 16 tensor sizes of [llm.c] 1.22. */
size_t gpt2_num_params(const gpt2_model* model);

/* Offsets and lengths (in floats) of the 16 parameter tensors inside the flat buffer, in
 * the order of [llm.c] 1.16 ParameterTensors: wte (V,C), wpe (maxT,C), ln1w (L,C), ln1b
 * (L,C), qkvw (L,3C,C), qkvb (L,3C), attprojw (L,C,C), attprojb (L,C), ln2w (L,C), ln2b
 * (L,C), fcw (L,4C,C), fcb (L,4C), fcprojw (L,C,4C), fcprojb (L,C), lnfw (C), lnfb (C).
 * Weight matrices are (out, in) and are applied as x . W^T ([llm.c] 1.5). */
int gpt2_param_layout(const gpt2_model* model, size_t off[16], size_t len[16]);

/* Copy num_params floats in the flat layout above into / out of the model. */
int gpt2_set_params(gpt2_model* model, const float* src, int src_is_device);
int gpt2_get_params(gpt2_model* model, float* dst, int dst_is_device);
/* Parameter gradients (flat layout) as accumulated by gpt2_backward. */
int gpt2_get_grads(gpt2_model* model, float* dst, int dst_is_device);
/* Overwrite the gradients (flat layout); lets a caller run gpt2_adamw_step on given grads. */
int gpt2_set_grads(gpt2_model* model, const float* src, int src_is_device);
/* GPT2_DTYPE_FP16 loss scaling (see GPT2_DTYPE_FP16): set the scale S (a power of two in
 * [1, 2^24]) and the growth interval (steps without overflow before S doubles; 0 keeps S
 * fixed, though an overflowing step is still skipped); waits for the stream. ERR_ARG for
 * other dtypes or bad values. gpt2_get_loss_scale waits for the stream and returns S and
 * whether the last gpt2_adamw_step was skipped (1) or applied (0); other dtypes report
 * S = 1, not skipped. Either output pointer may be NULL. */
int gpt2_set_loss_scale(gpt2_model* model, float scale, int growth_interval);
int gpt2_get_loss_scale(gpt2_model* model, float* scale, int* last_step_skipped);
/* AdamW first and second moments (flat layout); either pointer may be NULL. */
int gpt2_get_adam_state(gpt2_model* model, float* m, float* v, int dst_is_device);

/* ---------------------------------------------------------------------------------------
 * Training step: gpt2_zero_grad -> gpt2_forward(targets) -> gpt2_backward -> gpt2_adamw_step
 * ------------------------------------------------------------------------------------- */

/* Forward pass ([llm.c] 1.23 gpt2_forward). tokens and targets: device int32 (B,T),
 * caller-owned; they are copied into the model, so they may be reused once this returns.
 * targets may be NULL (no loss; backward is then refused). mean_loss: host float or NULL.
 * If non-NULL the call waits for the step and stores the mean cross-entropy over the B*T
 * positions, or -1 when targets is NULL; it also reports GPT2_ERR_TOKEN for a token or
 * target outside [0, V) (such entries are read as 0 so no access goes out of bounds).
 * If NULL nothing is waited for; the loss stays on the device (gpt2_get_losses).
 * Errors: ERR_ARG (T > maxT, B or T < 1), ERR_SHAPE (B,T differ from the allocation). */
int gpt2_forward(gpt2_model* model, const int32_t* tokens, const int32_t* targets, int B,
                 int T, float* mean_loss);

/* Per-position losses (B,T) and the logits (B,T,V) of the last forward. gpt2_get_logits is
 * valid only between a forward and the next backward (else ERR_STATE): the backward may
 * reuse the logits buffer for their gradient. */
int gpt2_get_losses(gpt2_model* model, float* dst, int dst_is_device);
int gpt2_get_logits(gpt2_model* model, float* dst, int dst_is_device);

/* Where the loss gradient of the logits ([llm.c] 1.15) is formed. With on = 1 (the default)
 * a forward with targets computes the losses and d(mean loss)/d(logits) in one pass over
 * the logits (gpt2_k_crossentropy_fused) into a buffer of its own, the size of the logits,
 * that the next gpt2_backward reads; with on = 0 the forward only computes the losses and
 * the backward forms the gradient in place of the logits (one more pass over them, no extra
 * buffer; for forward-only evaluation). Takes effect at the next forward; turning it on
 * after the first forward of a model built with it off is ERR_STATE (the buffer is sized
 * with the activations). Results agree to rounding either way. */
int gpt2_set_loss_grad_in_forward(gpt2_model* model, int on);

/* Set all parameter gradients to zero ([llm.c] 1.24 gpt2_zero_grad). The library writes,
 * rather than accumulates, every activation gradient, so only parameter gradients need
 * zeroing. */
int gpt2_zero_grad(gpt2_model* model);

/* Backward pass ([llm.c] 1.25 gpt2_backward) of the mean loss of the last forward, which
 * must have had targets (else ERR_STATE). Adds d(mean loss)/d(param) to the gradients. */
int gpt2_backward(gpt2_model* model);

/* One AdamW update of every parameter ([llm.c] 1.26 gpt2_update): m = b1 m + (1-b1) g;
 * v = b2 v + (1-b2) g^2; p -= lr (m/(1-b1^t) / (sqrt(v/(1-b2^t)) + eps) + wd p).
 * t is the 1-based step count (ERR_ARG if t < 1). */
int gpt2_adamw_step(gpt2_model* model, float lr, float beta1, float beta2, float eps,
                    float weight_decay, int t);

/* ---------------------------------------------------------------------------------------
 * Checkpoints, token files, sampling
 * ------------------------------------------------------------------------------------- */

/* Checkpoint files in the format [llm.c] 1.22 gpt2_build_from_checkpoint reads: 256 int32
 * (magic 20240326, version 1, maxT, V, L, NH, C, then zeros), followed by the fp32
 * parameters in the flat order of gpt2_param_layout ([llm.c] 1.16). Native byte order.
 * gpt2_checkpoint_info checks the header (magic, version, positive sizes) and that the file
 * holds exactly the parameters the header implies, and returns the configuration (any
 * output pointer may be NULL). gpt2_checkpoint_read reads the n = num_params floats into
 * host memory (ERR_ARG if n differs). gpt2_checkpoint_write writes a checkpoint from host
 * parameters (count implied by the sizes). Malformed or unreadable files: GPT2_ERR_IO.
 * These three need no GPU. */
int gpt2_checkpoint_info(const char* path, int* maxT, int* V, int* L, int* NH, int* C,
                         size_t* num_params);
int gpt2_checkpoint_read(const char* path, float* params, size_t n);
int gpt2_checkpoint_write(const char* path, int maxT, int V, int L, int NH, int C,
                          const float* params);
/* gpt2_build_ex with the configuration and parameters of a checkpoint file (the remaining
 * arguments as for gpt2_build_ex); *out is NULL on error. */
int gpt2_build_from_checkpoint(gpt2_model** out, const char* path, int dtype, int maxB,
                               int maxTseq, void* stream);
/* Write the model's current fp32 parameters as a checkpoint (waits for the stream). */
int gpt2_save_checkpoint(gpt2_model* model, const char* path);

/* Token files as [llm.c] 1.28 - 1.32 DataLoader reads them: a flat file of int32 tokens.
 * Each batch is the next window of B*T+1 tokens: inputs = window[0, B*T), targets =
 * window[1, B*T+1) (shifted by one); the window then advances by B*T tokens, and starts
 * again at the beginning of the file when the next window would run past its end.
 * gpt2_dataloader_init: ERR_IO if the file cannot be opened, ERR_ARG if it holds fewer than
 * B*T+1 tokens. gpt2_dataloader_num_batches: file size / (B*T*4), as the page counts.
 * gpt2_dataloader_next_batch copies the batch into inputs and targets (B*T int32 each; host
 * memory, or device memory when dst_is_device, copied on `stream` and waited for). Token
 * values are not checked here (gpt2_forward checks them against V). */
typedef struct gpt2_dataloader gpt2_dataloader;
int gpt2_dataloader_init(gpt2_dataloader** out, const char* path, int B, int T);
int gpt2_dataloader_num_batches(const gpt2_dataloader* loader);
int gpt2_dataloader_reset(gpt2_dataloader* loader);
int gpt2_dataloader_next_batch(gpt2_dataloader* loader, int32_t* inputs, int32_t* targets,
                               int dst_is_device, void* stream);
void gpt2_dataloader_free(gpt2_dataloader* loader);

/* [llm.c] 1.33 random_u32: xorshift* on a 64-bit state (shifts 12, 25, 27; the upper 32 bits
 * of the state times 0x2545F4914F6CDD1D). The state must not be 0. [llm.c] 1.34 random_f32:
 * the upper 24 bits of the next draw over 2^24, a float in [0, 1). Host functions. */
uint32_t gpt2_random_u32(uint64_t* state);
float gpt2_random_f32(uint64_t* state);

/* [llm.c] 1.35 sample_mult on the probabilities softmax(logits[b, t, :]) of the model's
 * last forward (valid between a forward and the next backward, else ERR_STATE): the
 * smallest token index i whose cumulative probability exceeds coin (coin in [0, 1), e.g.
 * from gpt2_random_f32), or V - 1 if rounding leaves every cumulative value at or below
 * coin. The probabilities and their running sum are fp32, the sum in index order within
 * fixed chunks. Waits for the stream and stores the index in *token (host). */
int gpt2_sample(gpt2_model* model, int b, int t, float coin, int32_t* token);

/* Launch profiler. gpt2_profile_enable(1) clears the record and from then on brackets every
 * kernel launch of the library with two HIP events on the launch's stream, tagged with the
 * kernel's name and that launch's algorithmic flops and HBM bytes; (2) does the same with
 * the problem shape appended to GEMM names; (0) stops recording.
 * gpt2_profile_summary waits for the recorded events and writes one line per kernel name,
 * "name<TAB>launches<TAB>total_ms<TAB>total_flop<TAB>total_bytes", into buf (ERR_ARG if
 * len is too small). Process-wide state; not thread-safe. */
int gpt2_profile_enable(int on);
int gpt2_profile_summary(char* buf, size_t len);
/* Restrict the profiler to launches whose recorded name equals `name` (a copy is kept);
 * NULL or "" records every launch again. Fewer events perturb the timed work less. */
int gpt2_profile_only(const char* name);

const char* gpt2_last_error(const gpt2_model* model);
const char* gpt2_last_global_error(void);
const char* gpt2_version(void);

/* ---------------------------------------------------------------------------------------
 * Per-kernel entry points: the production kernels on caller device buffers, enqueued on
 * `stream` (hipStream_t, NULL = null stream). They exist so each kernel can be checked
 * against a reference on its own. All pointers are device pointers unless stated.
 * ------------------------------------------------------------------------------------- */

/* [llm.c] 1.1: out (B,T,C) = wte[tok] + wpe[t]. tok (B,T) int32; entries outside [0,V)
 * read row 0 and set *err_flag (device int, may be NULL) to 1. */
int gpt2_k_encoder_forward(float* out, const int32_t* tok, const float* wte, const float* wpe,
                           int B, int T, int C, int V, int32_t* err_flag, void* stream);

/* [llm.c] 1.2: dwte[tok[b,t]] += dout[b,t]; dwpe[t] += sum_b dout[b,t]. Deterministic:
 * rows of one token are summed in ascending (b,t) order, in pieces cut at every multiple of
 * 32 in the order of positions sorted by (token, position), the piece sums added in order
 * and then to dwte. Tokens must be in [0,V) (others count as token 0); V below 2^21
 * (ERR_ARG otherwise). Allocates and frees its own scratch; synchronizes the stream. */
int gpt2_k_encoder_backward(float* dwte, float* dwpe, const float* dout, const int32_t* tok,
                            int B, int T, int C, int V, void* stream);

/* [llm.c] 1.3, [np60] Layer Norm: per row of x (N,C), out = (x-mean)*rstd*w + b with the
 * biased variance and rstd = 1/sqrt(var + 1e-5); mean, rstd (N) may be NULL. */
int gpt2_k_layernorm_forward(float* out, float* mean, float* rstd, const float* x,
                             const float* w, const float* b, int N, int C, void* stream);

/* [llm.c] 1.4: dx (N,C) += LN backward; dw, db (C) += column sums. Deterministic. */
int gpt2_k_layernorm_backward(float* dx, float* dw, float* db, const float* dout,
                              const float* x, const float* w, const float* mean,
                              const float* rstd, int N, int C, void* stream);

/* [llm.c] 1.5 (+1.9, 1.11 fused): out (N,OC) = inp (N,C) . W(OC,C)^T + bias (bias may be
 * NULL), then by `epilogue`: 0 store; 1 also out2 = gelu(out) (tanh form, [llm.c] 1.9);
 * 2 out = resid + result (resid (N,OC) may alias out). ld_out >= OC is out's row stride.
 * The fp32 GEMMs here and in gpt2_k_matmul_backward form each fp32 product as six bf16
 * MFMA products of an exact three-way bf16 split of the operands (within 2^-23 of the
 * exact product) with fp32 accumulation; the environment variable
 * GPT2_GEMM_F32_PRODUCTS=fp32 selects fp32 MFMA products instead. Leading dimensions must
 * be below 2^21 and multiples of 4 (-1 otherwise). */
int gpt2_k_matmul_forward(float* out, float* out2, const float* resid, const float* inp,
                          const float* W, const float* bias, int N, int C, int OC,
                          int ld_out, int epilogue, void* stream);

/* [llm.c] 1.6 (+1.10 fused): dinp (N,C) = dout (N,OC) . W (OC,C) -- written, not
 * accumulated; if gelu_pre != NULL, dinp = gelu'(gelu_pre) * (dout . W) (gelu_pre (N,C));
 * dW (OC,C) += dout^T . inp; dbias (OC) += column sums of dout (may be NULL).
 * ld_dout >= OC is dout's row stride. dinp may be NULL (skip), as may dW. */
int gpt2_k_matmul_backward(float* dinp, float* dW, float* dbias, const float* dout,
                           const float* inp, const float* W, const float* gelu_pre, int N,
                           int C, int OC, int ld_dout, void* stream);

/* Allocation-free form of gpt2_k_matmul_backward, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc). Same arguments, kernels and results as gpt2_k_matmul_backward; its scratch
 * (split-K partial products and bias-gradient partial sums) is a static device array of
 * GPT2_NOALLOC_SCRATCH_FLOATS floats (68 MiB) that each GPU the library runs on holds
 * until the process ends, located once per device at the first call on it. It calls no
 * allocator and never waits for the stream. A problem whose plan needs more scratch (for
 * example the tied lm_head weight gradient at B*T = 16384) is rejected with GPT2_ERR_ARG
 * before anything is enqueued. Every call on one GPU shares that GPU's array: calls that
 * overlap on one device (two streams, or two host threads) race and must not be issued;
 * calls in order on one stream are safe. */
#define GPT2_NOALLOC_SCRATCH_FLOATS (17 << 20)
int gpt2_k_matmul_backward_noalloc(float* dinp, float* dW, float* dbias, const float* dout,
                                   const float* inp, const float* W, const float* gelu_pre,
                                   int N, int C, int OC, int ld_dout, void* stream);

/* [llm.c] 1.7, [np60] Attention: qkv (B,T,3C) -> out (B,T,C), causal softmax attention
 * per head with scale 1/sqrt(C/NH). lse (B,NH,T) receives each query row's log-sum-exp
 * of the scaled scores (what the backward needs instead of the (B,NH,T,T) matrices).
 * For head sizes that are multiples of 8 the forward and the dQ products of the backward
 * (and the dK/dV products when the head size is also in (32, 64]) are formed as six bf16
 * MFMA products of exact three-way operand splits (fp32 accuracy, as for the GEMMs);
 * GPT2_ATTN_F32_PRODUCTS=fp32 selects fp32 MFMA products. */
int gpt2_k_attention_forward(float* out, float* lse, const float* qkv, int B, int T, int C,
                             int NH, void* stream);

/* [llm.c] 1.8: dqkv (B,T,3C) = gradient of the attention output w.r.t. qkv (written),
 * given dout (B,T,C), the forward's qkv, out and lse. */
int gpt2_k_attention_backward(float* dqkv, const float* dout, const float* qkv,
                              const float* out, const float* lse, int B, int T, int C,
                              int NH, void* stream);

/* [llm.c] 1.13 + 1.14: per row of logits (N rows of V, row stride ld >= V):
 * lse = logsumexp(row); loss = lse - row[target]. Writes losses (N) and lse (N); sets
 * *err_flag (may be NULL) to 1 for a target outside [0,V) and treats it as 0. */
int gpt2_k_crossentropy_forward(float* losses, float* lse, const float* logits,
                                const int32_t* targets, int N, int V, int ld,
                                int32_t* err_flag, void* stream);

/* [llm.c] 1.15: in place, logits[r,v] <- (exp(logits[r,v] - lse[r]) - [v == target[r]]) *
 * dloss for v < V, and 0 for V <= v < ld. */
int gpt2_k_crossentropy_backward(float* logits, const float* lse, const int32_t* targets,
                                 float dloss, int N, int V, int ld, void* stream);

/* [llm.c] 1.13 - 1.15 in one pass: per row as gpt2_k_crossentropy_forward (losses, lse,
 * err_flag), and dlogits[r,v] = (exp(logits[r,v] - lse[r]) - [v == target[r]]) * dloss for
 * v < V, 0 for V <= v < ld, written to dlogits (N x ld, distinct from logits, which are
 * left unchanged). ld must be at most 65536; ERR_ARG otherwise. */
int gpt2_k_crossentropy_fused(float* losses, float* lse, float* dlogits, const float* logits,
                              const int32_t* targets, float dloss, int N, int V, int ld,
                              int32_t* err_flag, void* stream);

/* [llm.c] 1.35 on one row of fp32 logits (device, V entries): *token (device int32) = the
 * index drawn with coin, as gpt2_sample. */
int gpt2_k_sample_mult(int32_t* token, const float* logits, int V, float coin, void* stream);

/* Mean of n floats into *out (device float), summed in a fixed order. */
int gpt2_k_mean(float* out, const float* x, int n, void* stream);

/* [llm.c] 1.26: AdamW over n elements of p, g, m, v (see gpt2_adamw_step). */
int gpt2_k_adamw(float* p, const float* g, float* m, float* v, size_t n, float lr,
                 float beta1, float beta2, float eps, float weight_decay, int t, void* stream);

/* ---------------------------------------------------------------------------------------
 * bf16 forms of the kernels used by GPT2_DTYPE_BF16. Tensors named bf16 are arrays of
 * uint16_t holding the upper half of an IEEE fp32 value; results rounded to bf16 use
 * round to nearest even. Statistics, losses, lse and gradients of parameters stay fp32.
 * ------------------------------------------------------------------------------------- */

/* [llm.c] 1.5, 1.6 (+1.9, 1.10, 1.11 fused) on bf16 operands with fp32 accumulation:
 * C (M,N) = op(A) . op(B). a_trans = 0: A stored (M,K) row-major (row stride lda);
 * 1: A stored (K,M). b_trans = 0: B stored (N,K) (a weight (out,in)); 1: B stored (K,N).
 * epilogue: 0 C = acc + bias; 1 C = acc + bias and C2 = gelu(acc + bias) (tanh form);
 * 2 C = R + acc + bias; 3 C += acc with C fp32 (gradient accumulation); 4 C = acc *
 * gelu'(R). C, C2 and R are bf16 with row stride ldc except for epilogue 3. bias (N, fp32)
 * may be NULL. colsum (M, fp32, may be NULL, needs a_trans) += sums over k of op(A)(m,k).
 * All pointers device, 16-byte aligned; lda, ldb multiples of 8; ldc a multiple of 8 (4
 * for epilogue 3). */
int gpt2_k_gemm_bf16(void* C, uint16_t* C2, const uint16_t* R, const uint16_t* A,
                     const uint16_t* B, const float* bias, float* colsum, int M, int N, int K,
                     int lda, int ldb, int ldc, int a_trans, int b_trans, int epilogue,
                     void* stream);

/* The same GEMM on fp16 operands (uint16_t arrays holding IEEE binary16 values; results
 * rounded to fp16 to nearest even) with fp16 MFMA and fp32 accumulation; arguments and
 * requirements as gpt2_k_gemm_bf16. */
int gpt2_k_gemm_f16(void* C, uint16_t* C2, const uint16_t* R, const uint16_t* A,
                    const uint16_t* B, const float* bias, float* colsum, int M, int N, int K,
                    int lda, int ldb, int ldc, int a_trans, int b_trans, int epilogue,
                    void* stream);

/* [llm.c] 1.7, 1.8 on fp16 qkv, out, dout and dqkv (lse fp32), as the bf16 forms: fp16
 * MFMA products for head sizes that are multiples of 8, P and dS rounded to fp16. */
int gpt2_k_attention_forward_f16(uint16_t* out, float* lse, const uint16_t* qkv, int B, int T,
                                 int C, int NH, void* stream);
int gpt2_k_attention_backward_f16(uint16_t* dqkv, const uint16_t* dout, const uint16_t* qkv,
                                  const uint16_t* out, const float* lse, int B, int T, int C,
                                  int NH, void* stream);

/* [llm.c] 1.1 with a bf16 result: out (B,T,C) bf16 = wte[tok] + wpe[t] (fp32 tables). */
int gpt2_k_encoder_forward_bf16(uint16_t* out, const int32_t* tok, const float* wte,
                                const float* wpe, int B, int T, int C, int V,
                                int32_t* err_flag, void* stream);

/* [llm.c] 1.3 on bf16 rows: x, out (N,C) bf16; w, b, mean, rstd fp32 (mean, rstd may be
 * NULL); statistics in fp32. */
int gpt2_k_layernorm_forward_bf16(uint16_t* out, float* mean, float* rstd, const uint16_t* x,
                                  const float* w, const float* b, int N, int C, void* stream);

/* [llm.c] 1.4 with bf16 dout and x: dx (N,C) fp32 += the LN backward, dx_copy (N,C) bf16
 * (may be NULL) receives the new dx rounded to bf16; dw, db (C) fp32 +=. */
int gpt2_k_layernorm_backward_bf16(float* dx, uint16_t* dx_copy, float* dw, float* db,
                                   const uint16_t* dout, const uint16_t* x, const float* w,
                                   const float* mean, const float* rstd, int N, int C,
                                   void* stream);

/* [llm.c] 1.7, 1.8 with bf16 qkv, out, dout and dqkv (lse fp32). For head sizes that are
 * multiples of 8 (at most 128) the products run on bf16 MFMA with fp32 accumulation: Q, K,
 * V and dO enter as stored, the probabilities P and the score gradients dS are rounded to
 * bf16 where they become MFMA operands, and the softmax statistics stay fp32. Other head
 * sizes widen the bf16 tensors and multiply on fp32 MFMA. */
int gpt2_k_attention_forward_bf16(uint16_t* out, float* lse, const uint16_t* qkv, int B, int T,
                                  int C, int NH, void* stream);
int gpt2_k_attention_backward_bf16(uint16_t* dqkv, const uint16_t* dout, const uint16_t* qkv,
                                   const uint16_t* out, const float* lse, int B, int T, int C,
                                   int NH, void* stream);

/* [llm.c] 1.13 - 1.15 on bf16 logits (row stride ld, a multiple of 4); losses, lse fp32;
 * the backward writes bf16 dlogits in place. */
int gpt2_k_crossentropy_forward_bf16(float* losses, float* lse, const uint16_t* logits,
                                     const int32_t* targets, int N, int V, int ld,
                                     int32_t* err_flag, void* stream);
int gpt2_k_crossentropy_backward_bf16(uint16_t* logits, const float* lse,
                                      const int32_t* targets, float dloss, int N, int V, int ld,
                                      void* stream);

/* AdamW as gpt2_k_adamw, also writing the updated parameters rounded to bf16 into p_bf16
 * (n elements, 8-byte aligned). */
int gpt2_k_adamw_bf16(float* p, uint16_t* p_bf16, const float* g, float* m, float* v, size_t n,
                      float lr, float beta1, float beta2, float eps, float weight_decay, int t,
                      void* stream);

/* dst (n, bf16) = src (n, fp32) rounded to nearest even. */
int gpt2_k_cast_bf16(uint16_t* dst, const float* src, size_t n, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* GPT2_MI355X_H */
