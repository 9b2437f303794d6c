// kernels.h -- launchers of the gfx950 kernels, shared by the model driver and the C ABI.
// Each returns 0 or a negative GPT2_ERR_* code; they only enqueue work on `stream`.
#pragma once

#include "common.h"

namespace gpt2 {

// ----- launch profiler (model.hip) --------------------------------------------------------
// When enabled (gpt2_profile_enable), every kernel launch made through a launcher below is
// bracketed by two HIP events on its stream and tagged with the kernel's name and the
// algorithmic flops and HBM bytes of that launch. Not thread-safe (one caller at a time).
bool profiling_on();
bool profiling_detail();  // names also carry the problem shape (gpt2_profile_enable(2))
struct ProfScope {
  ProfScope(const char* name, double flop, double bytes, hipStream_t s);
  ~ProfScope();
  int rec = -1;
  hipStream_t stream;
};

// ----- GEMM (gemm.hip) ------------------------------------------------------------------
enum Epilogue {
  EPI_STORE = 0,     // C = acc (+ bias)
  EPI_GELU = 1,      // C = acc + bias; C2 = gelu(C)
  EPI_RESID = 2,     // C = R + acc + bias
  EPI_ACCUM = 3,     // C += acc
  EPI_GELU_BWD = 4,  // C = acc * gelu'(R)
};

struct Gemm {
  // logical C(M,N) = A(M,K) . B(K,N)
  const float* A = nullptr;
  int lda = 0;
  bool a_trans = false;  // false: A stored (M,K) row-major; true: stored (K,M)
  const float* B = nullptr;
  int ldb = 0;
  bool b_trans = false;  // false: B stored (N,K) (a weight (out,in)); true: stored (K,N)
  float* C = nullptr;
  int ldc = 0;
  float* C2 = nullptr;        // EPI_GELU
  const float* R = nullptr;   // EPI_RESID (residual) / EPI_GELU_BWD (pre-activation), ldc
  const float* bias = nullptr;
  // optional, only with a_trans: colsum[m] += sum over k of A(m, k), i.e. the column sums
  // of the stored (K, M) operand -- the bias gradient of a weight-gradient GEMM, computed
  // from the A tiles already staged in LDS
  float* colsum = nullptr;
  int M = 0, N = 0, K = 0;
  Epilogue epi = EPI_STORE;
};

// Runs the GEMM; `workspace` (device, `ws_floats` floats) enables a deterministic split of
// K for grids too small to fill the chip (partials reduced in a fixed order). Pass
// nullptr/0 to disable splitting.
int gemm(const Gemm& g, float* workspace, size_t ws_floats, hipStream_t stream);
// floats of workspace gemm() may use for this problem (0 if it will not split)
size_t gemm_workspace_floats(const Gemm& g);

// column sums of x (N rows, C cols, row stride ld) added to out (C), fixed order;
// `partial` needs colsum_partial_floats(N, C) floats.
int colsum_accumulate(float* out, const float* x, int N, int C, int ld, float* partial,
                      hipStream_t stream);
size_t colsum_partial_floats(int N, int C);

// ----- 16-bit GEMM (gemm_bf16.hip) ------------------------------------------------------
// The same products with bf16 or fp16 operands (TS) and fp32 accumulation. C is TS for
// every epilogue except EPI_ACCUM, whose C is fp32 (the master gradients); R and C2 are TS
// with row stride ldc; bias and colsum are fp32.
template <typename TS>
struct GemmHalf {
  const TS* A = nullptr;
  int lda = 0;
  bool a_trans = false;
  const TS* B = nullptr;
  int ldb = 0;
  bool b_trans = false;
  void* C = nullptr;
  int ldc = 0;
  TS* C2 = nullptr;
  const TS* R = nullptr;
  const float* bias = nullptr;
  float* colsum = nullptr;
  int M = 0, N = 0, K = 0;
  Epilogue epi = EPI_STORE;
};
typedef GemmHalf<bf16_t> GemmBf16;
typedef GemmHalf<f16_t> GemmF16;
int gemm_bf16(const GemmBf16& g, float* workspace, size_t ws_floats, hipStream_t stream);
size_t gemm_bf16_workspace_floats(const GemmBf16& g);
int gemm_f16(const GemmF16& g, float* workspace, size_t ws_floats, hipStream_t stream);
size_t gemm_f16_workspace_floats(const GemmF16& g);

// ----- attention (attention.hip) --------------------------------------------------------
// qkv, out, dout, dqkv: fp32 or bf16 storage (overloads; the products run in fp32 either
// way); lse and the scratch buffers are fp32.
int attention_forward(float* out, float* lse, const float* qkv, int B, int T, int C, int NH,
                      hipStream_t stream);
int attention_forward(bf16_t* out, float* lse, const bf16_t* qkv, int B, int T, int C, int NH,
                      hipStream_t stream);
// bf16-MFMA attention (attention_bf16.hip), used by the bf16 overloads when the head size
// is a multiple of 8 (at most 128)
bool attention_bf16_mma_supported(int C, int NH);
// fp32 attention forward with split-operand products on bf16 MFMA (head size a multiple of
// 8, at most 128); the fp32 attention_forward uses it unless GPT2_ATTN_F32_PRODUCTS=fp32
int attention_forward_x6(float* out, float* lse, const float* qkv, int B, int T, int C, int NH,
                         hipStream_t stream);
// dQ = dS K of the fp32 attention backward from the fp32 dS tiles of attn_bwd_dkdv_kernel,
// with split-operand products (same conditions and switch as attention_forward_x6)
int attention_dq_x6(float* dqkv, const float* qkv, const float* ds_scratch, int B, int T, int C,
                    int NH, hipStream_t stream);
// dK, dV (and the fp32 dS tiles for attention_dq_x6) with split-operand products, for head
// sizes in (32, 64] that are multiples of 8; D = rowsum(dout * out) per (b, head, query)
bool attention_dkdv_x6_supported(int C, int NH);
int attention_dkdv_x6(float* dqkv, float* ds_scratch, const float* dout, const float* qkv,
                      const float* lse, const float* D, int B, int T, int C, int NH,
                      hipStream_t stream);
int attention_forward_bf16_mma(bf16_t* out, float* lse, const bf16_t* qkv, int B, int T, int C,
                               int NH, hipStream_t stream);
int attention_backward_bf16_mma(bf16_t* dqkv, const bf16_t* dout, const bf16_t* qkv,
                                const bf16_t* out, const float* lse, float* dscratch,
                                float* ds_scratch, int B, int T, int C, int NH,
                                hipStream_t stream);
int attention_forward_f16_mma(f16_t* out, float* lse, const f16_t* qkv, int B, int T, int C,
                              int NH, hipStream_t stream);
int attention_backward_f16_mma(f16_t* dqkv, const f16_t* dout, const f16_t* qkv,
                               const f16_t* out, const float* lse, float* dscratch,
                               float* ds_scratch, int B, int T, int C, int NH,
                               hipStream_t stream);
// D (B, NH, T) = rowsum over each head's columns of dout * out (fp32 sums)
int attention_rowdot(float* D, const bf16_t* dout, const bf16_t* out, int B, int T, int C,
                     int NH, hipStream_t stream);
int attention_rowdot(float* D, const f16_t* dout, const f16_t* out, int B, int T, int C,
                     int NH, hipStream_t stream);
// `dscratch` needs B*NH*T floats (row dot products of dout and out); `ds_scratch` needs
// attention_ds_scratch_floats(B, T, NH) floats (the causal 64x64 tiles of dS)
size_t attention_ds_scratch_floats(int B, int T, int NH);
int attention_backward(float* dqkv, const float* dout, const float* qkv, const float* out,
                       const float* lse, float* dscratch, float* ds_scratch, int B, int T, int C,
                       int NH, hipStream_t stream);
int attention_backward(bf16_t* dqkv, const bf16_t* dout, const bf16_t* qkv, const bf16_t* out,
                       const float* lse, float* dscratch, float* ds_scratch, int B, int T, int C,
                       int NH, hipStream_t stream);
int attention_forward(f16_t* out, float* lse, const f16_t* qkv, int B, int T, int C, int NH,
                      hipStream_t stream);
int attention_backward(f16_t* dqkv, const f16_t* dout, const f16_t* qkv, const f16_t* out,
                       const float* lse, float* dscratch, float* ds_scratch, int B, int T, int C,
                       int NH, hipStream_t stream);

// ----- memory-bound kernels (stream_ops.hip) ---------------------------------------------
// Activation tensors are fp32 or bf16 (overloads); statistics, losses, the residual-stream
// gradient and all parameter-shaped buffers are fp32.
int encoder_forward(float* out, const int32_t* tok, const float* wte, const float* wpe, int B,
                    int T, int C, int V, int32_t* err_flag, hipStream_t stream);
int encoder_forward(bf16_t* out, const int32_t* tok, const float* wte, const float* wpe, int B,
                    int T, int C, int V, int32_t* err_flag, hipStream_t stream);
int encoder_forward(f16_t* out, const int32_t* tok, const float* wte, const float* wpe, int B,
                    int T, int C, int V, int32_t* err_flag, hipStream_t stream);
// scratch of the embedding backward (sorted tokens, dwte partials):
// encoder_sort_scratch_ints(B*T, V, C) 4-byte words, 16-byte aligned
size_t encoder_sort_scratch_ints(int BT, int V, int C);
int encoder_backward(float* dwte, float* dwpe, const float* dout, const int32_t* tok, int B,
                     int T, int C, int V, int32_t* scratch, hipStream_t stream);
int layernorm_forward(float* out, float* mean, float* rstd, const float* x, const float* w,
                      const float* b, int N, int C, hipStream_t stream);
int layernorm_forward(bf16_t* out, float* mean, float* rstd, const bf16_t* x, const float* w,
                      const float* b, int N, int C, hipStream_t stream);
int layernorm_forward(f16_t* out, float* mean, float* rstd, const f16_t* x, const float* w,
                      const float* b, int N, int C, hipStream_t stream);
// `accumulate_dx`: dx += (true) or dx = (false). `partial` needs
// layernorm_partial_floats(N, C) floats. The bf16 form also writes dx rounded to bf16 into
// dx_copy (if not null).
int layernorm_backward(float* dx, float* dw, float* db, const float* dout, const float* x,
                       const float* w, const float* mean, const float* rstd, int N, int C,
                       bool accumulate_dx, float* partial, hipStream_t stream);
int layernorm_backward(float* dx, bf16_t* dx_copy, float* dw, float* db, const bf16_t* dout,
                       const bf16_t* x, const float* w, const float* mean, const float* rstd,
                       int N, int C, bool accumulate_dx, float* partial, hipStream_t stream);
int layernorm_backward(float* dx, f16_t* dx_copy, float* dw, float* db, const f16_t* dout,
                       const f16_t* x, const float* w, const float* mean, const float* rstd,
                       int N, int C, bool accumulate_dx, float* partial, hipStream_t stream);
size_t layernorm_partial_floats(int N, int C);
int crossentropy_forward(float* losses, float* lse, const float* logits, const int32_t* targets,
                         int N, int V, int ld, int32_t* err_flag, hipStream_t stream);
int crossentropy_forward(float* losses, float* lse, const bf16_t* logits, const int32_t* targets,
                         int N, int V, int ld, int32_t* err_flag, hipStream_t stream);
int crossentropy_backward(float* logits, const float* lse, const int32_t* targets, float dloss,
                          int N, int V, int ld, hipStream_t stream);
int crossentropy_backward(bf16_t* logits, const float* lse, const int32_t* targets, float dloss,
                          int N, int V, int ld, hipStream_t stream);
int crossentropy_forward(float* losses, float* lse, const f16_t* logits, const int32_t* targets,
                         int N, int V, int ld, int32_t* err_flag, hipStream_t stream);
// dscale (device, may be null): the gradient is also multiplied by *dscale (a loss scale)
int crossentropy_backward(f16_t* logits, const float* lse, const int32_t* targets, float dloss,
                          const float* dscale, int N, int V, int ld, hipStream_t stream);
// Cross-entropy forward and backward in one pass (losses, lse and dlogits =
// (softmax - onehot) * dloss [* *dscale], into a buffer apart from the logits); ld at most
// crossentropy_fused_max_ld()
int crossentropy_fused_max_ld();
int crossentropy_fused(float* losses, float* lse, float* dlogits, const float* logits,
                       const int32_t* targets, float dloss, const float* dscale, int N, int V,
                       int ld, int32_t* err_flag, hipStream_t stream);
int crossentropy_fused(float* losses, float* lse, bf16_t* dlogits, const bf16_t* logits,
                       const int32_t* targets, float dloss, const float* dscale, int N, int V,
                       int ld, int32_t* err_flag, hipStream_t stream);
int crossentropy_fused(float* losses, float* lse, f16_t* dlogits, const f16_t* logits,
                       const int32_t* targets, float dloss, const float* dscale, int N, int V,
                       int ld, int32_t* err_flag, hipStream_t stream);
int mean_reduce(float* out, const float* x, int n, hipStream_t stream);
// pbf (may be null): bf16 copy of the updated parameters
int adamw(float* p, const float* g, float* m, float* v, bf16_t* pbf, size_t n, float lr,
          float beta1, float beta2, float eps, float wd, int t, hipStream_t stream);
// fp16 copy of the parameters (pf16), gradients scaled by the loss scale (inv_scale: device
// 1/scale), and a device flag that skips the whole update when nonzero
int adamw(float* p, const float* g, float* m, float* v, f16_t* pf16, size_t n, float lr,
          float beta1, float beta2, float eps, float wd, int t, const float* inv_scale,
          const int32_t* skip, hipStream_t stream);
// *flag = 1 if any of g[0, n) is not finite (flag is not cleared)
int grads_nonfinite(int32_t* flag, const float* g, size_t n, hipStream_t stream);
// dynamic loss scale after a step: state {scale, 1/scale}, counters {overflow flag, good
// steps, last step skipped}; see stream_ops.hip
int loss_scaler_update(float* state, int32_t* counters, int growth_interval, hipStream_t stream);
// dst = src * (*factor) (device factor)
int scale_copy(float* dst, const float* src, const float* factor, size_t n, hipStream_t stream);
int cast_f32_to_bf16(bf16_t* dst, const float* src, size_t n, hipStream_t stream);
int cast_f32_to_f16(f16_t* dst, const float* src, size_t n, hipStream_t stream);
int cast_f16_to_f32(float* dst, const f16_t* src, size_t n, hipStream_t stream);
// ----- sampling (sampling.hip) ------------------------------------------------------------
// out (device int32) = the index drawn from softmax(logits[0, V)) with coin in [0, 1)
int sample_mult(int32_t* out, const float* logits, int V, float coin, hipStream_t stream);
int sample_mult(int32_t* out, const bf16_t* logits, int V, float coin, hipStream_t stream);
int sample_mult(int32_t* out, const f16_t* logits, int V, float coin, hipStream_t stream);
int cast_bf16_to_f32(float* dst, const bf16_t* src, size_t n, hipStream_t stream);

}  // namespace gpt2
