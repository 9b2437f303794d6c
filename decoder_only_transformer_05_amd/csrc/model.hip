// model.hip -- the GPT-2 model object and the C ABI declared in include/gpt2.h.
//
// Memory: parameters, gradients and the two AdamW moments live in one flat device block
// (4 x num_params floats), and every activation, activation gradient and scratch buffer in
// a second flat block sized once for (B, T) -- the "allocate everything up front" design of
// "llm.c 的中文注解-20240421" (sections 1.17 and 1.19). The 16 parameter tensors keep that
// page's order and shapes (section 1.16), so a flat fp32 parameter vector is portable.
//
// Launch sequence: gpt2_forward follows section 1.23, gpt2_backward section 1.25 (in
// reverse layer order), gpt2_adamw_step section 1.26. Every launch goes to the model's one
// stream; the only host synchronisation is the optional 4-byte loss readback.
#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <map>
#include <mutex>
#include <string>
#include <vector>

#include "gpt2.h"
#include "kernels.h"

namespace gpt2 {
static char g_err[512] = "";
static std::mutex g_err_mu;
void set_global_error(const char* fmt, ...) {
  std::lock_guard<std::mutex> lk(g_err_mu);
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
}

// ----- launch profiler -------------------------------------------------------------------
namespace {
struct ProfRec {
  std::string name;
  double flop, bytes;
  hipEvent_t a, b;
};
bool g_prof_on = false;
bool g_prof_detail = false;
std::string g_prof_only;  // record only launches of this name (empty: all)
std::vector<ProfRec> g_prof;
std::vector<hipEvent_t> g_event_pool;  // events reused across profiling sessions
size_t g_event_next = 0;

hipEvent_t next_event() {
  if (g_event_next == g_event_pool.size()) {
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    g_event_pool.push_back(e);
  }
  return g_event_pool[g_event_next++];
}
}  // namespace

bool profiling_on() { return g_prof_on; }
bool profiling_detail() { return g_prof_detail; }

ProfScope::ProfScope(const char* name, double flop, double bytes, hipStream_t s) : stream(s) {
  if (!g_prof_on) return;
  if (!g_prof_only.empty() && g_prof_only != name) return;
  hipEvent_t a = next_event(), b = next_event();
  if (!a || !b) return;
  if (hipEventRecord(a, s) != hipSuccess) return;
  g_prof.push_back(ProfRec{name, flop, bytes, a, b});
  rec = (int)g_prof.size() - 1;
}

ProfScope::~ProfScope() {
  if (rec >= 0) (void)hipEventRecord(g_prof[rec].b, stream);
}
}  // namespace gpt2

using namespace gpt2;

struct gpt2_model {
  int L = 0, C = 0, NH = 0, V = 0, maxT = 0, Vp = 0;
  int dtype = GPT2_DTYPE_FP32;
  int device = 0;
  hipStream_t stream = nullptr;  // NULL = the null stream
  size_t nparams = 0;
  size_t poff[16] = {}, plen[16] = {};
  float* pbuf = nullptr;
  float *params = nullptr, *grads = nullptr, *m = nullptr, *v = nullptr;
  bf16_t* pbf = nullptr;  // GPT2_DTYPE_BF16: bf16 copy of params (GEMM operands)
  f16_t* pf16 = nullptr;  // GPT2_DTYPE_FP16: fp16 copy of params (GEMM operands)
  // GPT2_DTYPE_FP16 loss scaling (device): {scale, 1/scale} and {overflow flag, good steps,
  // last step skipped}; growth interval 0 = fixed scale
  float* d_scale = nullptr;
  int32_t* d_scaler = nullptr;
  int growth_interval = 2000;

  int B = 0, T = 0;
  char* abuf = nullptr;
  // activation tensors: fp32 or bf16 storage by dtype (per layer where noted)
  void *encoded, *ln1, *qkv, *atty, *res2, *ln2, *fch, *fchg, *res3, *lnf, *logits;
  void *dbuf4, *dln, *datty, *dqkv;
  void* dlogits = nullptr;  // loss gradient of the logits, written by the forward (if enabled)
  // fp32 in both modes: statistics, losses, the residual-stream gradient, scratch
  float *ln1_mean, *ln1_rstd, *attn_lse, *ln2_mean, *ln2_rstd, *lnf_mean, *lnf_rstd, *losses,
      *xent_lse;
  float *dres, *attn_D, *attn_dS, *gemm_ws, *ln_ws, *d_loss;
  void* dres_h = nullptr;  // 16-bit dtypes: dres rounded to the activation type (a GEMM operand)
  size_t gemm_ws_floats = 0;
  int32_t *tok, *tgt, *sort_scratch, *d_err;

  bool fwd_targets = false;  // last forward had targets
  bool logits_valid = false; // logits buffer holds logits (not their gradient)
  bool loss_grad_in_forward = true;  // a forward with targets also writes dlogits
  bool dlogits_valid = false;        // dlogits holds the gradient for the last forward
  bool has_grads = false;    // a backward or set_grads happened since build
  char err[512] = "";
};

namespace {

enum { P_WTE, P_WPE, P_LN1W, P_LN1B, P_QKVW, P_QKVB, P_ATTPROJW, P_ATTPROJB, P_LN2W, P_LN2B,
       P_FCW, P_FCB, P_FCPROJW, P_FCPROJB, P_LNFW, P_LNFB };

int fail(gpt2_model* md, int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  if (md) snprintf(md->err, sizeof(md->err), "%s", buf);
  set_global_error("%s", buf);
  return code;
}

// propagate a kernel-launcher error code, copying the launcher's message into the model
int chk(gpt2_model* md, int rc) {
  if (rc) {
    std::lock_guard<std::mutex> lk(g_err_mu);
    snprintf(md->err, sizeof(md->err), "%s", g_err);
  }
  return rc;
}
#define CHK(expr)                    \
  do {                               \
    int rc_ = chk(md, (expr));       \
    if (rc_) return rc_;             \
  } while (0)
#define HIPCHK(expr)                                                                        \
  do {                                                                                      \
    hipError_t e_ = (expr);                                                                 \
    if (e_ != hipSuccess)                                                                   \
      return fail(md, GPT2_ERR_HIP, "%s: %s", #expr, hipGetErrorString(e_));                \
  } while (0)

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

float* P(gpt2_model* md, int k) { return md->params + md->poff[k]; }
float* G(gpt2_model* md, int k) { return md->grads + md->poff[k]; }

// storage of the weights that GEMMs read: the fp32 parameters, or their bf16 copy
template <typename T> const T* W(gpt2_model* md, int k);
template <> const float* W<float>(gpt2_model* md, int k) { return md->params + md->poff[k]; }
template <> const bf16_t* W<bf16_t>(gpt2_model* md, int k) { return md->pbf + md->poff[k]; }
template <> const f16_t* W<f16_t>(gpt2_model* md, int k) { return md->pf16 + md->poff[k]; }

template <typename T> T* act(void* p) { return static_cast<T*>(p); }

template <typename T> struct GemmOf;
template <> struct GemmOf<float> { using type = Gemm; };
template <> struct GemmOf<bf16_t> { using type = GemmBf16; };
template <> struct GemmOf<f16_t> { using type = GemmF16; };

size_t ws_floats(const Gemm& g) { return gemm_workspace_floats(g); }
size_t ws_floats(const GemmBf16& g) { return gemm_bf16_workspace_floats(g); }
size_t ws_floats(const GemmF16& g) { return gemm_f16_workspace_floats(g); }
int run_gemm(gpt2_model* md, const Gemm& g) {
  return gemm(g, md->gemm_ws, md->gemm_ws_floats, md->stream);
}
int run_gemm(gpt2_model* md, const GemmBf16& g) {
  return gemm_bf16(g, md->gemm_ws, md->gemm_ws_floats, md->stream);
}
int run_gemm(gpt2_model* md, const GemmF16& g) {
  return gemm_f16(g, md->gemm_ws, md->gemm_ws_floats, md->stream);
}
bool half_dtype(int dtype) { return dtype == GPT2_DTYPE_BF16 || dtype == GPT2_DTYPE_FP16; }

// the largest split-K workspace any GEMM of a step asks for
template <typename T>
size_t step_gemm_workspace(int BT, int C, int V) {
  using GT = typename GemmOf<T>::type;
  size_t ws = 0;
  const int oc[4] = {3 * C, C, 4 * C, C};
  const int in[4] = {C, C, C, 4 * C};
  for (int k = 0; k < 4; k++) {
    GT w;  // weight gradient (bias gradient fused)
    w.M = oc[k];
    w.N = in[k];
    w.K = BT;
    w.epi = EPI_ACCUM;
    w.a_trans = true;
    w.colsum = reinterpret_cast<float*>(16);  // only its presence matters when measuring
    ws = std::max(ws, ws_floats(w));
    GT d;  // input gradient
    d.M = BT;
    d.N = in[k];
    d.K = oc[k];
    ws = std::max(ws, ws_floats(d));
  }
  const int fn[5] = {3 * C, C, 4 * C, C, V};  // forward: qkv, attproj, fc, fcproj, lm_head
  const int fk[5] = {C, C, C, 4 * C, C};
  for (int k = 0; k < 5; k++) {
    GT f;
    f.M = BT;
    f.N = fn[k];
    f.K = fk[k];
    ws = std::max(ws, ws_floats(f));
  }
  GT d;  // dlnf = dlogits . wte
  d.M = BT;
  d.N = C;
  d.K = V;
  ws = std::max(ws, ws_floats(d));
  GT w;  // dwte += dlogits^T . lnf
  w.M = V;
  w.N = C;
  w.K = BT;
  w.epi = EPI_ACCUM;
  ws = std::max(ws, ws_floats(w));
  return ws;
}

// Carves the activation block for (B, T); with base == nullptr it only measures.
size_t carve_activations(gpt2_model* md, char* base, int B, int T) {
  const size_t L = md->L, C = md->C, NH = md->NH, BT = (size_t)B * T;
  size_t off = 0;
  auto take = [&](size_t bytes) -> char* {
    char* p = base ? base + off : nullptr;
    off += align_up(bytes, 256);
    return p;
  };
  auto F = [&](size_t n) { return reinterpret_cast<float*>(take(n * sizeof(float))); };
  const size_t es = half_dtype(md->dtype) ? 2 : 4;  // activation element size
  auto A = [&](size_t n) { return static_cast<void*>(take(n * es)); };
  md->encoded = A(BT * C);
  md->ln1 = A(L * BT * C);
  md->ln1_mean = F(L * BT);
  md->ln1_rstd = F(L * BT);
  md->qkv = A(L * BT * 3 * C);
  md->atty = A(L * BT * C);
  md->attn_lse = F(L * NH * BT);
  md->res2 = A(L * BT * C);
  md->ln2 = A(L * BT * C);
  md->ln2_mean = F(L * BT);
  md->ln2_rstd = F(L * BT);
  md->fch = A(L * BT * 4 * C);
  md->fchg = A(L * BT * 4 * C);
  md->res3 = A(L * BT * C);
  md->lnf = A(BT * C);
  md->lnf_mean = F(BT);
  md->lnf_rstd = F(BT);
  md->logits = A(BT * md->Vp);
  md->dlogits = md->loss_grad_in_forward && md->Vp <= crossentropy_fused_max_ld()
                    ? A(BT * md->Vp)
                    : nullptr;
  md->losses = F(BT);
  md->xent_lse = F(BT);
  md->dres = F(BT * C);
  md->dres_h = half_dtype(md->dtype) ? static_cast<void*>(take(BT * C * 2)) : nullptr;
  md->dbuf4 = A(BT * 4 * C);
  md->dln = A(BT * C);
  md->datty = A(BT * C);
  md->dqkv = A(BT * 3 * C);
  md->attn_D = F(NH * BT);
  md->attn_dS = F(attention_ds_scratch_floats(B, T, (int)NH));
  const size_t ws = md->dtype == GPT2_DTYPE_BF16
                        ? step_gemm_workspace<bf16_t>((int)BT, (int)C, md->V)
                    : md->dtype == GPT2_DTYPE_FP16
                        ? step_gemm_workspace<f16_t>((int)BT, (int)C, md->V)
                        : step_gemm_workspace<float>((int)BT, (int)C, md->V);
  md->gemm_ws_floats = ws;
  md->gemm_ws = F(ws ? ws : 1);
  md->ln_ws = F(layernorm_partial_floats((int)BT, (int)C));
  md->d_loss = F(1);
  md->tok = reinterpret_cast<int32_t*>(take(BT * sizeof(int32_t)));
  md->tgt = reinterpret_cast<int32_t*>(take(BT * sizeof(int32_t)));
  md->sort_scratch =
      reinterpret_cast<int32_t*>(take(encoder_sort_scratch_ints((int)BT, md->V, (int)C) * sizeof(int32_t)));
  md->d_err = reinterpret_cast<int32_t*>(take(sizeof(int32_t)));
  return off;
}

int alloc_activations(gpt2_model* md, int B, int T) {
  const size_t bytes = carve_activations(md, nullptr, B, T);
  void* p = nullptr;
  if (hipMalloc(&p, bytes) != hipSuccess || !p) {
    (void)hipGetLastError();
    return fail(md, GPT2_ERR_OOM, "cannot allocate %zu bytes of activations for B=%d T=%d",
                bytes, B, T);
  }
  md->abuf = static_cast<char*>(p);
  carve_activations(md, md->abuf, B, T);
  md->B = B;
  md->T = T;
  HIPCHK(hipMemsetAsync(md->d_err, 0, sizeof(int32_t), md->stream));
  return GPT2_OK;
}

int copy_floats(gpt2_model* md, float* dst, const float* src, size_t n, hipMemcpyKind kind) {
  HIPCHK(hipMemcpyAsync(dst, src, n * sizeof(float), kind, md->stream));
  if (kind == hipMemcpyDeviceToHost || kind == hipMemcpyHostToDevice)
    HIPCHK(hipStreamSynchronize(md->stream));
  return GPT2_OK;
}

int check_err_flag(gpt2_model* md) {
  int32_t e = 0;
  HIPCHK(hipMemcpyAsync(&e, md->d_err, sizeof(e), hipMemcpyDeviceToHost, md->stream));
  HIPCHK(hipStreamSynchronize(md->stream));
  if (e) {
    HIPCHK(hipMemsetAsync(md->d_err, 0, sizeof(int32_t), md->stream));
    return fail(md, GPT2_ERR_TOKEN, "a token or target was outside [0, %d)", md->V);
  }
  return GPT2_OK;
}

// ---------------------------------------------------------------------------------------
// the training step, for fp32 (T = float) or bf16 (T = bf16_t) activations
// ---------------------------------------------------------------------------------------
int ln_backward(gpt2_model* md, float* dx, float* dw, float* db, const float* dout,
                const float* x, const float* w, const float* mean, const float* rstd, int BT,
                bool acc) {
  return layernorm_backward(dx, dw, db, dout, x, w, mean, rstd, BT, md->C, acc, md->ln_ws,
                            md->stream);
}
int ln_backward(gpt2_model* md, float* dx, float* dw, float* db, const bf16_t* dout,
                const bf16_t* x, const float* w, const float* mean, const float* rstd, int BT,
                bool acc) {
  return layernorm_backward(dx, static_cast<bf16_t*>(md->dres_h), dw, db, dout, x, w, mean, rstd,
                            BT, md->C, acc, md->ln_ws, md->stream);
}
int ln_backward(gpt2_model* md, float* dx, float* dw, float* db, const f16_t* dout,
                const f16_t* x, const float* w, const float* mean, const float* rstd, int BT,
                bool acc) {
  return layernorm_backward(dx, static_cast<f16_t*>(md->dres_h), dw, db, dout, x, w, mean, rstd,
                            BT, md->C, acc, md->ln_ws, md->stream);
}
// softmax + cross-entropy backward in place; in fp16 the gradient carries the loss scale
int xent_backward(gpt2_model* md, float* logits, float dloss, int BT) {
  return crossentropy_backward(logits, md->xent_lse, md->tgt, dloss, BT, md->V, md->Vp,
                               md->stream);
}
int xent_backward(gpt2_model* md, bf16_t* logits, float dloss, int BT) {
  return crossentropy_backward(logits, md->xent_lse, md->tgt, dloss, BT, md->V, md->Vp,
                               md->stream);
}
int xent_backward(gpt2_model* md, f16_t* logits, float dloss, int BT) {
  return crossentropy_backward(logits, md->xent_lse, md->tgt, dloss, md->d_scale, BT, md->V,
                               md->Vp, md->stream);
}
// the residual-stream gradient as a GEMM operand
template <typename T> const T* dres_operand(gpt2_model* md);
template <> const float* dres_operand<float>(gpt2_model* md) { return md->dres; }
template <> const bf16_t* dres_operand<bf16_t>(gpt2_model* md) {
  return static_cast<const bf16_t*>(md->dres_h);
}
template <> const f16_t* dres_operand<f16_t>(gpt2_model* md) {
  return static_cast<const f16_t*>(md->dres_h);
}

// "llm.c 的中文注解-20240421" section 1.23 (gpt2_forward), on md->tok / md->tgt
template <typename T>
int forward_impl(gpt2_model* md, bool with_targets) {
  using GT = typename GemmOf<T>::type;
  const int B = md->B, T_ = md->T, L = md->L, C = md->C, NH = md->NH, V = md->V, BT = B * T_;
  const size_t NC = (size_t)BT * C;
  hipStream_t s = md->stream;
  T* encoded = act<T>(md->encoded);
  CHK(encoder_forward(encoded, md->tok, P(md, P_WTE), P(md, P_WPE), B, T_, C, V, md->d_err, s));
  for (int l = 0; l < L; l++) {
    const T* x = l == 0 ? encoded : act<T>(md->res3) + (l - 1) * NC;
    T* ln1 = act<T>(md->ln1) + l * NC;
    T* qkv = act<T>(md->qkv) + l * 3 * NC;
    T* atty = act<T>(md->atty) + l * NC;
    T* res2 = act<T>(md->res2) + l * NC;
    T* ln2 = act<T>(md->ln2) + l * NC;
    T* fch = act<T>(md->fch) + l * 4 * NC;
    T* fchg = act<T>(md->fchg) + l * 4 * NC;
    T* res3 = act<T>(md->res3) + l * NC;
    CHK(layernorm_forward(ln1, md->ln1_mean + (size_t)l * BT, md->ln1_rstd + (size_t)l * BT, x,
                          P(md, P_LN1W) + l * C, P(md, P_LN1B) + l * C, BT, C, s));
    GT g;  // qkv = ln1 . Wqkv^T + b
    g.A = ln1;
    g.lda = C;
    g.B = W<T>(md, P_QKVW) + (size_t)l * 3 * C * C;
    g.ldb = C;
    g.C = qkv;
    g.ldc = 3 * C;
    g.bias = P(md, P_QKVB) + (size_t)l * 3 * C;
    g.M = BT;
    g.N = 3 * C;
    g.K = C;
    CHK(run_gemm(md, g));
    CHK(attention_forward(atty, md->attn_lse + (size_t)l * NH * BT, qkv, B, T_, C, NH, s));
    GT pj;  // res2 = x + atty . Wproj^T + b
    pj.A = atty;
    pj.lda = C;
    pj.B = W<T>(md, P_ATTPROJW) + (size_t)l * C * C;
    pj.ldb = C;
    pj.C = res2;
    pj.ldc = C;
    pj.R = x;
    pj.bias = P(md, P_ATTPROJB) + (size_t)l * C;
    pj.M = BT;
    pj.N = C;
    pj.K = C;
    pj.epi = EPI_RESID;
    CHK(run_gemm(md, pj));
    CHK(layernorm_forward(ln2, md->ln2_mean + (size_t)l * BT, md->ln2_rstd + (size_t)l * BT, res2,
                          P(md, P_LN2W) + l * C, P(md, P_LN2B) + l * C, BT, C, s));
    GT fc;  // fch = ln2 . Wfc^T + b, fchg = gelu(fch)
    fc.A = ln2;
    fc.lda = C;
    fc.B = W<T>(md, P_FCW) + (size_t)l * 4 * C * C;
    fc.ldb = C;
    fc.C = fch;
    fc.C2 = fchg;
    fc.ldc = 4 * C;
    fc.bias = P(md, P_FCB) + (size_t)l * 4 * C;
    fc.M = BT;
    fc.N = 4 * C;
    fc.K = C;
    fc.epi = EPI_GELU;
    CHK(run_gemm(md, fc));
    GT fp;  // res3 = res2 + fchg . Wfcproj^T + b
    fp.A = fchg;
    fp.lda = 4 * C;
    fp.B = W<T>(md, P_FCPROJW) + (size_t)l * 4 * C * C;
    fp.ldb = 4 * C;
    fp.C = res3;
    fp.ldc = C;
    fp.R = res2;
    fp.bias = P(md, P_FCPROJB) + (size_t)l * C;
    fp.M = BT;
    fp.N = C;
    fp.K = 4 * C;
    fp.epi = EPI_RESID;
    CHK(run_gemm(md, fp));
  }
  T* lnf = act<T>(md->lnf);
  CHK(layernorm_forward(lnf, md->lnf_mean, md->lnf_rstd, act<T>(md->res3) + (L - 1) * NC,
                        P(md, P_LNFW), P(md, P_LNFB), BT, C, s));
  // tied lm_head: logits = lnf . wte^T, no bias (rows padded to Vp)
  T* logits = act<T>(md->logits);
  GT lm;
  lm.A = lnf;
  lm.lda = C;
  lm.B = W<T>(md, P_WTE);
  lm.ldb = C;
  lm.C = logits;
  lm.ldc = md->Vp;
  lm.M = BT;
  lm.N = V;
  lm.K = C;
  CHK(run_gemm(md, lm));
  if (with_targets) {
    if (md->dlogits && md->loss_grad_in_forward) {
      // losses and, for the backward, d(mean loss)/d(logits) (times the loss scale in fp16)
      CHK(crossentropy_fused(md->losses, md->xent_lse, act<T>(md->dlogits), logits, md->tgt,
                             1.0f / (float)BT,
                             md->dtype == GPT2_DTYPE_FP16 ? md->d_scale : nullptr, BT, V,
                             md->Vp, md->d_err, s));
      md->dlogits_valid = true;
    } else {
      CHK(crossentropy_forward(md->losses, md->xent_lse, logits, md->tgt, BT, V, md->Vp,
                               md->d_err, s));
    }
    CHK(mean_reduce(md->d_loss, md->losses, BT, s));
  }
  return GPT2_OK;
}

// section 1.25 (gpt2_backward): layers in reverse order; parameter gradients accumulate
template <typename T>
int backward_impl(gpt2_model* md) {
  using GT = typename GemmOf<T>::type;
  const int B = md->B, T_ = md->T, L = md->L, C = md->C, NH = md->NH, V = md->V, BT = B * T_;
  const size_t NC = (size_t)BT * C;
  hipStream_t s = md->stream;
  T* dln = act<T>(md->dln);
  // d(mean loss)/d(loss_bt) = 1/(B*T), through softmax + cross-entropy: written by the forward
  // into dlogits, else here, in place of the logits
  T* logits = act<T>(md->logits);
  if (!md->dlogits_valid) CHK(xent_backward(md, logits, 1.0f / (float)BT, BT));
  else logits = act<T>(md->dlogits);
  {
    GT d;  // dlnf = dlogits . wte
    d.A = logits;
    d.lda = md->Vp;
    d.B = W<T>(md, P_WTE);
    d.ldb = C;
    d.b_trans = true;
    d.C = dln;
    d.ldc = C;
    d.M = BT;
    d.N = C;
    d.K = V;
    CHK(run_gemm(md, d));
    GT w;  // dwte += dlogits^T . lnf
    w.A = logits;
    w.lda = md->Vp;
    w.a_trans = true;
    w.B = act<T>(md->lnf);
    w.ldb = C;
    w.b_trans = true;
    w.C = G(md, P_WTE);
    w.ldc = C;
    w.M = V;
    w.N = C;
    w.K = BT;
    w.epi = EPI_ACCUM;
    CHK(run_gemm(md, w));
  }
  CHK(ln_backward(md, md->dres, G(md, P_LNFW), G(md, P_LNFB), dln,
                  act<T>(md->res3) + (L - 1) * NC, P(md, P_LNFW), md->lnf_mean, md->lnf_rstd, BT,
                  false));

  // one linear layer's backward: dinp = dout . W (optionally times gelu'(pre)),
  // dW += dout^T . inp, and db += column sums of dout inside the same weight-gradient GEMM
  auto linear_bwd = [&](T* dinp, const T* gelu_pre, float* dW, float* db, const T* dout,
                        const T* inp, const T* Wt, int in, int out) -> int {
    GT d;
    d.A = dout;
    d.lda = out;
    d.B = Wt;
    d.ldb = in;
    d.b_trans = true;
    d.C = dinp;
    d.ldc = in;
    d.M = BT;
    d.N = in;
    d.K = out;
    if (gelu_pre) {
      d.epi = EPI_GELU_BWD;
      d.R = gelu_pre;
    }
    int rc = run_gemm(md, d);
    if (rc) return rc;
    GT w;
    w.A = dout;
    w.lda = out;
    w.a_trans = true;
    w.B = inp;
    w.ldb = in;
    w.b_trans = true;
    w.C = dW;
    w.ldc = in;
    w.M = out;
    w.N = in;
    w.K = BT;
    w.epi = EPI_ACCUM;
    w.colsum = db;
    return run_gemm(md, w);
  };

  T* dbuf4 = act<T>(md->dbuf4);
  T* datty = act<T>(md->datty);
  T* dqkv = act<T>(md->dqkv);
  const T* dres = dres_operand<T>(md);
  for (int l = L - 1; l >= 0; l--) {
    const T* x = l == 0 ? act<T>(md->encoded) : act<T>(md->res3) + (l - 1) * NC;
    // MLP: residual3 = residual2 + fcproj(gelu(fc(ln2(residual2))))
    CHK(linear_bwd(dbuf4, act<T>(md->fch) + l * 4 * NC, G(md, P_FCPROJW) + (size_t)l * 4 * C * C,
                   G(md, P_FCPROJB) + (size_t)l * C, dres, act<T>(md->fchg) + l * 4 * NC,
                   W<T>(md, P_FCPROJW) + (size_t)l * 4 * C * C, 4 * C, C));
    CHK(linear_bwd(dln, nullptr, G(md, P_FCW) + (size_t)l * 4 * C * C,
                   G(md, P_FCB) + (size_t)l * 4 * C, dbuf4, act<T>(md->ln2) + l * NC,
                   W<T>(md, P_FCW) + (size_t)l * 4 * C * C, C, 4 * C));
    CHK(ln_backward(md, md->dres, G(md, P_LN2W) + (size_t)l * C, G(md, P_LN2B) + (size_t)l * C,
                    dln, act<T>(md->res2) + l * NC, P(md, P_LN2W) + (size_t)l * C,
                    md->ln2_mean + (size_t)l * BT, md->ln2_rstd + (size_t)l * BT, BT, true));
    // attention: residual2 = x + attproj(attention(qkv(ln1(x))))
    CHK(linear_bwd(datty, nullptr, G(md, P_ATTPROJW) + (size_t)l * C * C,
                   G(md, P_ATTPROJB) + (size_t)l * C, dres, act<T>(md->atty) + l * NC,
                   W<T>(md, P_ATTPROJW) + (size_t)l * C * C, C, C));
    CHK(attention_backward(dqkv, datty, act<T>(md->qkv) + l * 3 * NC, act<T>(md->atty) + l * NC,
                           md->attn_lse + (size_t)l * NH * BT, md->attn_D, md->attn_dS, B, T_, C,
                           NH, s));
    CHK(linear_bwd(dln, nullptr, G(md, P_QKVW) + (size_t)l * 3 * C * C,
                   G(md, P_QKVB) + (size_t)l * 3 * C, dqkv, act<T>(md->ln1) + l * NC,
                   W<T>(md, P_QKVW) + (size_t)l * 3 * C * C, C, 3 * C));
    CHK(ln_backward(md, md->dres, G(md, P_LN1W) + (size_t)l * C, G(md, P_LN1B) + (size_t)l * C,
                    dln, x, P(md, P_LN1W) + (size_t)l * C, md->ln1_mean + (size_t)l * BT,
                    md->ln1_rstd + (size_t)l * BT, BT, true));
  }
  CHK(encoder_backward(G(md, P_WTE), G(md, P_WPE), md->dres, md->tok, B, T_, C, V,
                       md->sort_scratch, s));
  return GPT2_OK;
}

}  // namespace

extern "C" {

int gpt2_profile_enable(int on) {
  g_prof.clear();
  g_event_next = 0;
  g_prof_on = on != 0;
  g_prof_detail = on == 2;
  return GPT2_OK;
}

int gpt2_profile_only(const char* name) {
  g_prof_only = name ? name : "";
  return GPT2_OK;
}

int gpt2_profile_summary(char* buf, size_t len) {
  if (!buf || len == 0) return fail(nullptr, GPT2_ERR_ARG, "gpt2_profile_summary: no buffer");
  struct Agg {
    long long n = 0;
    double ms = 0, flop = 0, bytes = 0;
  };
  std::map<std::string, Agg> agg;
  for (auto& r : g_prof) {
    if (hipEventSynchronize(r.b) != hipSuccess)
      return fail(nullptr, GPT2_ERR_HIP, "gpt2_profile_summary: event wait failed");
    float ms = 0.f;
    if (hipEventElapsedTime(&ms, r.a, r.b) != hipSuccess)
      return fail(nullptr, GPT2_ERR_HIP, "gpt2_profile_summary: elapsed time failed");
    Agg& a = agg[r.name];
    a.n++;
    a.ms += ms;
    a.flop += r.flop;
    a.bytes += r.bytes;
  }
  size_t off = 0;
  buf[0] = 0;
  for (auto& kv : agg) {
    int w = snprintf(buf + off, len - off, "%s\t%lld\t%.6f\t%.6e\t%.6e\n", kv.first.c_str(),
                     kv.second.n, kv.second.ms, kv.second.flop, kv.second.bytes);
    if (w < 0 || (size_t)w >= len - off)
      return fail(nullptr, GPT2_ERR_ARG, "gpt2_profile_summary: buffer too small");
    off += (size_t)w;
  }
  return GPT2_OK;
}

const char* gpt2_version(void) {
  return "gpt2-mi355x 0.3 (gfx950; fp32, bf16 and fp16 MFMA)";
}

const char* gpt2_last_error(const gpt2_model* md) { return md ? md->err : gpt2::g_err; }

const char* gpt2_last_global_error(void) { return gpt2::g_err; }

int gpt2_build_ex(gpt2_model** out, int L, int C, int H, int V, int maxT, int dtype, int maxB,
                  int maxTseq, void* stream) {
  if (!out) return fail(nullptr, GPT2_ERR_ARG, "gpt2_build: out is NULL");
  *out = nullptr;
  if (L < 1 || C < 1 || H < 1 || V < 1 || maxT < 1)
    return fail(nullptr, GPT2_ERR_ARG, "gpt2_build: sizes must be >= 1");
  if (C % H || C % 4 || (C / H) % 4 || C / H > 128)
    return fail(nullptr, GPT2_ERR_ARG,
                "gpt2_build: need C %% H == 0, C %% 4 == 0, head size %% 4 == 0 and <= 128 "
                "(C=%d H=%d)", C, H);
  if ((C / 4 + 63) / 64 > 8)
    return fail(nullptr, GPT2_ERR_ARG, "gpt2_build: C=%d above the supported 2048", C);
  if (V >= (1 << 21))  // the embedding backward's token sort keeps tokens in 21 bits
    return fail(nullptr, GPT2_ERR_ARG, "gpt2_build: V=%d at or above the supported 2^21", V);
  if (dtype != GPT2_DTYPE_FP32 && dtype != GPT2_DTYPE_BF16 && dtype != GPT2_DTYPE_FP16)
    return fail(nullptr, GPT2_ERR_ARG, "gpt2_build: dtype %d is not supported", dtype);
  if ((maxB > 0) != (maxTseq > 0) || maxTseq > maxT)
    return fail(nullptr, GPT2_ERR_ARG, "gpt2_build: bad preallocation shape");

  gpt2_model* md = new gpt2_model();
  md->dtype = dtype;
  md->L = L;
  md->C = C;
  md->NH = H;
  md->V = V;
  md->maxT = maxT;
  md->Vp = (int)align_up((size_t)V, 64);
  if (hipGetDevice(&md->device) != hipSuccess) {
    delete md;
    return fail(nullptr, GPT2_ERR_HIP, "gpt2_build: no HIP device");
  }
  const size_t c = C, l = L;
  const size_t sizes[16] = {(size_t)V * c, (size_t)maxT * c, l * c, l * c, l * 3 * c * c,
                            l * 3 * c, l * c * c, l * c, l * c, l * c, l * 4 * c * c, l * 4 * c,
                            l * c * 4 * c, l * c, c, c};
  size_t o = 0;
  for (int k = 0; k < 16; k++) {
    md->poff[k] = o;
    md->plen[k] = sizes[k];
    o += sizes[k];
  }
  md->nparams = o;
  // every tensor offset must keep 16-byte alignment for the vector kernels (fp32 params;
  // 16-bit weight copy in mixed precision)
  const size_t align = half_dtype(dtype) ? 8 : 4;
  for (int k = 0; k < 16; k++)
    if (md->poff[k] % align) {
      delete md;
      return fail(nullptr, GPT2_ERR_ARG, "gpt2_build: tensor %d misaligned", k);
    }
  const size_t stride = align_up(md->nparams, 64);
  void* p = nullptr;
  if (hipMalloc(&p, 4 * stride * sizeof(float)) != hipSuccess || !p) {
    (void)hipGetLastError();
    delete md;
    return fail(nullptr, GPT2_ERR_OOM, "gpt2_build: cannot allocate %zu parameter floats",
                4 * stride);
  }
  md->pbuf = static_cast<float*>(p);
  md->params = md->pbuf;
  md->grads = md->pbuf + stride;
  md->m = md->pbuf + 2 * stride;
  md->v = md->pbuf + 3 * stride;
  md->stream = static_cast<hipStream_t>(stream);  // NULL: the null stream
  if (dtype == GPT2_DTYPE_BF16) {
    void* q = nullptr;
    if (hipMalloc(&q, stride * sizeof(bf16_t)) != hipSuccess || !q) {
      (void)hipGetLastError();
      gpt2_free(md);
      return fail(nullptr, GPT2_ERR_OOM, "gpt2_build: cannot allocate the bf16 weight copy");
    }
    md->pbf = static_cast<bf16_t*>(q);
    if (hipMemsetAsync(md->pbf, 0, stride * sizeof(bf16_t), md->stream) != hipSuccess) {
      gpt2_free(md);
      return fail(nullptr, GPT2_ERR_HIP, "gpt2_build: memset failed");
    }
  }
  if (dtype == GPT2_DTYPE_FP16) {
    // the fp16 weight copy, then 256 bytes for the loss scaler state
    void* q = nullptr;
    if (hipMalloc(&q, stride * sizeof(f16_t) + 256) != hipSuccess || !q) {
      (void)hipGetLastError();
      gpt2_free(md);
      return fail(nullptr, GPT2_ERR_OOM, "gpt2_build: cannot allocate the fp16 weight copy");
    }
    md->pf16 = static_cast<f16_t*>(q);
    md->d_scale = reinterpret_cast<float*>(static_cast<char*>(q) + stride * sizeof(f16_t));
    md->d_scaler = reinterpret_cast<int32_t*>(md->d_scale + 4);
    const float st[2] = {65536.f, 1.f / 65536.f};
    if (hipMemsetAsync(q, 0, stride * sizeof(f16_t) + 256, md->stream) != hipSuccess ||
        hipMemcpyAsync(md->d_scale, st, sizeof(st), hipMemcpyHostToDevice, md->stream) !=
            hipSuccess ||
        hipStreamSynchronize(md->stream) != hipSuccess) {
      gpt2_free(md);
      return fail(nullptr, GPT2_ERR_HIP, "gpt2_build: initialising the fp16 state failed");
    }
  }
  if (hipMemsetAsync(md->pbuf, 0, 4 * stride * sizeof(float), md->stream) != hipSuccess) {
    gpt2_free(md);
    return fail(nullptr, GPT2_ERR_HIP, "gpt2_build: memset failed");
  }
  if (maxB > 0) {
    int rc = alloc_activations(md, maxB, maxTseq);
    if (rc) {
      gpt2_free(md);
      return rc;
    }
  }
  if (hipStreamSynchronize(md->stream) != hipSuccess) {
    gpt2_free(md);
    return fail(nullptr, GPT2_ERR_HIP, "gpt2_build: synchronize failed");
  }
  *out = md;
  return GPT2_OK;
}

int gpt2_build(gpt2_model** out, int L, int C, int H, int V, int maxT) {
  return gpt2_build_ex(out, L, C, H, V, maxT, GPT2_DTYPE_FP32, 0, 0, nullptr);
}

void gpt2_free(gpt2_model* md) {
  if (!md) return;
  if (md->stream) (void)hipStreamSynchronize(md->stream);
  if (md->abuf) (void)hipFree(md->abuf);
  if (md->pbuf) (void)hipFree(md->pbuf);
  if (md->pbf) (void)hipFree(md->pbf);
  if (md->pf16) (void)hipFree(md->pf16);
  delete md;
}

int gpt2_set_stream(gpt2_model* md, void* stream) {
  if (!md) return fail(nullptr, GPT2_ERR_ARG, "NULL model");
  HIPCHK(hipStreamSynchronize(md->stream));
  md->stream = static_cast<hipStream_t>(stream);
  return GPT2_OK;
}

int gpt2_synchronize(gpt2_model* md) {
  if (!md) return fail(nullptr, GPT2_ERR_ARG, "NULL model");
  HIPCHK(hipStreamSynchronize(md->stream));
  if (md->abuf) return check_err_flag(md);
  return GPT2_OK;
}

size_t gpt2_num_params(const gpt2_model* md) { return md ? md->nparams : 0; }

int gpt2_get_config(const gpt2_model* md, int cfg[5]) {
  if (!md || !cfg) return fail(nullptr, GPT2_ERR_ARG, "gpt2_get_config: NULL");
  cfg[0] = md->L;
  cfg[1] = md->C;
  cfg[2] = md->NH;
  cfg[3] = md->V;
  cfg[4] = md->maxT;
  return GPT2_OK;
}

int gpt2_sample(gpt2_model* md, int b, int t, float coin, int32_t* token) {
  if (!md || !token) return fail(md, GPT2_ERR_ARG, "gpt2_sample: NULL");
  if (!md->logits_valid) return fail(md, GPT2_ERR_STATE, "gpt2_sample: logits are not available");
  if (b < 0 || b >= md->B || t < 0 || t >= md->T || !(coin >= 0.f && coin < 1.f))
    return fail(md, GPT2_ERR_ARG, "gpt2_sample: position (%d, %d) or coin %g out of range", b, t,
                (double)coin);
  const size_t row = ((size_t)b * md->T + t) * md->Vp;
  // the token-sort scratch is only used by the backward, which invalidates the logits
  int32_t* out = md->sort_scratch;
  if (md->dtype == GPT2_DTYPE_BF16)
    CHK(sample_mult(out, static_cast<const bf16_t*>(md->logits) + row, md->V, coin, md->stream));
  else if (md->dtype == GPT2_DTYPE_FP16)
    CHK(sample_mult(out, static_cast<const f16_t*>(md->logits) + row, md->V, coin, md->stream));
  else
    CHK(sample_mult(out, static_cast<const float*>(md->logits) + row, md->V, coin, md->stream));
  HIPCHK(hipMemcpyAsync(token, out, sizeof(int32_t), hipMemcpyDeviceToHost, md->stream));
  HIPCHK(hipStreamSynchronize(md->stream));
  return GPT2_OK;
}

int gpt2_param_layout(const gpt2_model* md, size_t off[16], size_t len[16]) {
  if (!md || !off || !len) return fail(nullptr, GPT2_ERR_ARG, "gpt2_param_layout: NULL");
  for (int k = 0; k < 16; k++) {
    off[k] = md->poff[k];
    len[k] = md->plen[k];
  }
  return GPT2_OK;
}

static int xfer(gpt2_model* md, float* dev, const float* src, float* dst, int is_device) {
  if (!md) return fail(nullptr, GPT2_ERR_ARG, "NULL model");
  if (src) return copy_floats(md, dev, src, md->nparams,
                              is_device ? hipMemcpyDeviceToDevice : hipMemcpyHostToDevice);
  if (!dst) return fail(md, GPT2_ERR_ARG, "NULL buffer");
  return copy_floats(md, dst, dev, md->nparams,
                     is_device ? hipMemcpyDeviceToDevice : hipMemcpyDeviceToHost);
}

int gpt2_set_params(gpt2_model* md, const float* src, int src_is_device) {
  if (md && !src) return fail(md, GPT2_ERR_ARG, "gpt2_set_params: NULL source");
  int rc = xfer(md, md ? md->params : nullptr, src, nullptr, src_is_device);
  if (!rc && md->pbf) CHK(cast_f32_to_bf16(md->pbf, md->params, md->nparams, md->stream));
  if (!rc && md->pf16) CHK(cast_f32_to_f16(md->pf16, md->params, md->nparams, md->stream));
  return rc;
}
int gpt2_get_params(gpt2_model* md, float* dst, int dst_is_device) {
  return xfer(md, md ? md->params : nullptr, nullptr, dst, dst_is_device);
}
int gpt2_get_grads(gpt2_model* md, float* dst, int dst_is_device) {
  if (md && md->dtype == GPT2_DTYPE_FP16) {
    // the stored gradients carry the loss scale: hand out grads / scale (exact: a power of 2)
    if (!dst) return fail(md, GPT2_ERR_ARG, "NULL buffer");
    if (dst_is_device) {
      CHK(scale_copy(dst, md->grads, md->d_scale + 1, md->nparams, md->stream));
      HIPCHK(hipStreamSynchronize(md->stream));
      return GPT2_OK;
    }
    float* tmp = nullptr;
    if (hipMalloc(&tmp, md->nparams * sizeof(float)) != hipSuccess) {
      (void)hipGetLastError();
      return fail(md, GPT2_ERR_OOM, "gpt2_get_grads: no memory to unscale the gradients");
    }
    int rc = chk(md, scale_copy(tmp, md->grads, md->d_scale + 1, md->nparams, md->stream));
    if (!rc) rc = copy_floats(md, dst, tmp, md->nparams, hipMemcpyDeviceToHost);
    (void)hipFree(tmp);
    return rc;
  }
  return xfer(md, md ? md->grads : nullptr, nullptr, dst, dst_is_device);
}
int gpt2_set_grads(gpt2_model* md, const float* src, int src_is_device) {
  if (md && !src) return fail(md, GPT2_ERR_ARG, "gpt2_set_grads: NULL source");
  int rc = xfer(md, md ? md->grads : nullptr, src, nullptr, src_is_device);
  if (!rc && md->dtype == GPT2_DTYPE_FP16)  // stored with the loss scale, as backward leaves them
    CHK(scale_copy(md->grads, md->grads, md->d_scale, md->nparams, md->stream));
  if (!rc) md->has_grads = true;
  return rc;
}

int gpt2_set_loss_grad_in_forward(gpt2_model* md, int on) {
  if (!md) return fail(nullptr, GPT2_ERR_ARG, "NULL model");
  if (on && md->abuf && !md->dlogits)
    return fail(md, GPT2_ERR_STATE, "gpt2_set_loss_grad_in_forward: the model was sized "
                "without the gradient buffer (turn it on before the first forward)");
  md->loss_grad_in_forward = on != 0;
  return GPT2_OK;
}

int gpt2_set_loss_scale(gpt2_model* md, float scale, int growth_interval) {
  if (!md) return fail(nullptr, GPT2_ERR_ARG, "NULL model");
  if (md->dtype != GPT2_DTYPE_FP16)
    return fail(md, GPT2_ERR_ARG, "gpt2_set_loss_scale: only fp16 models scale the loss");
  int e = 0;
  if (!(scale >= 1.f && scale <= 16777216.f) || std::frexp(scale, &e) != 0.5f ||
      growth_interval < 0)
    return fail(md, GPT2_ERR_ARG, "gpt2_set_loss_scale: scale must be a power of two in "
                "[1, 2^24] and growth_interval >= 0 (got %g, %d)", (double)scale,
                growth_interval);
  const float st[2] = {scale, 1.f / scale};
  const int32_t cnt[3] = {0, 0, 0};
  HIPCHK(hipMemcpyAsync(md->d_scale, st, sizeof(st), hipMemcpyHostToDevice, md->stream));
  HIPCHK(hipMemcpyAsync(md->d_scaler, cnt, sizeof(cnt), hipMemcpyHostToDevice, md->stream));
  HIPCHK(hipStreamSynchronize(md->stream));
  md->growth_interval = growth_interval;
  return GPT2_OK;
}

int gpt2_get_loss_scale(gpt2_model* md, float* scale, int* last_step_skipped) {
  if (!md) return fail(nullptr, GPT2_ERR_ARG, "NULL model");
  if (md->dtype != GPT2_DTYPE_FP16) {
    if (scale) *scale = 1.f;
    if (last_step_skipped) *last_step_skipped = 0;
    return GPT2_OK;
  }
  float st[2];
  int32_t cnt[3];
  HIPCHK(hipMemcpyAsync(st, md->d_scale, sizeof(st), hipMemcpyDeviceToHost, md->stream));
  HIPCHK(hipMemcpyAsync(cnt, md->d_scaler, sizeof(cnt), hipMemcpyDeviceToHost, md->stream));
  HIPCHK(hipStreamSynchronize(md->stream));
  if (scale) *scale = st[0];
  if (last_step_skipped) *last_step_skipped = cnt[2];
  return GPT2_OK;
}
int gpt2_get_adam_state(gpt2_model* md, float* m, float* v, int dst_is_device) {
  if (!md) return fail(nullptr, GPT2_ERR_ARG, "NULL model");
  if (m) {
    int rc = xfer(md, md->m, nullptr, m, dst_is_device);
    if (rc) return rc;
  }
  if (v) return xfer(md, md->v, nullptr, v, dst_is_device);
  return GPT2_OK;
}

int gpt2_get_losses(gpt2_model* md, float* dst, int dst_is_device) {
  if (!md || !dst) return fail(md, GPT2_ERR_ARG, "gpt2_get_losses: NULL");
  if (!md->fwd_targets) return fail(md, GPT2_ERR_STATE, "no forward with targets yet");
  return copy_floats(md, dst, md->losses, (size_t)md->B * md->T,
                     dst_is_device ? hipMemcpyDeviceToDevice : hipMemcpyDeviceToHost);
}

int gpt2_get_logits(gpt2_model* md, float* dst, int dst_is_device) {
  if (!md || !dst) return fail(md, GPT2_ERR_ARG, "gpt2_get_logits: NULL");
  if (!md->logits_valid) return fail(md, GPT2_ERR_STATE, "logits are not available");
  if (half_dtype(md->dtype)) {  // widen the 16-bit logits through a temporary
    const size_t n = (size_t)md->B * md->T * md->Vp;
    float* tmp = nullptr;
    if (hipMalloc(&tmp, n * sizeof(float)) != hipSuccess) {
      (void)hipGetLastError();
      return fail(md, GPT2_ERR_OOM, "gpt2_get_logits: no memory to widen the logits");
    }
    int rc = chk(md, md->dtype == GPT2_DTYPE_FP16
                         ? cast_f16_to_f32(tmp, static_cast<const f16_t*>(md->logits), n,
                                           md->stream)
                         : cast_bf16_to_f32(tmp, static_cast<const bf16_t*>(md->logits), n,
                                            md->stream));
    hipError_t e = rc ? hipSuccess
                      : hipMemcpy2DAsync(dst, (size_t)md->V * sizeof(float), tmp,
                                         (size_t)md->Vp * sizeof(float),
                                         (size_t)md->V * sizeof(float), (size_t)md->B * md->T,
                                         dst_is_device ? hipMemcpyDeviceToDevice
                                                       : hipMemcpyDeviceToHost,
                                         md->stream);
    if (e == hipSuccess) e = hipStreamSynchronize(md->stream);
    (void)hipFree(tmp);
    if (rc) return rc;
    if (e != hipSuccess) return fail(md, GPT2_ERR_HIP, "gpt2_get_logits: %s", hipGetErrorString(e));
    return GPT2_OK;
  }
  HIPCHK(hipMemcpy2DAsync(dst, (size_t)md->V * sizeof(float), md->logits,
                          (size_t)md->Vp * sizeof(float), (size_t)md->V * sizeof(float),
                          (size_t)md->B * md->T,
                          dst_is_device ? hipMemcpyDeviceToDevice : hipMemcpyDeviceToHost,
                          md->stream));
  HIPCHK(hipStreamSynchronize(md->stream));
  return GPT2_OK;
}

int gpt2_forward(gpt2_model* md, const int32_t* tokens, const int32_t* targets, int B, int T,
                 float* mean_loss) {
  if (!md) return fail(nullptr, GPT2_ERR_ARG, "NULL model");
  if (!tokens) return fail(md, GPT2_ERR_ARG, "gpt2_forward: tokens is NULL");
  if (B < 1 || T < 1 || T > md->maxT)
    return fail(md, GPT2_ERR_ARG, "gpt2_forward: need B >= 1 and 1 <= T <= %d (B=%d T=%d)",
                md->maxT, B, T);
  if (!md->abuf) {
    int rc = alloc_activations(md, B, T);
    if (rc) return rc;
  } else if (B != md->B || T != md->T) {
    return fail(md, GPT2_ERR_SHAPE, "gpt2_forward: model is sized for B=%d T=%d, got B=%d T=%d",
                md->B, md->T, B, T);
  }
  const int BT = B * T;
  hipStream_t s = md->stream;
  md->fwd_targets = false;
  md->logits_valid = false;
  md->dlogits_valid = false;
  HIPCHK(hipMemcpyAsync(md->tok, tokens, BT * sizeof(int32_t), hipMemcpyDeviceToDevice, s));
  if (targets)
    HIPCHK(hipMemcpyAsync(md->tgt, targets, BT * sizeof(int32_t), hipMemcpyDeviceToDevice, s));
  if (md->dtype == GPT2_DTYPE_BF16) CHK(forward_impl<bf16_t>(md, targets != nullptr));
  else if (md->dtype == GPT2_DTYPE_FP16) CHK(forward_impl<f16_t>(md, targets != nullptr));
  else CHK(forward_impl<float>(md, targets != nullptr));
  md->logits_valid = true;
  if (targets) md->fwd_targets = true;
  if (mean_loss) {
    float host = -1.0f;
    if (targets) {
      HIPCHK(hipMemcpyAsync(&host, md->d_loss, sizeof(float), hipMemcpyDeviceToHost, s));
    }
    int rc = check_err_flag(md);  // synchronises the stream
    if (rc) {
      md->fwd_targets = false;
      return rc;
    }
    *mean_loss = host;
  }
  return GPT2_OK;
}

int gpt2_zero_grad(gpt2_model* md) {
  if (!md) return fail(nullptr, GPT2_ERR_ARG, "NULL model");
  HIPCHK(hipMemsetAsync(md->grads, 0, md->nparams * sizeof(float), md->stream));
  return GPT2_OK;
}

int gpt2_backward(gpt2_model* md) {
  if (!md) return fail(nullptr, GPT2_ERR_ARG, "NULL model");
  if (!md->fwd_targets || !md->logits_valid)
    return fail(md, GPT2_ERR_STATE, "gpt2_backward: needs a forward with targets first");
  md->logits_valid = false;
  const int rc = md->dtype == GPT2_DTYPE_BF16   ? backward_impl<bf16_t>(md)
                 : md->dtype == GPT2_DTYPE_FP16 ? backward_impl<f16_t>(md)
                                                : backward_impl<float>(md);
  md->dlogits_valid = false;
  if (rc) return rc;
  md->has_grads = true;
  return GPT2_OK;
}

int gpt2_adamw_step(gpt2_model* md, float lr, float beta1, float beta2, float eps,
                    float weight_decay, int t) {
  if (!md) return fail(nullptr, GPT2_ERR_ARG, "NULL model");
  if (t < 1) return fail(md, GPT2_ERR_ARG, "gpt2_adamw_step: t must be >= 1 (got %d)", t);
  if (!md->has_grads) return fail(md, GPT2_ERR_STATE, "gpt2_adamw_step: no gradients yet");
  if (md->dtype == GPT2_DTYPE_FP16) {
    // skip the update if the scaled gradients overflowed, unscale them otherwise, then let
    // the scaler react
    CHK(grads_nonfinite(md->d_scaler, md->grads, md->nparams, md->stream));
    CHK(adamw(md->params, md->grads, md->m, md->v, md->pf16, md->nparams, lr, beta1, beta2, eps,
              weight_decay, t, md->d_scale + 1, md->d_scaler, md->stream));
    CHK(loss_scaler_update(md->d_scale, md->d_scaler, md->growth_interval, md->stream));
    return GPT2_OK;
  }
  CHK(adamw(md->params, md->grads, md->m, md->v, md->pbf, md->nparams, lr, beta1, beta2, eps,
            weight_decay, t, md->stream));
  return GPT2_OK;
}

// ---------------------------------------------------------------------------------------
// per-kernel entry points
// ---------------------------------------------------------------------------------------
#define KCHK(expr)                                                                          \
  do {                                                                                      \
    int rc_ = (expr);                                                                       \
    if (rc_) return rc_;                                                                    \
  } while (0)

static hipStream_t as_stream(void* s) { return static_cast<hipStream_t>(s); }

int gpt2_k_encoder_forward(float* out, const int32_t* tok, const float* wte, const float* wpe,
                           int B, int T, int C, int V, int32_t* err_flag, void* stream) {
  if (!out || !tok || !wte || !wpe) return fail(nullptr, GPT2_ERR_ARG, "NULL pointer");
  return encoder_forward(out, tok, wte, wpe, B, T, C, V, err_flag, as_stream(stream));
}

int gpt2_k_encoder_backward(float* dwte, float* dwpe, const float* dout, const int32_t* tok,
                            int B, int T, int C, int V, void* stream) {
  if (!dwte || !dwpe || !dout || !tok || B < 1 || T < 1 || V < 1)
    return fail(nullptr, GPT2_ERR_ARG, "bad argument");
  hipStream_t s = as_stream(stream);
  int32_t* scratch = nullptr;
  if (hipMalloc(&scratch, encoder_sort_scratch_ints(B * T, V, C) * sizeof(int32_t)) != hipSuccess)
    return fail(nullptr, GPT2_ERR_OOM, "scratch allocation failed");
  int rc = encoder_backward(dwte, dwpe, dout, tok, B, T, C, V, scratch, s);
  (void)hipStreamSynchronize(s);
  (void)hipFree(scratch);
  return rc;
}

int gpt2_k_layernorm_forward(float* out, float* mean, float* rstd, const float* x,
                             const float* w, const float* b, int N, int C, void* stream) {
  if (!out || !x || !w || !b) return fail(nullptr, GPT2_ERR_ARG, "NULL pointer");
  return layernorm_forward(out, mean, rstd, x, w, b, N, C, as_stream(stream));
}

int gpt2_k_layernorm_backward(float* dx, float* dw, float* db, const float* dout,
                              const float* x, const float* w, const float* mean,
                              const float* rstd, int N, int C, void* stream) {
  if (!dx || !dw || !db || !dout || !x || !w || !mean || !rstd || N < 1 || C < 1)
    return fail(nullptr, GPT2_ERR_ARG, "bad argument");
  hipStream_t s = as_stream(stream);
  float* partial = nullptr;
  if (hipMalloc(&partial, layernorm_partial_floats(N, C) * sizeof(float)) != hipSuccess)
    return fail(nullptr, GPT2_ERR_OOM, "scratch allocation failed");
  int rc = layernorm_backward(dx, dw, db, dout, x, w, mean, rstd, N, C, true, partial, s);
  (void)hipStreamSynchronize(s);
  (void)hipFree(partial);
  return rc;
}

int gpt2_k_matmul_forward(float* out, float* out2, const float* resid, const float* inp,
                          const float* W, const float* bias, int N, int C, int OC, int ld_out,
                          int epilogue, void* stream) {
  if (!out || !inp || !W || N < 1 || C < 1 || OC < 1 || ld_out < OC)
    return fail(nullptr, GPT2_ERR_ARG, "bad argument");
  Gemm g;
  g.A = inp;
  g.lda = C;
  g.B = W;
  g.ldb = C;
  g.C = out;
  g.ldc = ld_out;
  g.bias = bias;
  g.M = N;
  g.N = OC;
  g.K = C;
  if (epilogue == 1) {
    g.epi = EPI_GELU;
    g.C2 = out2;
  } else if (epilogue == 2) {
    g.epi = EPI_RESID;
    g.R = resid;
  } else if (epilogue != 0) {
    return fail(nullptr, GPT2_ERR_ARG, "unknown epilogue %d", epilogue);
  }
  return gemm(g, nullptr, 0, as_stream(stream));
}

// The two GEMMs of gpt2_k_matmul_backward for caller buffers, and the floats of scratch
// they need (split-K partials and column-sum partials).
struct MatmulBackward {
  Gemm d, w;
  size_t ws = 0;
};
static int plan_matmul_backward(MatmulBackward& mb, float* dinp, float* dW, float* dbias,
                                const float* dout, const float* inp, const float* W,
                                const float* gelu_pre, int N, int C, int OC, int ld_dout) {
  if (!dout || N < 1 || C < 1 || OC < 1 || ld_dout < OC || (dinp && !W) || (dW && !inp))
    return fail(nullptr, GPT2_ERR_ARG, "bad argument");
  Gemm& d = mb.d;
  d.A = dout;
  d.lda = ld_dout;
  d.B = W;
  d.ldb = C;
  d.b_trans = true;
  d.C = dinp;
  d.ldc = C;
  d.M = N;
  d.N = C;
  d.K = OC;
  if (gelu_pre) {
    d.epi = EPI_GELU_BWD;
    d.R = gelu_pre;
  }
  Gemm& w = mb.w;
  w.A = dout;
  w.lda = ld_dout;
  w.a_trans = true;
  w.B = inp;
  w.ldb = C;
  w.b_trans = true;
  w.C = dW;
  w.ldc = C;
  w.M = OC;
  w.N = C;
  w.K = N;
  w.epi = EPI_ACCUM;
  w.colsum = dbias;  // bias gradient fused into the weight-gradient GEMM
  size_t ws = std::max(dinp ? gemm_workspace_floats(d) : 0, dW ? gemm_workspace_floats(w) : 0);
  mb.ws = std::max(ws, colsum_partial_floats(N, OC));
  return 0;
}
static int run_matmul_backward(const MatmulBackward& mb, float* dbias, int N, int OC,
                               int ld_dout, float* buf, hipStream_t s) {
  int rc = 0;
  if (mb.d.C) rc = gemm(mb.d, buf, mb.ws, s);
  if (!rc && mb.w.C) rc = gemm(mb.w, buf, mb.ws, s);
  if (!rc && dbias && !mb.w.C) rc = colsum_accumulate(dbias, mb.d.A, N, OC, ld_dout, buf, s);
  return rc;
}

int gpt2_k_matmul_backward(float* dinp, float* dW, float* dbias, const float* dout,
                           const float* inp, const float* W, const float* gelu_pre, int N, int C,
                           int OC, int ld_dout, void* stream) {
  MatmulBackward mb;
  KCHK(plan_matmul_backward(mb, dinp, dW, dbias, dout, inp, W, gelu_pre, N, C, OC, ld_dout));
  hipStream_t s = as_stream(stream);
  float* buf = nullptr;
  if (hipMalloc(&buf, (mb.ws ? mb.ws : 1) * sizeof(float)) != hipSuccess)
    return fail(nullptr, GPT2_ERR_OOM, "scratch allocation failed");
  int rc = run_matmul_backward(mb, dbias, N, OC, ld_dout, buf, s);
  (void)hipStreamSynchronize(s);
  (void)hipFree(buf);
  return rc;
}

// ----- allocation-free matmul backward ----------------------------------------------------
// Scratch of gpt2_k_matmul_backward_noalloc: one static array per device, which each GPU the
// library runs on holds until the process ends. In host code `noalloc_scratch` names a host
// stand-in, not device memory, so kernels only ever receive the device address that
// hipGetSymbolAddress returns for the current device (looked up once per device).
static __device__ __align__(256) float noalloc_scratch[GPT2_NOALLOC_SCRATCH_FLOATS];
static std::mutex g_noalloc_mu;
static float* g_noalloc_ptr[64];

static int noalloc_scratch_ptr(float** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0)
    return fail(nullptr, GPT2_ERR_HIP, "gpt2_k_matmul_backward_noalloc: no current device");
  if (dev >= 64)
    return fail(nullptr, GPT2_ERR_ARG, "gpt2_k_matmul_backward_noalloc: device %d >= 64", dev);
  std::lock_guard<std::mutex> lk(g_noalloc_mu);
  if (!g_noalloc_ptr[dev]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(noalloc_scratch));
    if (e != hipSuccess || !p)
      return fail(nullptr, GPT2_ERR_HIP, "hipGetSymbolAddress(noalloc_scratch) failed: %s",
                  hipGetErrorString(e));
    g_noalloc_ptr[dev] = static_cast<float*>(p);
  }
  *out = g_noalloc_ptr[dev];
  return 0;
}

int gpt2_k_matmul_backward_noalloc(float* dinp, float* dW, float* dbias, const float* dout,
                                   const float* inp, const float* W, const float* gelu_pre, int N,
                                   int C, int OC, int ld_dout, void* stream) {
  MatmulBackward mb;
  KCHK(plan_matmul_backward(mb, dinp, dW, dbias, dout, inp, W, gelu_pre, N, C, OC, ld_dout));
  if (mb.ws > (size_t)GPT2_NOALLOC_SCRATCH_FLOATS)
    return fail(nullptr, GPT2_ERR_ARG,
                "gpt2_k_matmul_backward_noalloc: this problem needs %zu floats of scratch, "
                "above the %d the allocation-free entry point holds (use "
                "gpt2_k_matmul_backward)",
                mb.ws, (int)GPT2_NOALLOC_SCRATCH_FLOATS);
  float* scratch = nullptr;
  KCHK(noalloc_scratch_ptr(&scratch));
  // every scratch location a call reads (split partials, column-sum partials) is written
  // earlier in the same call, so nothing needs clearing between calls
  return run_matmul_backward(mb, dbias, N, OC, ld_dout, scratch, as_stream(stream));
}

int gpt2_k_attention_forward(float* out, float* lse, const float* qkv, int B, int T, int C,
                             int NH, void* stream) {
  if (!out || !lse || !qkv) return fail(nullptr, GPT2_ERR_ARG, "NULL pointer");
  return attention_forward(out, lse, qkv, B, T, C, NH, as_stream(stream));
}

int gpt2_k_attention_backward(float* dqkv, const float* dout, const float* qkv,
                              const float* out, const float* lse, int B, int T, int C, int NH,
                              void* stream) {
  if (!dqkv || !dout || !qkv || !out || !lse || B < 1 || T < 1 || NH < 1)
    return fail(nullptr, GPT2_ERR_ARG, "bad argument");
  hipStream_t s = as_stream(stream);
  float* D = nullptr;
  const size_t nD = (size_t)B * NH * T, nS = attention_ds_scratch_floats(B, T, NH);
  if (hipMalloc(&D, (nD + nS) * sizeof(float)) != hipSuccess)
    return fail(nullptr, GPT2_ERR_OOM, "scratch allocation failed");
  int rc = attention_backward(dqkv, dout, qkv, out, lse, D, D + nD, B, T, C, NH, s);
  (void)hipStreamSynchronize(s);
  (void)hipFree(D);
  return rc;
}

int gpt2_k_crossentropy_forward(float* losses, float* lse, const float* logits,
                                const int32_t* targets, int N, int V, int ld, int32_t* err_flag,
                                void* stream) {
  if (!losses || !lse || !logits || !targets) return fail(nullptr, GPT2_ERR_ARG, "NULL pointer");
  return crossentropy_forward(losses, lse, logits, targets, N, V, ld, err_flag, as_stream(stream));
}

int gpt2_k_crossentropy_backward(float* logits, const float* lse, const int32_t* targets,
                                 float dloss, int N, int V, int ld, void* stream) {
  if (!logits || !lse || !targets) return fail(nullptr, GPT2_ERR_ARG, "NULL pointer");
  return crossentropy_backward(logits, lse, targets, dloss, N, V, ld, as_stream(stream));
}

int gpt2_k_crossentropy_fused(float* losses, float* lse, float* dlogits, const float* logits,
                              const int32_t* targets, float dloss, int N, int V, int ld,
                              int32_t* err_flag, void* stream) {
  if (!losses || !lse || !dlogits || !logits || !targets)
    return fail(nullptr, GPT2_ERR_ARG, "NULL pointer");
  if (dlogits == logits)
    return fail(nullptr, GPT2_ERR_ARG, "gpt2_k_crossentropy_fused: dlogits must not alias logits");
  return crossentropy_fused(losses, lse, dlogits, logits, targets, dloss, nullptr, N, V, ld,
                            err_flag, as_stream(stream));
}

int gpt2_k_sample_mult(int32_t* token, const float* logits, int V, float coin, void* stream) {
  if (!token || !logits || V < 1 || !(coin >= 0.f && coin < 1.f))
    return fail(nullptr, GPT2_ERR_ARG, "gpt2_k_sample_mult: bad argument");
  return sample_mult(token, logits, V, coin, as_stream(stream));
}

int gpt2_k_mean(float* out, const float* x, int n, void* stream) {
  if (!out || !x) return fail(nullptr, GPT2_ERR_ARG, "NULL pointer");
  return mean_reduce(out, x, n, as_stream(stream));
}

int gpt2_k_gemm_bf16(void* C, uint16_t* C2, const uint16_t* R, const uint16_t* A,
                     const uint16_t* B, const float* bias, float* colsum, int M, int N, int K,
                     int lda, int ldb, int ldc, int a_trans, int b_trans, int epilogue,
                     void* stream) {
  if (!C || !A || !B || epilogue < 0 || epilogue > 4)
    return fail(nullptr, GPT2_ERR_ARG, "gpt2_k_gemm_bf16: bad argument");
  GemmBf16 g;
  g.A = A;
  g.lda = lda;
  g.a_trans = a_trans != 0;
  g.B = B;
  g.ldb = ldb;
  g.b_trans = b_trans != 0;
  g.C = C;
  g.ldc = ldc;
  g.C2 = C2;
  g.R = R;
  g.bias = bias;
  g.colsum = colsum;
  g.M = M;
  g.N = N;
  g.K = K;
  g.epi = static_cast<Epilogue>(epilogue);
  hipStream_t s = as_stream(stream);
  const size_t ws = M > 0 && N > 0 && K > 0 ? gemm_bf16_workspace_floats(g) : 0;
  float* buf = nullptr;
  if (ws && hipMalloc(&buf, ws * sizeof(float)) != hipSuccess)
    return fail(nullptr, GPT2_ERR_OOM, "scratch allocation failed");
  int rc = gemm_bf16(g, buf, ws, s);
  if (buf) {
    (void)hipStreamSynchronize(s);
    (void)hipFree(buf);
  }
  return rc;
}

int gpt2_k_gemm_f16(void* C, uint16_t* C2, const uint16_t* R, const uint16_t* A,
                     const uint16_t* B, const float* bias, float* colsum, int M, int N, int K,
                     int lda, int ldb, int ldc, int a_trans, int b_trans, int epilogue,
                     void* stream) {
  if (!C || !A || !B || epilogue < 0 || epilogue > 4)
    return fail(nullptr, GPT2_ERR_ARG, "gpt2_k_gemm_f16: bad argument");
  GemmF16 g;
  g.A = reinterpret_cast<const f16_t*>(A);
  g.lda = lda;
  g.a_trans = a_trans != 0;
  g.B = reinterpret_cast<const f16_t*>(B);
  g.ldb = ldb;
  g.b_trans = b_trans != 0;
  g.C = C;
  g.ldc = ldc;
  g.C2 = reinterpret_cast<f16_t*>(C2);
  g.R = reinterpret_cast<const f16_t*>(R);
  g.bias = bias;
  g.colsum = colsum;
  g.M = M;
  g.N = N;
  g.K = K;
  g.epi = static_cast<Epilogue>(epilogue);
  hipStream_t s = as_stream(stream);
  const size_t ws = M > 0 && N > 0 && K > 0 ? gemm_f16_workspace_floats(g) : 0;
  float* buf = nullptr;
  if (ws && hipMalloc(&buf, ws * sizeof(float)) != hipSuccess)
    return fail(nullptr, GPT2_ERR_OOM, "scratch allocation failed");
  int rc = gemm_f16(g, buf, ws, s);
  if (buf) {
    (void)hipStreamSynchronize(s);
    (void)hipFree(buf);
  }
  return rc;
}

int gpt2_k_encoder_forward_bf16(uint16_t* out, const int32_t* tok, const float* wte,
                                const float* wpe, int B, int T, int C, int V, int32_t* err_flag,
                                void* stream) {
  if (!out || !tok || !wte || !wpe) return fail(nullptr, GPT2_ERR_ARG, "NULL pointer");
  return encoder_forward(out, tok, wte, wpe, B, T, C, V, err_flag, as_stream(stream));
}

int gpt2_k_layernorm_forward_bf16(uint16_t* out, float* mean, float* rstd, const uint16_t* x,
                                  const float* w, const float* b, int N, int C, void* stream) {
  if (!out || !x || !w || !b) return fail(nullptr, GPT2_ERR_ARG, "NULL pointer");
  return layernorm_forward(out, mean, rstd, x, w, b, N, C, as_stream(stream));
}

int gpt2_k_layernorm_backward_bf16(float* dx, uint16_t* dx_copy, float* dw, float* db,
                                   const uint16_t* dout, const uint16_t* x, const float* w,
                                   const float* mean, const float* rstd, int N, int C,
                                   void* stream) {
  if (!dx || !dw || !db || !dout || !x || !w || !mean || !rstd || N < 1 || C < 1)
    return fail(nullptr, GPT2_ERR_ARG, "bad argument");
  hipStream_t s = as_stream(stream);
  float* partial = nullptr;
  if (hipMalloc(&partial, layernorm_partial_floats(N, C) * sizeof(float)) != hipSuccess)
    return fail(nullptr, GPT2_ERR_OOM, "scratch allocation failed");
  int rc = layernorm_backward(dx, dx_copy, dw, db, dout, x, w, mean, rstd, N, C, true, partial,
                              s);
  (void)hipStreamSynchronize(s);
  (void)hipFree(partial);
  return rc;
}

int gpt2_k_attention_forward_bf16(uint16_t* out, float* lse, const uint16_t* qkv, int B, int T,
                                  int C, int NH, void* stream) {
  if (!out || !lse || !qkv) return fail(nullptr, GPT2_ERR_ARG, "NULL pointer");
  return attention_forward(out, lse, qkv, B, T, C, NH, as_stream(stream));
}

int gpt2_k_attention_backward_bf16(uint16_t* dqkv, const uint16_t* dout, const uint16_t* qkv,
                                   const uint16_t* out, const float* lse, int B, int T, int C,
                                   int NH, void* stream) {
  if (!dqkv || !dout || !qkv || !out || !lse || B < 1 || T < 1 || NH < 1)
    return fail(nullptr, GPT2_ERR_ARG, "bad argument");
  hipStream_t s = as_stream(stream);
  float* D = nullptr;
  const size_t nD = (size_t)B * NH * T, nS = attention_ds_scratch_floats(B, T, NH);
  if (hipMalloc(&D, (nD + nS) * sizeof(float)) != hipSuccess)
    return fail(nullptr, GPT2_ERR_OOM, "scratch allocation failed");
  int rc = attention_backward(dqkv, dout, qkv, out, lse, D, D + nD, B, T, C, NH, s);
  (void)hipStreamSynchronize(s);
  (void)hipFree(D);
  return rc;
}

int gpt2_k_attention_forward_f16(uint16_t* out, float* lse, const uint16_t* qkv, int B, int T,
                                 int C, int NH, void* stream) {
  if (!out || !lse || !qkv) return fail(nullptr, GPT2_ERR_ARG, "NULL pointer");
  return attention_forward(reinterpret_cast<f16_t*>(out), lse,
                           reinterpret_cast<const f16_t*>(qkv), B, T, C, NH, as_stream(stream));
}

int gpt2_k_attention_backward_f16(uint16_t* dqkv, const uint16_t* dout, const uint16_t* qkv,
                                  const uint16_t* out, const float* lse, int B, int T, int C,
                                  int NH, void* stream) {
  if (!dqkv || !dout || !qkv || !out || !lse || B < 1 || T < 1 || NH < 1)
    return fail(nullptr, GPT2_ERR_ARG, "bad argument");
  hipStream_t s = as_stream(stream);
  const size_t nD = (size_t)B * NH * T, nS = attention_ds_scratch_floats(B, T, NH);
  float* D = nullptr;
  if (hipMalloc(&D, (nD + nS) * sizeof(float)) != hipSuccess)
    return fail(nullptr, GPT2_ERR_OOM, "scratch allocation failed");
  int rc = attention_backward(reinterpret_cast<f16_t*>(dqkv), reinterpret_cast<const f16_t*>(dout),
                              reinterpret_cast<const f16_t*>(qkv),
                              reinterpret_cast<const f16_t*>(out), lse, D, D + nD, B, T, C, NH, s);
  (void)hipStreamSynchronize(s);
  (void)hipFree(D);
  return rc;
}

int gpt2_k_crossentropy_forward_bf16(float* losses, float* lse, const uint16_t* logits,
                                     const int32_t* targets, int N, int V, int ld,
                                     int32_t* err_flag, void* stream) {
  if (!losses || !lse || !logits || !targets) return fail(nullptr, GPT2_ERR_ARG, "NULL pointer");
  return crossentropy_forward(losses, lse, logits, targets, N, V, ld, err_flag, as_stream(stream));
}

int gpt2_k_crossentropy_backward_bf16(uint16_t* logits, const float* lse,
                                      const int32_t* targets, float dloss, int N, int V, int ld,
                                      void* stream) {
  if (!logits || !lse || !targets) return fail(nullptr, GPT2_ERR_ARG, "NULL pointer");
  return crossentropy_backward(logits, lse, targets, dloss, N, V, ld, as_stream(stream));
}

int gpt2_k_adamw_bf16(float* p, uint16_t* p_bf16, const float* g, float* m, float* v, size_t n,
                      float lr, float beta1, float beta2, float eps, float weight_decay, int t,
                      void* stream) {
  if (!p || !p_bf16 || !g || !m || !v) return fail(nullptr, GPT2_ERR_ARG, "NULL pointer");
  return adamw(p, g, m, v, p_bf16, n, lr, beta1, beta2, eps, weight_decay, t,
               as_stream(stream));
}

int gpt2_k_cast_bf16(uint16_t* dst, const float* src, size_t n, void* stream) {
  if (!dst || !src) return fail(nullptr, GPT2_ERR_ARG, "NULL pointer");
  return cast_f32_to_bf16(dst, src, n, as_stream(stream));
}

int gpt2_k_adamw(float* p, const float* g, float* m, float* v, size_t n, float lr, float beta1,
                 float beta2, float eps, float weight_decay, int t, void* stream) {
  if (!p || !g || !m || !v) return fail(nullptr, GPT2_ERR_ARG, "NULL pointer");
  return adamw(p, g, m, v, nullptr, n, lr, beta1, beta2, eps, weight_decay, t,
               as_stream(stream));
}

}  // extern "C"
