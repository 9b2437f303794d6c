// gpt2_oracle.cpp -- TEST INFRASTRUCTURE, not part of the product.
//
// A plain, slow, single-threaded fp64 CPU implementation of one GPT-2 training step
// (embedding gather, pre-LayerNorm blocks with causal multi-head attention and a GELU MLP,
// tied lm_head with softmax cross-entropy, full backward, AdamW). It exists only to check
// the HIP implementation; it shares no code with it and only the test suite, the smoke
// check and the benchmark's CPU-baseline leg may load it.
//
// Sources (cited by page title and section):
//   [llm.c]  "llm.c 的中文注解-20240421" -- an annotated copy of llm.c's train_gpt2.c,
//            sections 1.1 .. 1.35 (per-layer forward/backward, model driver, AdamW).
//   [np60]   "高能技巧！60 行 NumPy 代码实现一个 GPT" -- GPT in 60 lines of NumPy,
//            sections GELU, Softmax, Layer Norm, Linear, Attention, causal mask.
//
// Everything is fp64. The pages' fp32 loops are approximations of the definitions below.
// Where the pages are silent or disagree, the reading taken is stated at the function.
// Parity status: every function here is pinned by the CPU tests (worked examples printed
// on the pages, closed forms, invariants, an independent library, finite differences);
// whole-model agreement with the pages' own PyTorch reference is unpinned (its data is not
// on the pages).

#include <cmath>
#include <cstdint>
#include <cstdlib>
#include <cstring>
#include <vector>

namespace {

// ---------------------------------------------------------------------------------------
// Per-layer operations.  Row-major tensors; "N" is the number of (b,t) positions.
// ---------------------------------------------------------------------------------------

// [llm.c] 1.1 encoder_forward: out[b,t,:] = wte[tok[b,t],:] + wpe[t,:].
void encoder_forward(double* out, const int* tok, const double* wte, const double* wpe,
                     int B, int T, int C) {
  for (int b = 0; b < B; b++)
    for (int t = 0; t < T; t++) {
      const double* we = wte + (int64_t)tok[b * T + t] * C;
      const double* pe = wpe + (int64_t)t * C;
      double* o = out + ((int64_t)b * T + t) * C;
      for (int c = 0; c < C; c++) o[c] = we[c] + pe[c];
    }
}

// [llm.c] 1.2 encoder_backward: dwte[tok] += dout, dwpe[t] += dout (accumulates).
void encoder_backward(double* dwte, double* dwpe, const double* dout, const int* tok,
                      int B, int T, int C) {
  for (int b = 0; b < B; b++)
    for (int t = 0; t < T; t++) {
      const double* d = dout + ((int64_t)b * T + t) * C;
      double* dw = dwte + (int64_t)tok[b * T + t] * C;
      double* dp = dwpe + (int64_t)t * C;
      for (int c = 0; c < C; c++) {
        dw[c] += d[c];
        dp[c] += d[c];
      }
    }
}

// [llm.c] 1.3 layernorm_forward, [np60] Layer Norm: per row, mean, biased variance,
// rstd = 1/sqrt(var + 1e-5), out = (x - mean) * rstd * w + b.
const double kLnEps = 1e-5;
void layernorm_forward(double* out, double* mean, double* rstd, const double* x,
                       const double* w, const double* bias, int64_t N, int C) {
  for (int64_t n = 0; n < N; n++) {
    const double* xr = x + n * C;
    double m = 0.0;
    for (int c = 0; c < C; c++) m += xr[c];
    m /= C;
    double v = 0.0;
    for (int c = 0; c < C; c++) v += (xr[c] - m) * (xr[c] - m);
    v /= C;
    double s = 1.0 / std::sqrt(v + kLnEps);
    double* o = out + n * C;
    for (int c = 0; c < C; c++) o[c] = (xr[c] - m) * s * w[c] + bias[c];
    if (mean) mean[n] = m;
    if (rstd) rstd[n] = s;
  }
}

// [llm.c] 1.4 layernorm_backward (accumulates into dx, dw, db), written from the
// derivative of y = n * w + b with n = (x - mean) * rstd. Per row, with g = w * dout (the
// gradient reaching n), the Jacobian of n with respect to x is rstd * (I - 1/C - n n^T / C),
// so dx = rstd * (g - <g> - n <g n>), where <.> is the mean over the C channels. The
// affine parameters collect dw = sum over rows of n * dout and db = sum of dout.
void layernorm_backward(double* dx, double* dw, double* db, const double* dout,
                        const double* x, const double* w, const double* mean,
                        const double* rstd, int64_t N, int C) {
  std::vector<double> nrm(C), g(C);
  for (int64_t r = 0; r < N; r++) {
    const double* dy = dout + r * C;
    const double* xr = x + r * C;
    for (int c = 0; c < C; c++) {
      nrm[c] = (xr[c] - mean[r]) * rstd[r];
      g[c] = w[c] * dy[c];
    }
    double g_avg = 0.0, gn_avg = 0.0;
    for (int c = 0; c < C; c++) g_avg += g[c];
    for (int c = 0; c < C; c++) gn_avg += g[c] * nrm[c];
    g_avg /= C;
    gn_avg /= C;
    double* dxr = dx + r * C;
    for (int c = 0; c < C; c++) dxr[c] += rstd[r] * (g[c] - g_avg - nrm[c] * gn_avg);
    for (int c = 0; c < C; c++) {
      dw[c] += nrm[c] * dy[c];
      db[c] += dy[c];
    }
  }
}

// Accumulating product used by the linear layers: for i < mi, j < nj,
//   out[i*ldo + j] += sum over k = 0, 1, ..., K-1 of a(i, k) * b(k, j),
// with a(i, k) = a[i*sa_i + k*sa_k] and b(k, j) = b[k*sb_k + j] (each |.| when ABS).
// Every output adds its K terms one at a time in ascending k, starting from its current
// value: the result is that of the plain triple loop. The outputs of a block (up to 4 x 8)
// are kept in registers while k runs, which only changes how fast this goes.
template <bool ABS>
inline double mag_or_value(double x) { return ABS ? std::fabs(x) : x; }

template <bool ABS, int MI, int NJ>
void block_product_acc(double* out, int64_t ldo, const double* a, int64_t sa_i, int64_t sa_k,
                       const double* b, int64_t sb_k, int64_t K) {
  double acc[MI][NJ];
  for (int i = 0; i < MI; i++)
    for (int j = 0; j < NJ; j++) acc[i][j] = out[i * ldo + j];
  for (int64_t k = 0; k < K; k++) {
    const double* bk = b + k * sb_k;
    for (int i = 0; i < MI; i++) {
      const double ai = mag_or_value<ABS>(a[i * sa_i + k * sa_k]);
      for (int j = 0; j < NJ; j++) acc[i][j] += ai * mag_or_value<ABS>(bk[j]);
    }
  }
  for (int i = 0; i < MI; i++)
    for (int j = 0; j < NJ; j++) out[i * ldo + j] = acc[i][j];
}

// The 4 x 8 block with the accumulators held as eight 4-wide vectors (GCC vector
// extensions: element-wise IEEE multiply and add, so the same operations as above).
typedef double f64x4 __attribute__((vector_size(32)));
typedef long long i64x4 __attribute__((vector_size(32)));
template <bool ABS>
inline f64x4 load4(const double* p) {
  f64x4 v;
  std::memcpy(&v, p, sizeof(v));
  if (ABS) {
    i64x4 bits = (i64x4)v & (i64x4){INT64_MAX, INT64_MAX, INT64_MAX, INT64_MAX};
    v = (f64x4)bits;
  }
  return v;
}
template <bool ABS>
void block_product_acc_4x8(double* out, int64_t ldo, const double* a, int64_t sa_i,
                           int64_t sa_k, const double* b, int64_t sb_k, int64_t K) {
  f64x4 c00 = load4<false>(out), c01 = load4<false>(out + 4);
  f64x4 c10 = load4<false>(out + ldo), c11 = load4<false>(out + ldo + 4);
  f64x4 c20 = load4<false>(out + 2 * ldo), c21 = load4<false>(out + 2 * ldo + 4);
  f64x4 c30 = load4<false>(out + 3 * ldo), c31 = load4<false>(out + 3 * ldo + 4);
  for (int64_t k = 0; k < K; k++) {
    const f64x4 b0 = load4<ABS>(b + k * sb_k), b1 = load4<ABS>(b + k * sb_k + 4);
    const double* ak = a + k * sa_k;
    const double a0 = mag_or_value<ABS>(ak[0]), a1 = mag_or_value<ABS>(ak[sa_i]),
                 a2 = mag_or_value<ABS>(ak[2 * sa_i]), a3 = mag_or_value<ABS>(ak[3 * sa_i]);
    c00 += a0 * b0;
    c01 += a0 * b1;
    c10 += a1 * b0;
    c11 += a1 * b1;
    c20 += a2 * b0;
    c21 += a2 * b1;
    c30 += a3 * b0;
    c31 += a3 * b1;
  }
  std::memcpy(out, &c00, 32);
  std::memcpy(out + 4, &c01, 32);
  std::memcpy(out + ldo, &c10, 32);
  std::memcpy(out + ldo + 4, &c11, 32);
  std::memcpy(out + 2 * ldo, &c20, 32);
  std::memcpy(out + 2 * ldo + 4, &c21, 32);
  std::memcpy(out + 3 * ldo, &c30, 32);
  std::memcpy(out + 3 * ldo + 4, &c31, 32);
}

// the same over an M x N output. k runs in ascending chunks of 256, and within a chunk the
// outputs are visited in panels of 256 columns, blocks of 4 x 8 and single entries at the
// edges, so the operand pieces in use stay in cache. Each output still receives its terms
// in ascending k (a chunk continues from the value the previous chunk stored).
template <bool ABS>
void product_acc(double* out, int64_t ldo, const double* a, int64_t sa_i, int64_t sa_k,
                 const double* b, int64_t sb_k, int64_t M, int64_t N, int64_t K) {
  const int64_t KC = 256, NP = 256;
  const int64_t M4 = M / 4 * 4;
  for (int64_t k0 = 0; k0 < K; k0 += KC) {
    const int64_t kn = K - k0 < KC ? K - k0 : KC;
    const double* ak = a + k0 * sa_k;
    const double* bk = b + k0 * sb_k;
    for (int64_t j0 = 0; j0 < N; j0 += NP) {
      const int64_t j1 = N - j0 < NP ? N : j0 + NP;
      const int64_t j8 = j0 + (j1 - j0) / 8 * 8;
      for (int64_t i = 0; i < M4; i += 4)
        for (int64_t j = j0; j < j8; j += 8)
          block_product_acc_4x8<ABS>(out + i * ldo + j, ldo, ak + i * sa_i, sa_i, sa_k,
                                     bk + j, sb_k, kn);
      for (int64_t i = 0; i < M; i++)
        for (int64_t j = (i < M4 ? j8 : j0); j < j1; j++)
          block_product_acc<ABS, 1, 1>(out + i * ldo + j, ldo, ak + i * sa_i, sa_i, sa_k,
                                       bk + j, sb_k, kn);
    }
  }
}

// [llm.c] 1.5 matmul_forward, [np60] Linear: out(N,OC) = inp(N,C) . W(OC,C)^T + bias(OC).
// W is stored (OC, C) row-major as on the llm.c page (the NumPy page stores [in, out];
// same function). bias may be null. Each output is bias + sum over c in ascending order.
void matmul_forward(double* out, const double* inp, const double* W, const double* bias,
                    int64_t N, int C, int OC) {
  // W^T, so a block of outputs reads contiguous columns
  std::vector<double> WT((size_t)C * OC);
  for (int o = 0; o < OC; o++)
    for (int c = 0; c < C; c++) WT[(size_t)c * OC + o] = W[(size_t)o * C + c];
  for (int64_t n = 0; n < N; n++) {
    double* orow = out + n * OC;
    for (int o = 0; o < OC; o++) orow[o] = bias ? bias[o] : 0.0;
  }
  // out[n][o] += sum_c inp[n][c] * WT[c][o]
  product_acc<false>(out, OC, inp, C, 1, WT.data(), OC, N, OC, C);
}

// [llm.c] 1.6 matmul_backward (accumulates): dinp += dout . W; dW += dout^T . inp;
// dbias += column sums of dout. dbias may be null. Every sum runs in ascending order of
// its index (o for dinp, n for dW and dbias).
void matmul_backward(double* dinp, double* dW, double* dbias, const double* dout,
                     const double* inp, const double* W, int64_t N, int C, int OC) {
  // dinp[n][c] += sum_o dout[n][o] * W[o][c]
  product_acc<false>(dinp, C, dout, OC, 1, W, C, N, C, OC);
  // dW[o][c] += sum_n dout[n][o] * inp[n][c]
  product_acc<false>(dW, C, dout, 1, OC, inp, C, OC, C, N);
  if (dbias)
    for (int64_t n = 0; n < N; n++)
      for (int o = 0; o < OC; o++) dbias[o] += dout[n * OC + o];
}

// [llm.c] 1.7 attention_forward, [np60] Attention + causal mask.
// qkv is (B,T,3C): Q = columns [0,C), K = [C,2C), V = [2C,3C); head h owns columns
// [h*hs, (h+1)*hs) of each. For each (b,h,t): s[t2] = q_t.k_t2 / sqrt(hs) for t2 <= t;
// att[t,:] = softmax over t2 <= t (exactly zero for t2 > t); out_t = sum_t2 att * v_t2.
// Readings: the row max is the true maximum (the page starts it at -10000, marked TODO),
// and the causal mask excludes t2 > t exactly (the NumPy page adds -1e10 instead).
// att (B,NH,T,T) is written when non-null (the backward needs it).
void attention_forward(double* out, double* att, const double* qkv, int B, int T, int C,
                       int NH) {
  const int hs = C / NH;
  const int64_t C3 = 3 * (int64_t)C;
  const double scale = 1.0 / std::sqrt((double)hs);
  std::vector<double> s(T), p(T);
  // one head's q, k, v rows gathered into contiguous (T, hs) arrays (a copy, for locality)
  std::vector<double> Q((size_t)T * hs), K((size_t)T * hs), Vv((size_t)T * hs);
  for (int b = 0; b < B; b++)
    for (int h = 0; h < NH; h++) {
      for (int t = 0; t < T; t++)
        for (int i = 0; i < hs; i++) {
          const double* row = qkv + ((int64_t)b * T + t) * C3 + h * hs + i;
          Q[(size_t)t * hs + i] = row[0];
          K[(size_t)t * hs + i] = row[C];
          Vv[(size_t)t * hs + i] = row[2 * C];
        }
      for (int t = 0; t < T; t++) {
        const double* q = Q.data() + (size_t)t * hs;
        double mx = -INFINITY;
        for (int t2 = 0; t2 <= t; t2++) {
          const double* k = K.data() + (size_t)t2 * hs;
          double dot = 0.0;
          for (int i = 0; i < hs; i++) dot += q[i] * k[i];
          s[t2] = dot * scale;
          if (s[t2] > mx) mx = s[t2];
        }
        double sum = 0.0;
        for (int t2 = 0; t2 <= t; t2++) {
          p[t2] = std::exp(s[t2] - mx);
          sum += p[t2];
        }
        for (int t2 = 0; t2 <= t; t2++) p[t2] /= sum;
        double* o = out + ((int64_t)b * T + t) * C + h * hs;
        for (int i = 0; i < hs; i++) o[i] = 0.0;
        for (int t2 = 0; t2 <= t; t2++) {
          const double* v = Vv.data() + (size_t)t2 * hs;
          for (int i = 0; i < hs; i++) o[i] += p[t2] * v[i];
        }
        if (att) {
          double* a = att + (((int64_t)b * NH + h) * T + t) * T;
          for (int t2 = 0; t2 < T; t2++) a[t2] = t2 <= t ? p[t2] : 0.0;
        }
      }
    }
}

// [llm.c] 1.8 attention_backward (accumulates into dqkv), with the softmax Jacobian
// contracted in closed form: datt[t2] = dout_t . v_t2; dv_t2 += att[t2] * dout_t;
// dpre[t2] = att[t2] * (datt[t2] - sum_t3 att[t3] * datt[t3]);
// dq_t += scale * sum dpre[t2] k_t2; dk_t2 += scale * dpre[t2] q_t.
// The page's double loop over (t2, t3) computes the same dpre (the tests check this).
void attention_backward(double* dqkv, const double* dout, const double* qkv, const double* att,
                        int B, int T, int C, int NH) {
  const int hs = C / NH;
  const int64_t C3 = 3 * (int64_t)C;
  const double scale = 1.0 / std::sqrt((double)hs);
  std::vector<double> datt(T), dpre(T);
  // one head's q, k, v and their gradients in contiguous (T, hs) arrays (gathered from and
  // written back to qkv / dqkv, so every accumulation continues from dqkv's contents)
  const size_t TH = (size_t)T * hs;
  std::vector<double> Q(TH), K(TH), Vv(TH), dQ(TH), dK(TH), dV(TH);
  for (int b = 0; b < B; b++)
    for (int h = 0; h < NH; h++) {
      for (int t = 0; t < T; t++)
        for (int i = 0; i < hs; i++) {
          const int64_t r = ((int64_t)b * T + t) * C3 + h * hs + i;
          const size_t j = (size_t)t * hs + i;
          Q[j] = qkv[r];
          K[j] = qkv[r + C];
          Vv[j] = qkv[r + 2 * C];
          dQ[j] = dqkv[r];
          dK[j] = dqkv[r + C];
          dV[j] = dqkv[r + 2 * C];
        }
      for (int t = 0; t < T; t++) {
        const double* a = att + (((int64_t)b * NH + h) * T + t) * T;
        const double* dO = dout + ((int64_t)b * T + t) * C + h * hs;
        const double* q = Q.data() + (size_t)t * hs;
        double* dq = dQ.data() + (size_t)t * hs;
        double dot_ad = 0.0;
        for (int t2 = 0; t2 <= t; t2++) {
          const double* v = Vv.data() + (size_t)t2 * hs;
          double* dv = dV.data() + (size_t)t2 * hs;
          double acc = 0.0;
          for (int i = 0; i < hs; i++) {
            acc += v[i] * dO[i];
            dv[i] += a[t2] * dO[i];
          }
          datt[t2] = acc;
          dot_ad += a[t2] * acc;
        }
        for (int t2 = 0; t2 <= t; t2++) dpre[t2] = a[t2] * (datt[t2] - dot_ad);
        for (int t2 = 0; t2 <= t; t2++) {
          const double* k = K.data() + (size_t)t2 * hs;
          double* dk = dK.data() + (size_t)t2 * hs;
          for (int i = 0; i < hs; i++) {
            dq[i] += scale * dpre[t2] * k[i];
            dk[i] += scale * dpre[t2] * q[i];
          }
        }
      }
      for (int t = 0; t < T; t++)
        for (int i = 0; i < hs; i++) {
          const int64_t r = ((int64_t)b * T + t) * C3 + h * hs + i;
          const size_t j = (size_t)t * hs + i;
          dqkv[r] = dQ[j];
          dqkv[r + C] = dK[j];
          dqkv[r + 2 * C] = dV[j];
        }
    }
}

// [llm.c] 1.9 gelu_forward, [np60] GELU: the tanh approximation
// gelu(x) = 0.5 x (1 + tanh(sqrt(2/pi) (x + 0.044715 x^3))).
const double kGeluS = 0.79788456080286535587989211986876;  // sqrt(2/pi)
double gelu(double x) { return 0.5 * x * (1.0 + std::tanh(kGeluS * (x + 0.044715 * x * x * x))); }

// [llm.c] 1.10 gelu_backward: d/dx of the tanh form. The page writes sech^2 as
// 1/cosh^2; 1 - tanh^2 is the same function and cannot overflow.
double gelu_grad(double x) {
  double u = kGeluS * (x + 0.044715 * x * x * x);
  double th = std::tanh(u);
  return 0.5 * (1.0 + th) + 0.5 * x * (1.0 - th * th) * kGeluS * (1.0 + 3.0 * 0.044715 * x * x);
}

// log(sum_v exp(z_v)) with the maximum subtracted first ([llm.c] 1.13, [np60] Softmax).
double logsumexp(const double* z, int V) {
  double mx = -INFINITY;
  for (int v = 0; v < V; v++)
    if (z[v] > mx) mx = z[v];
  double sum = 0.0;
  for (int v = 0; v < V; v++) sum += std::exp(z[v] - mx);
  return mx + std::log(sum);
}

// ---------------------------------------------------------------------------------------
// Magnitude envelopes for the parity gates: each parameter gradient is a sum over
// positions of products; these helpers form the same sums over absolute values, which
// bound how much rounding (and error in the summed factors) the sum can carry when its
// terms cancel. They do not take part in the training step itself.
// ---------------------------------------------------------------------------------------

// linear layer ([llm.c] 1.6): dWmag[o,c] += sum_n |dout[n,o]| |inp[n,c]|,
// dbmag[o] += sum_n |dout[n,o]| (dbmag may be null)
void matmul_param_grad_mag(double* dWmag, double* dbmag, const double* dout, const double* inp,
                           int64_t N, int C, int OC) {
  product_acc<true>(dWmag, C, dout, 1, OC, inp, C, OC, C, N);
  if (dbmag)
    for (int64_t n = 0; n < N; n++)
      for (int o = 0; o < OC; o++) dbmag[o] += std::fabs(dout[n * OC + o]);
}

// LayerNorm affine parameters ([llm.c] 1.4): dwmag[c] += sum |n * dout|, dbmag[c] += sum |dout|
void layernorm_param_grad_mag(double* dwmag, double* dbmag, const double* dout,
                              const double* x, const double* mean, const double* rstd,
                              int64_t N, int C) {
  for (int64_t r = 0; r < N; r++)
    for (int c = 0; c < C; c++) {
      const double dy = dout[r * C + c];
      dwmag[c] += std::fabs((x[r * C + c] - mean[r]) * rstd[r] * dy);
      dbmag[c] += std::fabs(dy);
    }
}

// ---------------------------------------------------------------------------------------
// Model layout ([llm.c] 1.16 ParameterTensors, 1.22 sizes): 16 tensors in one flat buffer.
// ---------------------------------------------------------------------------------------
struct Sizes {
  int64_t n[16];
  int64_t off[16];
  int64_t total;
};

Sizes param_sizes(int L, int C, int V, int maxT) {
  Sizes s;
  int64_t c = C, l = L;
  int64_t n[16] = {(int64_t)V * c, (int64_t)maxT * c, l * c,         l * c,
                   l * 3 * c * c,  l * 3 * c,          l * c * c,     l * c,
                   l * c,          l * c,              l * 4 * c * c, l * 4 * c,
                   l * c * 4 * c,  l * c,              c,             c};
  int64_t o = 0;
  for (int i = 0; i < 16; i++) {
    s.n[i] = n[i];
    s.off[i] = o;
    o += n[i];
  }
  s.total = o;
  return s;
}

enum { WTE, WPE, LN1W, LN1B, QKVW, QKVB, ATTPROJW, ATTPROJB, LN2W, LN2B, FCW, FCB,
       FCPROJW, FCPROJB, LNFW, LNFB };

}  // namespace

extern "C" {

// ----- op-level entry points (for the pins and for per-kernel parity) -------------------
void oracle_encoder_forward(double* out, const int* tok, const double* wte,
                            const double* wpe, int B, int T, int C) {
  encoder_forward(out, tok, wte, wpe, B, T, C);
}
void oracle_encoder_backward(double* dwte, double* dwpe, const double* dout, const int* tok,
                             int B, int T, int C) {
  encoder_backward(dwte, dwpe, dout, tok, B, T, C);
}
void oracle_layernorm_forward(double* out, double* mean, double* rstd, const double* x,
                              const double* w, const double* b, int64_t N, int C) {
  layernorm_forward(out, mean, rstd, x, w, b, N, C);
}
void oracle_layernorm_backward(double* dx, double* dw, double* db, const double* dout,
                               const double* x, const double* w, const double* mean,
                               const double* rstd, int64_t N, int C) {
  layernorm_backward(dx, dw, db, dout, x, w, mean, rstd, N, C);
}
void oracle_matmul_forward(double* out, const double* inp, const double* W, const double* b,
                           int64_t N, int C, int OC) {
  matmul_forward(out, inp, W, b, N, C, OC);
}
void oracle_matmul_backward(double* dinp, double* dW, double* db, const double* dout,
                            const double* inp, const double* W, int64_t N, int C, int OC) {
  matmul_backward(dinp, dW, db, dout, inp, W, N, C, OC);
}
void oracle_attention_forward(double* out, double* att, const double* qkv, int B, int T,
                              int C, int NH) {
  attention_forward(out, att, qkv, B, T, C, NH);
}
void oracle_attention_backward(double* dqkv, const double* dout, const double* qkv,
                               const double* att, int B, int T, int C, int NH) {
  attention_backward(dqkv, dout, qkv, att, B, T, C, NH);
}

// The llm.c page's own form of the softmax backward (section 1.8): for each query row,
// dpre[t3] += att[t2] * ([t2 == t3] - att[t3]) * datt[t2] over all t2, t3 <= t, i.e. the
// explicit Jacobian, O(T^3) per head. Used only to show it equals the closed form above.
void oracle_softmax_jacobian_backward(double* dpre, const double* att, const double* datt,
                                      int T) {
  for (int t = 0; t < T; t++) {
    const double* a = att + (int64_t)t * T;
    const double* da = datt + (int64_t)t * T;
    double* dp = dpre + (int64_t)t * T;
    for (int t2 = 0; t2 <= t; t2++)
      for (int t3 = 0; t3 <= t; t3++) {
        double ind = t2 == t3 ? 1.0 : 0.0;
        dp[t3] += a[t2] * (ind - a[t3]) * da[t2];
      }
  }
}
// closed form of the same: dpre[t2] += att[t2] * (datt[t2] - sum_t3 att[t3] datt[t3])
void oracle_softmax_closed_backward(double* dpre, const double* att, const double* datt,
                                    int T) {
  for (int t = 0; t < T; t++) {
    const double* a = att + (int64_t)t * T;
    const double* da = datt + (int64_t)t * T;
    double* dp = dpre + (int64_t)t * T;
    double dot = 0.0;
    for (int t2 = 0; t2 <= t; t2++) dot += a[t2] * da[t2];
    for (int t2 = 0; t2 <= t; t2++) dp[t2] += a[t2] * (da[t2] - dot);
  }
}

void oracle_gelu_forward(double* out, const double* x, int64_t n) {
  for (int64_t i = 0; i < n; i++) out[i] = gelu(x[i]);
}
// accumulates dx += gelu'(x) * dout ([llm.c] 1.10)
void oracle_gelu_backward(double* dx, const double* x, const double* dout, int64_t n) {
  for (int64_t i = 0; i < n; i++) dx[i] += gelu_grad(x[i]) * dout[i];
}
// [llm.c] 1.13 softmax_forward, [np60] Softmax: probs = exp(z - max) / sum.
void oracle_softmax_forward(double* probs, const double* logits, int64_t N, int V) {
  for (int64_t n = 0; n < N; n++) {
    const double* z = logits + n * V;
    double lse = logsumexp(z, V);
    for (int v = 0; v < V; v++) probs[n * V + v] = std::exp(z[v] - lse);
  }
}
// [llm.c] 1.14 crossentropy_forward: loss = -log softmax(z)[target], evaluated as
// logsumexp(z) - z[target] (equal in exact arithmetic; the NumPy page names log-softmax
// as the stable form). Returns nonzero if a target is outside [0, V).
int oracle_crossentropy_forward(double* losses, const double* logits, const int* targets,
                                int64_t N, int V) {
  for (int64_t n = 0; n < N; n++) {
    int y = targets[n];
    if (y < 0 || y >= V) return 1;
    const double* z = logits + n * V;
    losses[n] = logsumexp(z, V) - z[y];
  }
  return 0;
}
// [llm.c] 1.15 crossentropy_softmax_backward (accumulates):
// dlogits += (softmax(z) - onehot(target)) * dloss.
void oracle_crossentropy_softmax_backward(double* dlogits, const double* logits,
                                          const int* targets, const double* dlosses,
                                          int64_t N, int V) {
  for (int64_t n = 0; n < N; n++) {
    const double* z = logits + n * V;
    double lse = logsumexp(z, V);
    for (int v = 0; v < V; v++) {
      double p = std::exp(z[v] - lse);
      dlogits[n * V + v] += (p - (v == targets[n] ? 1.0 : 0.0)) * dlosses[n];
    }
  }
}

// [llm.c] 1.35 sample_mult: walk the cumulative distribution of probs (which sum to 1) and
// return the first index whose cumulative value exceeds coin (coin in [0, 1)); if rounding
// leaves every cumulative value at or below coin, the last index.
int oracle_sample_mult(const double* probs, int n, double coin) {
  double cdf = 0.0;
  for (int i = 0; i < n; i++) {
    cdf += probs[i];
    if (coin < cdf) return i;
  }
  return n - 1;
}

// [llm.c] 1.26 gpt2_update (AdamW, as torch.optim.AdamW which the page cites):
// m = b1 m + (1-b1) g; v = b2 v + (1-b2) g^2; mhat = m/(1-b1^t); vhat = v/(1-b2^t);
// p -= lr (mhat / (sqrt(vhat) + eps) + wd p), with p the value before this update.
void oracle_adamw(int64_t n, double* p, const double* g, double* m, double* v, double lr,
                  double b1, double b2, double eps, double wd, int t) {
  const double c1 = 1.0 - std::pow(b1, t), c2 = 1.0 - std::pow(b2, t);
  for (int64_t i = 0; i < n; i++) {
    m[i] = b1 * m[i] + (1.0 - b1) * g[i];
    v[i] = b2 * v[i] + (1.0 - b2) * g[i] * g[i];
    double mhat = m[i] / c1, vhat = v[i] / c2;
    p[i] -= lr * (mhat / (std::sqrt(vhat) + eps) + wd * p[i]);
  }
}

int64_t oracle_num_params(int L, int C, int V, int maxT) {
  return param_sizes(L, C, V, maxT).total;
}

// One training step's forward and (if grads != null) backward ([llm.c] 1.23 gpt2_forward,
// 1.25 gpt2_backward). params: flat fp64 in the 16-tensor order. tokens/targets: (B,T).
// Outputs (each may be null): mean_loss, losses (B*T), logits (B*T*V), grads (flat,
// overwritten, not accumulated). Returns 0, or 1 for bad shapes/tokens.
// grad_mag (flat, like grads) and logit_mag (B*T*V), each optional, receive the sums over
// absolute values of the final contraction that forms each gradient entry and each logit
// (see matmul_param_grad_mag); grad_mag needs grads.
int oracle_gpt2_step_mag(int L, int C, int NH, int V, int maxT, const double* params,
                         const int* tokens, const int* targets, int B, int T, double* mean_loss,
                         double* losses_out, double* logits_out, double* grads,
                         double* grad_mag, double* logit_mag) {
  if (L < 1 || C < 1 || NH < 1 || C % NH || V < 1 || B < 1 || T < 1 || T > maxT) return 1;
  for (int64_t i = 0; i < (int64_t)B * T; i++) {
    if (tokens[i] < 0 || tokens[i] >= V) return 1;
    if (targets && (targets[i] < 0 || targets[i] >= V)) return 1;
  }
  if (grads && !targets) return 1;
  if (grad_mag && !grads) return 1;
  const Sizes S = param_sizes(L, C, V, maxT);
  const int64_t N = (int64_t)B * T, NC = N * C;
  auto P = [&](int k) { return params + S.off[k]; };

  // ---- forward, keeping what the backward needs (per layer, as [llm.c] 1.18) ----
  std::vector<double> encoded(NC);
  std::vector<double> ln1((size_t)L * NC), ln1m((size_t)L * N), ln1r((size_t)L * N);
  std::vector<double> qkv((size_t)L * 3 * NC), atty((size_t)L * NC);
  std::vector<double> att((size_t)L * B * NH * T * T);
  std::vector<double> res2((size_t)L * NC), ln2((size_t)L * NC), ln2m((size_t)L * N),
      ln2r((size_t)L * N);
  std::vector<double> fch((size_t)L * 4 * NC), fchg((size_t)L * 4 * NC);
  std::vector<double> res3((size_t)L * NC);
  std::vector<double> lnf(NC), lnfm(N), lnfr(N);
  std::vector<double> logits((size_t)N * V);
  std::vector<double> tmp(NC);

  encoder_forward(encoded.data(), tokens, P(WTE), P(WPE), B, T, C);
  for (int l = 0; l < L; l++) {
    const double* x = l == 0 ? encoded.data() : res3.data() + (l - 1) * NC;
    double* l_ln1 = ln1.data() + l * NC;
    double* l_qkv = qkv.data() + l * 3 * NC;
    double* l_atty = atty.data() + l * NC;
    double* l_att = att.data() + (size_t)l * B * NH * T * T;
    double* l_res2 = res2.data() + l * NC;
    double* l_ln2 = ln2.data() + l * NC;
    double* l_fch = fch.data() + l * 4 * NC;
    double* l_fchg = fchg.data() + l * 4 * NC;
    double* l_res3 = res3.data() + l * NC;
    layernorm_forward(l_ln1, ln1m.data() + l * N, ln1r.data() + l * N, x, P(LN1W) + l * C,
                      P(LN1B) + l * C, N, C);
    matmul_forward(l_qkv, l_ln1, P(QKVW) + (int64_t)l * 3 * C * C, P(QKVB) + l * 3 * C, N, C,
                   3 * C);
    attention_forward(l_atty, l_att, l_qkv, B, T, C, NH);
    matmul_forward(tmp.data(), l_atty, P(ATTPROJW) + (int64_t)l * C * C, P(ATTPROJB) + l * C,
                   N, C, C);
    for (int64_t i = 0; i < NC; i++) l_res2[i] = x[i] + tmp[i];  // [llm.c] 1.11 residual
    layernorm_forward(l_ln2, ln2m.data() + l * N, ln2r.data() + l * N, l_res2,
                      P(LN2W) + l * C, P(LN2B) + l * C, N, C);
    matmul_forward(l_fch, l_ln2, P(FCW) + (int64_t)l * 4 * C * C, P(FCB) + l * 4 * C, N, C,
                   4 * C);
    for (int64_t i = 0; i < 4 * NC; i++) l_fchg[i] = gelu(l_fch[i]);
    matmul_forward(tmp.data(), l_fchg, P(FCPROJW) + (int64_t)l * 4 * C * C,
                   P(FCPROJB) + l * C, N, 4 * C, C);
    for (int64_t i = 0; i < NC; i++) l_res3[i] = l_res2[i] + tmp[i];
  }
  const double* xL = res3.data() + (L - 1) * NC;
  layernorm_forward(lnf.data(), lnfm.data(), lnfr.data(), xL, P(LNFW), P(LNFB), N, C);
  // tied lm_head: logits = lnf . wte^T, no bias ([llm.c] 1.23; [np60] "x @ wte.T")
  matmul_forward(logits.data(), lnf.data(), P(WTE), nullptr, N, C, V);
  if (logits_out) std::memcpy(logits_out, logits.data(), sizeof(double) * N * V);
  if (logit_mag) {
    std::vector<double> alnf(NC), awte((size_t)V * C);
    for (int64_t i = 0; i < NC; i++) alnf[i] = std::fabs(lnf[i]);
    for (int64_t i = 0; i < (int64_t)V * C; i++) awte[i] = std::fabs(P(WTE)[i]);
    matmul_forward(logit_mag, alnf.data(), awte.data(), nullptr, N, C, V);
  }

  if (!targets) {
    if (mean_loss) *mean_loss = -1.0;  // [llm.c] 1.23: no targets, no loss
    return 0;
  }
  std::vector<double> losses(N);
  oracle_crossentropy_forward(losses.data(), logits.data(), targets, N, V);
  double mean = 0.0;
  for (int64_t i = 0; i < N; i++) mean += losses[i];
  mean /= (double)N;
  if (mean_loss) *mean_loss = mean;
  if (losses_out) std::memcpy(losses_out, losses.data(), sizeof(double) * N);
  if (!grads) return 0;

  // ---- backward ([llm.c] 1.25): reverse order, activation grads one layer at a time ----
  std::memset(grads, 0, sizeof(double) * S.total);
  auto G = [&](int k) { return grads + S.off[k]; };
  std::vector<double> dlosses(N, 1.0 / (double)N);  // d(mean)/d(loss_bt)
  std::vector<double> dlogits((size_t)N * V, 0.0);
  oracle_crossentropy_softmax_backward(dlogits.data(), logits.data(), targets, dlosses.data(),
                                       N, V);
  std::vector<double> dlnf(NC, 0.0);
  matmul_backward(dlnf.data(), G(WTE), nullptr, dlogits.data(), lnf.data(), P(WTE), N, C, V);
  double* M = grad_mag;  // envelopes, or null
  if (M) {
    std::memset(M, 0, sizeof(double) * S.total);
    matmul_param_grad_mag(M + S.off[WTE], nullptr, dlogits.data(), lnf.data(), N, C, V);
  }
  dlogits.clear();
  dlogits.shrink_to_fit();
  // dres holds d(loss)/d(residual stream) entering the layer being processed
  std::vector<double> dres(NC, 0.0);
  layernorm_backward(dres.data(), G(LNFW), G(LNFB), dlnf.data(), xL, P(LNFW), lnfm.data(),
                     lnfr.data(), N, C);
  if (M)
    layernorm_param_grad_mag(M + S.off[LNFW], M + S.off[LNFB], dlnf.data(), xL, lnfm.data(),
                             lnfr.data(), N, C);
  std::vector<double> dfchg(4 * NC), dfch(4 * NC), dln(NC), datty(NC), dqkv(3 * NC);
  for (int l = L - 1; l >= 0; l--) {
    const double* x = l == 0 ? encoded.data() : res3.data() + (l - 1) * NC;
    // residual3 = residual2 + fcproj: both receive dres ([llm.c] 1.12 residual_backward)
    std::fill(dfchg.begin(), dfchg.end(), 0.0);
    matmul_backward(dfchg.data(), G(FCPROJW) + (int64_t)l * 4 * C * C, G(FCPROJB) + l * C,
                    dres.data(), fchg.data() + l * 4 * NC, P(FCPROJW) + (int64_t)l * 4 * C * C,
                    N, 4 * C, C);
    if (M)
      matmul_param_grad_mag(M + S.off[FCPROJW] + (int64_t)l * 4 * C * C,
                            M + S.off[FCPROJB] + l * C, dres.data(), fchg.data() + l * 4 * NC,
                            N, 4 * C, C);
    std::fill(dfch.begin(), dfch.end(), 0.0);
    oracle_gelu_backward(dfch.data(), fch.data() + l * 4 * NC, dfchg.data(), 4 * NC);
    std::fill(dln.begin(), dln.end(), 0.0);
    matmul_backward(dln.data(), G(FCW) + (int64_t)l * 4 * C * C, G(FCB) + l * 4 * C,
                    dfch.data(), ln2.data() + l * NC, P(FCW) + (int64_t)l * 4 * C * C, N, C,
                    4 * C);
    if (M)
      matmul_param_grad_mag(M + S.off[FCW] + (int64_t)l * 4 * C * C, M + S.off[FCB] + l * 4 * C,
                            dfch.data(), ln2.data() + l * NC, N, C, 4 * C);
    if (M)
      layernorm_param_grad_mag(M + S.off[LN2W] + l * C, M + S.off[LN2B] + l * C, dln.data(),
                               res2.data() + l * NC, ln2m.data() + l * N, ln2r.data() + l * N,
                               N, C);
    // dres now also collects the ln2 branch: d residual2 = d residual3 + LN2 backward
    layernorm_backward(dres.data(), G(LN2W) + l * C, G(LN2B) + l * C, dln.data(),
                       res2.data() + l * NC, P(LN2W) + l * C, ln2m.data() + l * N,
                       ln2r.data() + l * N, N, C);
    // residual2 = x + attproj: both receive d residual2
    std::fill(datty.begin(), datty.end(), 0.0);
    matmul_backward(datty.data(), G(ATTPROJW) + (int64_t)l * C * C, G(ATTPROJB) + l * C,
                    dres.data(), atty.data() + l * NC, P(ATTPROJW) + (int64_t)l * C * C, N, C,
                    C);
    if (M)
      matmul_param_grad_mag(M + S.off[ATTPROJW] + (int64_t)l * C * C, M + S.off[ATTPROJB] + l * C,
                            dres.data(), atty.data() + l * NC, N, C, C);
    std::fill(dqkv.begin(), dqkv.end(), 0.0);
    attention_backward(dqkv.data(), datty.data(), qkv.data() + l * 3 * NC,
                       att.data() + (size_t)l * B * NH * T * T, B, T, C, NH);
    std::fill(dln.begin(), dln.end(), 0.0);
    matmul_backward(dln.data(), G(QKVW) + (int64_t)l * 3 * C * C, G(QKVB) + l * 3 * C,
                    dqkv.data(), ln1.data() + l * NC, P(QKVW) + (int64_t)l * 3 * C * C, N, C,
                    3 * C);
    if (M) {
      matmul_param_grad_mag(M + S.off[QKVW] + (int64_t)l * 3 * C * C, M + S.off[QKVB] + l * 3 * C,
                            dqkv.data(), ln1.data() + l * NC, N, C, 3 * C);
      layernorm_param_grad_mag(M + S.off[LN1W] + l * C, M + S.off[LN1B] + l * C, dln.data(), x,
                               ln1m.data() + l * N, ln1r.data() + l * N, N, C);
    }
    layernorm_backward(dres.data(), G(LN1W) + l * C, G(LN1B) + l * C, dln.data(), x,
                       P(LN1W) + l * C, ln1m.data() + l * N, ln1r.data() + l * N, N, C);
  }
  // dres is now d(loss)/d(encoded); the encoder term adds to the lm_head term of dwte
  encoder_backward(G(WTE), G(WPE), dres.data(), tokens, B, T, C);
  if (M) {
    for (int64_t i = 0; i < NC; i++) dres[i] = std::fabs(dres[i]);
    encoder_backward(M + S.off[WTE], M + S.off[WPE], dres.data(), tokens, B, T, C);
  }
  return 0;
}

int oracle_gpt2_step(int L, int C, int NH, int V, int maxT, const double* params,
                     const int* tokens, const int* targets, int B, int T, double* mean_loss,
                     double* losses_out, double* logits_out, double* grads) {
  return oracle_gpt2_step_mag(L, C, NH, V, maxT, params, tokens, targets, B, T, mean_loss,
                              losses_out, logits_out, grads, nullptr, nullptr);
}

}  // extern "C"
