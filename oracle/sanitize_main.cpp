// sanitize_main.cpp -- TEST INFRASTRUCTURE: a stand-alone driver for the oracle, built
// together with gpt2_oracle.cpp under AddressSanitizer and UndefinedBehaviorSanitizer by
// the CPU test suite. It reads one problem from a binary file, runs the whole training
// step (every layer's forward and backward, envelopes included) plus the entry points the
// step does not use, and writes the results, so the test can compare them with the
// ordinary build's.
//
// Input file (native endianness): int32 L, C, NH, V, maxT, B, T; int64 P; P doubles of
// parameters; B*T int32 tokens; B*T int32 targets.
// Output file: double loss; B*T losses; B*T*V logits; P grads; P grad envelopes;
// B*T*V logit envelopes; P parameters after one AdamW step (wd 0.1) from those gradients;
// T*T softmax-Jacobian backward of a synthetic attention row block.
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <vector>

extern "C" {
int oracle_gpt2_step_mag(int L, int C, int NH, int V, int maxT, const double* params,
                         const int* tokens, const int* targets, int B, int T, double* mean_loss,
                         double* losses_out, double* logits_out, double* grads,
                         double* grad_mag, double* logit_mag);
void oracle_adamw(int64_t n, double* p, const double* g, double* m, double* v, double lr,
                  double b1, double b2, double eps, double wd, int t);
void oracle_softmax_jacobian_backward(double* dpre, const double* att, const double* datt,
                                      int T);
void oracle_softmax_forward(double* probs, const double* logits, int64_t N, int V);
}

template <typename X>
static bool rd(FILE* f, X* p, size_t n) { return fread(p, sizeof(X), n, f) == n; }
template <typename X>
static void wr(FILE* f, const X* p, size_t n) { fwrite(p, sizeof(X), n, f); }

int main(int argc, char** argv) {
  if (argc != 3) {
    fprintf(stderr, "usage: %s input output\n", argv[0]);
    return 2;
  }
  FILE* f = fopen(argv[1], "rb");
  if (!f) return 2;
  int32_t d[7];
  int64_t P = 0;
  if (!rd(f, d, 7) || !rd(f, &P, 1)) return 2;
  const int L = d[0], C = d[1], NH = d[2], V = d[3], maxT = d[4], B = d[5], T = d[6];
  const size_t N = (size_t)B * T;
  std::vector<double> params(P);
  std::vector<int> tok(N), tgt(N);
  if (!rd(f, params.data(), P) || !rd(f, tok.data(), N) || !rd(f, tgt.data(), N)) return 2;
  fclose(f);

  double loss = 0.0;
  std::vector<double> losses(N), logits(N * V), grads(P), gmag(P), lmag(N * V);
  if (oracle_gpt2_step_mag(L, C, NH, V, maxT, params.data(), tok.data(), tgt.data(), B, T,
                           &loss, losses.data(), logits.data(), grads.data(), gmag.data(),
                           lmag.data()))
    return 3;
  std::vector<double> p2(params), m(P, 0.0), v(P, 0.0);
  oracle_adamw(P, p2.data(), grads.data(), m.data(), v.data(), 1e-3, 0.9, 0.999, 1e-8, 0.1, 1);
  // a causal attention block: softmax of the first T*T logits row by row, masked
  std::vector<double> att((size_t)T * T, 0.0), datt((size_t)T * T), dpre((size_t)T * T, 0.0);
  for (int t = 0; t < T; t++) {
    std::vector<double> row(logits.begin() + (size_t)t * V, logits.begin() + (size_t)t * V + t + 1);
    oracle_softmax_forward(att.data() + (size_t)t * T, row.data(), 1, t + 1);
    for (int t2 = 0; t2 < T; t2++) datt[(size_t)t * T + t2] = logits[(size_t)t2 * V + t];
  }
  oracle_softmax_jacobian_backward(dpre.data(), att.data(), datt.data(), T);

  FILE* o = fopen(argv[2], "wb");
  if (!o) return 2;
  wr(o, &loss, 1);
  wr(o, losses.data(), N);
  wr(o, logits.data(), N * V);
  wr(o, grads.data(), P);
  wr(o, gmag.data(), P);
  wr(o, lmag.data(), N * V);
  wr(o, p2.data(), P);
  wr(o, dpre.data(), (size_t)T * T);
  fclose(o);
  return 0;
}
