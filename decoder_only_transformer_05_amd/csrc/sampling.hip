// sampling.hip -- drawing the next token from the logits of one position ("llm.c 的中文注解-
// 20240421", section 1.35 sample_mult, applied to the probabilities of section 1.13's
// softmax): with p = softmax(z), the result is the smallest index i whose cumulative
// probability p_0 + ... + p_i exceeds coin (coin in [0, 1)), or the last index if rounding
// leaves every cumulative value at or below coin.
//
// One workgroup of 1024 threads per row: each thread owns a contiguous chunk of the row;
// the row maximum and the sum of exp(z - max) are reduced in a fixed order, each chunk's
// probability mass is summed in index order and the chunk prefix sums are formed by one
// thread in chunk order, so the cumulative value seen at index i -- and the result -- does
// not depend on scheduling. The thread whose chunk holds the crossing walks it in order.
#include "kernels.h"

namespace gpt2 {
namespace {

constexpr int SAMPLE_THREADS = 1024;

template <typename TS>
__global__ __launch_bounds__(SAMPLE_THREADS) void sample_mult_kernel(int32_t* __restrict__ out,
                                                                     const TS* __restrict__ z,
                                                                     int V, float coin) {
  __shared__ float red[SAMPLE_THREADS];
  __shared__ float prefix[SAMPLE_THREADS];
  __shared__ int first;
  const int tid = threadIdx.x;
  const int chunk = (V + SAMPLE_THREADS - 1) / SAMPLE_THREADS;
  const int i0 = min(V, tid * chunk), i1 = min(V, i0 + chunk);

  float mx = -INFINITY;
  for (int i = i0; i < i1; i++) mx = fmaxf(mx, ld1(z + i));
  red[tid] = mx;
  if (tid == 0) first = V;
  __syncthreads();
  for (int s = SAMPLE_THREADS / 2; s > 0; s >>= 1) {
    if (tid < s) red[tid] = fmaxf(red[tid], red[tid + s]);
    __syncthreads();
  }
  mx = red[0];
  __syncthreads();

  float sum = 0.f;
  for (int i = i0; i < i1; i++) sum += expf(ld1(z + i) - mx);
  red[tid] = sum;
  __syncthreads();
  for (int s = SAMPLE_THREADS / 2; s > 0; s >>= 1) {
    if (tid < s) red[tid] += red[tid + s];
    __syncthreads();
  }
  const float total = red[0];
  __syncthreads();

  // probability mass of this thread's chunk, in index order
  float mass = 0.f;
  for (int i = i0; i < i1; i++) mass += expf(ld1(z + i) - mx) / total;
  prefix[tid] = mass;
  __syncthreads();
  if (tid == 0) {  // exclusive prefix sums of the chunk masses, in chunk order
    float run = 0.f;
    for (int t = 0; t < SAMPLE_THREADS; t++) {
      const float m = prefix[t];
      prefix[t] = run;
      run += m;
    }
  }
  __syncthreads();
  float cdf = prefix[tid];
  for (int i = i0; i < i1; i++) {
    cdf += expf(ld1(z + i) - mx) / total;
    if (coin < cdf) {
      atomicMin(&first, i);
      break;
    }
  }
  __syncthreads();
  if (tid == 0) out[0] = first < V ? first : V - 1;
}

}  // namespace

template <typename TS>
static int sample_mult_launch(int32_t* out, const TS* logits, int V, float coin,
                              hipStream_t stream) {
  if (!out || !logits || V < 1) {
    set_global_error("sample_mult: bad argument");
    return -1;
  }
  ProfScope ps("sample_mult_kernel", 0.0, (double)V * sizeof(TS), stream);
  sample_mult_kernel<TS><<<1, SAMPLE_THREADS, 0, stream>>>(out, logits, V, coin);
  GPT2_HIP_OK(hipGetLastError());
  return 0;
}

int sample_mult(int32_t* out, const float* logits, int V, float coin, hipStream_t stream) {
  return sample_mult_launch(out, logits, V, coin, stream);
}
int sample_mult(int32_t* out, const bf16_t* logits, int V, float coin, hipStream_t stream) {
  return sample_mult_launch(out, logits, V, coin, stream);
}
int sample_mult(int32_t* out, const f16_t* logits, int V, float coin, hipStream_t stream) {
  return sample_mult_launch(out, logits, V, coin, stream);
}

}  // namespace gpt2
