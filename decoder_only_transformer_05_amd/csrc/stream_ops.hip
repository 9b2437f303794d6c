// stream_ops.hip -- the memory-bound kernels of the training step: embedding gather and
// scatter, LayerNorm forward/backward, softmax cross-entropy forward/backward, the mean
// loss and AdamW. Each streams its tensors once with 16-byte accesses; row reductions use
// wave64 shuffles, column reductions are split into fixed-order partial sums so results do
// not depend on scheduling.
//
// Definitions follow "llm.c 的中文注解-20240421": 1.1 encoder_forward, 1.2 encoder_backward,
// 1.3 layernorm_forward, 1.4 layernorm_backward, 1.13 softmax_forward, 1.14
// crossentropy_forward, 1.15 crossentropy_softmax_backward, 1.26 gpt2_update (AdamW).
#include <cmath>

#include "kernels.h"

namespace gpt2 {
namespace {

// tokens outside [0, V) were reported by the forward; here they read as 0 so that no
// index leaves its buffer
GPT2_DEVICE_INLINE int clamp_tok(int v, int V) { return (v < 0 || v >= V) ? 0 : v; }

// Loads and stores marked nontemporal (not kept in the caches), for the AdamW streams, which
// are read and written once per step and not read again soon. A probe on this GPU: an
// AdamW-shaped stream of 124M parameters (four reads, three writes) at 5.30 TB/s with plain
// accesses, 5.50 TB/s nontemporal; AdamW itself 642 -> 583 us at 124M. (The one-pass
// cross-entropy was 2% slower with them and keeps plain accesses.)
GPT2_DEVICE_INLINE f32x4 ld4_nt(const float* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
}
GPT2_DEVICE_INLINE void st4_nt(float* p, f32x4 v) {
  __builtin_nontemporal_store(v, reinterpret_cast<f32x4*>(p));
}
GPT2_DEVICE_INLINE void st4_nt(bf16_t* p, f32x4 v) {
  const uint32_t lo = (uint32_t)f32_to_bf16(v[0]) | ((uint32_t)f32_to_bf16(v[1]) << 16);
  const uint32_t hi = (uint32_t)f32_to_bf16(v[2]) | ((uint32_t)f32_to_bf16(v[3]) << 16);
  __builtin_nontemporal_store(u32x2_t{lo, hi}, reinterpret_cast<u32x2_t*>(p));
}
GPT2_DEVICE_INLINE void st4_nt(f16_t* p, f32x4 v) {
  __builtin_nontemporal_store(__builtin_convertvector(v, f16x4_t), reinterpret_cast<f16x4_t*>(p));
}

int blocks_for(long long n, int per_block, int cap) {
  long long b = (n + per_block - 1) / per_block;
  if (b > cap) b = cap;
  return b < 1 ? 1 : (int)b;
}

// ---------------------------------------------------------------------------------------
// encoder
// ---------------------------------------------------------------------------------------
template <typename TO>
__global__ void encoder_fwd_kernel(TO* __restrict__ out, const int32_t* __restrict__ tok,
                                   const float* __restrict__ wte, const float* __restrict__ wpe,
                                   int BT, int T, int C, int V, int32_t* err) {
  const int C4 = C / 4;
  const long long total = (long long)BT * C4;
  for (long long idx = (long long)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
       idx += (long long)gridDim.x * blockDim.x) {
    const int row = (int)(idx / C4), c = 4 * (int)(idx % C4);
    int v = tok[row];
    if (v < 0 || v >= V) {
      if (err) *err = 1;
      v = 0;
    }
    const int t = row % T;
    f32x4 a = ld4(wte + (long long)v * C + c), p = ld4(wpe + (long long)t * C + c);
    st4(out + (long long)row * C + c, a + p);
  }
}

// dwpe[t] += sum over b of dout[b, t] (b ascending)
__global__ void encoder_bwd_wpe_kernel(float* __restrict__ dwpe, const float* __restrict__ dout,
                                       int B, int T, int C) {
  const int C4 = C / 4;
  const long long total = (long long)T * C4;
  for (long long idx = (long long)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
       idx += (long long)gridDim.x * blockDim.x) {
    const int t = (int)(idx / C4), c = 4 * (int)(idx % C4);
    f32x4 s = {0.f, 0.f, 0.f, 0.f};
    for (int b = 0; b < B; b++) s += ld4(dout + ((long long)b * T + t) * C + c);
    float* p = dwpe + (long long)t * C + c;
    st4(p, ld4(p) + s);
  }
}

// Stable sort of positions by token, in two fully parallel steps.
// token_chunk_sort_kernel: one 1024-thread workgroup per chunk of 1024 consecutive
// positions sorts the chunk's keys (token << 10 | position in the chunk) with a bitonic
// network in LDS; the last chunk is padded with keys above every real key.
// token_merge_kernel: the place of a key in the whole sorted order is its index in its own
// chunk plus, for every earlier chunk, the number of keys with a token at most its own and,
// for every later chunk, the number with a token below its own (lower bounds by binary
// search in the sorted chunks, eight chunks searched in lockstep). Equal tokens thus keep
// position order, and the result is a function of the tokens alone.
// scratch: sorted[BT], keys[nchunks * 1024].
constexpr int SORT_THREADS = 1024;
constexpr int32_t SORT_PAD = 0x7FFFFFFF;
__global__ __launch_bounds__(SORT_THREADS) void token_chunk_sort_kernel(
    int32_t* __restrict__ keys, const int32_t* __restrict__ tok, int BT, int V) {
  __shared__ int32_t key_s[SORT_THREADS];
  const int tid = threadIdx.x;
  const int c0 = blockIdx.x * SORT_THREADS, i = c0 + tid;
  key_s[tid] = i < BT ? (clamp_tok(tok[i], V) << 10) | tid : SORT_PAD;
  __syncthreads();
  for (int k = 2; k <= SORT_THREADS; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      const int partner = tid ^ j;
      if (partner > tid) {
        const int a = key_s[tid], b = key_s[partner];
        const bool up = (tid & k) == 0;
        if ((a > b) == up) {
          key_s[tid] = b;
          key_s[partner] = a;
        }
      }
      __syncthreads();
    }
  }
  keys[c0 + tid] = key_s[tid];
}

__global__ __launch_bounds__(SORT_THREADS) void token_merge_kernel(
    int32_t* __restrict__ sorted, const int32_t* __restrict__ keys, int nchunks) {
  constexpr int G = 8;  // chunks searched together
  const int c = blockIdx.x, j = threadIdx.x;
  const int key = keys[c * SORT_THREADS + j];
  if (key == SORT_PAD) return;
  const int v = key >> 10;
  int dest = j;
  for (int g0 = 0; g0 < nchunks; g0 += G) {
    int lo[G];
#pragma unroll
    for (int u = 0; u < G; u++) lo[u] = 0;
#pragma unroll
    for (int step = SORT_THREADS / 2; step > 0; step >>= 1) {
#pragma unroll
      for (int u = 0; u < G; u++) {
        const int c2 = g0 + u;
        if (c2 < nchunks && c2 != c) {
          const int bound = c2 < c ? (v + 1) << 10 : v << 10;
          if (keys[c2 * SORT_THREADS + lo[u] + step - 1] < bound) lo[u] += step;
        }
      }
    }
#pragma unroll
    for (int u = 0; u < G; u++) {
      const int c2 = g0 + u;
      if (c2 < nchunks && c2 != c) {
        const int bound = c2 < c ? (v + 1) << 10 : v << 10;
        dest += lo[u] + (keys[c2 * SORT_THREADS + lo[u]] < bound ? 1 : 0);
      }
    }
  }
  sorted[dest] = c * SORT_THREADS + (key & 1023);
}

// dwte: positions sorted by (token, position) form one run per token. Runs are cut at every
// multiple of WTE_CHUNK sorted indices, so no wave sums more than WTE_CHUNK rows however
// skewed the tokens are (a frequent token of real text repeats hundreds of times in a
// batch). One wave per sorted index j; the waves at a run start or at a chunk boundary
// inside a run each sum their piece of rows in ascending position order. A piece that is a
// whole run is added to the token's dwte row at once; the pieces of a run that crosses
// chunk boundaries go to a partial buffer (per chunk: the piece that starts it, continuing
// an earlier run, and the piece of the run that starts in it and goes on past its end),
// and encoder_bwd_wte_span_kernel adds them up in chunk order. Fixed summation order, no
// atomics: bitwise reproducible.
constexpr int WTE_CHUNK = 32;
__global__ void encoder_bwd_wte_kernel(float* __restrict__ dwte, float* __restrict__ part,
                                       const float* __restrict__ dout,
                                       const int32_t* __restrict__ tok,
                                       const int32_t* __restrict__ sorted, int BT, int C,
                                       int V) {
  const int j = blockIdx.x * (blockDim.x / 64) + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (j >= BT) return;  // wave-uniform
  // lane l looks at sorted index j - 1 + l, l = 0 .. WTE_CHUNK + 1
  const int k = j - 1 + lane;
  const bool in = lane <= WTE_CHUNK + 1 && k >= 0 && k < BT;
  const int pos = in ? sorted[k] : 0;
  const int t = in ? clamp_tok(tok[pos], V) : -1;
  const int v = __shfl(t, 1, 64);          // token at j
  const bool head = __shfl(t, 0, 64) == v;  // the run began before j (lane 0 holds -1 if j = 0)
  if (head && j % WTE_CHUNK != 0) return;   // neither a run start nor a chunk boundary
  // the piece ends at the first index e > j holding another token, at BT, or at the next chunk
  // boundary (always within lanes 2 .. WTE_CHUNK + 1)
  const bool stop = lane >= 2 && lane <= WTE_CHUNK + 1 &&
                    (k >= BT || t != v || k % WTE_CHUNK == 0);
  const int le = __ffsll((unsigned long long)__ballot(stop)) - 1;
  const int e = j - 1 + le;
  const bool tail = e < BT && __shfl(t, le, 64) == v;  // the run goes on past the boundary e
  const int nrow = e - j;
  const int chunk = j / WTE_CHUNK;
  float* dst = !head && !tail ? dwte + (long long)v * C
                              : part + (2LL * chunk + (head ? 0 : 1)) * C;
  for (int c = 4 * lane; c < C; c += 256) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int r = 0; r < nrow; r++) {
      const int p = __builtin_amdgcn_readlane(pos, r + 1);
      acc += ld4(dout + (long long)p * C + c);
    }
    if (!head && !tail) st4(dst + c, ld4(dst + c) + acc);
    else st4(dst + c, acc);
  }
}

// One wave per chunk: if a run starts in the chunk and goes on past its end, add its piece
// in this chunk and the leading pieces of the following chunks it covers, in that order, to
// the token's dwte row.
__global__ void encoder_bwd_wte_span_kernel(float* __restrict__ dwte,
                                            const float* __restrict__ part,
                                            const int32_t* __restrict__ tok,
                                            const int32_t* __restrict__ sorted, int BT, int C,
                                            int V) {
  const int nch = (BT + WTE_CHUNK - 1) / WTE_CHUNK;
  const int c = blockIdx.x * (blockDim.x / 64) + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (c >= nch) return;
  const int jl = min(BT, (c + 1) * WTE_CHUNK) - 1;  // last index of the chunk
  if (jl + 1 >= BT) return;
  const int u = clamp_tok(tok[sorted[jl]], V);
  if (clamp_tok(tok[sorted[jl + 1]], V) != u) return;                       // ends here
  if (c > 0 && clamp_tok(tok[sorted[c * WTE_CHUNK - 1]], V) == u) return;   // began earlier
  // last chunk of the run: the first chunk c2 > c whose next chunk does not start with u
  int last = -1;
  for (int base = c + 1; last < 0; base += 64) {
    const int c2 = base + lane;
    const int nx = (c2 + 1) * WTE_CHUNK;
    const bool more = c2 < nch && nx < BT && clamp_tok(tok[sorted[nx]], V) == u;
    const unsigned long long m = __ballot(c2 < nch && !more);
    if (m) last = base + __ffsll(m) - 1;
  }
  float* dst = dwte + (long long)u * C;
  for (int col = 4 * lane; col < C; col += 256) {
    f32x4 acc = ld4(part + (2LL * c + 1) * C + col);
    for (int c2 = c + 1; c2 <= last; c2++) acc += ld4(part + 2LL * c2 * C + col);
    st4(dst + col, ld4(dst + col) + acc);
  }
}

// ---------------------------------------------------------------------------------------
// LayerNorm: one wave per row, VPL float4 per lane held in registers
// ---------------------------------------------------------------------------------------
template <int VPL, typename T>
__global__ __launch_bounds__(256) void layernorm_fwd_kernel(T* __restrict__ out,
                                                            float* __restrict__ mean,
                                                            float* __restrict__ rstd,
                                                            const T* __restrict__ x,
                                                            const float* __restrict__ w,
                                                            const float* __restrict__ bias,
                                                            int N, int C) {
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= N) return;
  const int C4 = C / 4;
  const T* xr = x + (long long)row * C;
  f32x4 v[VPL];
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < VPL; i++) {
    const int c4 = lane + 64 * i;
    v[i] = c4 < C4 ? ld4(xr + 4 * c4) : f32x4{0.f, 0.f, 0.f, 0.f};
    s += (v[i][0] + v[i][1]) + (v[i][2] + v[i][3]);
  }
  const float m = warp_sum(s) / C;
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < VPL; i++) {
    if (lane + 64 * i < C4) {
      f32x4 d = v[i] - m;
      ss += (d[0] * d[0] + d[1] * d[1]) + (d[2] * d[2] + d[3] * d[3]);
    }
  }
  const float rs = 1.0f / sqrtf(warp_sum(ss) / C + 1e-5f);
  T* orow = out + (long long)row * C;
#pragma unroll
  for (int i = 0; i < VPL; i++) {
    const int c4 = lane + 64 * i;
    if (c4 < C4) st4(orow + 4 * c4, (v[i] - m) * rs * ld4(w + 4 * c4) + ld4(bias + 4 * c4));
  }
  if (lane == 0) {
    if (mean) mean[row] = m;
    if (rstd) rstd[row] = rs;
  }
}

// rows per workgroup in the backward: 32, halved (down to 4) until there are at least 512
// workgroups, so short batches still fill the chip (fewer workgroups, fewer partial sums
// for the column reduction)
int lnb_rows(int N) {
  int rows = 32;
  while (rows > 4 && (N + rows - 1) / rows < 512) rows /= 2;
  return rows;
}

// one row's dout and x for the LayerNorm backward, held in registers as stored (zeros past C)
template <int VPL, typename T, typename R>
GPT2_DEVICE_INLINE void lnb_fetch(R (&dy)[VPL], R (&xv)[VPL], const T* dout, const T* x,
                                  int row, int C, int lane) {
  const int C4 = C / 4;
#pragma unroll
  for (int i = 0; i < VPL; i++) {
    const int c4 = lane + 64 * i;
    const long long o = (long long)row * C + 4 * c4;
    dy[i] = c4 < C4 ? raw4(dout + o) : R{};
    xv[i] = c4 < C4 ? raw4(x + o) : R{};
  }
}

// dx (+)= rstd * (g - mean(g) - n * mean(g*n)), g = w * dout, n = (x - mean) * rstd;
// per workgroup, partial[blk][0][:] = sum of n*dout, partial[blk][1][:] = sum of dout over
// its rows. Each wave sums its rows in order into its own LDS slice (so the column sums
// take no registers across rows), then the four slices are added in wave order. A wave's
// next row of dout and x, and the dx that row accumulates into, are loaded while the
// current row is computed.
// dx is fp32; with 16-bit activations dx_copy (if not null) receives dx rounded to T.
template <int VPL, typename T>
__global__ __launch_bounds__(256) void layernorm_bwd_kernel(
    float* __restrict__ dx, T* __restrict__ dx_copy, float* __restrict__ partial,
    const T* __restrict__ dout, const T* __restrict__ x, const float* __restrict__ w,
    const float* __restrict__ mean, const float* __restrict__ rstd, int N, int C,
    int accumulate, int rows_per_block) {
  extern __shared__ float red[];  // [4 waves][2][C]
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int C4 = C / 4;
  float* rdw = red + (wave * 2 + 0) * C;
  float* rdb = red + (wave * 2 + 1) * C;
  f32x4 wv[VPL];
#pragma unroll
  for (int i = 0; i < VPL; i++) {
    const int c4 = lane + 64 * i;
    wv[i] = c4 < C4 ? ld4(w + 4 * c4) : f32x4{0.f, 0.f, 0.f, 0.f};
    if (c4 < C4) {
      st4(rdw + 4 * c4, f32x4{0.f, 0.f, 0.f, 0.f});
      st4(rdb + 4 * c4, f32x4{0.f, 0.f, 0.f, 0.f});
    }
  }
  const int r0 = blockIdx.x * rows_per_block;
  const int r1 = min(N, r0 + rows_per_block);
  typename Raw4<T>::type dyn[VPL], xn[VPL];  // the next row, as stored
  f32x4 dxn[VPL];                             // and the dx it accumulates into
  float mun = 0.f, rsn = 0.f;
  int row = r0 + wave;
  auto fetch_dx = [&](int rw) {
#pragma unroll
    for (int i = 0; i < VPL; i++) {
      const int c4 = lane + 64 * i;
      dxn[i] = c4 < C4 && accumulate ? ld4(dx + (long long)rw * C + 4 * c4)
                                     : f32x4{0.f, 0.f, 0.f, 0.f};
    }
  };
  if (row < r1) {
    lnb_fetch<VPL>(dyn, xn, dout, x, row, C, lane);
    fetch_dx(row);
    mun = mean[row];
    rsn = rstd[row];
  }
  for (; row < r1; row += 4) {
    f32x4 dy[VPL], nv[VPL], dxo[VPL];
    const float mu = mun, rs = rsn;
#pragma unroll
    for (int i = 0; i < VPL; i++) {
      dy[i] = widen4(dyn[i]);
      nv[i] = widen4(xn[i]);
      dxo[i] = dxn[i];
    }
    float* dxr = dx + (long long)row * C;
    if (row + 4 < r1) {
      lnb_fetch<VPL>(dyn, xn, dout, x, row + 4, C, lane);
      fetch_dx(row + 4);
      mun = mean[row + 4];
      rsn = rstd[row + 4];
    }
    float sg = 0.f, sgn = 0.f;
#pragma unroll
    for (int i = 0; i < VPL; i++) {
      if (lane + 64 * i < C4) {
        nv[i] = (nv[i] - mu) * rs;
        f32x4 g = wv[i] * dy[i];
        sg += (g[0] + g[1]) + (g[2] + g[3]);
        f32x4 gn = g * nv[i];
        sgn += (gn[0] + gn[1]) + (gn[2] + gn[3]);
      } else {
        nv[i] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
    }
    const float mg = warp_sum(sg) / C, mgn = warp_sum(sgn) / C;
#pragma unroll
    for (int i = 0; i < VPL; i++) {
      const int c4 = lane + 64 * i;
      if (c4 < C4) {
        f32x4 d = (wv[i] * dy[i] - mg - nv[i] * mgn) * rs;
        if (accumulate) d += dxo[i];
        st4(dxr + 4 * c4, d);
        if (dx_copy) st4(dx_copy + (long long)row * C + 4 * c4, d);
        st4(rdw + 4 * c4, ld4(rdw + 4 * c4) + nv[i] * dy[i]);
        st4(rdb + 4 * c4, ld4(rdb + 4 * c4) + dy[i]);
      }
    }
  }
  __syncthreads();
  for (int c = threadIdx.x; c < 2 * C; c += 256) {
    const int which = c / C, cc = c % C;
    float s = red[(0 * 2 + which) * C + cc];
    s += red[(1 * 2 + which) * C + cc];
    s += red[(2 * 2 + which) * C + cc];
    s += red[(3 * 2 + which) * C + cc];
    partial[((long long)blockIdx.x * 2 + which) * C + cc] = s;
  }
}

// dw[c] += sum_k partial[k][0][c], db[c] += sum_k partial[k][1][c]. A workgroup owns 8 of
// the 2C columns; its 32 thread groups each sum every 32nd partial (in order, four loads in
// flight), and the 32 group sums are then added in group order.
constexpr int LNF_COLS = 8, LNF_GROUPS = 32;
__global__ __launch_bounds__(256) void layernorm_bwd_final_kernel(float* __restrict__ dw,
                                                                  float* __restrict__ db,
                                                                  const float* __restrict__ partial,
                                                                  int blocks, int C) {
  __shared__ float red[LNF_GROUPS][LNF_COLS];
  const int cl = threadIdx.x % LNF_COLS, grp = threadIdx.x / LNF_COLS;
  const int c = blockIdx.x * LNF_COLS + cl;
  const int which = c / C, cc = c - which * C;
  float s = 0.f;
  if (c < 2 * C) {
    const float* p = partial + (long long)which * C + cc;
    const long long st = 2LL * C;  // between consecutive partials
    constexpr int G = LNF_GROUPS;
    int k = grp;
    for (; k + 3 * G < blocks; k += 4 * G) {
      const float a0 = p[(long long)k * st], a1 = p[(long long)(k + G) * st];
      const float a2 = p[(long long)(k + 2 * G) * st], a3 = p[(long long)(k + 3 * G) * st];
      s += a0;
      s += a1;
      s += a2;
      s += a3;
    }
    for (; k < blocks; k += G) s += p[(long long)k * st];
  }
  red[grp][cl] = s;
  __syncthreads();
  if (grp == 0 && c < 2 * C) {
    float t = red[0][cl];
#pragma unroll
    for (int k = 1; k < LNF_GROUPS; k++) t += red[k][cl];
    if (which == 0) dw[cc] += t;
    else db[cc] += t;
  }
}

// ---------------------------------------------------------------------------------------
// softmax cross-entropy over the vocabulary: one workgroup per row
// ---------------------------------------------------------------------------------------
GPT2_DEVICE_INLINE void lse_merge(float& m, float& s, float m2, float s2) {
  const float mn = fmaxf(m, m2);
  if (mn == -INFINITY) return;
  s = s * __expf(m - mn) + s2 * __expf(m2 - mn);
  m = mn;
}

template <typename T>
__global__ __launch_bounds__(256) void xent_fwd_kernel(float* __restrict__ losses,
                                                       float* __restrict__ lse_out,
                                                       const T* __restrict__ logits,
                                                       const int32_t* __restrict__ targets,
                                                       int N, int V, int ld, int32_t* err) {
  __shared__ float sm[4], ss[4];
  const int row = blockIdx.x;
  const T* z = logits + (long long)row * ld;
  float m = -INFINITY, s = 0.f;
  const int V4 = (V + 3) / 4;
  for (int c4 = threadIdx.x; c4 < V4; c4 += 256) {
    f32x4 v = ld4(z + 4 * c4);
    const int c = 4 * c4;
    if (c + 3 >= V) {
      if (c + 1 >= V) v[1] = -INFINITY;
      if (c + 2 >= V) v[2] = -INFINITY;
      if (c + 3 >= V) v[3] = -INFINITY;
    }
    const float mx = fmaxf(fmaxf(v[0], v[1]), fmaxf(v[2], v[3]));
    if (mx > m) {
      s *= __expf(m - mx);
      m = mx;
    }
    s += (__expf(v[0] - m) + __expf(v[1] - m)) + (__expf(v[2] - m) + __expf(v[3] - m));
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float m2 = __shfl_xor(m, o, 64), s2 = __shfl_xor(s, o, 64);
    lse_merge(m, s, m2, s2);
  }
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  if (lane == 0) {
    sm[wave] = m;
    ss[wave] = s;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    float M = sm[0], S = ss[0];
    for (int k = 1; k < 4; k++) lse_merge(M, S, sm[k], ss[k]);
    const float lse = M + logf(S);
    int y = targets[row];
    if (y < 0 || y >= V) {
      if (err) *err = 1;
      y = 0;
    }
    losses[row] = lse - ld1(z + y);
    lse_out[row] = lse;
  }
}

// in place: logits[r, v] <- (softmax - onehot(target)) * dloss for v < V, 0 on the padding;
// with dscale (device, may be null) the factor is dloss * *dscale (a loss scale).
// One 16-byte vector per thread over a flat grid: a workgroup covers 256 vectors of one row
// (`chunks` workgroups per row), so the whole matrix streams in address order.
template <typename T>
__global__ __launch_bounds__(256) void xent_bwd_kernel(T* __restrict__ logits,
                                                       const float* __restrict__ lse,
                                                       const int32_t* __restrict__ targets,
                                                       float dloss, const float* dscale, int V,
                                                       int ld, int chunks) {
  constexpr int G = 16 / (4 * sizeof(T));  // groups of 4 elements per thread
  if (dscale) dloss *= *dscale;
  const int row = blockIdx.x / chunks;
  const int c0 = ((blockIdx.x - row * chunks) * 256 + threadIdx.x) * 4 * G;
  if (c0 >= ld) return;
  T* z = logits + (long long)row * ld;
  const float l = lse[row];
  int y = targets[row];
  if (y < 0 || y >= V) y = 0;
  f32x4 v[G];
#pragma unroll
  for (int k = 0; k < G; k++)
    if (c0 + 4 * k < ld) v[k] = ld4(z + c0 + 4 * k);
#pragma unroll
  for (int k = 0; k < G; k++) {
    const int c = c0 + 4 * k;
    if (c >= ld) break;
    f32x4 o;
#pragma unroll
    for (int j = 0; j < 4; j++)
      o[j] = c + j < V ? (__expf(v[k][j] - l) - (c + j == y ? 1.f : 0.f)) * dloss : 0.f;
    st4(z + c, o);
  }
}

// Forward and backward of the softmax cross-entropy in one pass over the logits: per row the
// log-sum-exp, the loss lse - z[target] (as xent_fwd_kernel) and the gradient
// dlogits = (softmax - onehot(target)) * dloss (as xent_bwd_kernel, zero on the padding),
// written to a separate buffer so the logits stay. One 1024-thread workgroup per row keeps
// the row in registers (CH vectors of 4 per thread, vector c4 = thread + 1024 k), so the
// logits are read once and the gradient written once; the row's running (max, sum) pairs
// are merged across the 16 waves in wave order.
constexpr int XF_THREADS = 1024;
template <typename T, int CH>
__global__ __launch_bounds__(XF_THREADS) void xent_fused_kernel(
    float* __restrict__ losses, float* __restrict__ lse_out, T* __restrict__ dlogits,
    const T* __restrict__ logits, const int32_t* __restrict__ targets, float dloss,
    const float* dscale, int V, int ld, int32_t* err) {
  __shared__ float sm[XF_THREADS / 64], ss[XF_THREADS / 64];
  const int row = blockIdx.x;
  const T* z = logits + (long long)row * ld;
  T* dz = dlogits + (long long)row * ld;
  const int L4 = ld / 4;
  f32x4 v[CH];
#pragma unroll
  for (int k = 0; k < CH; k++) {
    const int c4 = threadIdx.x + XF_THREADS * k;
    v[k] = c4 < L4 ? ld4(z + 4 * c4) : f32x4{0.f, 0.f, 0.f, 0.f};
  }
  float m = -INFINITY, s = 0.f;
#pragma unroll
  for (int k = 0; k < CH; k++) {
    const int c = 4 * (threadIdx.x + XF_THREADS * k);
    if (c >= V) break;
    f32x4 w = v[k];
    if (c + 3 >= V) {
      if (c + 1 >= V) w[1] = -INFINITY;
      if (c + 2 >= V) w[2] = -INFINITY;
      if (c + 3 >= V) w[3] = -INFINITY;
    }
    const float mx = fmaxf(fmaxf(w[0], w[1]), fmaxf(w[2], w[3]));
    if (mx > m) {
      s *= __expf(m - mx);
      m = mx;
    }
    s += (__expf(w[0] - m) + __expf(w[1] - m)) + (__expf(w[2] - m) + __expf(w[3] - m));
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float m2 = __shfl_xor(m, o, 64), s2 = __shfl_xor(s, o, 64);
    lse_merge(m, s, m2, s2);
  }
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  if (lane == 0) {
    sm[wave] = m;
    ss[wave] = s;
  }
  __syncthreads();
  float M = sm[0], S = ss[0];
  for (int k = 1; k < XF_THREADS / 64; k++) lse_merge(M, S, sm[k], ss[k]);
  const float lse = M + logf(S);
  int y = targets[row];
  if (y < 0 || y >= V) {
    if (err && threadIdx.x == 0) *err = 1;
    y = 0;
  }
  if (threadIdx.x == 0) {
    losses[row] = lse - ld1(z + y);
    lse_out[row] = lse;
  }
  if (dscale) dloss *= *dscale;
#pragma unroll
  for (int k = 0; k < CH; k++) {
    const int c4 = threadIdx.x + XF_THREADS * k;
    if (c4 >= L4) break;
    const int c = 4 * c4;
    f32x4 o;
#pragma unroll
    for (int j = 0; j < 4; j++)
      o[j] = c + j < V ? (__expf(v[k][j] - lse) - (c + j == y ? 1.f : 0.f)) * dloss : 0.f;
    st4(dz + c, o);
  }
}

// mean of n values by one workgroup, in a fixed order
__global__ __launch_bounds__(1024) void mean_kernel(float* __restrict__ out,
                                                    const float* __restrict__ x, int n) {
  __shared__ float part[16];
  float s = 0.f;
  for (int i = threadIdx.x; i < n; i += 1024) s += x[i];
  s = warp_sum(s);
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = s;
  __syncthreads();
  if (threadIdx.x == 0) {
    float t = 0.f;
    for (int k = 0; k < 16; k++) t += part[k];
    *out = t / n;
  }
}

// ---------------------------------------------------------------------------------------
// AdamW
// ---------------------------------------------------------------------------------------
// One float4 of parameters per thread over a flat grid (streams HBM faster than a
// grid-stride loop); threads n4 ... n4 + (n % 4) - 1 take the scalar tail. pbf (if not null)
// receives the updated parameters rounded to bf16.
GPT2_DEVICE_INLINE float adamw_one(float& p, float g, float& m, float& v, float lr, float b1,
                                   float b2, float eps, float wd, float inv_c1, float inv_c2) {
  m = b1 * m + (1.f - b1) * g;
  v = b2 * v + (1.f - b2) * g * g;
  const float mh = m * inv_c1, vh = v * inv_c2;
  p -= lr * (mh / (sqrtf(vh) + eps) + wd * p);
  return p;
}

// With a loss scale (inv_scale, device, may be null) the gradients are the scaled ones and
// are multiplied by *inv_scale first; a nonzero *skip (device, may be null) leaves every
// parameter and moment unchanged (the step's gradients overflowed).
template <typename TP>
__global__ __launch_bounds__(256) void adamw_kernel(float* __restrict__ p,
                                                    const float* __restrict__ g,
                                                    float* __restrict__ m, float* __restrict__ v,
                                                    TP* __restrict__ pbf, long long n4,
                                                    long long n, float lr, float b1, float b2,
                                                    float eps, float wd, float inv_c1,
                                                    float inv_c2, const float* inv_scale,
                                                    const int32_t* skip) {
  if (skip && *skip) return;
  const float gs = inv_scale ? *inv_scale : 1.f;
  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
  if (i < n4) {
    f32x4 pp = ld4_nt(p + 4 * i), gg = ld4_nt(g + 4 * i), mm = ld4_nt(m + 4 * i),
          vv = ld4_nt(v + 4 * i);
    if (inv_scale) gg *= gs;
#pragma unroll
    for (int j = 0; j < 4; j++) {
      float pj = pp[j], mj = mm[j], vj = vv[j];
      adamw_one(pj, gg[j], mj, vj, lr, b1, b2, eps, wd, inv_c1, inv_c2);
      pp[j] = pj;
      mm[j] = mj;
      vv[j] = vj;
    }
    st4_nt(p + 4 * i, pp);
    st4_nt(m + 4 * i, mm);
    st4_nt(v + 4 * i, vv);
    if (pbf) st4_nt(pbf + 4 * i, pp);
  } else {
    const long long e = 4 * n4 + (i - n4);
    if (e >= n) return;
    float pe = p[e], me = m[e], ve = v[e];
    adamw_one(pe, inv_scale ? g[e] * gs : g[e], me, ve, lr, b1, b2, eps, wd, inv_c1, inv_c2);
    p[e] = pe;
    m[e] = me;
    v[e] = ve;
    if (pbf) st1(pbf + e, pe);
  }
}

// flag = 1 if any of the n gradients is an infinity or a NaN (the loss-scaled backward
// overflowed); one float4 per thread
__global__ __launch_bounds__(256) void nonfinite_kernel(int32_t* __restrict__ flag,
                                                        const float* __restrict__ g, long long n4,
                                                        long long n) {
  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
  bool bad = false;
  if (i < n4) {
    const f32x4 x = ld4(g + 4 * i);
    bad = !(isfinite(x[0]) && isfinite(x[1]) && isfinite(x[2]) && isfinite(x[3]));
  } else {
    const long long e = 4 * n4 + (i - n4);
    if (e < n) bad = !isfinite(g[e]);
  }
  if (bad) *flag = 1;  // every writer stores the same value
}

// Dynamic loss scale, after each step's check: state = {scale, 1/scale}, counters =
// {overflow flag, good steps since the last change, last step skipped}. An overflow halves
// the scale (not below 1) and marks the step skipped; growth_interval steps in a row without
// one double it (not above 2^24); growth_interval 0 keeps the scale fixed. The flag is
// cleared for the next step.
__global__ void scaler_update_kernel(float* __restrict__ state, int32_t* __restrict__ cnt,
                                     int growth_interval) {
  const int overflow = cnt[0];
  cnt[2] = overflow;
  cnt[0] = 0;
  float s = state[0];
  if (overflow) {
    if (growth_interval > 0) s = fmaxf(1.f, s * 0.5f);
    cnt[1] = 0;
  } else if (growth_interval > 0 && ++cnt[1] >= growth_interval) {
    s = fminf(16777216.f, s * 2.f);
    cnt[1] = 0;
  }
  state[0] = s;
  state[1] = 1.f / s;
}

// dst = src * (*factor), n floats (a power-of-two loss scale: exact)
__global__ void scale_copy_kernel(float* __restrict__ dst, const float* __restrict__ src,
                                  const float* __restrict__ factor, long long n) {
  const float f = *factor;
  for (long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (long long)gridDim.x * blockDim.x)
    dst[i] = src[i] * f;
}

// fp32 <-> 16-bit copies (round to nearest even)
template <typename TD, typename TS>
__global__ void cast_kernel(TD* __restrict__ dst, const TS* __restrict__ src, long long n) {
  const long long n4 = n / 4;
  for (long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x; i < n4;
       i += (long long)gridDim.x * blockDim.x)
    st4(dst + 4 * i, ld4(src + 4 * i));
  if (blockIdx.x == 0 && threadIdx.x < n - 4 * n4) {
    const long long i = 4 * n4 + threadIdx.x;
    st1(dst + i, ld1(src + i));
  }
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15) == 0; }

}  // namespace

namespace {
template <typename TO>
int encoder_forward_t(TO* out, const int32_t* tok, const float* wte, const float* wpe, int B,
                      int T, int C, int V, int32_t* err_flag, hipStream_t stream,
                      const char* name) {
  if (B < 1 || T < 1 || C < 4 || C % 4 || V < 1 || !aligned16(out) || !aligned16(wte) ||
      !aligned16(wpe)) {
    set_global_error("encoder_forward: bad arguments");
    return -1;
  }
  const long long n = (long long)B * T * (C / 4);
  ProfScope ps(name, (double)B * T * C, (8.0 + sizeof(TO)) * B * T * C + 4.0 * B * T, stream);
  encoder_fwd_kernel<TO><<<blocks_for(n, 256, 8192), 256, 0, stream>>>(out, tok, wte, wpe, B * T,
                                                                      T, C, V, err_flag);
  GPT2_HIP_OK(hipGetLastError());
  return 0;
}
}  // namespace

int encoder_forward(float* out, const int32_t* tok, const float* wte, const float* wpe, int B,
                    int T, int C, int V, int32_t* err_flag, hipStream_t stream) {
  return encoder_forward_t(out, tok, wte, wpe, B, T, C, V, err_flag, stream, "encoder_fwd_kernel");
}
int encoder_forward(bf16_t* out, const int32_t* tok, const float* wte, const float* wpe, int B,
                    int T, int C, int V, int32_t* err_flag, hipStream_t stream) {
  return encoder_forward_t(out, tok, wte, wpe, B, T, C, V, err_flag, stream,
                           "encoder_fwd_bf16_kernel");
}
int encoder_forward(f16_t* out, const int32_t* tok, const float* wte, const float* wpe, int B,
                    int T, int C, int V, int32_t* err_flag, hipStream_t stream) {
  return encoder_forward_t(out, tok, wte, wpe, B, T, C, V, err_flag, stream,
                           "encoder_fwd_f16_kernel");
}

size_t encoder_sort_scratch_ints(int BT, int V, int C) {
  (void)V;
  const size_t padded = (size_t)(BT + SORT_THREADS - 1) / SORT_THREADS * SORT_THREADS;
  const size_t nch = (size_t)(BT + WTE_CHUNK - 1) / WTE_CHUNK;
  return 2 * nch * (size_t)C + (size_t)BT + padded;
}

int encoder_backward(float* dwte, float* dwpe, const float* dout, const int32_t* tok, int B,
                     int T, int C, int V, int32_t* scratch, hipStream_t stream) {
  if (B < 1 || T < 1 || C < 4 || C % 4 || V < 1) {
    set_global_error("encoder_backward: bad arguments");
    return -1;
  }
  const int BT = B * T;
  if (V >= (1 << 21)) {  // keys hold the token in their upper 21 bits
    set_global_error("encoder_backward: vocabulary of %d tokens is too large", V);
    return -1;
  }
  // scratch: dwte partials (2 per chunk of WTE_CHUNK sorted indices, C floats each), the
  // sorted positions, the sort keys
  const int nwch = (BT + WTE_CHUNK - 1) / WTE_CHUNK;
  float* part = reinterpret_cast<float*>(scratch);
  int32_t* sorted = scratch + 2LL * nwch * C;
  const int nchunks = (BT + SORT_THREADS - 1) / SORT_THREADS;
  int32_t* keys = sorted + BT;
  {
    ProfScope ps("encoder_bwd_wpe_kernel", (double)BT * C, 4.0 * ((double)BT * C + 2.0 * T * C),
                 stream);
    encoder_bwd_wpe_kernel<<<blocks_for((long long)T * (C / 4), 256, 8192), 256, 0, stream>>>(
        dwpe, dout, B, T, C);
  }
  {
    ProfScope ps("token_chunk_sort_kernel", 0.0, 4.0 * 2.0 * BT, stream);
    token_chunk_sort_kernel<<<nchunks, SORT_THREADS, 0, stream>>>(keys, tok, BT, V);
  }
  {
    ProfScope ps("token_merge_kernel", 0.0, 4.0 * 2.0 * BT, stream);
    token_merge_kernel<<<nchunks, SORT_THREADS, 0, stream>>>(sorted, keys, nchunks);
  }
  {
    ProfScope ps("encoder_bwd_wte_kernel", (double)BT * C, 4.0 * (3.0 * BT * C + 2.0 * BT),
                 stream);
    encoder_bwd_wte_kernel<<<(BT + 3) / 4, 256, 0, stream>>>(dwte, part, dout, tok, sorted, BT,
                                                            C, V);
  }
  ProfScope ps("encoder_bwd_wte_span_kernel", 0.0, 4.0 * 2.0 * nwch, stream);
  encoder_bwd_wte_span_kernel<<<(nwch + 3) / 4, 256, 0, stream>>>(dwte, part, tok, sorted, BT, C,
                                                                 V);
  GPT2_HIP_OK(hipGetLastError());
  return 0;
}

#define GPT2_LN_DISPATCH(VPLV, ...) \
  switch (VPLV) {                   \
    case 1: __VA_ARGS__(1); break;  \
    case 2: __VA_ARGS__(2); break;  \
    case 3: __VA_ARGS__(3); break;  \
    case 4: __VA_ARGS__(4); break;  \
    case 5: __VA_ARGS__(5); break;  \
    case 6: __VA_ARGS__(6); break;  \
    case 7: __VA_ARGS__(7); break;  \
    case 8: __VA_ARGS__(8); break;  \
    default: break;                 \
  }

namespace {
template <typename T>
int layernorm_forward_t(T* out, float* mean, float* rstd, const T* x, const float* w,
                        const float* b, int N, int C, hipStream_t stream, const char* name) {
  const int vpl = (C / 4 + 63) / 64;
  if (N < 1 || C < 4 || C % 4 || vpl > 8 || !aligned16(out) || !aligned16(x)) {
    set_global_error("layernorm_forward: unsupported N=%d C=%d", N, C);
    return -1;
  }
  const int grid = (N + 3) / 4;
  ProfScope ps(name, 8.0 * N * C, 2.0 * sizeof(T) * N * C + 8.0 * N + 8.0 * C, stream);
#define GPT2_LNF(V) \
  layernorm_fwd_kernel<V, T><<<grid, 256, 0, stream>>>(out, mean, rstd, x, w, b, N, C)
  GPT2_LN_DISPATCH(vpl, GPT2_LNF)
#undef GPT2_LNF
  GPT2_HIP_OK(hipGetLastError());
  return 0;
}
}  // namespace

int layernorm_forward(float* out, float* mean, float* rstd, const float* x, const float* w,
                      const float* b, int N, int C, hipStream_t stream) {
  return layernorm_forward_t(out, mean, rstd, x, w, b, N, C, stream, "layernorm_fwd_kernel");
}
int layernorm_forward(bf16_t* out, float* mean, float* rstd, const bf16_t* x, const float* w,
                      const float* b, int N, int C, hipStream_t stream) {
  return layernorm_forward_t(out, mean, rstd, x, w, b, N, C, stream,
                             "layernorm_fwd_bf16_kernel");
}
int layernorm_forward(f16_t* out, float* mean, float* rstd, const f16_t* x, const float* w,
                      const float* b, int N, int C, hipStream_t stream) {
  return layernorm_forward_t(out, mean, rstd, x, w, b, N, C, stream,
                             "layernorm_fwd_f16_kernel");
}

size_t layernorm_partial_floats(int N, int C) {
  const int rows = lnb_rows(N);
  return (size_t)((N + rows - 1) / rows) * 2 * C;
}

namespace {
template <typename T>
int layernorm_backward_t(float* dx, T* dx_copy, float* dw, float* db, const T* dout,
                         const T* x, const float* w, const float* mean, const float* rstd, int N,
                         int C, bool accumulate_dx, float* partial, hipStream_t stream,
                         const char* name) {
  const int vpl = (C / 4 + 63) / 64;
  if (N < 1 || C < 4 || C % 4 || vpl > 8) {
    set_global_error("layernorm_backward: unsupported N=%d C=%d", N, C);
    return -1;
  }
  const int rows = lnb_rows(N);
  const int blocks = (N + rows - 1) / rows;
  const size_t lds = (size_t)8 * C * sizeof(float);
  {
    ProfScope ps(name, 14.0 * N * C,
                 (2.0 * sizeof(T) + (accumulate_dx ? 8.0 : 4.0) + (dx_copy ? 2.0 : 0.0)) * N * C +
                     8.0 * N + 8.0 * blocks * C,
                 stream);
#define GPT2_LNB(V)                                                                          \
  layernorm_bwd_kernel<V, T><<<blocks, 256, lds, stream>>>(dx, dx_copy, partial, dout, x, w,   \
                                                           mean, rstd, N, C, accumulate_dx ? 1 : 0, \
                                                           rows)
    GPT2_LN_DISPATCH(vpl, GPT2_LNB)
#undef GPT2_LNB
  }
  ProfScope ps("layernorm_bwd_final_kernel", 2.0 * blocks * C, 4.0 * (2.0 * blocks * C + 4.0 * C),
               stream);
  layernorm_bwd_final_kernel<<<(2 * C + LNF_COLS - 1) / LNF_COLS, 256, 0, stream>>>(dw, db, partial,
                                                                                  blocks, C);
  GPT2_HIP_OK(hipGetLastError());
  return 0;
}
}  // namespace

int layernorm_backward(float* dx, float* dw, float* db, const float* dout, const float* x,
                       const float* w, const float* mean, const float* rstd, int N, int C,
                       bool accumulate_dx, float* partial, hipStream_t stream) {
  return layernorm_backward_t(dx, (float*)nullptr, dw, db, dout, x, w, mean, rstd, N, C,
                              accumulate_dx, partial, stream, "layernorm_bwd_kernel");
}
int layernorm_backward(float* dx, bf16_t* dx_copy, float* dw, float* db, const bf16_t* dout,
                       const bf16_t* x, const float* w, const float* mean, const float* rstd,
                       int N, int C, bool accumulate_dx, float* partial, hipStream_t stream) {
  return layernorm_backward_t(dx, dx_copy, dw, db, dout, x, w, mean, rstd, N, C, accumulate_dx,
                              partial, stream, "layernorm_bwd_bf16_kernel");
}
int layernorm_backward(float* dx, f16_t* dx_copy, float* dw, float* db, const f16_t* dout,
                       const f16_t* x, const float* w, const float* mean, const float* rstd,
                       int N, int C, bool accumulate_dx, float* partial, hipStream_t stream) {
  return layernorm_backward_t(dx, dx_copy, dw, db, dout, x, w, mean, rstd, N, C, accumulate_dx,
                              partial, stream, "layernorm_bwd_f16_kernel");
}

namespace {
template <typename T>
int crossentropy_forward_t(float* losses, float* lse, const T* logits, const int32_t* targets,
                           int N, int V, int ld, int32_t* err_flag, hipStream_t stream,
                           const char* name) {
  if (N < 1 || V < 1 || ld < V || ld % 4 || !aligned16(logits)) {
    set_global_error("crossentropy_forward: bad arguments");
    return -1;
  }
  ProfScope ps(name, 3.0 * N * V, (double)sizeof(T) * N * V + 12.0 * N, stream);
  xent_fwd_kernel<T><<<N, 256, 0, stream>>>(losses, lse, logits, targets, N, V, ld, err_flag);
  GPT2_HIP_OK(hipGetLastError());
  return 0;
}

template <typename T>
int crossentropy_backward_t(T* logits, const float* lse, const int32_t* targets, float dloss,
                            const float* dscale, int N, int V, int ld, hipStream_t stream,
                            const char* name) {
  if (N < 1 || V < 1 || ld < V || ld % 4 || !aligned16(logits)) {
    set_global_error("crossentropy_backward: bad arguments");
    return -1;
  }
  const int per_block = 256 * 16 / (int)sizeof(T);  // elements one workgroup covers
  const int chunks = (ld + per_block - 1) / per_block;
  if ((long long)N * chunks >= (1LL << 31)) {
    set_global_error("crossentropy_backward: too many rows");
    return -1;
  }
  ProfScope ps(name, 3.0 * N * V, 2.0 * sizeof(T) * N * ld + 8.0 * N, stream);
  xent_bwd_kernel<T><<<N * chunks, 256, 0, stream>>>(logits, lse, targets, dloss, dscale, V, ld,
                                                     chunks);
  GPT2_HIP_OK(hipGetLastError());
  return 0;
}

template <typename T>
int crossentropy_fused_t(float* losses, float* lse, T* dlogits, const T* logits,
                         const int32_t* targets, float dloss, const float* dscale, int N, int V,
                         int ld, int32_t* err_flag, hipStream_t stream, const char* name) {
  if (N < 1 || V < 1 || ld < V || ld % 4 || !aligned16(logits) || !aligned16(dlogits) ||
      ld > crossentropy_fused_max_ld()) {
    set_global_error("crossentropy_fused: bad arguments (V=%d ld=%d)", V, ld);
    return -1;
  }
  ProfScope ps(name, 4.0 * N * V, 2.0 * sizeof(T) * N * ld + 12.0 * N, stream);
  const int per = (ld / 4 + XF_THREADS - 1) / XF_THREADS;  // vectors of 4 per thread
#define XF_LAUNCH(CH)                                                                      \
  xent_fused_kernel<T, CH><<<N, XF_THREADS, 0, stream>>>(losses, lse, dlogits, logits,     \
                                                         targets, dloss, dscale, V, ld, err_flag)
  if (per <= 1) XF_LAUNCH(1);
  else if (per <= 2) XF_LAUNCH(2);
  else if (per <= 4) XF_LAUNCH(4);
  else if (per <= 8) XF_LAUNCH(8);
  else if (per <= 13) XF_LAUNCH(13);
  else XF_LAUNCH(16);
#undef XF_LAUNCH
  GPT2_HIP_OK(hipGetLastError());
  return 0;
}
}  // namespace

int crossentropy_forward(float* losses, float* lse, const float* logits, const int32_t* targets,
                         int N, int V, int ld, int32_t* err_flag, hipStream_t stream) {
  return crossentropy_forward_t(losses, lse, logits, targets, N, V, ld, err_flag, stream,
                                "xent_fwd_kernel");
}
int crossentropy_forward(float* losses, float* lse, const bf16_t* logits, const int32_t* targets,
                         int N, int V, int ld, int32_t* err_flag, hipStream_t stream) {
  return crossentropy_forward_t(losses, lse, logits, targets, N, V, ld, err_flag, stream,
                                "xent_fwd_bf16_kernel");
}
int crossentropy_backward(float* logits, const float* lse, const int32_t* targets, float dloss,
                          int N, int V, int ld, hipStream_t stream) {
  return crossentropy_backward_t(logits, lse, targets, dloss, (const float*)nullptr, N, V, ld,
                                 stream, "xent_bwd_kernel");
}
int crossentropy_backward(bf16_t* logits, const float* lse, const int32_t* targets, float dloss,
                          int N, int V, int ld, hipStream_t stream) {
  return crossentropy_backward_t(logits, lse, targets, dloss, (const float*)nullptr, N, V, ld,
                                 stream, "xent_bwd_bf16_kernel");
}
int crossentropy_forward(float* losses, float* lse, const f16_t* logits, const int32_t* targets,
                         int N, int V, int ld, int32_t* err_flag, hipStream_t stream) {
  return crossentropy_forward_t(losses, lse, logits, targets, N, V, ld, err_flag, stream,
                                "xent_fwd_f16_kernel");
}
int crossentropy_backward(f16_t* logits, const float* lse, const int32_t* targets, float dloss,
                          const float* dscale, int N, int V, int ld, hipStream_t stream) {
  return crossentropy_backward_t(logits, lse, targets, dloss, dscale, N, V, ld, stream,
                                 "xent_bwd_f16_kernel");
}

int crossentropy_fused_max_ld() { return 16 * 4 * XF_THREADS; }
int crossentropy_fused(float* losses, float* lse, float* dlogits, const float* logits,
                       const int32_t* targets, float dloss, const float* dscale, int N, int V,
                       int ld, int32_t* err_flag, hipStream_t stream) {
  return crossentropy_fused_t(losses, lse, dlogits, logits, targets, dloss, dscale, N, V, ld,
                              err_flag, stream, "xent_fused_kernel");
}
int crossentropy_fused(float* losses, float* lse, bf16_t* dlogits, const bf16_t* logits,
                       const int32_t* targets, float dloss, const float* dscale, int N, int V,
                       int ld, int32_t* err_flag, hipStream_t stream) {
  return crossentropy_fused_t(losses, lse, dlogits, logits, targets, dloss, dscale, N, V, ld,
                              err_flag, stream, "xent_fused_bf16_kernel");
}
int crossentropy_fused(float* losses, float* lse, f16_t* dlogits, const f16_t* logits,
                       const int32_t* targets, float dloss, const float* dscale, int N, int V,
                       int ld, int32_t* err_flag, hipStream_t stream) {
  return crossentropy_fused_t(losses, lse, dlogits, logits, targets, dloss, dscale, N, V, ld,
                              err_flag, stream, "xent_fused_f16_kernel");
}

int mean_reduce(float* out, const float* x, int n, hipStream_t stream) {
  if (n < 1) return -1;
  ProfScope ps("mean_kernel", (double)n, 4.0 * (n + 1.0), stream);
  mean_kernel<<<1, 1024, 0, stream>>>(out, x, n);
  GPT2_HIP_OK(hipGetLastError());
  return 0;
}

namespace {
template <typename TP>
int adamw_t(float* p, const float* g, float* m, float* v, TP* pbf, size_t n, float lr,
            float beta1, float beta2, float eps, float wd, int t, const float* inv_scale,
            const int32_t* skip, hipStream_t stream) {
  if (t < 1 || !aligned16(p) || !aligned16(g) || !aligned16(m) || !aligned16(v) ||
      (pbf && ((uintptr_t)pbf & 7))) {
    set_global_error("adamw: bad arguments (t=%d)", t);
    return -1;
  }
  const long long n4 = (long long)(n / 4);
  const float inv_c1 = (float)(1.0 / (1.0 - pow((double)beta1, t)));
  const float inv_c2 = (float)(1.0 / (1.0 - pow((double)beta2, t)));
  ProfScope ps("adamw_kernel", 12.0 * n, (pbf ? 30.0 : 28.0) * n, stream);
  const long long threads = n4 + (long long)(n - 4 * n4);
  if (threads == 0) return 0;
  adamw_kernel<TP><<<(unsigned)((threads + 255) / 256), 256, 0, stream>>>(
      p, g, m, v, pbf, n4, (long long)n, lr, beta1, beta2, eps, wd, inv_c1, inv_c2, inv_scale,
      skip);
  GPT2_HIP_OK(hipGetLastError());
  return 0;
}
}  // namespace

int adamw(float* p, const float* g, float* m, float* v, bf16_t* pbf, size_t n, float lr,
          float beta1, float beta2, float eps, float wd, int t, hipStream_t stream) {
  return adamw_t(p, g, m, v, pbf, n, lr, beta1, beta2, eps, wd, t, nullptr, nullptr, stream);
}
int adamw(float* p, const float* g, float* m, float* v, f16_t* pf16, size_t n, float lr,
          float beta1, float beta2, float eps, float wd, int t, const float* inv_scale,
          const int32_t* skip, hipStream_t stream) {
  return adamw_t(p, g, m, v, pf16, n, lr, beta1, beta2, eps, wd, t, inv_scale, skip, stream);
}

int grads_nonfinite(int32_t* flag, const float* g, size_t n, hipStream_t stream) {
  if (!aligned16(g)) {
    set_global_error("grads_nonfinite: misaligned gradients");
    return -1;
  }
  const long long n4 = (long long)(n / 4), threads = n4 + (long long)(n - 4 * n4);
  if (threads == 0) return 0;
  ProfScope ps("nonfinite_kernel", 0.0, 4.0 * n, stream);
  nonfinite_kernel<<<(unsigned)((threads + 255) / 256), 256, 0, stream>>>(flag, g, n4,
                                                                         (long long)n);
  GPT2_HIP_OK(hipGetLastError());
  return 0;
}

int loss_scaler_update(float* state, int32_t* counters, int growth_interval,
                       hipStream_t stream) {
  scaler_update_kernel<<<1, 1, 0, stream>>>(state, counters, growth_interval);
  GPT2_HIP_OK(hipGetLastError());
  return 0;
}

int scale_copy(float* dst, const float* src, const float* factor, size_t n, hipStream_t stream) {
  if (n == 0) return 0;
  ProfScope ps("scale_copy_kernel", (double)n, 8.0 * n, stream);
  scale_copy_kernel<<<blocks_for((long long)n, 256, 16384), 256, 0, stream>>>(dst, src, factor,
                                                                              (long long)n);
  GPT2_HIP_OK(hipGetLastError());
  return 0;
}

int cast_f32_to_bf16(bf16_t* dst, const float* src, size_t n, hipStream_t stream) {
  if (((uintptr_t)dst & 7) || !aligned16(src)) {
    set_global_error("cast: misaligned buffers");
    return -1;
  }
  if (n == 0) return 0;
  ProfScope ps("cast_kernel", 0.0, 6.0 * n, stream);
  cast_kernel<<<blocks_for((long long)n / 4 + 1, 256, 16384), 256, 0, stream>>>(dst, src,
                                                                                 (long long)n);
  GPT2_HIP_OK(hipGetLastError());
  return 0;
}

int cast_f32_to_f16(f16_t* dst, const float* src, size_t n, hipStream_t stream) {
  if (((uintptr_t)dst & 7) || !aligned16(src)) {
    set_global_error("cast: misaligned buffers");
    return -1;
  }
  if (n == 0) return 0;
  ProfScope ps("cast_kernel", 0.0, 6.0 * n, stream);
  cast_kernel<<<blocks_for((long long)n / 4 + 1, 256, 16384), 256, 0, stream>>>(dst, src,
                                                                                 (long long)n);
  GPT2_HIP_OK(hipGetLastError());
  return 0;
}

int cast_f16_to_f32(float* dst, const f16_t* src, size_t n, hipStream_t stream) {
  if (!aligned16(dst) || ((uintptr_t)src & 7)) {
    set_global_error("cast: misaligned buffers");
    return -1;
  }
  if (n == 0) return 0;
  ProfScope ps("cast_kernel", 0.0, 6.0 * n, stream);
  cast_kernel<<<blocks_for((long long)n / 4 + 1, 256, 16384), 256, 0, stream>>>(dst, src,
                                                                                 (long long)n);
  GPT2_HIP_OK(hipGetLastError());
  return 0;
}

int cast_bf16_to_f32(float* dst, const bf16_t* src, size_t n, hipStream_t stream) {
  if (!aligned16(dst) || ((uintptr_t)src & 7)) {
    set_global_error("cast: misaligned buffers");
    return -1;
  }
  if (n == 0) return 0;
  ProfScope ps("cast_kernel", 0.0, 6.0 * n, stream);
  cast_kernel<<<blocks_for((long long)n / 4 + 1, 256, 16384), 256, 0, stream>>>(dst, src,
                                                                                 (long long)n);
  GPT2_HIP_OK(hipGetLastError());
  return 0;
}

}  // namespace gpt2
