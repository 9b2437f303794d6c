// gemm.hip -- fp32 GEMMs of the training step on gfx950 MFMA (v_mfma_f32_32x32x2_f32).
//
// Every linear layer of "llm.c 的中文注解-20240421" (section 1.5 matmul_forward,
// section 1.6 matmul_backward) is one of three storage patterns of C = A . B:
//   forward      out  = inp . W^T   A (M,K) row-major, B = W stored (N,K)     ("NT")
//   grad input   dinp = dout . W    A (M,K) row-major, B = W stored (K,N)     ("NN")
//   grad weight  dW  += dout^T.inp  A = dout stored (K,M), B = inp (K,N)      ("TN")
// with fused epilogues: bias, bias+GELU (section 1.9), bias+residual (section 1.11),
// accumulate, and the GELU backward (section 1.10).
//
// Tiling: a 256-thread workgroup owns a 128x128 tile of C; its four waves own 64x64
// sub-tiles, i.e. 2x2 MFMA blocks of 32x32. K advances 16 at a time through two LDS
// buffers: global loads for the next K-slab are issued before the MFMAs of the current one
// and written to the other buffer afterwards, so one barrier per slab suffices.
// LDS holds both operands K-major ([k][m] and [k][n], row stride 130 floats): a lane's two
// MFMA blocks along M take adjacent rows m = 2r and 2r+1, so one 8-byte LDS read feeds two
// MFMAs, and the results are un-interleaved in the epilogue.
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>

#include "kernels.h"

namespace gpt2 {
namespace {

#ifndef GPT2_GEMM_BK
#define GPT2_GEMM_BK 16
#endif
constexpr int BM = 128, BN = 128, BK = GPT2_GEMM_BK;
constexpr int LDSA = BM + 2, LDSB = BN + 2;
constexpr int NTHREADS = 256;

struct Args {
  const float* A;
  const float* B;
  float* C;
  float* C2;
  const float* R;
  const float* bias;
  int lda, ldb, ldc;
  int M, N, K;
  float* colsum;     // see Gemm::colsum (or its per-split partials)
  int k_split;       // K elements per split (multiple of BK)
  int splits;
  long long c_zstride;       // floats between the partial outputs of successive splits
  long long colsum_zstride;  // floats between per-split colsum partials (0: accumulate)
};

constexpr int GROUP_M = 8;  // m-tiles that sweep the n-tiles together (L2 reuse of A and B)
// word 3 of a raw (untyped, unswizzled) buffer resource on gfx9-family GPUs
constexpr int kBufferFlags = 0x00020000;

// Loads one K-slab of an operand into registers (4 float4 per thread) and later stores it to
// LDS in [k][row] order. `rows` is M (for A) or N (for B).
//  trans == false: operand stored (rows, K) row-major: thread -> (row = tid/8 + 32i, k4 = tid%8)
//  trans == true : operand stored (K, rows):          thread -> (k = tid/32 + 8i, r4 = tid%32)
// The loads carry no branches and no use of their values before the LDS store, so all eight
// of a thread's loads stay in flight across the MFMAs of the current slab. Addresses are
// clamped into the operand: a row past `rows` reads the last row (its products only reach
// outputs that are never stored). A slab that lies wholly below `kend` is loaded from a
// uniform per-slab base plus per-thread byte offsets computed once (`init`), with no clamps
// or masks; only a slab that reaches past `kend` clamps its K indices (to a valid element
// whose value is replaced by zero when the slab is written to LDS). The host keeps the byte
// offsets below 2^32.
template <bool TRANS>
struct SlabLoader {
  // float4 loads per thread per slab: 128 x BK floats / (256 threads x 4)
  static constexpr int NV = BM * BK / (4 * NTHREADS);
  static constexpr int F4_PER_ROW = BK / 4;              // !TRANS: float4s along K per row
  static constexpr int ROWS_PER_PASS = NTHREADS / F4_PER_ROW;
  static constexpr int K_PER_PASS = NTHREADS / (BM / 4);  // TRANS: K rows per pass (8)
  f32x4 v[NV];
  int k0, kend;
  uint32_t voff[NV];  // byte offsets of this thread's float4s from the slab base
  const float* base0;  // !TRANS: row row0 of the operand; TRANS: the operand itself
  int ld;

  __device__ __forceinline__ void init(const float* __restrict__ P, int ld_, int row0, int rows,
                                       int tid) {
    ld = ld_;
#pragma unroll
    for (int i = 0; i < NV; i++) {
      if (!TRANS) {
        const int r = min(row0 + tid / F4_PER_ROW + ROWS_PER_PASS * i, rows - 1) - row0;
        voff[i] = (uint32_t)(r * ld + 4 * (tid % F4_PER_ROW)) * 4u;
      } else {
        const int k = tid / (BM / 4) + K_PER_PASS * i;
        const int r = min(row0 + 4 * (tid % (BM / 4)), (rows - 1) & ~3);
        voff[i] = (uint32_t)(k * ld + r) * 4u;
      }
    }
    base0 = TRANS ? P : P + (long long)row0 * ld;
  }

  // a slab wholly below kend: buffer loads from a scalar base (the slab's buffer resource)
  // plus this thread's 32-bit offsets, so the loop spends no vector ALU on addresses
  __device__ __forceinline__ void load_full(int k0_, int kend_) {
    k0 = k0_;
    kend = kend_;
    const float* b = TRANS ? base0 + (long long)k0 * ld : base0 + k0;
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(b), (short)0, -1, kBufferFlags);
#pragma unroll
    for (int i = 0; i < NV; i++)
      v[i] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, voff[i], 0, 0));
  }

  __device__ __forceinline__ void load(const float* __restrict__ P, int ld, int row0, int rows,
                                       int k0_, int kend_, int tid) {
    k0 = k0_;
    kend = kend_;
#pragma unroll
    for (int i = 0; i < NV; i++) {
      if (!TRANS) {
        const int r = min(row0 + tid / F4_PER_ROW + ROWS_PER_PASS * i, rows - 1);
        const int k = min(k0 + 4 * (tid % F4_PER_ROW), (kend - 1) & ~3);
        v[i] = *reinterpret_cast<const f32x4*>(P + (long long)r * ld + k);
      } else {
        const int k = min(k0 + tid / (BM / 4) + K_PER_PASS * i, kend - 1);
        const int r = min(row0 + 4 * (tid % (BM / 4)), (rows - 1) & ~3);
        v[i] = *reinterpret_cast<const f32x4*>(P + (long long)k * ld + r);
      }
    }
  }

  template <int LDS>
  __device__ __forceinline__ void store(float (*S)[LDS], int tid) const {
    if (k0 + BK <= kend) {  // full slab (uniform): no masks
#pragma unroll
      for (int i = 0; i < NV; i++) {
        if (!TRANS) {
          const int r = tid / F4_PER_ROW + ROWS_PER_PASS * i;
          const int k = 4 * (tid % F4_PER_ROW);
#pragma unroll
          for (int j = 0; j < 4; j++) S[k + j][r] = v[i][j];
        } else {
          const int k = tid / (BM / 4) + K_PER_PASS * i;
          const int r = 4 * (tid % (BM / 4));
          *reinterpret_cast<f32x2*>(&S[k][r]) = f32x2{v[i][0], v[i][1]};
          *reinterpret_cast<f32x2*>(&S[k][r + 2]) = f32x2{v[i][2], v[i][3]};
        }
      }
      return;
    }
#pragma unroll
    for (int i = 0; i < NV; i++) {
      if (!TRANS) {
        const int r = tid / F4_PER_ROW + ROWS_PER_PASS * i;
        const int k = 4 * (tid % F4_PER_ROW);
        const int kg = k0 + k;  // global K index of element 0
#pragma unroll
        for (int j = 0; j < 4; j++) S[k + j][r] = kg + j < kend ? v[i][j] : 0.f;
      } else {
        const int k = tid / (BM / 4) + K_PER_PASS * i;
        const int r = 4 * (tid % (BM / 4));
        const bool ok = k0 + k < kend;
        *reinterpret_cast<f32x2*>(&S[k][r]) = ok ? f32x2{v[i][0], v[i][1]} : f32x2{0.f, 0.f};
        *reinterpret_cast<f32x2*>(&S[k][r + 2]) = ok ? f32x2{v[i][2], v[i][3]} : f32x2{0.f, 0.f};
      }
    }
  }
};

template <int EPI>
__device__ __forceinline__ void epilogue_pair(const Args& g, float* C, int m, int n, float v0,
                                              float v1) {
  if (m >= g.M || n >= g.N) return;
  const bool two = n + 1 < g.N;
  long long off = (long long)m * g.ldc + n;
  if (EPI == EPI_STORE || EPI == EPI_GELU || EPI == EPI_RESID) {
    if (g.bias) {
      v0 += g.bias[n];
      if (two) v1 += g.bias[n + 1];
    }
  }
  if (EPI == EPI_RESID) {
    if (two) {
      f32x2 r = *reinterpret_cast<const f32x2*>(g.R + off);
      v0 += r[0];
      v1 += r[1];
    } else {
      v0 += g.R[off];
    }
  }
  if (EPI == EPI_ACCUM) {
    if (two) {
      f32x2 c = *reinterpret_cast<const f32x2*>(C + off);
      v0 += c[0];
      v1 += c[1];
    } else {
      v0 += C[off];
    }
  }
  if (EPI == EPI_GELU_BWD) {
    if (two) {
      f32x2 r = *reinterpret_cast<const f32x2*>(g.R + off);
      v0 *= gelu_bwd(r[0]);
      v1 *= gelu_bwd(r[1]);
    } else {
      v0 *= gelu_bwd(g.R[off]);
    }
  }
  if (two) {
    *reinterpret_cast<f32x2*>(C + off) = f32x2{v0, v1};
    if (EPI == EPI_GELU) *reinterpret_cast<f32x2*>(g.C2 + off) = f32x2{gelu_fwd(v0), gelu_fwd(v1)};
  } else {
    C[off] = v0;
    if (EPI == EPI_GELU) g.C2[off] = gelu_fwd(v0);
  }
}

template <bool AT, bool BT, int EPI>
__global__ __launch_bounds__(NTHREADS, 2) void gemm_kernel(Args g) {
  __shared__ float As[2][BK][LDSA];
  __shared__ float Bs[2][BK][LDSB];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int r = lane & 31, h = lane >> 5;
  // 1-D grid: logical block -> (split z, m-tile, n-tile), XCD-local and grouped
  const int nM = (g.M + BM - 1) / BM, nN = (g.N + BN - 1) / BN;
  const int tiles = nM * nN;
  const int lid = xcd_logical_block(blockIdx.x, gridDim.x);
  const int z = lid / tiles;
  const int t = lid - z * tiles;
  const int group = t / (GROUP_M * nN);
  const int first_m = group * GROUP_M;
  const int gsz = min(nM - first_m, GROUP_M);
  const int tin = t - group * GROUP_M * nN;
  const int mt = first_m + tin % gsz, nt = tin / gsz;
  const int m0 = mt * BM, n0 = nt * BN;
  const int wm0 = (wave >> 1) * 64, wn0 = (wave & 1) * 64;
  const bool do_colsum = AT && g.colsum != nullptr && nt == 0;  // uniform per workgroup
  float csum = 0.f;

  const int kbeg = z * g.k_split;
  const int kend = min(g.K, kbeg + g.k_split);
  const int klen = kend > kbeg ? kend - kbeg : 0;
  const int ntiles = (klen + BK - 1) / BK;

  f32x16 acc[2][2];
#pragma unroll
  for (int a = 0; a < 2; a++)
#pragma unroll
    for (int b = 0; b < 2; b++)
#pragma unroll
      for (int i = 0; i < 16; i++) acc[a][b][i] = 0.f;

  SlabLoader<AT> la;
  SlabLoader<BT> lb;
  la.init(g.A, g.lda, m0, g.M, tid);
  lb.init(g.B, g.ldb, n0, g.N, tid);
  auto load_slab = [&](int kt) {
    const int k0 = kbeg + kt * BK;
    if (k0 + BK <= kend) {  // uniform
      la.load_full(k0, kend);
      lb.load_full(k0, kend);
    } else {
      la.load(g.A, g.lda, m0, g.M, k0, kend, tid);
      lb.load(g.B, g.ldb, n0, g.N, k0, kend, tid);
    }
  };
  if (ntiles > 0) {
    load_slab(0);
    la.template store<LDSA>(As[0], tid);
    lb.template store<LDSB>(Bs[0], tid);
  }
  __syncthreads();

  for (int kt = 0; kt < ntiles; kt++) {
    const int cur = kt & 1;
    const bool more = kt + 1 < ntiles;
    if (more) load_slab(kt + 1);
    // all of this slab's fragments first, then its 64 MFMAs
    f32x2 af[BK / 2], bf[BK / 2];
#pragma unroll
    for (int kk2 = 0; kk2 < BK / 2; kk2++) {
      const int kk = 2 * kk2 + h;
      af[kk2] = *reinterpret_cast<const f32x2*>(&As[cur][kk][wm0 + 2 * r]);
      bf[kk2] = *reinterpret_cast<const f32x2*>(&Bs[cur][kk][wn0 + 2 * r]);
    }
#pragma unroll
    for (int kk2 = 0; kk2 < BK / 2; kk2++) {
      acc[0][0] = mfma32x32x2(af[kk2][0], bf[kk2][0], acc[0][0]);
      acc[0][1] = mfma32x32x2(af[kk2][0], bf[kk2][1], acc[0][1]);
      acc[1][0] = mfma32x32x2(af[kk2][1], bf[kk2][0], acc[1][0]);
      acc[1][1] = mfma32x32x2(af[kk2][1], bf[kk2][1], acc[1][1]);
    }
    if (do_colsum) {  // column c of the A tile: rows 16*half .. 16*half+15 of this slab
      const int c = tid & (BM - 1), half = tid >> 7;
#pragma unroll
      for (int kk = 0; kk < BK / 2; kk++) csum += As[cur][half * (BK / 2) + kk][c];
    }
    if (more) {
      la.template store<LDSA>(As[cur ^ 1], tid);
      lb.template store<LDSB>(Bs[cur ^ 1], tid);
    }
    __syncthreads();
  }

  if (do_colsum) {
    float* red = &As[0][0][0];
    if (tid >= BM) red[tid - BM] = csum;
    __syncthreads();
    if (tid < BM && m0 + tid < g.M) {
      const float total = csum + red[tid];
      if (g.colsum_zstride) g.colsum[(long long)z * g.colsum_zstride + m0 + tid] = total;
      else g.colsum[m0 + tid] += total;
    }
  }

  float* C = g.C + (long long)z * g.c_zstride;
#pragma unroll
  for (int bm = 0; bm < 2; bm++)
#pragma unroll
    for (int i = 0; i < 16; i++) {
      const int row = 8 * (i / 4) + 4 * h + (i % 4);
      const int m = m0 + wm0 + 2 * row + bm;
      const int n = n0 + wn0 + 2 * r;
      epilogue_pair<EPI>(g, C, m, n, acc[bm][0][i], acc[bm][1][i]);
    }
}

// The epilogue `EPI` of one output element of a split-K GEMM (only EPI_STORE-with-bias,
// EPI_ACCUM and EPI_GELU_BWD are used with splits) applied to the sum s of its partials.
template <int EPI>
__device__ __forceinline__ float split_epilogue(const Args& g, long long off, int n, float s) {
  if (EPI == EPI_ACCUM) return g.C[off] + s;
  if (EPI == EPI_GELU_BWD) return s * gelu_bwd(g.R[off]);
  s += g.bias ? g.bias[n] : 0.f;
  if (EPI == EPI_RESID) s += g.R[off];
  return s;
}

// Sums `splits` partial results (each M x N, row stride wld) into C with the epilogue `EPI`,
// adding the partials in split order; four consecutive columns per thread, with all of a
// group's partial loads issued before the adds. With vec4 (ldc a multiple of 4, every output
// and epilogue operand 16-byte aligned) the epilogue reads and writes whole float4s. With
// colsum_part, the last workgroups instead add the per-split column sums (split order) into
// g.colsum. The host keeps M * ceil(N / 4) below 2^31.
template <int EPI>
__global__ __launch_bounds__(256) void split_reduce_kernel(Args g, const float* __restrict__ ws,
                                                           int splits, int wld,
                                                           const float* __restrict__ colsum_part,
                                                           int vec4) {
  // the last ceil(M / blockDim) workgroups reduce the column sums, one m per thread
  const int ncs = colsum_part ? (g.M + blockDim.x - 1) / blockDim.x : 0;
  const int nb = gridDim.x - ncs;
  if ((int)blockIdx.x >= nb) {
    const int m = (blockIdx.x - nb) * blockDim.x + threadIdx.x;
    if (m < g.M) {
      float cs = 0.f;
      for (int z = 0; z < splits; z++) cs += colsum_part[(long long)z * g.M + m];
      g.colsum[m] += cs;
    }
    return;
  }
  const int N4 = (g.N + 3) / 4;
  const int total = g.M * N4;
  const long long zstride = (long long)g.M * wld;
  for (int idx = blockIdx.x * blockDim.x + threadIdx.x; idx < total; idx += nb * blockDim.x) {
    const int m = idx / N4, n = 4 * (idx - m * N4);
    const float* src = ws + (long long)m * wld + n;
    const bool full = n + 3 < g.N;
    f32x4 s = {0.f, 0.f, 0.f, 0.f};
    int z = 0;
    if (full) {
      for (; z + 4 <= splits; z += 4) {
        f32x4 p0 = *reinterpret_cast<const f32x4*>(src + (long long)(z + 0) * zstride);
        f32x4 p1 = *reinterpret_cast<const f32x4*>(src + (long long)(z + 1) * zstride);
        f32x4 p2 = *reinterpret_cast<const f32x4*>(src + (long long)(z + 2) * zstride);
        f32x4 p3 = *reinterpret_cast<const f32x4*>(src + (long long)(z + 3) * zstride);
        s += p0;
        s += p1;
        s += p2;
        s += p3;
      }
      for (; z < splits; z++) s += *reinterpret_cast<const f32x4*>(src + (long long)z * zstride);
    } else {
      for (; z < splits; z++)
        for (int j = 0; j < 4 && n + j < g.N; j++) s[j] += src[(long long)z * zstride + j];
    }
    const long long off = (long long)m * g.ldc + n;
    if (full && vec4) {
      f32x4 v;
      if (EPI == EPI_ACCUM) {
        v = ld4(g.C + off) + s;
      } else if (EPI == EPI_GELU_BWD) {
        const f32x4 r = ld4(g.R + off);
#pragma unroll
        for (int j = 0; j < 4; j++) v[j] = s[j] * gelu_bwd(r[j]);
      } else {
        v = s;
        if (g.bias) v += ld4(g.bias + n);
        if (EPI == EPI_RESID) v += ld4(g.R + off);
      }
      st4(g.C + off, v);
      if (EPI == EPI_GELU) {
        f32x4 gv;
#pragma unroll
        for (int j = 0; j < 4; j++) gv[j] = gelu_fwd(v[j]);
        st4(g.C2 + off, gv);
      }
    } else {
#pragma unroll
      for (int j = 0; j < 4; j++) {
        if (n + j >= g.N) break;
        const float v = split_epilogue<EPI>(g, off + j, n + j, s[j]);
        g.C[off + j] = v;
        if (EPI == EPI_GELU) g.C2[off + j] = gelu_fwd(v);
      }
    }
  }
}

template <bool AT, bool BT>
void launch_tn(const Args& a, int epi, dim3 grid, hipStream_t s) {
  switch (epi) {
    case EPI_STORE: gemm_kernel<AT, BT, EPI_STORE><<<grid, NTHREADS, 0, s>>>(a); break;
    case EPI_GELU: gemm_kernel<AT, BT, EPI_GELU><<<grid, NTHREADS, 0, s>>>(a); break;
    case EPI_RESID: gemm_kernel<AT, BT, EPI_RESID><<<grid, NTHREADS, 0, s>>>(a); break;
    case EPI_ACCUM: gemm_kernel<AT, BT, EPI_ACCUM><<<grid, NTHREADS, 0, s>>>(a); break;
    case EPI_GELU_BWD: gemm_kernel<AT, BT, EPI_GELU_BWD><<<grid, NTHREADS, 0, s>>>(a); break;
  }
}

void launch(const Args& a, bool at, bool bt, int epi, dim3 grid, hipStream_t s) {
  if (!at && !bt) launch_tn<false, false>(a, epi, grid, s);
  else if (!at && bt) launch_tn<false, true>(a, epi, grid, s);
  else if (at && bt) launch_tn<true, true>(a, epi, grid, s);
  else launch_tn<true, false>(a, epi, grid, s);
}

int ceil_div(long long a, long long b) { return (int)((a + b - 1) / b); }

// Number of K splits for a problem, from a cost model fitted to measurements on MI355X.
// Four 256-thread workgroups fit on each of the 256 CUs (1024 slots). A launch of n
// workgroups runs ceil(n/1024) rounds of the same length, so relative to perfectly packed
// work it costs q = ceil(n/1024) / (n/1024); splitting K multiplies n by the split count and
// adds a pass that reads the partials and applies the epilogue (the partials themselves are
// written while the GEMM computes).
// Compute time is estimated at 90% of the fp32 MFMA peak, memory at 5 TB/s.
int choose_splits(const Gemm& g) {
#ifdef GPT2_SPLIT_OVERRIDE
  if (const char* e = getenv("GPT2_SPLITS")) return atoi(e);
#endif
  const double tiles = (double)ceil_div(g.M, BM) * ceil_div(g.N, BN);
  const int kt = ceil_div(g.K, BK);
  const double mn = (double)g.M * g.N;
  const double t_mfma = 2.0 * mn * g.K / (0.9 * 157.3e12);
  double best = 1e30;
  int best_s = 1;
  for (int s = 1; s <= 32; s++) {
    const int kper = ceil_div(kt, s);
    if (s > 1 && kper < 4) break;
    if (s > 1 && ceil_div(kt, kper) != s) continue;
    const double rounds = tiles * s / 1024.0;
    const double q = std::ceil(rounds) / rounds;
    double cost = t_mfma * q;
    if (s > 1) cost += 4.0 * mn * (s + 2.0) / 5e12;  // partials are written during the GEMM
    if (cost < best * 0.95) {  // prefer fewer splits unless clearly cheaper
      best = cost;
      best_s = s;
    }
  }
  return best_s;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15) == 0; }

}  // namespace

// partial results of a split GEMM are stored with a row stride that is a multiple of 4
// (16-byte loads in the reduction)
int split_ld(int N) { return (N + 3) & ~3; }

size_t gemm_workspace_floats(const Gemm& g) {
  int s = choose_splits(g);
  if (s <= 1) return 0;
  return (size_t)s * g.M * split_ld(g.N) + (g.colsum ? (size_t)s * g.M : 0);
}


int gemm(const Gemm& g, float* workspace, size_t ws_floats, hipStream_t stream) {
  if (g.M <= 0 || g.N <= 0 || g.K <= 0) {
    set_global_error("gemm: non-positive size M=%d N=%d K=%d", g.M, g.N, g.K);
    return -1;
  }
  // float4 operand loads: 16-byte aligned bases and leading dimensions that are multiples
  // of 4 (which also keeps the last float4 of a row inside the row's storage)
  // (and leading dimensions below 2^23, so a slab's per-thread byte offsets fit 32 bits)
  const int a_cols = g.a_trans ? g.M : g.K, b_cols = g.b_trans ? g.N : g.K;
  if (!aligned16(g.A) || !aligned16(g.B) || !aligned16(g.C) || g.lda % 4 || g.ldb % 4 ||
      g.ldc % 2 || g.lda < a_cols || g.ldb < b_cols || g.ldc < g.N || g.lda >= (1 << 23) ||
      g.ldb >= (1 << 23)) {
    set_global_error("gemm: unsupported alignment or leading dimension (lda=%d ldb=%d ldc=%d)",
                     g.lda, g.ldb, g.ldc);
    return -1;
  }
  if ((g.epi == EPI_GELU && !g.C2) || ((g.epi == EPI_RESID || g.epi == EPI_GELU_BWD) && !g.R) ||
      (g.colsum && !g.a_trans)) {
    set_global_error("gemm: epilogue %d is missing an operand", (int)g.epi);
    return -1;
  }
  Args a;
  a.A = g.A;
  a.B = g.B;
  a.C = g.C;
  a.C2 = g.C2;
  a.R = g.R;
  a.bias = g.bias;
  a.colsum = g.colsum;
  a.lda = g.lda;
  a.ldb = g.ldb;
  a.ldc = g.ldc;
  a.M = g.M;
  a.N = g.N;
  a.K = g.K;
  a.c_zstride = 0;
  a.colsum_zstride = 0;

  int splits = choose_splits(g);
  if (splits > 1 && (!workspace || ws_floats < gemm_workspace_floats(g))) splits = 1;
  const int kt = ceil_div(g.K, BK);
  const int kt_per = ceil_div(kt, splits);
  splits = ceil_div(kt, kt_per);
  a.k_split = kt_per * BK;
  a.splits = splits;
  const int tiles = ceil_div(g.M, BM) * ceil_div(g.N, BN);

  const double MN = (double)g.M * g.N;
  const double flop = 2.0 * MN * g.K;
  const double in_bytes = 4.0 * ((double)g.M * g.K + (double)g.N * g.K);
  // output traffic of an epilogue: stores, plus the extra tensor it reads or writes
  const double out_factor = g.epi == EPI_STORE ? 1.0 : 2.0;
  char name[64];
  if (splits == 1) {
    snprintf(name, sizeof(name), "gemm_kernel<%d,%d,%d>", (int)g.a_trans, (int)g.b_trans,
             (int)g.epi);
    if (profiling_detail())
      snprintf(name + strlen(name), sizeof(name) - strlen(name), " %dx%dx%d", g.M, g.N, g.K);
    ProfScope ps(name, flop, in_bytes + 4.0 * MN * out_factor, stream);
    launch(a, g.a_trans, g.b_trans, g.epi, dim3(tiles), stream);
  } else {
    // the reduction indexes the M x ceil(N/4) output groups with 32-bit integers
    const long long total = (long long)g.M * ((g.N + 3) / 4);
    if (total >= (1LL << 31) - 65536LL * 256) {
      set_global_error("gemm: split-K output too large (%d x %d)", g.M, g.N);
      return -1;
    }
    Args p = a;
    p.C = workspace;
    p.ldc = split_ld(g.N);
    p.c_zstride = (long long)g.M * p.ldc;
    p.bias = nullptr;
    float* colsum_part = workspace + (size_t)splits * g.M * p.ldc;
    if (g.colsum) {
      p.colsum = colsum_part;
      p.colsum_zstride = g.M;
    }
    snprintf(name, sizeof(name), "gemm_kernel<%d,%d,0>", (int)g.a_trans, (int)g.b_trans);
    if (profiling_detail())
      snprintf(name + strlen(name), sizeof(name) - strlen(name), " %dx%dx%d/%d", g.M, g.N, g.K,
               splits);
    {
      ProfScope ps(name, flop, in_bytes + 4.0 * MN * splits, stream);
      launch(p, g.a_trans, g.b_trans, EPI_STORE, dim3(tiles * splits), stream);
    }
    int blocks = (int)((total + 255) / 256);
    if (blocks > 65536) blocks = 65536;
    auto al = [](const void* q) { return ((uintptr_t)q & 15) == 0; };
    const int vec4 = g.ldc % 4 == 0 && al(g.C) && (!g.C2 || al(g.C2)) && (!g.R || al(g.R)) &&
                     (!g.bias || al(g.bias));
    snprintf(name, sizeof(name), "split_reduce_kernel<%d>", (int)g.epi);
    {
      const float* cp = g.colsum ? colsum_part : nullptr;
      const int nblk = blocks + (cp ? ceil_div(g.M, 256) : 0);
      ProfScope ps(name, 0.0,
                   4.0 * MN * (splits + out_factor) + (cp ? 4.0 * (splits + 2.0) * g.M : 0.0),
                   stream);
      switch (g.epi) {
        case EPI_ACCUM: split_reduce_kernel<EPI_ACCUM><<<nblk, 256, 0, stream>>>(a, workspace, splits, p.ldc, cp, vec4); break;
        case EPI_GELU_BWD: split_reduce_kernel<EPI_GELU_BWD><<<nblk, 256, 0, stream>>>(a, workspace, splits, p.ldc, cp, vec4); break;
        case EPI_GELU: split_reduce_kernel<EPI_GELU><<<nblk, 256, 0, stream>>>(a, workspace, splits, p.ldc, cp, vec4); break;
        case EPI_RESID: split_reduce_kernel<EPI_RESID><<<nblk, 256, 0, stream>>>(a, workspace, splits, p.ldc, cp, vec4); break;
        default: split_reduce_kernel<EPI_STORE><<<nblk, 256, 0, stream>>>(a, workspace, splits, p.ldc, cp, vec4); break;
      }
    }
  }
  GPT2_HIP_OK(hipGetLastError());
  return 0;
}

// ----- bias gradients: deterministic column sums -----------------------------------------
namespace {
constexpr int COLSUM_ROWS = 256;  // rows summed per workgroup before the second pass

// partial[blockIdx.y][c] = sum of x[r][c] for r in this workgroup's row chunk (ascending)
__global__ void colsum_partial_kernel(float* __restrict__ partial, const float* __restrict__ x,
                                      int N, int C, int ld) {
  const int c = blockIdx.x * blockDim.x + threadIdx.x;
  if (c >= C) return;
  const int r0 = blockIdx.y * COLSUM_ROWS;
  const int r1 = min(N, r0 + COLSUM_ROWS);
  float s = 0.f;
  for (int r = r0; r < r1; r++) s += x[(long long)r * ld + c];
  partial[(long long)blockIdx.y * C + c] = s;
}

__global__ void colsum_final_kernel(float* __restrict__ out, const float* __restrict__ partial,
                                    int chunks, int C) {
  const int c = blockIdx.x * blockDim.x + threadIdx.x;
  if (c >= C) return;
  float s = 0.f;
  for (int k = 0; k < chunks; k++) s += partial[(long long)k * C + c];
  out[c] += s;
}
}  // namespace

size_t colsum_partial_floats(int N, int C) {
  return (size_t)((N + COLSUM_ROWS - 1) / COLSUM_ROWS) * C;
}

int colsum_accumulate(float* out, const float* x, int N, int C, int ld, float* partial,
                      hipStream_t stream) {
  if (N <= 0 || C <= 0) return -1;
  const int chunks = (N + COLSUM_ROWS - 1) / COLSUM_ROWS;
  dim3 g1((C + 255) / 256, chunks);
  {
    ProfScope ps("colsum_partial_kernel", (double)N * C, 4.0 * ((double)N * C + (double)chunks * C),
                 stream);
    colsum_partial_kernel<<<g1, 256, 0, stream>>>(partial, x, N, C, ld);
  }
  ProfScope ps("colsum_final_kernel", (double)chunks * C, 4.0 * ((double)chunks * C + 2.0 * C),
               stream);
  colsum_final_kernel<<<(C + 255) / 256, 256, 0, stream>>>(out, partial, chunks, C);
  GPT2_HIP_OK(hipGetLastError());
  return 0;
}

}  // namespace gpt2
