// gemm_bf16.hip -- the GEMMs of the mixed-precision step: bf16 operands, fp32 accumulation
// (v_mfma_f32_32x32x16_bf16 on gfx950), bf16 or fp32 results.
//
// Same three storage patterns as the fp32 GEMMs ("llm.c 的中文注解-20240421", sections 1.5
// and 1.6), C = op(A) . op(B):
//   forward      out  = inp . W^T   A (M,K) row-major, B = W stored (N,K)
//   grad input   dinp = dout . W    A (M,K) row-major, B = W stored (K,N)   (b_trans)
//   grad weight  dW  += dout^T.inp  A = dout stored (K,M), B = inp (K,N)   (a_trans, b_trans)
// and the same fused epilogues (bias, bias+GELU, bias+residual, fp32 accumulate into the
// master gradients, GELU backward), computed in fp32 and rounded once to bf16 on store.
//
// Tiling: 256-thread workgroups own 128x128 tiles of C, each wave a 64x64 sub-tile (2x2
// MFMA blocks of 32x32); K advances 64 at a time through one LDS buffer per operand. Both
// operands sit in LDS as [row][k] with k contiguous (128-byte rows), because each lane of
// the bf16 MFMA supplies 8 consecutive k of one row. Operands stored with K contiguous are
// copied in 16-byte pieces; operands stored (K, rows) are transposed on the way: a thread
// loads 4 k-rows of 8 consecutive row elements and writes 8 rows of 4 k (8 bytes each).
// The 16-byte chunks of row r are placed at chunk c ^ ((r ^ r/8) & 7), which keeps both the
// fragment reads (32 rows, same chunk) and the transposing writes (rows 8 apart) spread
// over the LDS banks.
// The MFMA takes the B tile as its first operand, so a lane ends up holding four runs of 4
// consecutive output columns of one row: epilogue loads and stores are 8- or 16-byte
// vectors.
#include <cmath>
#include <cstdio>
#include <cstring>

#include "kernels.h"

namespace gpt2 {
namespace {

constexpr int BM = 128, BN = 128, BK = 64;
constexpr int NTHREADS = 256;
constexpr int GROUP_M = 8;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

struct Args {
  const bf16_t* A;
  const bf16_t* B;
  void* C;
  bf16_t* C2;
  const bf16_t* R;
  const float* bias;
  float* colsum;
  int lda, ldb, ldc;
  int M, N, K;
  int k_split;
  int splits;
  long long c_zstride;
  long long colsum_zstride;
};

GPT2_DEVICE_INLINE int swz(int row) { return (row ^ (row >> 3)) & 7; }
// bf16 offset of the 16-byte chunk c (8 k values) of LDS row `row`
GPT2_DEVICE_INLINE int lds_off(int row, int c) { return row * BK + ((c ^ swz(row)) << 3); }

// zero the 16-bit halves of x whose k index (k0 + 2*i + half) is >= kend
GPT2_DEVICE_INLINE uint32_t mask_pair(uint32_t x, int k, int kend) {
  const uint32_t lo = k < kend ? 0xFFFFu : 0u, hi = k + 1 < kend ? 0xFFFF0000u : 0u;
  return x & (lo | hi);
}

// word 3 of a raw (untyped, unswizzled) buffer resource on gfx9-family GPUs
constexpr int kBufferFlags = 0x00020000;

// A slab of an interior tile (no row past the operand's edge) wholly below kend is loaded
// with buffer loads from a scalar per-slab base: a per-thread 32-bit byte offset computed
// once (`init`) plus a uniform offset per load, so no vector ALU goes to addresses. Other
// slabs take `load`, which clamps their indices. The host keeps the byte offsets below 2^32.
template <bool TRANS>
struct SlabLoader {
  u32x4 v[4];
  int k0, kend;
  uint32_t voff;        // byte offset of this thread's first piece from the slab base
  const bf16_t* base0;  // !TRANS: row row0 of the operand; TRANS: column row0
  int ld;

  __device__ __forceinline__ void init(const bf16_t* __restrict__ P, int ld_, int row0,
                                       int tid) {
    ld = ld_;
    if (!TRANS) voff = (uint32_t)((tid >> 3) * ld + 8 * (tid & 7)) * 2u;
    else voff = (uint32_t)(4 * (tid >> 4) * ld + 8 * (tid & 15)) * 2u;
    base0 = TRANS ? P + row0 : P + (long long)row0 * ld;
  }

  __device__ __forceinline__ void load_full(int k0_, int kend_) {
    k0 = k0_;
    kend = kend_;
    const bf16_t* b = TRANS ? base0 + (long long)k0 * ld : base0 + k0;
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<bf16_t*>(b), (short)0, -1, kBufferFlags);
    // !TRANS: piece i is 32 rows further; TRANS: piece j is one k row further
    const int step = TRANS ? ld * 2 : 64 * ld;
#pragma unroll
    for (int i = 0; i < 4; i++)
      v[i] = __builtin_bit_cast(u32x4,
                                __builtin_amdgcn_raw_buffer_load_b128(rs, voff, i * step, 0));
  }

  // !TRANS: operand stored (rows, K): thread -> rows tid/8 + 32i, k chunk tid%8 (8 k)
  //  TRANS: operand stored (K, rows): thread -> k rows 4*(tid/16) .. +3, rows 8*(tid%16) .. +7
  __device__ __forceinline__ void load(const bf16_t* __restrict__ P, int ld, int row0,
                                       int rows, int k0_, int kend_, int tid) {
    k0 = k0_;
    kend = kend_;
    if (!TRANS) {
      const int c = tid & 7;
      const int kc = min(k0 + 8 * c, (kend - 1) & ~7);
#pragma unroll
      for (int i = 0; i < 4; i++) {
        const int r = min(row0 + (tid >> 3) + 32 * i, rows - 1);
        v[i] = *reinterpret_cast<const u32x4*>(P + (long long)r * ld + kc);
      }
    } else {
      const int rg = tid & 15, kq = tid >> 4;
      const int r = min(row0 + 8 * rg, (rows - 1) & ~7);
#pragma unroll
      for (int j = 0; j < 4; j++) {
        const int k = min(k0 + 4 * kq + j, kend - 1);
        v[j] = *reinterpret_cast<const u32x4*>(P + (long long)k * ld + r);
      }
    }
  }

  // `tail`: this slab reaches past kend (the same for the whole workgroup)
  __device__ __forceinline__ void store(bf16_t* S, int tid, bool tail) const {
    if (!TRANS) {
      const int c = tid & 7;
      const int kg = k0 + 8 * c;
#pragma unroll
      for (int i = 0; i < 4; i++) {
        const int row = (tid >> 3) + 32 * i;
        u32x4 x = v[i];
        if (tail) {
#pragma unroll
          for (int q = 0; q < 4; q++) x[q] = mask_pair(x[q], kg + 2 * q, kend);
        }
        *reinterpret_cast<u32x4*>(S + lds_off(row, c)) = x;
      }
    } else {
      const int rg = tid & 15, kq = tid >> 4;
      const int kg = k0 + 4 * kq;
      u32x4 x[4];
#pragma unroll
      for (int j = 0; j < 4; j++) x[j] = (!tail || kg + j < kend) ? v[j] : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
      for (int e = 0; e < 8; e++) {
        const int q = e >> 1;
        uint32_t lo, hi;
        if ((e & 1) == 0) {
          lo = (x[0][q] & 0xFFFFu) | (x[1][q] << 16);
          hi = (x[2][q] & 0xFFFFu) | (x[3][q] << 16);
        } else {
          lo = (x[0][q] >> 16) | (x[1][q] & 0xFFFF0000u);
          hi = (x[2][q] >> 16) | (x[3][q] & 0xFFFF0000u);
        }
        const int row = 8 * rg + e;
        *reinterpret_cast<u32x2*>(S + lds_off(row, kq >> 1) + 4 * (kq & 1)) = u32x2{lo, hi};
      }
    }
  }
};

// Epilogue of four consecutive columns n..n+3 of row m (n % 4 == 0, m < M, n < N).
template <int EPI, bool CF32>
__device__ __forceinline__ void epilogue4(const Args& g, void* Cv, int m, int n, f32x4 v) {
  const long long off = (long long)m * g.ldc + n;
  const int cnt = min(4, g.N - n);
  if (EPI == EPI_STORE || EPI == EPI_GELU || EPI == EPI_RESID) {
    if (g.bias) {
      if (cnt == 4) {
        v += *reinterpret_cast<const f32x4*>(g.bias + n);
      } else {
        for (int j = 0; j < cnt; j++) v[j] += g.bias[n + j];
      }
    }
  }
  if (EPI == EPI_RESID || EPI == EPI_GELU_BWD) {
    f32x4 r;
    if (cnt == 4) {
      r = ld4(g.R + off);
    } else {
      for (int j = 0; j < 4; j++) r[j] = j < cnt ? bf16_to_f32(g.R[off + j]) : 0.f;
    }
    if (EPI == EPI_RESID) v += r;
    else
#pragma unroll
      for (int j = 0; j < 4; j++) v[j] *= gelu_bwd(r[j]);
  }
  if (CF32) {
    float* C = static_cast<float*>(Cv);
    if (cnt == 4) {
      if (EPI == EPI_ACCUM) v += *reinterpret_cast<const f32x4*>(C + off);
      *reinterpret_cast<f32x4*>(C + off) = v;
    } else {
      for (int j = 0; j < cnt; j++) C[off + j] = EPI == EPI_ACCUM ? C[off + j] + v[j] : v[j];
    }
  } else {
    bf16_t* C = static_cast<bf16_t*>(Cv);
    if (cnt == 4) {
      st4(C + off, v);
      if (EPI == EPI_GELU)
        st4(g.C2 + off, f32x4{gelu_fwd(v[0]), gelu_fwd(v[1]), gelu_fwd(v[2]),
                                       gelu_fwd(v[3])});
    } else {
      for (int j = 0; j < cnt; j++) {
        C[off + j] = f32_to_bf16(v[j]);
        if (EPI == EPI_GELU) g.C2[off + j] = f32_to_bf16(gelu_fwd(v[j]));
      }
    }
  }
}

template <bool AT, bool BT, bool CF32, int EPI>
__global__ __launch_bounds__(NTHREADS, 3) void gemm_bf16_kernel(Args g) {
  __shared__ __attribute__((aligned(16))) bf16_t As[1][BM * BK];
  __shared__ __attribute__((aligned(16))) bf16_t Bs[1][BN * BK];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int r = lane & 31, h = lane >> 5;
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
  const int nslabs = (klen + BK - 1) / BK;

  f32x16 acc[2][2];
#pragma unroll
  for (int a = 0; a < 2; a++)
#pragma unroll
    for (int b = 0; b < 2; b++)
#pragma unroll
      for (int i = 0; i < 16; i++) acc[a][b][i] = 0.f;

  // One LDS buffer (32 KB), so three workgroups fit on a CU: the next slab's global loads
  // are issued into registers before the current slab's MFMAs and written to LDS after a
  // barrier.
  SlabLoader<AT> la;
  SlabLoader<BT> lb;
  la.init(g.A, g.lda, m0, tid);
  lb.init(g.B, g.ldb, n0, tid);
  const bool interior = m0 + BM <= g.M && n0 + BN <= g.N;  // uniform
  auto load_slab = [&](int k0) {
    if (interior && k0 + BK <= kend) {  // uniform
      la.load_full(k0, kend);
      lb.load_full(k0, kend);
    } else {
      la.load(g.A, g.lda, m0, g.M, k0, kend, tid);
      lb.load(g.B, g.ldb, n0, g.N, k0, kend, tid);
    }
  };
  auto compute = [&]() {
    // the compiler's MFMA / LDS-read interleaving strategy 1 (measured 1% faster per step
    // than its default schedule on the 774M shapes; strategy 0 and explicit prefetch depth
    // 2 or 3 were slower)
    __builtin_amdgcn_iglp_opt(1);
#pragma unroll
    for (int ks = 0; ks < BK / 16; ks++) {
      const int c = 2 * ks + h;
      bf16x8 af[2], bfr[2];
#pragma unroll
      for (int q = 0; q < 2; q++) {
        af[q] = *reinterpret_cast<const bf16x8*>(&As[0][lds_off(wm0 + 32 * q + r, c)]);
        bfr[q] = *reinterpret_cast<const bf16x8*>(&Bs[0][lds_off(wn0 + 32 * q + r, c)]);
      }
#pragma unroll
      for (int tm = 0; tm < 2; tm++)
#pragma unroll
        for (int tn = 0; tn < 2; tn++)
          acc[tm][tn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr[tn], af[tm], acc[tm][tn],
                                                                0, 0, 0);
    }
    if (do_colsum) {  // row m of the A tile, k chunks 4*half .. 4*half+3 of this slab
      const int m = tid & (BM - 1), half = tid >> 7;
#pragma unroll
      for (int cc = 0; cc < 4; cc++) {
        const u32x4 x = *reinterpret_cast<const u32x4*>(&As[0][lds_off(m, 4 * half + cc)]);
#pragma unroll
        for (int q = 0; q < 4; q++)
          csum += __uint_as_float(x[q] << 16) + __uint_as_float(x[q] & 0xFFFF0000u);
      }
    }
  };
  if (nslabs > 0) {
    load_slab(kbeg);
    la.store(As[0], tid, kbeg + BK > kend);
    lb.store(Bs[0], tid, kbeg + BK > kend);
  }
  __syncthreads();
  for (int kt = 0; kt < nslabs; kt++) {
    const bool more = kt + 1 < nslabs;
    if (more) load_slab(kbeg + (kt + 1) * BK);
    compute();
    __syncthreads();
    if (more) {
      const bool tail = kbeg + (kt + 2) * BK > kend;
      la.store(As[0], tid, tail);
      lb.store(Bs[0], tid, tail);
      __syncthreads();
    }
  }

  if (do_colsum) {
    float* red = reinterpret_cast<float*>(&As[0][0]);
    if (tid >= BM) red[tid - BM] = csum;
    __syncthreads();
    if (tid < BM && m0 + tid < g.M) {
      const float total = csum + red[tid];
      if (g.colsum_zstride) g.colsum[(long long)z * g.colsum_zstride + m0 + tid] = total;
      else g.colsum[m0 + tid] += total;
    }
  }

  void* C = CF32 ? static_cast<void*>(static_cast<float*>(g.C) + (long long)z * g.c_zstride)
                 : g.C;
  // acc[tm][tn][4q + j]: row m = m0 + wm0 + 32 tm + r, column n = n0 + wn0 + 32 tn + 8q + 4h + j
#pragma unroll
  for (int tm = 0; tm < 2; tm++) {
    const int m = m0 + wm0 + 32 * tm + r;
    if (m >= g.M) continue;
#pragma unroll
    for (int tn = 0; tn < 2; tn++)
#pragma unroll
      for (int q = 0; q < 4; q++) {
        const int n = n0 + wn0 + 32 * tn + 8 * q + 4 * h;
        if (n >= g.N) continue;
        epilogue4<EPI, CF32>(g, C, m, n,
                             f32x4{acc[tm][tn][4 * q], acc[tm][tn][4 * q + 1],
                                   acc[tm][tn][4 * q + 2], acc[tm][tn][4 * q + 3]});
      }
  }
}

// Adds `splits` fp32 partials (each M x N, row stride wld) in split order, then applies the
// epilogue into the real output; four consecutive columns per thread.
// With colsum_part, the last workgroups instead add the per-split column sums (split order)
// into g.colsum.
template <int EPI, bool CF32>
__global__ void split_reduce_bf16_kernel(Args g, const float* __restrict__ ws, int splits,
                                         int wld, const float* __restrict__ colsum_part) {
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
  const long long total = (long long)g.M * N4;
  const long long zstride = (long long)g.M * wld;
  for (long long idx = (long long)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
       idx += (long long)nb * blockDim.x) {
    const int m = (int)(idx / N4), n = 4 * (int)(idx % N4);
    const float* src = ws + (long long)m * wld + n;
    f32x4 s = {0.f, 0.f, 0.f, 0.f};
    int z = 0;
    for (; z + 4 <= splits; z += 4) {
      const f32x4 p0 = *reinterpret_cast<const f32x4*>(src + (long long)(z + 0) * zstride);
      const f32x4 p1 = *reinterpret_cast<const f32x4*>(src + (long long)(z + 1) * zstride);
      const f32x4 p2 = *reinterpret_cast<const f32x4*>(src + (long long)(z + 2) * zstride);
      const f32x4 p3 = *reinterpret_cast<const f32x4*>(src + (long long)(z + 3) * zstride);
      s += p0;
      s += p1;
      s += p2;
      s += p3;
    }
    for (; z < splits; z++) s += *reinterpret_cast<const f32x4*>(src + (long long)z * zstride);
    epilogue4<EPI, CF32>(g, g.C, m, n, s);
  }
}


template <bool AT, bool BT, bool CF32>
void launch_epi(const Args& a, int epi, dim3 grid, hipStream_t s) {
  switch (epi) {
    case EPI_STORE: gemm_bf16_kernel<AT, BT, CF32, EPI_STORE><<<grid, NTHREADS, 0, s>>>(a); break;
    case EPI_GELU: gemm_bf16_kernel<AT, BT, false, EPI_GELU><<<grid, NTHREADS, 0, s>>>(a); break;
    case EPI_RESID: gemm_bf16_kernel<AT, BT, false, EPI_RESID><<<grid, NTHREADS, 0, s>>>(a); break;
    case EPI_ACCUM: gemm_bf16_kernel<AT, BT, true, EPI_ACCUM><<<grid, NTHREADS, 0, s>>>(a); break;
    case EPI_GELU_BWD: gemm_bf16_kernel<AT, BT, false, EPI_GELU_BWD><<<grid, NTHREADS, 0, s>>>(a); break;
  }
}

template <bool AT, bool BT>
void launch_c(const Args& a, int epi, bool cf32, dim3 grid, hipStream_t s) {
  if (cf32) launch_epi<AT, BT, true>(a, epi, grid, s);
  else launch_epi<AT, BT, false>(a, epi, grid, s);
}

void launch(const Args& a, bool at, bool bt, int epi, bool cf32, dim3 grid, hipStream_t s) {
  if (!at && !bt) launch_c<false, false>(a, epi, cf32, grid, s);
  else if (!at && bt) launch_c<false, true>(a, epi, cf32, grid, s);
  else if (at && bt) launch_c<true, true>(a, epi, cf32, grid, s);
  else launch_c<true, false>(a, epi, cf32, grid, s);
}

int ceil_div(long long a, long long b) { return (int)((a + b - 1) / b); }

// K splits from a wave-quantisation cost model (three 256-thread workgroups per CU, 768
// slots), compute at half the bf16 MFMA peak, split partials and their reduction at 5 TB/s.
int choose_splits(const GemmBf16& g) {
  const double tiles = (double)ceil_div(g.M, BM) * ceil_div(g.N, BN);
  const int kt = ceil_div(g.K, BK);
  const double mn = (double)g.M * g.N;
  const double t_mfma = 2.0 * mn * g.K / (0.5 * 2516.6e12);
  double best = 1e30;
  int best_s = 1;
  for (int s = 1; s <= 16; s++) {
    const int kper = ceil_div(kt, s);
    if (s > 1 && kper < 4) break;
    if (s > 1 && ceil_div(kt, kper) != s) continue;
    const double rounds = tiles * s / 768.0;
    const double q = std::ceil(rounds) / rounds;
    double cost = t_mfma * q;
    if (s > 1) cost += 4.0 * mn * (s + 2.0) / 5e12;
    if (cost < best * 0.95) {
      best = cost;
      best_s = s;
    }
  }
  return best_s;
}

int split_ld(int N) { return (N + 3) & ~3; }

bool aligned16(const void* p) { return ((uintptr_t)p & 15) == 0; }

}  // namespace

size_t gemm_bf16_workspace_floats(const GemmBf16& g) {
  const int s = choose_splits(g);
  if (s <= 1) return 0;
  return (size_t)s * g.M * split_ld(g.N) + (g.colsum ? (size_t)s * g.M : 0);
}

int gemm_bf16(const GemmBf16& g, float* workspace, size_t ws_floats, hipStream_t stream) {
  if (g.M <= 0 || g.N <= 0 || g.K <= 0) {
    set_global_error("gemm_bf16: non-positive size M=%d N=%d K=%d", g.M, g.N, g.K);
    return -1;
  }
  // 16-byte operand loads need 16-byte aligned bases and leading dimensions that are
  // multiples of 8 elements; the epilogue's vector stores need ldc % 8 (bf16) or % 4 (fp32)
  const bool cf32 = g.epi == EPI_ACCUM;
  const int a_cols = g.a_trans ? g.M : g.K, b_cols = g.b_trans ? g.N : g.K;
  // (and leading dimensions below 2^24, so a slab's per-thread byte offsets fit 32 bits)
  if (!aligned16(g.A) || !aligned16(g.B) || !aligned16(g.C) || g.lda % 8 || g.ldb % 8 ||
      g.ldc % (cf32 ? 4 : 8) || g.lda < a_cols || g.ldb < b_cols || g.ldc < g.N ||
      (g.bias && !aligned16(g.bias)) || g.lda >= (1 << 24) || g.ldb >= (1 << 24)) {
    set_global_error("gemm_bf16: unsupported alignment or leading dimension (lda=%d ldb=%d "
                     "ldc=%d)", g.lda, g.ldb, g.ldc);
    return -1;
  }
  if ((g.epi == EPI_GELU && !g.C2) || ((g.epi == EPI_RESID || g.epi == EPI_GELU_BWD) && !g.R) ||
      (g.colsum && !g.a_trans)) {
    set_global_error("gemm_bf16: epilogue %d is missing an operand", (int)g.epi);
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
  if (splits > 1 && (!workspace || ws_floats < gemm_bf16_workspace_floats(g))) splits = 1;
  const int kt = ceil_div(g.K, BK);
  const int kt_per = ceil_div(kt, splits);
  splits = ceil_div(kt, kt_per);
  a.k_split = kt_per * BK;
  a.splits = splits;
  const int tiles = ceil_div(g.M, BM) * ceil_div(g.N, BN);

  const double MN = (double)g.M * g.N;
  const double flop = 2.0 * MN * g.K;
  const double in_bytes = 2.0 * ((double)g.M * g.K + (double)g.N * g.K);
  const double cb = cf32 ? 4.0 : 2.0;
  const double out_bytes = g.epi == EPI_STORE ? cb * MN : 2.0 * cb * MN;
  char name[80];
  if (splits == 1) {
    snprintf(name, sizeof(name), "gemm_bf16_kernel<%d,%d,%d>", (int)g.a_trans, (int)g.b_trans,
             (int)g.epi);
    if (profiling_detail())
      snprintf(name + strlen(name), sizeof(name) - strlen(name), " %dx%dx%d", g.M, g.N, g.K);
    ProfScope ps(name, flop, in_bytes + out_bytes, stream);
    launch(a, g.a_trans, g.b_trans, g.epi, cf32, dim3(tiles), stream);
  } else {
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
    snprintf(name, sizeof(name), "gemm_bf16_kernel<%d,%d,0>", (int)g.a_trans, (int)g.b_trans);
    if (profiling_detail())
      snprintf(name + strlen(name), sizeof(name) - strlen(name), " %dx%dx%d/%d", g.M, g.N, g.K,
               splits);
    {
      ProfScope ps(name, flop, in_bytes + 4.0 * MN * splits, stream);
      launch(p, g.a_trans, g.b_trans, EPI_STORE, true, dim3(tiles * splits), stream);
    }
    const long long total = (long long)g.M * ((g.N + 3) / 4);
    int blocks = (int)((total + 255) / 256);
    if (blocks > 8192) blocks = 8192;
    snprintf(name, sizeof(name), "split_reduce_bf16_kernel<%d>", (int)g.epi);
    const float* cp = g.colsum ? colsum_part : nullptr;
    const int nblk = blocks + (cp ? ceil_div(g.M, 256) : 0);
    ProfScope ps(name, 0.0, 4.0 * MN * splits + out_bytes + (cp ? 4.0 * (splits + 2.0) * g.M : 0.0),
                 stream);
    switch (g.epi) {
      case EPI_ACCUM: split_reduce_bf16_kernel<EPI_ACCUM, true><<<nblk, 256, 0, stream>>>(a, workspace, splits, p.ldc, cp); break;
      case EPI_GELU_BWD: split_reduce_bf16_kernel<EPI_GELU_BWD, false><<<nblk, 256, 0, stream>>>(a, workspace, splits, p.ldc, cp); break;
      case EPI_GELU: split_reduce_bf16_kernel<EPI_GELU, false><<<nblk, 256, 0, stream>>>(a, workspace, splits, p.ldc, cp); break;
      case EPI_RESID: split_reduce_bf16_kernel<EPI_RESID, false><<<nblk, 256, 0, stream>>>(a, workspace, splits, p.ldc, cp); break;
      default: split_reduce_bf16_kernel<EPI_STORE, false><<<nblk, 256, 0, stream>>>(a, workspace, splits, p.ldc, cp); break;
    }
  }
  GPT2_HIP_OK(hipGetLastError());
  return 0;
}

}  // namespace gpt2
