// gemm.hip -- fp32 GEMMs of the training step on gfx950 MFMA.
//
// Every linear layer of "llm.c 的中文注解-20240421" (section 1.5 matmul_forward,
// section 1.6 matmul_backward) is one of three storage patterns of C = A . B:
//   forward      out  = inp . W^T   A (M,K) row-major, B = W stored (N,K)     ("NT")
//   grad input   dinp = dout . W    A (M,K) row-major, B = W stored (K,N)     ("NN")
//   grad weight  dW  += dout^T.inp  A = dout stored (K,M), B = inp (K,N)      ("TN")
// with fused epilogues: bias, bias+GELU (section 1.9), bias+residual (section 1.11),
// accumulate, and the GELU backward (section 1.10).
//
// Two kernels compute them, with the same epilogues and split-K planning:
// - gemm_x6_kernel (used by default): fp32 operands and fp32 accumulation, the products
//   formed on bf16 MFMA (v_mfma_f32_32x32x16_bf16) from an exact three-way bf16 split of each
//   operand value, six partial products per fp32 product, which keeps each product within
//   2^-23 of its exact value (fp32 accuracy) at 16/6 times the fp32 MFMA rate. 256x256 tiles;
//   each slab of 16 k is loaded through registers, split once per workgroup and written to
//   LDS as three bf16 planes per operand.
// - gemm_kernel: fp32 MFMA (v_mfma_f32_32x32x2_f32). A 256-thread workgroup owns a 128x128
//   tile of C; its four waves own 64x64 sub-tiles, i.e. 2x2 MFMA blocks of 32x32. K advances
//   in slabs of 16 that go from global memory straight into LDS (buffer loads with the LDS as
//   destination, no staging registers), the next slab in flight while the current one is
//   used, one LDS object per stage. An operand stored with K contiguous is kept [row][k] in
//   LDS and read 16 bytes (four k) per lane, feeding four MFMAs: the products take the K
//   order in which lane half h supplies k = 8h + s at step s. An operand stored (K, rows) is
//   kept as stored, [k][row], and read 4 bytes per lane.
// In both the MFMA takes the B fragment as its first operand, so a lane ends up holding runs
// of 4 consecutive output columns of one row: the epilogue works on float4s.
#include <cmath>
#include <cstdio>
#include <type_traits>
#include <cstdlib>
#include <cstring>

#include "kernels.h"

namespace gpt2 {
namespace {

// Slab depth (build option): K advances BK at a time through LDS.
#ifndef GPT2_GEMM_BK
#define GPT2_GEMM_BK 16
#endif
constexpr int BK = GPT2_GEMM_BK;
static_assert(BK == 16 || BK == 32, "slab depth");
constexpr int HALF = BK / 2;  // k per lane half in a slab

// Shape of one GEMM kernel: a workgroup owns BM x BN outputs; WAVES_M x WAVES_N waves own
// (BM / WAVES_M) x (BN / WAVES_N) each, i.e. TM x TN MFMA blocks of 32x32; at least OCC
// waves per SIMD (the register budget). X6 false: fp32 MFMA products, NSTAGE fp32 slabs in
// LDS. X6 true: split-operand bf16 MFMA products (see gemm_x6s_body), two LDS buffers of
// three bf16 planes per operand (NSTAGE must be 2). WG_PER_CU workgroups fit on a CU; RATE
// is the throughput (flop/s) the split planner assumes for the kernel.
template <int BM_, int BN_, int WAVES_M_, int WAVES_N_, int NSTAGE_, int OCC_, bool X6_>
struct Cfg {
  static constexpr int BM = BM_, BN = BN_, WAVES_M = WAVES_M_, WAVES_N = WAVES_N_;
  static constexpr int NWAVES = WAVES_M * WAVES_N, NTHREADS = 64 * NWAVES;
  static constexpr int TM = BM / WAVES_M / 32, TN = BN / WAVES_N / 32;
  static constexpr int NSTAGE = NSTAGE_, OCC = OCC_;
  static constexpr bool X6 = X6_;
  static constexpr int LDS_BYTES = X6 ? 2 * 3 * (BM + BN) * BK * 2 : NSTAGE * (BM + BN) * BK * 4;
  static constexpr int WG_PER_CU = (OCC * 4 / NWAVES) < (160 * 1024 / LDS_BYTES)
                                       ? OCC * 4 / NWAVES : 160 * 1024 / LDS_BYTES;
  static constexpr double RATE = X6 ? 0.4 * 2.5e15 / 6 : 0.9 * 157.3e12;
  static_assert(TM * WAVES_M * 32 == BM && TN * WAVES_N * 32 == BN, "whole MFMA blocks");
  static_assert(NSTAGE == 2 || (NSTAGE == 3 && !X6), "two or three LDS stages");
  static_assert(NTHREADS == BM || NTHREADS == 2 * BM, "column sums: one or two threads per m");
  static_assert(WG_PER_CU >= 1, "fits a CU");
};

// fp32 MFMA kernel: BM x 128 tiles (BM a build option), waves of 64 x 64, two LDS stages
// (16 KB each at BM 128) and four workgroups per CU, or three stages and three.
#ifndef GPT2_GEMM_BM
#define GPT2_GEMM_BM 128
#endif
#ifndef GPT2_GEMM_STAGES
#define GPT2_GEMM_STAGES 2
#endif
typedef Cfg<GPT2_GEMM_BM, 128, GPT2_GEMM_BM / 64, 2, GPT2_GEMM_STAGES,
            (GPT2_GEMM_STAGES == 2 ? 4 : 3) * 128 / GPT2_GEMM_BM * 16 / BK, false>
    CfgF32;
// split-operand kernel: 256 x 256 tiles of eight waves of 128 x 64 (96 KB of LDS), or
// 256 x 192 tiles of eight waves of 64 x 96 (84 KB; for output widths that 192 divides and
// 256 does not), one workgroup per CU (two waves per SIMD)
typedef Cfg<256, 256, 2, 4, 2, 2, true> CfgX6W;
typedef Cfg<256, 192, 4, 2, 2, 2, true> CfgX6N;
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

typedef __attribute__((address_space(3))) void lds_void_t;

// 16 bytes per lane from a buffer into LDS (lane l writes lds + 16 l); `lds` is wave-uniform
GPT2_DEVICE_INLINE void copy_to_lds16(__amdgpu_buffer_rsrc_t rs, char* lds, uint32_t voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void_t*)lds, 16, voff, 0, 0, 0);
}

// LDS placement of an operand stored with K contiguous: [row][k], rows of BK k (64 or 128
// bytes); the 16-byte chunk c of row r holds the row's chunk c ^ kswz(r), which spreads the
// 16-byte fragment reads (32 consecutive rows, one chunk) over all banks. An operand stored
// (K, rows) keeps that layout, [k][row], and is read 4 bytes per lane from consecutive rows
// (no conflicts, no swizzle).
GPT2_DEVICE_INLINE int kswz(int row) {
  return BK == 16 ? ((row >> 1) ^ (row >> 3)) & 3 : (row ^ (row >> 3)) & 7;
}

// One operand's share of the slab pipeline: a slab (BK k x R rows) is copied from global
// memory straight into LDS, 1 KB per wave-wide buffer load (lane l fills bytes
// 16 l .. 16 l + 15 of the KB), without passing through registers, shared among NWAVES. The
// buffer resource of a slab ends where the operand ends, so rows past its last row (and,
// for an operand stored (K, rows), k past K) read as zero; a K tail inside a row is masked
// in the fragments. The extent is clamped to 32 bits: only a slab whose extent is small
// (the last rows or the last k) ever reaches past the operand. Per-lane byte offsets are
// computed once; the host keeps them below 2^32.
template <bool TRANS, int R, int NWAVES>
struct SlabCopy {
  static constexpr int PER_WAVE = R * BK * 4 / 1024 / NWAVES;
  static_assert(PER_WAVE * NWAVES * 1024 == R * BK * 4, "whole 1 KB copies per wave");
  const char* tile;  // operand at this tile's first row (!TRANS) or column (TRANS), k = kbeg
  long long step;    // bytes between consecutive slabs
  long long remain;  // bytes from `tile` to the end of the operand
  uint32_t voff[PER_WAVE];

  __device__ __forceinline__ void init(const float* P, int ld, int row0, long long total,
                                       int wave, int lane) {
    const long long at = TRANS ? (long long)row0 : (long long)row0 * ld;
    tile = reinterpret_cast<const char*>(P + at);
    remain = 4 * (total - at);
    step = TRANS ? 4LL * BK * ld : 4LL * BK;
#pragma unroll
    for (int j = 0; j < PER_WAVE; j++) {
      const int b = (j * NWAVES + wave) * 1024 + 16 * lane;  // LDS byte within the slab
      if (!TRANS) {
        const int row = b / (4 * BK), p = (b % (4 * BK)) >> 4;
        voff[j] = (uint32_t)(row * ld + 4 * (p ^ kswz(row))) * 4u;
      } else {
        const int k = b / (4 * R), p = (b % (4 * R)) >> 4;
        voff[j] = (uint32_t)(k * ld + 4 * p) * 4u;
      }
    }
  }

  // `live` false: a copy past the last slab, given an empty range (it reads nothing and
  // writes zeros), so that every pipeline step issues the same number of copies
  __device__ __forceinline__ void issue(int kt, bool live, float* lds, int wave) const {
    const long long off = live ? (long long)kt * step : 0;
    const long long left = live ? remain - off : 0;
    const int nrec = (int)(uint32_t)(left > 0xFFFFFFFFLL ? 0xFFFFFFFFLL : left > 0 ? left : 0);
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<char*>(tile + off), (short)0, nrec, kBufferFlags);
#pragma unroll
    for (int j = 0; j < PER_WAVE; j++)
      copy_to_lds16(rs, reinterpret_cast<char*>(lds) + (j * NWAVES + wave) * 1024, voff[j]);
  }
};

// workgroup barrier without a memory fence: the slab copies still in flight must not be
// waited for here (the fence of __syncthreads would wait for all of them); the clobber keeps
// the compiler from moving LDS accesses across it
GPT2_DEVICE_INLINE void lds_barrier() { asm volatile("s_barrier" ::: "memory"); }
// wait until at most n vector-memory operations of this wave are outstanding (n < 16)
template <int n>
GPT2_DEVICE_INLINE void wait_vmcnt() {
  static_assert(n >= 0 && n < 16, "vmcnt");
  __builtin_amdgcn_s_waitcnt(0x0F70 | n);  // expcnt and lgkmcnt at their no-wait maxima
}

// Epilogue of four consecutive columns n..n+3 of row m (n % 4 == 0, m < M, n < N): bias,
// GELU, residual, accumulate or GELU backward, then the store (16-byte vectors when the
// row stride keeps them aligned).
template <int EPI>
__device__ __forceinline__ void epilogue4(const Args& g, float* C, int m, int n, f32x4 v) {
  const long long off = (long long)m * g.ldc + n;
  const int cnt = min(4, g.N - n);
  const bool vec = cnt == 4 && (g.ldc & 3) == 0;
  if (EPI == EPI_STORE || EPI == EPI_GELU || EPI == EPI_RESID) {
    if (g.bias) {
      if (cnt == 4) v += *reinterpret_cast<const f32x4*>(g.bias + n);
      else
        for (int j = 0; j < cnt; j++) v[j] += g.bias[n + j];
    }
  }
  if (EPI == EPI_RESID || EPI == EPI_GELU_BWD || EPI == EPI_ACCUM) {
    const float* src = EPI == EPI_ACCUM ? C : g.R;
    f32x4 r;
    if (vec) r = *reinterpret_cast<const f32x4*>(src + off);
    else
      for (int j = 0; j < 4; j++) r[j] = j < cnt ? src[off + j] : 0.f;
    if (EPI == EPI_GELU_BWD) {
#pragma unroll
      for (int j = 0; j < 4; j++) v[j] *= gelu_bwd(r[j]);
    } else {
      v += r;
    }
  }
  if (vec) {
    *reinterpret_cast<f32x4*>(C + off) = v;
    if (EPI == EPI_GELU)
      *reinterpret_cast<f32x4*>(g.C2 + off) =
          f32x4{gelu_fwd(v[0]), gelu_fwd(v[1]), gelu_fwd(v[2]), gelu_fwd(v[3])};
  } else {
    for (int j = 0; j < cnt; j++) {
      C[off + j] = v[j];
      if (EPI == EPI_GELU) g.C2[off + j] = gelu_fwd(v[j]);
    }
  }
}

// zero the elements of a 4-k fragment at or past `lim` (its first element being k = 0)
GPT2_DEVICE_INLINE f32x4 kmask4(f32x4 v, int lim) {
#pragma unroll
  for (int e = 0; e < 4; e++) v[e] = e < lim ? v[e] : 0.f;
  return v;
}

// fp32 MFMA kernel body. K order of the products: at MFMA step s (0..BK/2-1) of a slab, lane
// half h supplies k = (BK/2) h + s for both operands (each lane supplies one k per 32x32x2
// MFMA; any bijection contracts the same sum), so a lane's four consecutive k of a row
// stored with K contiguous are one 16-byte LDS read feeding four MFMAs.
template <class CFG, bool AT, bool BT, int EPI>
__device__ __forceinline__ void gemm_body(const Args& g) {
  constexpr int BM = CFG::BM, BN = CFG::BN, TM = CFG::TM, TN = CFG::TN;
  constexpr int NSTAGE = CFG::NSTAGE, NWAVES = CFG::NWAVES;
  // one LDS object per pipeline stage, so the compiler can tell which copies a read waits
  // for (the third is a placeholder with two stages)
  constexpr int SA3 = NSTAGE > 2 ? BM * BK : 4, SB3 = NSTAGE > 2 ? BN * BK : 4;
  __shared__ __attribute__((aligned(1024))) float As0[BM * BK], As1[BM * BK];
  __shared__ __attribute__((aligned(1024))) float Bs0[BN * BK], Bs1[BN * BK];
  __shared__ __attribute__((aligned(1024))) float As2[SA3], Bs2[SB3];

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
  const int wm0 = (wave / CFG::WAVES_N) * (32 * TM), wn0 = (wave % CFG::WAVES_N) * (32 * TN);
  const bool do_colsum = AT && g.colsum != nullptr && nt == 0;  // uniform per workgroup
  float csum = 0.f;

  const int kbeg = z * g.k_split;
  const int kend = min(g.K, kbeg + g.k_split);
  const int klen = kend > kbeg ? kend - kbeg : 0;
  const int nslabs = (klen + BK - 1) / BK;

  f32x16 acc[TM][TN];
#pragma unroll
  for (int a = 0; a < TM; a++)
#pragma unroll
    for (int b = 0; b < TN; b++)
#pragma unroll
      for (int i = 0; i < 16; i++) acc[a][b][i] = 0.f;

  SlabCopy<AT, BM, NWAVES> ca;
  SlabCopy<BT, BN, NWAVES> cb;
  ca.init(g.A + (AT ? (long long)kbeg * g.lda : kbeg), g.lda, m0,
          AT ? (long long)(g.K - kbeg) * g.lda : (long long)g.M * g.lda - kbeg, wave, lane);
  cb.init(g.B + (BT ? (long long)kbeg * g.ldb : kbeg), g.ldb, n0,
          BT ? (long long)(g.K - kbeg) * g.ldb : (long long)g.N * g.ldb - kbeg, wave, lane);

  // per-lane fragment read offsets (bytes within a stage): K-contiguous operands, the chunk
  // of k = HALF h .. HALF h + 3 (the j-th next four k: offset ^ 16 j); (K, rows) operands,
  // k-row HALF h
  int rda[TM], rdb[TN];
#pragma unroll
  for (int q = 0; q < TM; q++) {
    const int ra = wm0 + 32 * q + r;
    rda[q] = AT ? (HALF * h * BM + ra) * 4 : ra * 4 * BK + 16 * (((HALF / 4) * h) ^ kswz(ra));
  }
#pragma unroll
  for (int q = 0; q < TN; q++) {
    const int rb = wn0 + 32 * q + r;
    rdb[q] = BT ? (HALF * h * BN + rb) * 4 : rb * 4 * BK + 16 * (((HALF / 4) * h) ^ kswz(rb));
  }

  auto stage_a = [&](int s) -> float* { return s == 0 ? As0 : s == 1 ? As1 : As2; };
  auto stage_b = [&](int s) -> float* { return s == 0 ? Bs0 : s == 1 ? Bs1 : Bs2; };
  auto issue = [&](int kt, int s) {
    ca.issue(kt, kt < nslabs, stage_a(s), wave);
    cb.issue(kt, kt < nslabs, stage_b(s), wave);
  };
  auto frag = [&](const char* p, int rd, int j, bool trans, int rows) -> f32x4 {
    if (!trans) return *reinterpret_cast<const f32x4*>(p + (rd ^ (16 * j)));
    f32x4 v;
#pragma unroll
    for (int e = 0; e < 4; e++)
      v[e] = *reinterpret_cast<const float*>(p + rd + (4 * j + e) * rows * 4);
    return v;
  };
  auto compute = [&](const float* As, const float* Bs, int kt) {
    const char* pa = reinterpret_cast<const char*>(As);
    const char* pb = reinterpret_cast<const char*>(Bs);
    const int k0 = kbeg + kt * BK;
    const bool tail = k0 + BK > kend;  // uniform
    f32x4 af[HALF / 4][TM], bfr[HALF / 4][TN];
#pragma unroll
    for (int j = 0; j < HALF / 4; j++) {
#pragma unroll
      for (int q = 0; q < TM; q++) af[j][q] = frag(pa, rda[q], j, AT, BM);
#pragma unroll
      for (int q = 0; q < TN; q++) bfr[j][q] = frag(pb, rdb[q], j, BT, BN);
      if (tail) {
        const int lim = kend - (k0 + HALF * h + 4 * j);
#pragma unroll
        for (int q = 0; q < TM; q++) af[j][q] = kmask4(af[j][q], lim);
#pragma unroll
        for (int q = 0; q < TN; q++) bfr[j][q] = kmask4(bfr[j][q], lim);
      }
    }
#pragma unroll
    for (int j = 0; j < HALF / 4; j++)
#pragma unroll
      for (int e = 0; e < 4; e++)
#pragma unroll
        for (int tm = 0; tm < TM; tm++)
#pragma unroll
          for (int tn = 0; tn < TN; tn++)
            acc[tm][tn] = mfma32x32x2(bfr[j][tn][e], af[j][tm][e], acc[tm][tn]);
    if (do_colsum) {  // column m of the A tile ([k][m] in LDS): this thread's share of k
      constexpr int KP = BK * BM / CFG::NTHREADS;
      const int m = tid % BM, part = tid / BM;
#pragma unroll
      for (int kk = 0; kk < KP; kk++) csum += As[(part * KP + kk) * BM + m];
    }
  };
  // Stage of slab kt: kt % NSTAGE; slab kt + NSTAGE - 1 is issued while slab kt is used. The
  // loop is unrolled by NSTAGE so every LDS access names its stage statically, and every
  // step issues the same copies (empty ones past the last slab): the compiler's own waits
  // for the copies then follow them exactly.
  constexpr int COPIES =
      SlabCopy<AT, BM, NWAVES>::PER_WAVE + SlabCopy<BT, BN, NWAVES>::PER_WAVE;
  auto step = [&](int s, int kt) {  // s: a constant at every call
    // this wave's copies of slab kt have landed (those of the NSTAGE - 2 later slabs may not)
    wait_vmcnt<COPIES * (NSTAGE - 2)>();
    lds_barrier();  // so have every wave's; and every wave is done with slab kt - 1
    issue(kt + NSTAGE - 1, (s + NSTAGE - 1) % NSTAGE);
    compute(stage_a(s), stage_b(s), kt);
  };
  if (nslabs > 0) {
#pragma unroll
    for (int s = 0; s < NSTAGE - 1; s++) issue(s, s);
    int kt = 0;
    for (; kt + NSTAGE <= nslabs; kt += NSTAGE) {
#pragma unroll
      for (int s = 0; s < NSTAGE; s++) step(s, kt + s);
    }
#pragma unroll
    for (int s = 0; s < NSTAGE - 1; s++)
      if (kt + s < nslabs) step(s, kt + s);
    wait_vmcnt<0>();  // the empty copies past the end still write their zeros
  }

  if (do_colsum) {
    float* red = As0;
    if (CFG::NTHREADS == 2 * BM) {  // the second thread of each m hands its share over
      lds_barrier();
      if (tid >= BM) red[tid - BM] = csum;
      __syncthreads();
    }
    if (tid < BM && m0 + tid < g.M) {
      const float total = CFG::NTHREADS == 2 * BM ? csum + red[tid] : csum;
      if (g.colsum_zstride) g.colsum[(long long)z * g.colsum_zstride + m0 + tid] = total;
      else g.colsum[m0 + tid] += total;
    }
  }

  float* C = g.C + (long long)z * g.c_zstride;
  // acc[tm][tn][4q + j]: row m = m0 + wm0 + 32 tm + r, column n = n0 + wn0 + 32 tn + 8q + 4h + j
#pragma unroll
  for (int tm = 0; tm < TM; tm++) {
    const int m = m0 + wm0 + 32 * tm + r;
    if (m >= g.M) continue;
#pragma unroll
    for (int tn = 0; tn < TN; tn++)
#pragma unroll
      for (int q = 0; q < 4; q++) {
        const int n = n0 + wn0 + 32 * tn + 8 * q + 4 * h;
        if (n >= g.N) continue;
        epilogue4<EPI>(g, C, m, n,
                       f32x4{acc[tm][tn][4 * q], acc[tm][tn][4 * q + 1], acc[tm][tn][4 * q + 2],
                             acc[tm][tn][4 * q + 3]});
      }
  }
}

// ---- split-operand kernel ----------------------------------------------------------------
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

// One wave64 bf16 MFMA: acc(32x32) += A(32x16) * B(16x32), fp32 accumulation. Lane l
// supplies A[l % 32][8 (l / 32) .. + 7] and B[8 (l / 32) .. + 7][l % 32]; the result layout
// is that of mfma32x32x2.
GPT2_DEVICE_INLINE f32x16 mfma_bf16(bf16x8 a, bf16x8 b, f32x16 acc) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc, 0, 0, 0);
}


// Products: with a = ah + am + al and b = bh + bm + bl (the exact split of common.h),
// a b = ah bh + (ah bm + am bh) + (ah bl + al bh + am bm) + (am bl + al bm) + al bl; the six
// terms of the first three groups are formed on bf16 MFMA (each exact, 8 x 8 significand
// bits, accumulated in fp32) and the last three dropped, which changes a b by at most
// 2^-23 |a b|, the size of one or two fp32 roundings of the product. The fp32 accumulation
// of the K-term sum then dominates the error, as it does with fp32 products. The MFMA's 16-k
// step takes, in lane half h, the k 8h .. 8h + 7 of a 16-k slab.
//
// The workgroup stages each slab through registers: every thread loads 8 consecutive fp32
// values of each operand (two 16-byte buffer loads; rows or k past the operand's end read
// as zero), splits them into their bf16 parts and writes the three parts to three LDS
// planes, so each value is split once rather than once per wave that reads it. Planes are
// double-buffered (slab kt + 1 is written while slab kt is read) with one barrier per slab,
// and the global loads of slab kt + 3 are in flight during the products of slabs kt + 1 and
// kt + 2 (two register sets).
// Plane layouts (bf16): an operand stored with K contiguous as [row][16 k], 32-byte rows,
// chunk c (8 k) of row r at chunk c ^ ((r >> 3) & 1), so the 16-byte fragment reads of 32
// consecutive rows cover all banks; an operand stored (K, rows) as [k][row], chunk c (8 rows)
// of k-row k at chunk c ^ rswz<R>(k % 4), read with transposing reads, whose four k-rows
// then fall on disjoint banks. gfx950's LDS has 64 four-byte banks and serves a transposing
// read 32 lanes at a time: four k-rows of 64 bytes each. With R = 256 (512-byte k-rows) the
// XOR moves the four by 0, 96, 192 and 160 bytes; with R = 192 (384-byte k-rows, every other
// one 128 bytes on) by 0, 32, 64 and 96, so the two k-rows of each parity differ by 64
// bytes (the XOR stays inside the row's 24 chunks). The earlier 0, 0, 32, 32 was
// conflict-free for 16 lanes at a time but not for 32 (SQ_LDS_BANK_CONFLICT counted 0.66
// conflict cycles per LDS cycle in the grad-input GEMMs).
template <int R>
GPT2_DEVICE_INLINE int rswz(int j) {
  static_assert(R == 256 || R == 192, "k-row length");
  return R == 256 ? (0xAC60 >> (4 * j)) & 15 : (0x6420 >> (4 * j)) & 15;
}

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4_t;

// Fragment of an operand stored (K, rows): two transposing 8-byte reads
// (ds_read_b64_tr_b16). In each 16-lane group, lane i receives column i of the 4 x 16 block
// whose k-row j is read by lanes 4j .. 4j + 3 (4 columns each).
GPT2_DEVICE_INLINE bf16x8 frag_tr(const char* p, int kstride4) {
  const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(p));
  const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(p + kstride4));
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// One operand's staging. The slab is cut into R BK / 8 chunks of 8 values; chunk f is, for
// an operand stored with K contiguous, row f / 2 at k 8 (f % 2) .. + 7 of the slab, for one
// stored (K, rows), k-row f / (R / 8) at rows 8 (f % (R / 8)) .. + 7. Thread t stages chunks
// t, t + NT, ... below R BK / 8 (whole waves take part or skip). The buffer resource of a
// slab ends where the operand ends.
template <bool TRANS, int R, int NT>
struct StageX6 {
  static constexpr int CPR = R / 8;                  // 8-row chunks per k-row (TRANS)
  static constexpr int NCH = R * BK / 8;             // chunks per slab
  static constexpr int CH = (NCH + NT - 1) / NT;     // chunks per thread (at most)
  static_assert(NCH % 64 == 0, "whole waves");
  // whether chunk i of thread tid exists (wave-uniform)
  static __device__ __forceinline__ bool live(int i, int tid) {
    return NCH % NT == 0 || tid + NT * i < NCH;
  }
  const char* tile;     // operand at this tile's first row / column, k = kbeg
  long long step;       // bytes between consecutive slabs
  long long remain;     // bytes from `tile` to the end of the operand
  uint32_t voff[CH];    // byte offsets of this thread's chunks within a slab
  int kofs[CH];         // k (first k) of each chunk within a slab
  int lds_off[CH];      // byte offset of each chunk within a plane

  __device__ __forceinline__ void init(const float* P, int ld, int row0, long long total,
                                       int tid) {
    const long long at = TRANS ? (long long)row0 : (long long)row0 * ld;
    tile = reinterpret_cast<const char*>(P + at);
    remain = 4 * (total - at);
    step = TRANS ? 4LL * BK * ld : 4LL * BK;
#pragma unroll
    for (int i = 0; i < CH; i++) {
      const int f = tid + NT * i;
      if (!TRANS) {
        const int row = f >> 1, c = f & 1;
        voff[i] = (uint32_t)(row * ld + 8 * c) * 4u;
        kofs[i] = 8 * c;
        lds_off[i] = row * 2 * BK + 16 * (c ^ ((row >> 3) & 1));
      } else {
        const int kk = f / CPR, c = f % CPR;
        voff[i] = (uint32_t)(kk * ld + 8 * c) * 4u;
        kofs[i] = kk;
        lds_off[i] = kk * 2 * R + 16 * (c ^ rswz<R>(kk & 3));
      }
    }
  }
  // v: 2 CH float4s
  __device__ __forceinline__ void load(int kt, f32x4* v, int tid) const {
    const long long off = (long long)kt * step;
    const long long left = remain - off;
    const int nrec = (int)(uint32_t)(left > 0xFFFFFFFFLL ? 0xFFFFFFFFLL : left > 0 ? left : 0);
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<char*>(tile + off), (short)0, nrec, kBufferFlags);
#pragma unroll
    for (int i = 0; i < CH; i++) {
      if (!live(i, tid)) break;
      v[2 * i] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, voff[i], 0, 0));
      v[2 * i + 1] =
          __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, voff[i] + 16, 0, 0));
    }
  }
  // with MASKED, zero k at or past kend (k0: first k of the slab); with COLSUM, add the
  // values to cs (column sums of an operand stored (K, rows); 8 per chunk); split, and write
  // the three parts
  template <bool COLSUM, bool MASKED>
  __device__ __forceinline__ void store(const f32x4* v, char* planes, int k0, int kend,
                                        float* cs, int tid) const {
    constexpr int PLANE = R * BK * 2;
#pragma unroll
    for (int i = 0; i < CH; i++) {
      if (!live(i, tid)) break;
      f32x4 a = v[2 * i], b = v[2 * i + 1];
      if (MASKED && !TRANS) {
        const int lim = kend - (k0 + kofs[i]);
        a = kmask4(a, lim);
        b = kmask4(b, lim - 4);
      } else if (MASKED && k0 + kofs[i] >= kend) {
        a = f32x4{0.f, 0.f, 0.f, 0.f};
        b = a;
      }
      if (COLSUM) {
#pragma unroll
        for (int e = 0; e < 4; e++) {
          cs[8 * i + e] += a[e];
          cs[8 * i + 4 + e] += b[e];
        }
      }
      u32x4 hi, mid, lo;
      split8(a, b, hi, mid, lo);
      *reinterpret_cast<u32x4*>(planes + lds_off[i]) = hi;
      *reinterpret_cast<u32x4*>(planes + PLANE + lds_off[i]) = mid;
      *reinterpret_cast<u32x4*>(planes + 2 * PLANE + lds_off[i]) = lo;
    }
  }
};

template <class CFG, bool AT, bool BT, int EPI>
__device__ __forceinline__ void gemm_x6s_body(const Args& g) {
  constexpr int BM = CFG::BM, BN = CFG::BN, TM = CFG::TM, TN = CFG::TN;
  constexpr int NT = CFG::NTHREADS;
  static_assert(BK == 16, "one bf16 MFMA step per slab");
  static_assert(BM * BK >= 8 * NT, "every thread stages A (its column sums)");
  constexpr int PA = BM * BK * 2, PB = BN * BK * 2;  // bytes of one plane
  constexpr int BUF = 3 * (PA + PB);
  __shared__ __attribute__((aligned(1024))) char lds[2 * BUF];

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
  const int wm0 = (wave / CFG::WAVES_N) * (32 * TM), wn0 = (wave % CFG::WAVES_N) * (32 * TN);
  const bool do_colsum = AT && g.colsum != nullptr && nt == 0;  // uniform per workgroup

  const int kbeg = z * g.k_split;
  const int kend = min(g.K, kbeg + g.k_split);
  const int klen = kend > kbeg ? kend - kbeg : 0;
  const int nslabs = (klen + BK - 1) / BK;

  f32x16 acc[TM][TN];
#pragma unroll
  for (int a = 0; a < TM; a++)
#pragma unroll
    for (int b = 0; b < TN; b++)
#pragma unroll
      for (int i = 0; i < 16; i++) acc[a][b][i] = 0.f;
  StageX6<AT, BM, NT> sa;
  StageX6<BT, BN, NT> sb;
  constexpr int CHA = StageX6<AT, BM, NT>::CH, CHB = StageX6<BT, BN, NT>::CH;
  float cs[8 * CHA];
#pragma unroll
  for (int i = 0; i < 8 * CHA; i++) cs[i] = 0.f;
  sa.init(g.A + (AT ? (long long)kbeg * g.lda : kbeg), g.lda, m0,
          AT ? (long long)(g.K - kbeg) * g.lda : (long long)g.M * g.lda - kbeg, tid);
  sb.init(g.B + (BT ? (long long)kbeg * g.ldb : kbeg), g.ldb, n0,
          BT ? (long long)(g.K - kbeg) * g.ldb : (long long)g.N * g.ldb - kbeg, tid);

  // per-lane fragment read offsets within a plane
  const int g16 = lane >> 4, i16 = lane & 15;
  int rda[TM], rdb[TN];
#pragma unroll
  for (int q = 0; q < TM; q++) {
    const int row = wm0 + 32 * q + r;
    const int n = wm0 + 32 * q + 16 * (g16 & 1) + 4 * (i16 & 3);
    rda[q] = !AT ? row * 2 * BK + 16 * (h ^ ((row >> 3) & 1))
                 : (8 * h + (i16 >> 2)) * 2 * BM + 16 * ((n >> 3) ^ rswz<BM>(i16 >> 2)) +
                       8 * (i16 & 1);
  }
#pragma unroll
  for (int q = 0; q < TN; q++) {
    const int row = wn0 + 32 * q + r;
    const int n = wn0 + 32 * q + 16 * (g16 & 1) + 4 * (i16 & 3);
    rdb[q] = !BT ? row * 2 * BK + 16 * (h ^ ((row >> 3) & 1))
                 : (8 * h + (i16 >> 2)) * 2 * BN + 16 * ((n >> 3) ^ rswz<BN>(i16 >> 2)) +
                       8 * (i16 & 1);
  }
  auto fa = [&](const char* pl, int q) -> bf16x8 {
    if (!AT) return *reinterpret_cast<const bf16x8*>(pl + rda[q]);
    return frag_tr(pl + rda[q], 4 * 2 * BM);
  };
  auto fb = [&](const char* pl, int q) -> bf16x8 {
    if (!BT) return *reinterpret_cast<const bf16x8*>(pl + rdb[q]);
    return frag_tr(pl + rdb[q], 4 * 2 * BN);
  };
  f32x4 va[2][2 * CHA], vb[2][2 * CHB];  // two register sets of staged values
  auto load = [&](int kt, int set) {
    sa.load(kt, va[set], tid);
    sb.load(kt, vb[set], tid);
  };
  // COLSUM: column sums of A wanted; MASKED: the last slab ends before BK (a K tail)
  auto stage = [&](auto colsum, auto masked, int set, char* buf, int kt) {
    constexpr bool COLSUM = decltype(colsum)::value, MASKED = decltype(masked)::value;
    const int k0 = kbeg + kt * BK;
    sa.template store<COLSUM, MASKED>(va[set], buf, k0, kend, cs, tid);
    sb.template store<false, MASKED>(vb[set], buf + 3 * PA, k0, kend, cs, tid);
  };
  auto compute = [&](const char* buf) {
    const char* pa = buf;
    const char* pb = buf + 3 * PA;
    bf16x8 bh[TN], bm[TN], bl[TN];
#pragma unroll
    for (int tn = 0; tn < TN; tn++) {
      bh[tn] = fb(pb, tn);
      bm[tn] = fb(pb + PB, tn);
      bl[tn] = fb(pb + 2 * PB, tn);
    }
#pragma unroll
    for (int tm = 0; tm < TM; tm++) {
      const bf16x8 ah = fa(pa, tm), am = fa(pa + PA, tm), al = fa(pa + 2 * PA, tm);
      // the B fragment is the MFMA's first operand (a lane then holds runs of 4
      // consecutive output columns); the smaller terms go first
#pragma unroll
      for (int tn = 0; tn < TN; tn++) acc[tm][tn] = mfma_bf16(bm[tn], am, acc[tm][tn]);
#pragma unroll
      for (int tn = 0; tn < TN; tn++) acc[tm][tn] = mfma_bf16(bl[tn], ah, acc[tm][tn]);
#pragma unroll
      for (int tn = 0; tn < TN; tn++) acc[tm][tn] = mfma_bf16(bh[tn], al, acc[tm][tn]);
#pragma unroll
      for (int tn = 0; tn < TN; tn++) acc[tm][tn] = mfma_bf16(bm[tn], ah, acc[tm][tn]);
#pragma unroll
      for (int tn = 0; tn < TN; tn++) acc[tm][tn] = mfma_bf16(bh[tn], am, acc[tm][tn]);
#pragma unroll
      for (int tn = 0; tn < TN; tn++) acc[tm][tn] = mfma_bf16(bh[tn], ah, acc[tm][tn]);
    }
  };

  // Slab kt is read from plane buffer kt % 2; its values arrive in register set kt % 2. The
  // loop is unrolled by two so that both name their buffer and set statically, and its
  // steady state (every step stages and loads) has no conditions, so the products, the
  // splitting and the LDS traffic of a step form one block the compiler can interleave.
  // Masking and column sums are compile-time choices of the loop (both uniform).
  char* const buf0 = lds;
  char* const buf1 = lds + BUF;
  auto run = [&](auto colsum, auto masked) {
    load(0, 0);
    if (nslabs > 1) load(1, 1);
    stage(colsum, masked, 0, buf0, 0);
    if (nslabs > 2) load(2, 0);
    __syncthreads();
    int kt = 0;
    for (; kt + 5 <= nslabs; kt += 2) {
      compute(buf0);  // slab kt
      stage(colsum, masked, 1, buf1, kt + 1);
      __syncthreads();  // slab kt + 1 is written; every wave is done with slab kt
      load(kt + 3, 1);
      compute(buf1);  // slab kt + 1
      stage(colsum, masked, 0, buf0, kt + 2);
      __syncthreads();
      load(kt + 4, 0);
    }
    for (; kt + 2 <= nslabs; kt += 2) {
      compute(buf0);
      stage(colsum, masked, 1, buf1, kt + 1);
      __syncthreads();
      if (kt + 3 < nslabs) load(kt + 3, 1);
      compute(buf1);
      if (kt + 2 < nslabs) stage(colsum, masked, 0, buf0, kt + 2);
      __syncthreads();
      if (kt + 4 < nslabs) load(kt + 4, 0);
    }
    if (kt < nslabs) compute(buf0);  // an odd last slab
  };
  typedef std::integral_constant<bool, true> yes;
  typedef std::integral_constant<bool, false> no;
  if (nslabs > 0) {
    const bool tail = klen % BK != 0;
    if (AT && do_colsum) {
      if (tail) run(yes{}, yes{});
      else run(yes{}, no{});
    } else {
      if (tail) run(no{}, yes{});
      else run(no{}, no{});
    }
  }

  if (do_colsum) {  // the BK k-row partial sums of each m, added in k-row order
    float* red = reinterpret_cast<float*>(lds);
    constexpr int CPR = BM / 8;
    __syncthreads();  // every wave is done reading the planes (an odd last slab has no barrier)
#pragma unroll
    for (int i = 0; i < CHA; i++) {
      const int f = tid + NT * i, kk = f / CPR, c = f % CPR;
#pragma unroll
      for (int e = 0; e < 8; e++) red[kk * BM + 8 * c + e] = cs[8 * i + e];
    }
    __syncthreads();
    for (int m = tid; m < BM; m += NT) {
      if (m0 + m >= g.M) break;
      float total = 0.f;
      for (int j = 0; j < BK; j++) total += red[j * BM + m];
      if (g.colsum_zstride) g.colsum[(long long)z * g.colsum_zstride + m0 + m] = total;
      else g.colsum[m0 + m] += total;
    }
  }

  float* C = g.C + (long long)z * g.c_zstride;
  // Epilogue. On gfx9 the vector-memory counter covers stores as well as loads, so a load
  // waited for between stores also waits for every store issued before it. The bias of the
  // thread's columns is therefore added before any store, and the operand rows an epilogue
  // reads (residual, GELU pre-activation, or C itself) are loaded for the next 32-row block
  // before the current block is stored. The arithmetic is that of epilogue4, in the same
  // order.
  constexpr bool HAS_BIAS = EPI == EPI_STORE || EPI == EPI_GELU || EPI == EPI_RESID;
  constexpr bool READS = EPI == EPI_RESID || EPI == EPI_GELU_BWD || EPI == EPI_ACCUM;
  const bool vec = (g.ldc & 3) == 0;
  auto col = [&](int tn, int q) { return n0 + wn0 + 32 * tn + 8 * q + 4 * h; };
  auto row = [&](int tm) { return m0 + wm0 + 32 * tm + r; };
  // the bias of each column, added into the accumulators before anything is stored
  if (HAS_BIAS && g.bias) {
#pragma unroll
    for (int tn = 0; tn < TN; tn++)
#pragma unroll
      for (int q = 0; q < 4; q++) {
        const int n = col(tn, q);
        f32x4 bv = {0.f, 0.f, 0.f, 0.f};
        if (n + 3 < g.N) bv = *reinterpret_cast<const f32x4*>(g.bias + n);
        else
          for (int j = 0; j < 4; j++)
            if (n + j < g.N) bv[j] = g.bias[n + j];
#pragma unroll
        for (int tm = 0; tm < TM; tm++)
#pragma unroll
          for (int j = 0; j < 4; j++) acc[tm][tn][4 * q + j] += bv[j];
      }
  }
  const float* rsrc = EPI == EPI_ACCUM ? C : g.R;
  f32x4 rv[TN][4];  // operand values of one row block
  auto load_rows = [&](int tm) {
    const int m = row(tm);
#pragma unroll
    for (int tn = 0; tn < TN; tn++)
#pragma unroll
      for (int q = 0; q < 4; q++) {
        const int n = col(tn, q);
        rv[tn][q] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (m >= g.M || n >= g.N) continue;
        const long long off = (long long)m * g.ldc + n;
        if (vec && n + 3 < g.N) rv[tn][q] = *reinterpret_cast<const f32x4*>(rsrc + off);
        else
          for (int j = 0; j < 4; j++)
            if (n + j < g.N) rv[tn][q][j] = rsrc[off + j];
      }
  };
  // per row block: the values are combined into the accumulators, then the next block's
  // operand loads are issued, then this block's stores (so a later wait for those loads
  // never waits for these stores)
  if (READS) load_rows(0);
#pragma unroll
  for (int tm = 0; tm < TM; tm++) {
#pragma unroll
    for (int tn = 0; tn < TN; tn++)
#pragma unroll
      for (int q = 0; q < 4; q++) {
        f32x4 v = {acc[tm][tn][4 * q], acc[tm][tn][4 * q + 1], acc[tm][tn][4 * q + 2],
                   acc[tm][tn][4 * q + 3]};
        if (READS) {
          if (EPI == EPI_GELU_BWD) {
#pragma unroll
            for (int j = 0; j < 4; j++) v[j] *= gelu_bwd(rv[tn][q][j]);
          } else {
            v += rv[tn][q];
          }
        }
#pragma unroll
        for (int j = 0; j < 4; j++) acc[tm][tn][4 * q + j] = v[j];
      }
    if (READS && tm + 1 < TM) load_rows(tm + 1);
    const int m = row(tm);
    if (m >= g.M) continue;
#pragma unroll
    for (int tn = 0; tn < TN; tn++)
#pragma unroll
      for (int q = 0; q < 4; q++) {
        const int n = col(tn, q);
        if (n >= g.N) continue;
        const f32x4 v = {acc[tm][tn][4 * q], acc[tm][tn][4 * q + 1], acc[tm][tn][4 * q + 2],
                         acc[tm][tn][4 * q + 3]};
        const long long off = (long long)m * g.ldc + n;
        if (vec && n + 3 < g.N) *reinterpret_cast<f32x4*>(C + off) = v;
        else
          for (int j = 0; j < 4; j++)
            if (n + j < g.N) C[off + j] = v[j];
      }
  }
  // GELU: the activation of the (biased) pre-activation now in acc, written in a second pass
  // over the tile (interleaved with the pre-activation, the two streams of partial lines had
  // cost extra write traffic)
  if (EPI == EPI_GELU) {
#pragma unroll
    for (int tm = 0; tm < TM; tm++) {
      const int m = row(tm);
      if (m >= g.M) continue;
#pragma unroll
      for (int tn = 0; tn < TN; tn++)
#pragma unroll
        for (int q = 0; q < 4; q++) {
          const int n = col(tn, q);
          if (n >= g.N) continue;
          const f32x4 v = {acc[tm][tn][4 * q], acc[tm][tn][4 * q + 1], acc[tm][tn][4 * q + 2],
                           acc[tm][tn][4 * q + 3]};
          const long long off = (long long)m * g.ldc + n;
          if (vec && n + 3 < g.N)
            *reinterpret_cast<f32x4*>(g.C2 + off) =
                f32x4{gelu_fwd(v[0]), gelu_fwd(v[1]), gelu_fwd(v[2]), gelu_fwd(v[3])};
          else
            for (int j = 0; j < 4; j++)
              if (n + j < g.N) g.C2[off + j] = gelu_fwd(v[j]);
        }
    }
  }
}

// the two GEMM kernels: fp32 MFMA products, and split-operand bf16 MFMA products
template <bool AT, bool BT, int EPI>
__global__ __launch_bounds__(CfgF32::NTHREADS, CfgF32::OCC) void gemm_kernel(Args g) {
  gemm_body<CfgF32, AT, BT, EPI>(g);
}
template <int BNX, bool AT, bool BT, int EPI>
__global__ __launch_bounds__(512, 2) void gemm_x6_kernel(Args g) {
  static_assert(CfgX6W::NTHREADS == 512 && CfgX6N::NTHREADS == 512 && CfgX6W::OCC == 2 &&
                CfgX6N::OCC == 2, "launch bounds");
  if constexpr (BNX == 256) gemm_x6s_body<CfgX6W, AT, BT, EPI>(g);
  else gemm_x6s_body<CfgX6N, AT, BT, EPI>(g);
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

// the kernels and tile shapes a GEMM can run with
enum GemmKind { KIND_F32 = 0, KIND_X6W = 1, KIND_X6N = 2 };

template <bool AT, bool BT, int EPI>
void launch_e(const Args& a, int kind, dim3 grid, hipStream_t s) {
  if (kind == KIND_X6W) gemm_x6_kernel<256, AT, BT, EPI><<<grid, 512, 0, s>>>(a);
  else if (kind == KIND_X6N) gemm_x6_kernel<192, AT, BT, EPI><<<grid, 512, 0, s>>>(a);
  else gemm_kernel<AT, BT, EPI><<<grid, CfgF32::NTHREADS, 0, s>>>(a);
}

template <bool AT, bool BT>
void launch_tn(const Args& a, int kind, int epi, dim3 grid, hipStream_t s) {
  switch (epi) {
    case EPI_STORE: launch_e<AT, BT, EPI_STORE>(a, kind, grid, s); break;
    case EPI_GELU: launch_e<AT, BT, EPI_GELU>(a, kind, grid, s); break;
    case EPI_RESID: launch_e<AT, BT, EPI_RESID>(a, kind, grid, s); break;
    case EPI_ACCUM: launch_e<AT, BT, EPI_ACCUM>(a, kind, grid, s); break;
    case EPI_GELU_BWD: launch_e<AT, BT, EPI_GELU_BWD>(a, kind, grid, s); break;
  }
}

void launch(const Args& a, int kind, bool at, bool bt, int epi, dim3 grid, hipStream_t s) {
  if (!at && !bt) launch_tn<false, false>(a, kind, epi, grid, s);
  else if (!at && bt) launch_tn<false, true>(a, kind, epi, grid, s);
  else if (at && bt) launch_tn<true, true>(a, kind, epi, grid, s);
  else launch_tn<true, false>(a, kind, epi, grid, s);
}

// The kernels for the fp32 GEMMs: the split-operand bf16 kernel, unless the environment
// variable GPT2_GEMM_F32_PRODUCTS is "fp32" (the fp32 MFMA kernel, kept for comparison);
// GPT2_GEMM_X6_TILE = 256 or 192 restricts it to one tile width (for tests).
bool use_x6() {
  const char* e = getenv("GPT2_GEMM_F32_PRODUCTS");
  return !(e && strcmp(e, "fp32") == 0);
}
int forced_x6_width() {
  const char* e = getenv("GPT2_GEMM_X6_TILE");
  const int v = e ? atoi(e) : 0;
  return v == 256 || v == 192 ? v : 0;
}

// tile shape, workgroups per CU and planning rate of a kernel
struct KernelShape {
  int bm, bn, wg_per_cu;
  double rate;
};
template <class CFG>
KernelShape shape_of(double derate = 1.0) {
  return KernelShape{CFG::BM, CFG::BN, CFG::WG_PER_CU, CFG::RATE * derate};
}
// the narrower split-operand tile reads more LDS per product: planned at 95% of the rate
KernelShape kernel_shape(int kind) {
  return kind == KIND_X6W ? shape_of<CfgX6W>()
                          : kind == KIND_X6N ? shape_of<CfgX6N>(0.95) : shape_of<CfgF32>();
}

int ceil_div(long long a, long long b) { return (int)((a + b - 1) / b); }

// Kernel, tile shape and number of K splits for a problem, from a cost model fitted to
// measurements on MI355X. wg_per_cu workgroups of a kernel fit on each of the 256 CUs; a
// launch of n workgroups runs ceil(n / slots) rounds, each as long as one tile's products at
// the kernel's planning rate (tiles padded to whole tiles). Splitting K multiplies n by the
// split count and adds a pass that reads the partials and applies the epilogue (the
// partials themselves are written while the GEMM computes), costed at 5 TB/s. More splits,
// or the narrower tile, only when clearly (5%) cheaper.
struct Plan {
  int kind, splits;
};
Plan choose_plan(const Gemm& g) {
  int kinds[2] = {use_x6() ? (int)KIND_X6W : (int)KIND_F32, (int)KIND_X6N};
  int nkinds = use_x6() ? 2 : 1;
  if (use_x6() && forced_x6_width()) {
    kinds[0] = forced_x6_width() == 256 ? KIND_X6W : KIND_X6N;
    nkinds = 1;
  }
  const int kt = ceil_div(g.K, BK);
  const double mn = (double)g.M * g.N;
  double best = 1e30;
  Plan plan{kinds[0], 1};
  for (int ki = 0; ki < nkinds; ki++) {
    const KernelShape ks = kernel_shape(kinds[ki]);
    const double tiles = (double)ceil_div(g.M, ks.bm) * ceil_div(g.N, ks.bn);
    const double slots = 256.0 * ks.wg_per_cu;
    for (int s = 1; s <= 32; s++) {
      const int kper = ceil_div(kt, s);
      if (s > 1 && kper < 4) break;
      if (s > 1 && ceil_div(kt, kper) != s) continue;
      double cost = std::ceil(tiles * s / slots) * 2.0 * ks.bm * ks.bn * (double)kper * BK *
                    slots / ks.rate;
      if (s > 1) cost += 4.0 * mn * (s + 2.0) / 5e12;
      if (cost < best * 0.95) {
        best = cost;
        plan = Plan{kinds[ki], s};
      }
    }
  }
#ifdef GPT2_SPLIT_OVERRIDE
  if (const char* e = getenv("GPT2_SPLITS")) plan.splits = atoi(e);
#endif
  return plan;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15) == 0; }

}  // namespace

// partial results of a split GEMM are stored with a row stride that is a multiple of 4
// (16-byte loads in the reduction)
int split_ld(int N) { return (N + 3) & ~3; }

size_t gemm_workspace_floats(const Gemm& g) {
  const int s = choose_plan(g).splits;
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
  // (and leading dimensions below 2^21, so the per-thread byte offsets within a slab of
  // 256 rows fit 32 bits)
  const int a_cols = g.a_trans ? g.M : g.K, b_cols = g.b_trans ? g.N : g.K;
  if (!aligned16(g.A) || !aligned16(g.B) || !aligned16(g.C) || g.lda % 4 || g.ldb % 4 ||
      g.ldc % 2 || g.lda < a_cols || g.ldb < b_cols || g.ldc < g.N || g.lda >= (1 << 21) ||
      g.ldb >= (1 << 21)) {
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

  const Plan plan = choose_plan(g);
  const KernelShape ks = kernel_shape(plan.kind);
  int splits = plan.splits;
  if (splits > 1 && (!workspace || ws_floats < gemm_workspace_floats(g))) splits = 1;
  const int kt = ceil_div(g.K, BK);
  const int kt_per = ceil_div(kt, splits);
  splits = ceil_div(kt, kt_per);
  a.k_split = kt_per * BK;
  a.splits = splits;
  const int tiles = ceil_div(g.M, ks.bm) * ceil_div(g.N, ks.bn);
  // kernel name as profilers show it (template arguments: tile width for the split-operand
  // kernel, then the operand layouts)
  char kname[32];
  if (plan.kind == KIND_F32) snprintf(kname, sizeof(kname), "gemm_kernel<");
  else snprintf(kname, sizeof(kname), "gemm_x6_kernel<%d,", ks.bn);

  const double MN = (double)g.M * g.N;
  const double flop = 2.0 * MN * g.K;
  const double in_bytes = 4.0 * ((double)g.M * g.K + (double)g.N * g.K);
  // output traffic of an epilogue: stores, plus the extra tensor it reads or writes
  const double out_factor = g.epi == EPI_STORE ? 1.0 : 2.0;
  char name[64];
  if (splits == 1) {
    snprintf(name, sizeof(name), "%s%d,%d,%d>", kname, (int)g.a_trans, (int)g.b_trans,
             (int)g.epi);
    if (profiling_detail())
      snprintf(name + strlen(name), sizeof(name) - strlen(name), " %dx%dx%d", g.M, g.N, g.K);
    ProfScope ps(name, flop, in_bytes + 4.0 * MN * out_factor, stream);
    launch(a, plan.kind, g.a_trans, g.b_trans, g.epi, dim3(tiles), stream);
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
    snprintf(name, sizeof(name), "%s%d,%d,0>", kname, (int)g.a_trans, (int)g.b_trans);
    if (profiling_detail())
      snprintf(name + strlen(name), sizeof(name) - strlen(name), " %dx%dx%d/%d", g.M, g.N, g.K,
               splits);
    {
      ProfScope ps(name, flop, in_bytes + 4.0 * MN * splits, stream);
      launch(p, plan.kind, g.a_trans, g.b_trans, EPI_STORE, dim3(tiles * splits), stream);
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
