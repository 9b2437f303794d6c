// gemm_bf16.hip -- the GEMMs of the mixed-precision steps: 16-bit operands (bf16 or fp16),
// fp32 accumulation (v_mfma_f32_32x32x16_bf16 / v_mfma_f32_32x32x16_f16 on gfx950), 16-bit
// or fp32 results. The two formats share every line but the MFMA instruction and the
// conversions, so the kernels are templated on the storage type TS.
//
// Same three storage patterns as the fp32 GEMMs ("llm.c 的中文注解-20240421", sections 1.5
// and 1.6), C = op(A) . op(B):
//   forward      out  = inp . W^T   A (M,K) row-major, B = W stored (N,K)
//   grad input   dinp = dout . W    A (M,K) row-major, B = W stored (K,N)   (b_trans)
//   grad weight  dW  += dout^T.inp  A = dout stored (K,M), B = inp (K,N)   (a_trans, b_trans)
// and the same fused epilogues (bias, bias+GELU, bias+residual, fp32 accumulate into the
// master gradients, GELU backward), computed in fp32 and rounded once to TS on store.
//
// Tiling: workgroups own 256x256 tiles of C (8 waves of 128x64) or, for grids too small to
// fill the chip, 128x128 tiles (4 waves of 64x64); each wave holds WM x WN blocks of 32x32
// accumulators. K advances in slabs that go from global memory straight into LDS (buffer
// loads with the LDS as destination, no staging registers), several slabs in flight, one
// LDS object per pipeline stage. Each lane of the bf16 MFMA supplies 8 consecutive k of one
// row: an operand stored with K contiguous is kept [row][k] in LDS and read with 16-byte
// loads; an operand stored (K, rows) is kept as stored, [k][row], and read with the
// transposing LDS load of gfx950 (ds_read_b64_tr_b16), so no thread transposes anything.
// XOR swizzles of the 16-byte chunks (applied on the global side of the copy) keep both
// kinds of fragment read free of LDS bank conflicts.
// The MFMA takes the B tile as its first operand, so a lane ends up holding four runs of 4
// consecutive output columns of one row: epilogue loads and stores are 8- or 16-byte
// vectors.
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <type_traits>

#include "kernels.h"

namespace gpt2 {
namespace {

// Tile shapes: BM x BN per workgroup of WGM x WGN waves (each wave WM x WN blocks of 32 x 32),
// slabs of BK k, NSTAGE slabs in LDS, OCC workgroups per CU.
template <int BM_, int BN_, int BK_, int WGM_, int WGN_, int NSTAGE_, int OCC_, int GROUP_M_>
struct TileCfg {
  static constexpr int BM = BM_, BN = BN_, BK = BK_, WGM = WGM_, WGN = WGN_, GROUP_M = GROUP_M_;
  static constexpr int NWAVES = WGM * WGN, NT = 64 * NWAVES;
  static constexpr int WM = BM / 32 / WGM, WN = BN / 32 / WGN;
  static constexpr int NSTAGE = NSTAGE_, OCC = OCC_;
  static_assert(NSTAGE >= 2 && NSTAGE <= 5, "two to five LDS stages");
  static_assert(BK == 32 || BK == 64, "slab depth");
};
// 128 x 128: 4 waves of 64 x 64, slabs of 32 k, 3 stages of 16 KB, three workgroups per CU
// (small grids: more workgroups than the large tile)
typedef TileCfg<128, 128, 32, 2, 2, 3, 3, 8> Tile128;
// 256 x 256: 8 waves of 128 x 64, slabs of 64 k (128-byte pieces of rows stored with K
// contiguous), 2 stages of 64 KB, one workgroup per CU: half the operand bytes per flop of
// the 128 x 128 tile
typedef TileCfg<256, 256, 64, 2, 4, 2, 1, 8> Tile256;
// 256 x 192: 8 waves of 64 x 96, slabs of 64 k, 2 stages of 56 KB, one workgroup per CU:
// 8192 x 1280 outputs in 224 tiles (one round, no split of K) where 256 x 256 leaves 160
typedef TileCfg<256, 192, 64, 4, 2, 2, 1, 8> Tile192;
// 256 x 320: 8 waves of 64 x 160, slabs of 64 k, 2 stages of 72 KB, one workgroup per CU:
// 8192 x 5120 outputs in 512 tiles (two whole rounds) where 256 x 256 needs 2.5
typedef TileCfg<256, 320, 64, 4, 2, 2, 1, 8> Tile320;
// Epilogues that read a tensor (residual, GELU pre-activation, the fp32 C they accumulate
// into) load the next row block's values while the current one is stored. With the 10
// accumulator blocks of the 256 x 320 tile those values do not fit beside the accumulators
// (the kernels spill hundreds of registers), so that tile runs only the epilogues that read
// nothing; the planner gives it no other.
template <class CFG>
constexpr bool kReadingEpilogues = CFG::WM * CFG::WN <= 8;
bool epi_reads(int epi) { return epi == EPI_RESID || epi == EPI_GELU_BWD || epi == EPI_ACCUM; }

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));  // 8 x 16 bits of either format
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

// acc += a . b on the MFMA of the storage format (fragments carry the raw 16-bit patterns)
template <typename TS>
GPT2_DEVICE_INLINE f32x16 mfma16(bf16x8 a, bf16x8 b, f32x16 acc) {
  if constexpr (std::is_same<TS, f16_t>::value)
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), acc, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc, 0, 0, 0);
}
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4_t;

template <typename TS>
struct Args {
  const TS* A;
  const TS* B;
  void* C;
  TS* C2;
  const TS* R;
  const float* bias;
  float* colsum;
  int lda, ldb, ldc;
  int M, N, K;
  int k_split;
  int splits;
  long long c_zstride;
  long long colsum_zstride;
};

// LDS placement. An operand stored with K contiguous sits in LDS as [row][k] (rows of BK k);
// the 16-byte chunk c of row r holds the row's chunk c ^ kswz(r), which spreads the 16-byte
// fragment reads (consecutive rows, one chunk) over all banks. An operand stored
// (K, rows) keeps that layout in LDS, [k][row] (R elements per k); chunk c of k-row k holds
// chunk c ^ rswz<R>(k % 4), so the four k-rows that one transposing read touches fall on
// different banks. A transposing read serves 32 lanes at a time: four k-rows of 64 bytes
// each, which must cover disjoint banks (64 banks of 4 bytes). k-rows of 256 or 512 bytes
// start on the same bank: the XOR moves the four by 0, 96, 192 and 160 bytes. k-rows of 384
// bytes (R = 192) start 128 bytes apart in turn: the XOR moves them by 0, 32, 64 and 96
// bytes, so the two k-rows of each parity differ by 64 bytes, and every chunk stays inside
// its row's 24.
template <int BK>
GPT2_DEVICE_INLINE int kswz(int row) {
  return BK == 32 ? ((row >> 1) ^ (row >> 3)) & 3 : (row ^ (row >> 3)) & 7;
}
template <int R>
GPT2_DEVICE_INLINE int rswz(int j) {
  static_assert(R == 128 || R == 256 || R == 192 || R == 320, "k-row length");
  return R == 192 || R == 320 ? (0x6420 >> (4 * j)) & 15 : (0xAC60 >> (4 * j)) & 15;
}

// word 3 of a raw (untyped, unswizzled) buffer resource on gfx9-family GPUs
constexpr int kBufferFlags = 0x00020000;

// 16 bytes per lane from a buffer into LDS (lane l writes lds + 16 l); `lds` is wave-uniform
GPT2_DEVICE_INLINE void copy_to_lds16(__amdgpu_buffer_rsrc_t rs, char* lds, uint32_t voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void_t*)lds, 16, voff, 0, 0, 0);
}

// One operand's share of the slab pipeline: a slab (BK k x R rows, 2 R BK bytes) is copied
// from global memory straight into LDS, 1 KB per wave-wide buffer load (lane l fills bytes
// 16 l .. 16 l + 15 of the KB), without passing through registers. The buffer resource of a
// slab ends where the operand ends, so rows past its last row (and, for an operand stored
// (K, rows), k past K) read as zero. Per-lane byte offsets are computed once.
template <bool TRANS, int R, int NWAVES, int BK>
struct SlabCopy {
  static constexpr int PER_WAVE = R * BK * 2 / 1024 / NWAVES;
  static_assert(PER_WAVE * NWAVES * 1024 == R * BK * 2, "whole 1 KB copies per wave");
  const char* tile;     // operand at this tile's first row (!TRANS) or column (TRANS), k = 0
  long long step;       // bytes between consecutive slabs
  long long remain;     // bytes from `tile` to the end of the operand
  uint32_t voff[PER_WAVE];

  __device__ __forceinline__ void init(const void* P, int ld, int row0, long long total,
                                       int wave, int lane) {
    const long long at = TRANS ? (long long)row0 : (long long)row0 * ld;
    tile = reinterpret_cast<const char*>(P) + 2 * at;
    remain = 2 * (total - at);
    step = TRANS ? 2LL * BK * ld : 2LL * BK;
#pragma unroll
    for (int j = 0; j < PER_WAVE; j++) {
      const int b = (j * NWAVES + wave) * 1024 + 16 * lane;  // LDS byte within the slab
      if (!TRANS) {
        const int row = b / (2 * BK), p = (b % (2 * BK)) >> 4;
        voff[j] = (uint32_t)(row * ld + 8 * (p ^ kswz<BK>(row))) * 2u;
      } else {
        const int k = b / (2 * R), p = (b % (2 * R)) >> 4;
        voff[j] = (uint32_t)(k * ld + 8 * (p ^ rswz<R>(k & 3))) * 2u;
      }
    }
  }

  // `live` false: a copy past the last slab, given an empty range (it reads nothing and
  // writes zeros), so that every pipeline step issues the same number of copies
  __device__ __forceinline__ void issue(int kt, bool live, void* lds, int wave) const {
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

// Fragment of the bf16 MFMA for a lane: row r = lane % 32 of a 32-row block, k = 8 h .. 8 h + 7
// with h = lane / 32 (within a 16-k step).
// Operand stored with K contiguous: one 16-byte read. `rd` = byte of (row base + r, chunk of
// step 0); step 1 is the chunk 2 further, which the swizzle maps to rd ^ 32 within the row.
// Operand stored (K, rows): two transposing 8-byte reads (ds_read_b64_tr_b16). In each
// 16-lane group, lane i receives column i of the 4 x 16 block whose k-row j is read by lanes
// 4j .. 4j + 3 (4 columns each), so a group covers 16 columns x 4 k.
GPT2_DEVICE_INLINE bf16x8 frag_tr(const char* p, int kstride4) {
  const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(p));
  const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(p + kstride4));
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// zero the k values of a fragment at or past `lim` (its first element being k = 0)
GPT2_DEVICE_INLINE bf16x8 kmask(bf16x8 v, int lim) {
  u32x4 u = __builtin_bit_cast(u32x4, v);
#pragma unroll
  for (int q = 0; q < 4; q++)
    u[q] &= (2 * q < lim ? 0xFFFFu : 0u) | (2 * q + 1 < lim ? 0xFFFF0000u : 0u);
  return __builtin_bit_cast(bf16x8, u);
}

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

// Epilogue of four consecutive columns n..n+3 of row m (n % 4 == 0, m < M, n < N).
template <typename TS, int EPI, bool CF32>
__device__ __forceinline__ void epilogue4(const Args<TS>& g, void* Cv, int m, int n, f32x4 v) {
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
      for (int j = 0; j < 4; j++) r[j] = j < cnt ? ld1(g.R + off + j) : 0.f;
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
    TS* C = static_cast<TS*>(Cv);
    if (cnt == 4) {
      st4(C + off, v);
      if (EPI == EPI_GELU)
        st4(g.C2 + off, f32x4{gelu_fwd(v[0]), gelu_fwd(v[1]), gelu_fwd(v[2]),
                                       gelu_fwd(v[3])});
    } else {
      for (int j = 0; j < cnt; j++) {
        st1(C + off + j, v[j]);
        if (EPI == EPI_GELU) st1(g.C2 + off + j, gelu_fwd(v[j]));
      }
    }
  }
}

// epilogue4 with the bias already in v and the values the epilogue reads (residual, GELU
// pre-activation, or the fp32 C to accumulate into) passed in as r
template <typename TS, int EPI, bool CF32>
__device__ __forceinline__ void epilogue4_pre(const Args<TS>& g, void* Cv, int m, int n, f32x4 v,
                                              f32x4 r) {
  const long long off = (long long)m * g.ldc + n;
  const int cnt = min(4, g.N - n);
  if (EPI == EPI_RESID) v += r;
  if (EPI == EPI_GELU_BWD)
#pragma unroll
    for (int j = 0; j < 4; j++) v[j] *= gelu_bwd(r[j]);
  if (CF32) {
    float* C = static_cast<float*>(Cv);
    if (EPI == EPI_ACCUM) v += r;
    if (cnt == 4) {
      *reinterpret_cast<f32x4*>(C + off) = v;
    } else {
      for (int j = 0; j < cnt; j++) C[off + j] = v[j];
    }
  } else {
    TS* C = static_cast<TS*>(Cv);
    if (cnt == 4) {
      st4(C + off, v);
      if (EPI == EPI_GELU)
        st4(g.C2 + off, f32x4{gelu_fwd(v[0]), gelu_fwd(v[1]), gelu_fwd(v[2]),
                                       gelu_fwd(v[3])});
    } else {
      for (int j = 0; j < cnt; j++) {
        st1(C + off + j, v[j]);
        if (EPI == EPI_GELU) st1(g.C2 + off + j, gelu_fwd(v[j]));
      }
    }
  }
}

template <typename TS, class CFG, bool AT, bool BT, bool CF32, int EPI>
__global__ __launch_bounds__(CFG::NT, CFG::OCC) void gemm16_kernel(Args<TS> g) {
  constexpr int BM = CFG::BM, BN = CFG::BN, BK = CFG::BK, WM = CFG::WM, WN = CFG::WN;
  constexpr int NT = CFG::NT;
  constexpr int NSTAGE = CFG::NSTAGE, NWAVES = CFG::NWAVES;
  // one LDS object per pipeline stage, so the compiler can tell which copies a read waits for
  // (stages past NSTAGE are 16-byte placeholders)
  constexpr int SA = BM * BK, SB = BN * BK;
  constexpr int SA3 = NSTAGE > 3 ? SA : 8, SB3 = NSTAGE > 3 ? SB : 8;
  constexpr int SA4 = NSTAGE > 4 ? SA : 8, SB4 = NSTAGE > 4 ? SB : 8;
  __shared__ __attribute__((aligned(1024))) uint16_t As0[SA], As1[SA], As2[SA];
  __shared__ __attribute__((aligned(1024))) uint16_t Bs0[SB], Bs1[SB], Bs2[SB];
  __shared__ __attribute__((aligned(16))) uint16_t As3[SA3], Bs3[SB3], As4[SA4], Bs4[SB4];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int r = lane & 31, h = lane >> 5;
  const int nM = (g.M + BM - 1) / BM, nN = (g.N + BN - 1) / BN;
  const int tiles = nM * nN;
  const int lid = xcd_logical_block(blockIdx.x, gridDim.x);
  const int z = lid / tiles;
  const int t = lid - z * tiles;
  constexpr int GROUP_M = CFG::GROUP_M;
  const int group = t / (GROUP_M * nN);
  const int first_m = group * GROUP_M;
  const int gsz = min(nM - first_m, GROUP_M);
  const int tin = t - group * GROUP_M * nN;
  const int mt = first_m + tin % gsz, nt = tin / gsz;
  const int m0 = mt * BM, n0 = nt * BN;
  const int wm0 = (wave / CFG::WGN) * 32 * WM, wn0 = (wave % CFG::WGN) * 32 * WN;
  const bool do_colsum = AT && g.colsum != nullptr && nt == 0;  // uniform per workgroup
  // column sums: thread -> 8 consecutive m (chunk tid % CHUNKS) of every KG-th k-row
  constexpr int CHUNKS = BM / 8, KG = NT / CHUNKS;
  static_assert(BK % KG == 0 && KG * BM * 4 <= SA * 2, "column-sum layout");
  float csum[8];
#pragma unroll
  for (int e = 0; e < 8; e++) csum[e] = 0.f;

  const int kbeg = z * g.k_split;
  const int kend = min(g.K, kbeg + g.k_split);
  const int klen = kend > kbeg ? kend - kbeg : 0;
  const int nslabs = (klen + BK - 1) / BK;

  f32x16 acc[WM][WN];
#pragma unroll
  for (int a = 0; a < WM; a++)
#pragma unroll
    for (int b = 0; b < WN; b++)
#pragma unroll
      for (int i = 0; i < 16; i++) acc[a][b][i] = 0.f;

  SlabCopy<AT, BM, NWAVES, BK> ca;
  SlabCopy<BT, BN, NWAVES, BK> cb;
  ca.init(g.A + (AT ? (long long)kbeg * g.lda : kbeg), g.lda, m0,
          AT ? (long long)(g.K - kbeg) * g.lda : (long long)g.M * g.lda - kbeg, wave, lane);
  cb.init(g.B + (BT ? (long long)kbeg * g.ldb : kbeg), g.ldb, n0,
          BT ? (long long)(g.K - kbeg) * g.ldb : (long long)g.N * g.ldb - kbeg, wave, lane);

  // per-lane fragment read offsets (bytes within a stage)
  const int g16 = lane >> 4, i16 = lane & 15;
  int rda[WM], rdb[WN];
#pragma unroll
  for (int q = 0; q < WM; q++) {
    if (!AT) rda[q] = (wm0 + 32 * q + r) * 2 * BK + 16 * (h ^ kswz<BK>(wm0 + 32 * q + r));
    else {
      const int n = wm0 + 32 * q + 16 * (g16 & 1) + 4 * (i16 & 3);
      rda[q] = (8 * h + (i16 >> 2)) * 2 * BM + 16 * ((n >> 3) ^ rswz<BM>(i16 >> 2)) + 8 * (i16 & 1);
    }
  }
#pragma unroll
  for (int q = 0; q < WN; q++) {
    if (!BT) rdb[q] = (wn0 + 32 * q + r) * 2 * BK + 16 * (h ^ kswz<BK>(wn0 + 32 * q + r));
    else {
      const int n = wn0 + 32 * q + 16 * (g16 & 1) + 4 * (i16 & 3);
      rdb[q] = (8 * h + (i16 >> 2)) * 2 * BN + 16 * ((n >> 3) ^ rswz<BN>(i16 >> 2)) + 8 * (i16 & 1);
    }
  }

  auto stage_a = [&](int s) -> uint16_t* {
    return s == 0 ? As0 : s == 1 ? As1 : s == 2 ? As2 : s == 3 ? As3 : As4;
  };
  auto stage_b = [&](int s) -> uint16_t* {
    return s == 0 ? Bs0 : s == 1 ? Bs1 : s == 2 ? Bs2 : s == 3 ? Bs3 : Bs4;
  };
  auto issue = [&](int kt, int s) {
    ca.issue(kt, kt < nslabs, stage_a(s), wave);
    cb.issue(kt, kt < nslabs, stage_b(s), wave);
  };
  auto compute = [&](const uint16_t* As, const uint16_t* Bs, int kt) {
    const char* pa = reinterpret_cast<const char*>(As);
    const char* pb = reinterpret_cast<const char*>(Bs);
    const int k0 = kbeg + kt * BK;
    const bool tail = k0 + BK > kend;  // uniform
#pragma unroll
    for (int ks = 0; ks < BK / 16; ks++) {
      bf16x8 af[WM], bfr[WN];
#pragma unroll
      for (int q = 0; q < WM; q++) {
        if (!AT) af[q] = *reinterpret_cast<const bf16x8*>(pa + (rda[q] ^ (32 * ks)));
        else af[q] = frag_tr(pa + rda[q] + 16 * ks * 2 * BM, 4 * 2 * BM);
      }
#pragma unroll
      for (int q = 0; q < WN; q++) {
        if (!BT) bfr[q] = *reinterpret_cast<const bf16x8*>(pb + (rdb[q] ^ (32 * ks)));
        else bfr[q] = frag_tr(pb + rdb[q] + 16 * ks * 2 * BN, 4 * 2 * BN);
      }
      if (tail) {
        const int lim = kend - (k0 + 16 * ks + 8 * h);
#pragma unroll
        for (int q = 0; q < WM; q++) af[q] = kmask(af[q], lim);
#pragma unroll
        for (int q = 0; q < WN; q++) bfr[q] = kmask(bfr[q], lim);
      }
#pragma unroll
      for (int tm = 0; tm < WM; tm++)
#pragma unroll
        for (int tn = 0; tn < WN; tn++)
          acc[tm][tn] = mfma16<TS>(bfr[tn], af[tm], acc[tm][tn]);
    }
    if (do_colsum) {
      // A is stored (K, M): LDS [k][m] (k past K reads as zero: the copy stops at the
      // operand's end)
#pragma unroll
      for (int j = 0; j < BK / KG; j++) {
        const int k = tid / CHUNKS + KG * j, mc = tid % CHUNKS;
        const u32x4 x = *reinterpret_cast<const u32x4*>(pa + k * 2 * BM +
                                                         16 * (mc ^ rswz<BM>(k & 3)));
#pragma unroll
        for (int q = 0; q < 4; q++) {
          csum[2 * q] += Half16<TS>::lo(x[q]);
          csum[2 * q + 1] += Half16<TS>::hi(x[q]);
        }
      }
    }
  };
  // Stage of slab kt: kt % NSTAGE. Slab kt + NSTAGE - 1 is issued while slab kt is used. The
  // loop is unrolled by NSTAGE so every LDS access names its stage statically, and every step
  // issues the same copies (empty ones past the last slab).
  constexpr int COPIES =
      SlabCopy<AT, BM, NWAVES, BK>::PER_WAVE + SlabCopy<BT, BN, NWAVES, BK>::PER_WAVE;
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
    // whole groups of NSTAGE steps in the loop: every path round the loop issues the same
    // copies in the same order, so the compiler's waits before reading a stage need only that
    // stage's copies; the remaining steps follow the loop
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
    // reduce the KG k-row groups of each m through LDS (stage 0 of A: KG x BM floats)
    float* red = reinterpret_cast<float*>(As0);
    lds_barrier();
#pragma unroll
    for (int e = 0; e < 8; e++) red[(tid / CHUNKS) * BM + 8 * (tid % CHUNKS) + e] = csum[e];
    __syncthreads();
    if (tid < BM && m0 + tid < g.M) {
      float total = 0.f;
      for (int j = 0; j < KG; j++) total += red[j * BM + tid];
      if (g.colsum_zstride) g.colsum[(long long)z * g.colsum_zstride + m0 + tid] = total;
      else g.colsum[m0 + tid] += total;
    }
  }

  void* C = CF32 ? static_cast<void*>(static_cast<float*>(g.C) + (long long)z * g.c_zstride)
                 : g.C;
  // acc[tm][tn][4q + j]: row m = m0 + wm0 + 32 tm + r, column n = n0 + wn0 + 32 tn + 8q + 4h + j.
  // One vector-memory counter covers loads and stores, so a load waited for between stores
  // also waits for every store issued before it: the bias is added into the accumulators
  // before anything is stored, and the rows an epilogue reads (residual, GELU pre-activation,
  // or the fp32 C it accumulates into) are loaded for the next 32-row block before the
  // current block is stored. epilogue4 then runs with the bias already applied and the row
  // values passed in; the arithmetic and its order are unchanged.
  constexpr bool HAS_BIAS = EPI == EPI_STORE || EPI == EPI_GELU || EPI == EPI_RESID;
  constexpr bool READS = EPI == EPI_RESID || EPI == EPI_GELU_BWD || (CF32 && EPI == EPI_ACCUM);
  auto col = [&](int tn, int q) { return n0 + wn0 + 32 * tn + 8 * q + 4 * h; };
  if (HAS_BIAS && g.bias) {
#pragma unroll
    for (int tn = 0; tn < WN; tn++)
#pragma unroll
      for (int q = 0; q < 4; q++) {
        const int n = col(tn, q);
        f32x4 bv = {0.f, 0.f, 0.f, 0.f};
        if (n + 3 < g.N) bv = *reinterpret_cast<const f32x4*>(g.bias + n);
        else
          for (int j = 0; j < 4; j++)
            if (n + j < g.N) bv[j] = g.bias[n + j];
#pragma unroll
        for (int tm = 0; tm < WM; tm++)
#pragma unroll
          for (int j = 0; j < 4; j++) acc[tm][tn][4 * q + j] += bv[j];
      }
  }
  f32x4 rv[WN][4];
  auto load_rows = [&](int tm) {
    const int m = m0 + wm0 + 32 * tm + r;
#pragma unroll
    for (int tn = 0; tn < WN; tn++)
#pragma unroll
      for (int q = 0; q < 4; q++) {
        const int n = col(tn, q);
        rv[tn][q] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (m >= g.M || n >= g.N) continue;
        const long long off = (long long)m * g.ldc + n;
        const int cnt = min(4, g.N - n);
        if (EPI == EPI_ACCUM) {
          const float* Cf = static_cast<const float*>(C);
          if (cnt == 4) rv[tn][q] = *reinterpret_cast<const f32x4*>(Cf + off);
          else
            for (int j = 0; j < cnt; j++) rv[tn][q][j] = Cf[off + j];
        } else {
          if (cnt == 4) rv[tn][q] = ld4(g.R + off);
          else
            for (int j = 0; j < cnt; j++) rv[tn][q][j] = ld1(g.R + off + j);
        }
      }
  };
  if (READS) load_rows(0);
#pragma unroll
  for (int tm = 0; tm < WM; tm++) {
    const int m = m0 + wm0 + 32 * tm + r;
    f32x4 rcur[WN][4];
#pragma unroll
    for (int tn = 0; tn < WN; tn++)
#pragma unroll
      for (int q = 0; q < 4; q++) rcur[tn][q] = rv[tn][q];
    if (READS && tm + 1 < WM) load_rows(tm + 1);
    if (m >= g.M) continue;
#pragma unroll
    for (int tn = 0; tn < WN; tn++)
#pragma unroll
      for (int q = 0; q < 4; q++) {
        const int n = col(tn, q);
        if (n >= g.N) continue;
        epilogue4_pre<TS, EPI, CF32>(g, C, m, n,
                                     f32x4{acc[tm][tn][4 * q], acc[tm][tn][4 * q + 1],
                                           acc[tm][tn][4 * q + 2], acc[tm][tn][4 * q + 3]},
                                     rcur[tn][q]);
      }
  }
}

// Adds `splits` fp32 partials (each M x N, row stride wld) in split order, then applies the
// epilogue into the real output; four consecutive columns per thread.
// With colsum_part, the last workgroups instead add the per-split column sums (split order)
// into g.colsum.
template <typename TS, int EPI, bool CF32>
__global__ void split_reduce_bf16_kernel(Args<TS> g, const float* __restrict__ ws, int splits,
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
    epilogue4<TS, EPI, CF32>(g, g.C, m, n, s);
  }
}


template <typename TS, class CFG, bool AT, bool BT, bool CF32>
void launch_epi(const Args<TS>& a, int epi, dim3 grid, hipStream_t s) {
  constexpr int NT = CFG::NT;
  switch (epi) {
    case EPI_STORE: gemm16_kernel<TS, CFG, AT, BT, CF32, EPI_STORE><<<grid, NT, 0, s>>>(a); break;
    case EPI_GELU: gemm16_kernel<TS, CFG, AT, BT, false, EPI_GELU><<<grid, NT, 0, s>>>(a); break;
    case EPI_RESID:
      if constexpr (kReadingEpilogues<CFG>)
        gemm16_kernel<TS, CFG, AT, BT, false, EPI_RESID><<<grid, NT, 0, s>>>(a);
      break;
    case EPI_ACCUM:
      if constexpr (kReadingEpilogues<CFG>)
        gemm16_kernel<TS, CFG, AT, BT, true, EPI_ACCUM><<<grid, NT, 0, s>>>(a);
      break;
    case EPI_GELU_BWD:
      if constexpr (kReadingEpilogues<CFG>)
        gemm16_kernel<TS, CFG, AT, BT, false, EPI_GELU_BWD><<<grid, NT, 0, s>>>(a);
      break;
  }
}

template <typename TS, class CFG, bool AT, bool BT>
void launch_c(const Args<TS>& a, int epi, bool cf32, dim3 grid, hipStream_t s) {
  if (cf32) launch_epi<TS, CFG, AT, BT, true>(a, epi, grid, s);
  else launch_epi<TS, CFG, AT, BT, false>(a, epi, grid, s);
}

template <class CFG, typename TS>
void launch(const Args<TS>& a, bool at, bool bt, int epi, bool cf32, dim3 grid, hipStream_t s) {
  if (!at && !bt) launch_c<TS, CFG, false, false>(a, epi, cf32, grid, s);
  else if (!at && bt) launch_c<TS, CFG, false, true>(a, epi, cf32, grid, s);
  else if (at && bt) launch_c<TS, CFG, true, true>(a, epi, cf32, grid, s);
  else launch_c<TS, CFG, true, false>(a, epi, cf32, grid, s);
}

int ceil_div(long long a, long long b) { return (int)((a + b - 1) / b); }

// Tile shape and K splits from a wave-quantisation cost model: each shape's workgroups run
// in rounds of OCC per CU (256 CUs) at that shape's measured fraction of the bf16 MFMA peak;
// split partials and their reduction move at 5 TB/s.
enum TileKind { T128 = 1, T256 = 2, T192 = 3, T320 = 4 };
struct Plan {
  int tile;    // TileKind
  int splits;
};
struct TileInfo {
  int bm, bn, bk, occ;
  double eff;  // measured fraction of the peak on the 774M shapes
};
TileInfo tile_info(int t) {
  if (t == T128) return {Tile128::BM, Tile128::BN, Tile128::BK, Tile128::OCC, 0.26};
  if (t == T192) return {Tile192::BM, Tile192::BN, Tile192::BK, Tile192::OCC, 0.33};
  if (t == T320) return {Tile320::BM, Tile320::BN, Tile320::BK, Tile320::OCC, 0.34};
  return {Tile256::BM, Tile256::BN, Tile256::BK, Tile256::OCC, 0.34};
}
// GPT2_GEMM_BF16_TILE=1 (128 x 128), 2 (256 x 256), 3 (256 x 192) or 4 (256 x 320) in the
// environment pins the tile shape (tests of every kernel, measurements; pinned to 256 x 320,
// an epilogue that reads a tensor runs split or on the default 128 x 128 tile); anything
// else leaves the choice to the model
int forced_tile() {
  const char* e = getenv("GPT2_GEMM_BF16_TILE");
  const int v = e ? atoi(e) : 0;
  return v >= T128 && v <= T320 ? v : 0;
}
template <typename TS>
Plan choose_plan(const GemmHalf<TS>& g) {
  const double mn = (double)g.M * g.N;
  Plan best_p{T128, 1};
  double best = 1e30;
  for (int t = T128; t <= T320; t++) {
    if (forced_tile() && t != forced_tile()) continue;
    const TileInfo ti = tile_info(t);
    const int kt = ceil_div(g.K, ti.bk);
    const double tiles = (double)ceil_div(g.M, ti.bm) * ceil_div(g.N, ti.bn);
    for (int s = 1; s <= 16; s++) {
      if (t == T320 && s == 1 && epi_reads(g.epi)) continue;  // (split launches store only)
      const int kper = ceil_div(kt, s);
      if (s > 1 && kper * ti.bk < 128) break;
      if (s > 1 && ceil_div(kt, kper) != s) continue;
      const double rounds = std::ceil(tiles * s / (256.0 * ti.occ));
      double cost = rounds * ti.occ * 2.0 * ti.bm * ti.bn * (double)kper * ti.bk /
                    (ti.eff * 2516.6e12 / 256);
      if (s > 1) cost += 4.0 * mn * (s + 2.0) / 5e12;
      if (cost < best * 0.97) {
        best = cost;
        best_p = Plan{t, s};
      }
    }
  }
  return best_p;
}

int split_ld(int N) { return (N + 3) & ~3; }

bool aligned16(const void* p) { return ((uintptr_t)p & 15) == 0; }

}  // namespace

template <typename TS>
size_t gemm16_workspace_floats(const GemmHalf<TS>& g) {
  const int s = choose_plan(g).splits;
  if (s <= 1) return 0;
  return (size_t)s * g.M * split_ld(g.N) + (g.colsum ? (size_t)s * g.M : 0);
}

template <typename TS>
int gemm16(const GemmHalf<TS>& g, float* workspace, size_t ws_floats, hipStream_t stream) {
  constexpr bool F16 = std::is_same<TS, f16_t>::value;
  const char* fmt = F16 ? "f16" : "bf16";
  if (g.M <= 0 || g.N <= 0 || g.K <= 0) {
    set_global_error("gemm_%s: non-positive size M=%d N=%d K=%d", fmt, g.M, g.N, g.K);
    return -1;
  }
  // 16-byte operand loads need 16-byte aligned bases and leading dimensions that are
  // multiples of 8 elements; the epilogue's vector stores need ldc % 8 (bf16) or % 4 (fp32)
  const bool cf32 = g.epi == EPI_ACCUM;
  const int a_cols = g.a_trans ? g.M : g.K, b_cols = g.b_trans ? g.N : g.K;
  // (and leading dimensions below 2^24 and operands below 4 GiB, so the byte offsets and
  // the extent of a slab's buffer resource fit 32 bits)
  if (!aligned16(g.A) || !aligned16(g.B) || !aligned16(g.C) || g.lda % 8 || g.ldb % 8 ||
      g.ldc % (cf32 ? 4 : 8) || g.lda < a_cols || g.ldb < b_cols || g.ldc < g.N ||
      (g.bias && !aligned16(g.bias)) || g.lda >= (1 << 24) || g.ldb >= (1 << 24) ||
      2.0 * (g.a_trans ? g.K : g.M) * g.lda >= 4294967295.0 ||
      2.0 * (g.b_trans ? g.K : g.N) * g.ldb >= 4294967295.0) {
    set_global_error("gemm_%s: unsupported alignment or leading dimension (lda=%d ldb=%d "
                     "ldc=%d)", fmt, g.lda, g.ldb, g.ldc);
    return -1;
  }
  if ((g.epi == EPI_GELU && !g.C2) || ((g.epi == EPI_RESID || g.epi == EPI_GELU_BWD) && !g.R) ||
      (g.colsum && !g.a_trans)) {
    set_global_error("gemm_%s: epilogue %d is missing an operand", fmt, (int)g.epi);
    return -1;
  }
  Args<TS> a;
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
  const TileInfo ti = tile_info(plan.tile);
  int splits = plan.splits;
  if (splits > 1 && (!workspace || ws_floats < gemm16_workspace_floats(g))) splits = 1;
  const int kt = ceil_div(g.K, ti.bk);
  const int kt_per = ceil_div(kt, splits);
  splits = ceil_div(kt, kt_per);
  a.k_split = kt_per * ti.bk;
  a.splits = splits;
  const int tiles = ceil_div(g.M, ti.bm) * ceil_div(g.N, ti.bn);
  auto run = [&](const Args<TS>& x, int epi, bool f32out, int grid) {
    const bool at = g.a_trans, bt = g.b_trans;
    if (plan.tile == T128) launch<Tile128>(x, at, bt, epi, f32out, dim3(grid), stream);
    else if (plan.tile == T192) launch<Tile192>(x, at, bt, epi, f32out, dim3(grid), stream);
    else if (plan.tile == T320) launch<Tile320>(x, at, bt, epi, f32out, dim3(grid), stream);
    else launch<Tile256>(x, at, bt, epi, f32out, dim3(grid), stream);
  };

  const double MN = (double)g.M * g.N;
  const double flop = 2.0 * MN * g.K;
  const double in_bytes = 2.0 * ((double)g.M * g.K + (double)g.N * g.K);
  const double cb = cf32 ? 4.0 : 2.0;
  const double out_bytes = g.epi == EPI_STORE ? cb * MN : 2.0 * cb * MN;
  char name[80];
  if (splits == 1) {
    snprintf(name, sizeof(name), "gemm_%s_kernel<%d,%d,%d>", fmt, (int)g.a_trans,
             (int)g.b_trans, (int)g.epi);
    if (profiling_detail())
      snprintf(name + strlen(name), sizeof(name) - strlen(name), " %dx%dx%d", g.M, g.N, g.K);
    ProfScope ps(name, flop, in_bytes + out_bytes, stream);
    run(a, g.epi, cf32, tiles);
  } else {
    Args<TS> p = a;
    p.C = workspace;
    p.ldc = split_ld(g.N);
    p.c_zstride = (long long)g.M * p.ldc;
    p.bias = nullptr;
    float* colsum_part = workspace + (size_t)splits * g.M * p.ldc;
    if (g.colsum) {
      p.colsum = colsum_part;
      p.colsum_zstride = g.M;
    }
    snprintf(name, sizeof(name), "gemm_%s_kernel<%d,%d,0>", fmt, (int)g.a_trans, (int)g.b_trans);
    if (profiling_detail())
      snprintf(name + strlen(name), sizeof(name) - strlen(name), " %dx%dx%d/%d", g.M, g.N, g.K,
               splits);
    {
      ProfScope ps(name, flop, in_bytes + 4.0 * MN * splits, stream);
      run(p, EPI_STORE, true, tiles * splits);
    }
    const long long total = (long long)g.M * ((g.N + 3) / 4);
    int blocks = (int)((total + 255) / 256);
    if (blocks > 8192) blocks = 8192;
    snprintf(name, sizeof(name), "split_reduce_%s_kernel<%d>", fmt, (int)g.epi);
    const float* cp = g.colsum ? colsum_part : nullptr;
    const int nblk = blocks + (cp ? ceil_div(g.M, 256) : 0);
    ProfScope ps(name, 0.0, 4.0 * MN * splits + out_bytes + (cp ? 4.0 * (splits + 2.0) * g.M : 0.0),
                 stream);
    switch (g.epi) {
      case EPI_ACCUM: split_reduce_bf16_kernel<TS, EPI_ACCUM, true><<<nblk, 256, 0, stream>>>(a, workspace, splits, p.ldc, cp); break;
      case EPI_GELU_BWD: split_reduce_bf16_kernel<TS, EPI_GELU_BWD, false><<<nblk, 256, 0, stream>>>(a, workspace, splits, p.ldc, cp); break;
      case EPI_GELU: split_reduce_bf16_kernel<TS, EPI_GELU, false><<<nblk, 256, 0, stream>>>(a, workspace, splits, p.ldc, cp); break;
      case EPI_RESID: split_reduce_bf16_kernel<TS, EPI_RESID, false><<<nblk, 256, 0, stream>>>(a, workspace, splits, p.ldc, cp); break;
      default: split_reduce_bf16_kernel<TS, EPI_STORE, false><<<nblk, 256, 0, stream>>>(a, workspace, splits, p.ldc, cp); break;
    }
  }
  GPT2_HIP_OK(hipGetLastError());
  return 0;
}

size_t gemm_bf16_workspace_floats(const GemmBf16& g) { return gemm16_workspace_floats(g); }
size_t gemm_f16_workspace_floats(const GemmF16& g) { return gemm16_workspace_floats(g); }
int gemm_bf16(const GemmBf16& g, float* workspace, size_t ws_floats, hipStream_t stream) {
  return gemm16(g, workspace, ws_floats, stream);
}
int gemm_f16(const GemmF16& g, float* workspace, size_t ws_floats, hipStream_t stream) {
  return gemm16(g, workspace, ws_floats, stream);
}

}  // namespace gpt2
