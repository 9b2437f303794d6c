// attention_bf16.hip -- causal attention of the mixed-precision steps on 16-bit MFMA
// (v_mfma_f32_32x32x16_bf16 or v_mfma_f32_32x32x16_f16, fp32 accumulation), and the fp32
// attention forward and dQ with split-operand products on bf16 MFMA.
//
// Same computation as attention.hip ("llm.c 的中文注解-20240421" sections 1.7 and 1.8;
// flash-style: online softmax forward keeping only the row log-sum-exp, recomputation in
// the backward), for 16-bit (bf16 or fp16: the storage type TS) Q, K, V, O, dO and dQKV.
// The score products take 16-bit operands with exact products and fp32 sums, as in fp32
// arithmetic on the same inputs; the probabilities P and the score gradients dS are rounded
// to TS where they become MFMA operands. Softmax statistics, lse and rowsum(dO*O) stay
// fp32; the dS tiles handed from the dK/dV kernel to the dQ kernel are TS.
//
// Register layouts. Each lane of the bf16 MFMA supplies 8 consecutive k of one row of A and
// of one column of B; the result tile gives lane l the column l % 32 and the rows
// 8*(i/4) + 4*(l/32) + i%4 of acc[i]. Scores are computed transposed (keys down the rows,
// one query per lane column), so for a 16-wide k step the 16 accumulator entries
// 8h .. 8h+7 of lanes l and l+32 together hold 16 consecutive keys of the lane's query:
// lane l < 32 keys 16h + {0..3, 8..11}, lane l+32 keys 16h + {4..7, 12..15}. That is
// directly the B operand of the next product if the other operand orders its keys the same
// way, which V^T (and, in the backward, dO^T and Q^T) do by being stored in LDS at the
// permuted key position kpos() below: each lane's 8 keys are then one 16-byte read.
#include <cmath>
#include <type_traits>

#include "attn_order.h"
#include "kernels.h"

namespace gpt2 {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int TILE = 64;   // queries per workgroup, keys per tile
constexpr int NTHR = 128;  // two waves of 32 queries (or keys)

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4_t;

GPT2_DEVICE_INLINE f32x16 mfma_bf16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
// the MFMA of storage format TS on fragments holding its raw 16-bit patterns
template <typename TS>
GPT2_DEVICE_INLINE f32x16 mfma16(bf16x8 a, bf16x8 b, f32x16 c) {
  if constexpr (std::is_same<TS, f16_t>::value)
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  else
    return mfma_bf16(a, b, c);
}

// position of key k (0..63 within a tile) in a permuted row: groups of 4 keys stay
// together, and lane-half lh of k step (kb, h) finds its 8 keys at 32kb + 16h + 8lh .. +7
GPT2_DEVICE_INLINE int kpos(int k) {
  const int r = k & 15;
  return (k & ~15) + 8 * ((r >> 2) & 1) + (r & 3) + 4 * (r >> 3);
}

// LDS tiles of ROWS rows x COLS 16-bit values (COLS a multiple of 8): 16-byte chunk c of row r is
// stored at chunk c ^ swz(r), which spreads 32 rows read at the same chunk, and rows 8
// apart written at the same chunk, over the banks.
template <int COLS>
GPT2_DEVICE_INLINE int loff(int row, int c) {
  constexpr int CPR = COLS / 8;
  return row * COLS + ((c ^ ((row ^ (row >> 3)) & (CPR - 1))) << 3);
}

// 16 bytes (8 values of a 16-bit format) of row t, columns d..d+7 of a strided tensor; rows
// past the end and columns past hs read as zero (addresses clamped into the tensor)
template <typename P>
GPT2_DEVICE_INLINE u32x4 load8(const P* base, long long ld, int t, int d, int T, int hs) {
  static_assert(sizeof(P) == 2, "16-bit storage");
  const int tc = min(t, T - 1), dc = min(d, hs - 8);
  const u32x4 x = *reinterpret_cast<const u32x4*>(base + (long long)tc * ld + dc);
  return (t < T && d < hs) ? x : u32x4{0u, 0u, 0u, 0u};
}
// The same load with the zeroing left to the caller (returns whether the values are real):
// the tile structs below apply it when they store, so the loads of the next tile stay in
// flight until then (a select right after the load makes the compiler wait for it there).
template <typename P>
GPT2_DEVICE_INLINE bool load8_raw(const P* base, long long ld, int t, int d, int T, int hs,
                                  u32x4& x) {
  static_assert(sizeof(P) == 2, "16-bit storage");
  const int tc = min(t, T - 1), dc = min(d, hs - 8);
  x = *reinterpret_cast<const u32x4*>(base + (long long)tc * ld + dc);
  return t < T && d < hs;
}

// Natural tile: rows row0 .. row0+63 of the tensor -> S[row][d] (HSP columns). load()
// fills registers, store() writes them, so a tile can be fetched ahead of its use.
template <int HSP>
struct RowsTile {
  static constexpr int CPR = HSP / 8, NI = TILE * CPR / NTHR;
  u32x4 v[NI];
  uint32_t ok;  // bit i: chunk i holds values (else it is stored as zeros)
  template <typename P>
  __device__ __forceinline__ void load(const P* base, long long ld, int row0, int T, int hs,
                                       int tid) {
    ok = 0;
#pragma unroll
    for (int i = 0; i < NI; i++) {
      const int f = tid + NTHR * i;
      ok |= (uint32_t)load8_raw(base, ld, row0 + f / CPR, 8 * (f % CPR), T, hs, v[i]) << i;
    }
  }
  __device__ __forceinline__ void store(uint16_t* S, int tid) const {
#pragma unroll
    for (int i = 0; i < NI; i++) {
      const int f = tid + NTHR * i;
      *reinterpret_cast<u32x4*>(S + loff<HSP>(f / CPR, f % CPR)) =
          (ok >> i) & 1 ? v[i] : u32x4{0u, 0u, 0u, 0u};
    }
  }
};

// Transposed tile: rows row0 .. row0+63 of the tensor -> S[d][kpos(row)] (64 columns). A
// thread moves blocks of 4 rows x 8 columns: four 16-byte loads, eight 8-byte stores.
template <int HSP>
struct ColsTile {
  static constexpr int DG = HSP / 8;             // 8-column groups
  static constexpr int BLOCKS = (TILE / 4) * DG;  // 4x8 blocks in the tile
  static constexpr int NI = (BLOCKS + NTHR - 1) / NTHR;
  u32x4 x[NI][4];
  uint32_t ok;  // bit 4 i + j: row j of block i holds values (else it is stored as zeros)
  template <typename P>
  __device__ __forceinline__ void load(const P* base, long long ld, int row0, int T, int hs,
                                       int tid) {
    ok = 0;
#pragma unroll
    for (int i = 0; i < NI; i++) {
      const int b = tid + NTHR * i;
      if (BLOCKS % NTHR && b >= BLOCKS) break;
      const int dg = b % DG, rq = b / DG;  // columns 8dg .. +7, rows 4rq .. +3
#pragma unroll
      for (int j = 0; j < 4; j++)
        ok |= (uint32_t)load8_raw(base, ld, row0 + 4 * rq + j, 8 * dg, T, hs, x[i][j])
              << (4 * i + j);
    }
  }
  __device__ __forceinline__ void store(uint16_t* S, int tid) {
#pragma unroll
    for (int i = 0; i < NI; i++) {
      const int b = tid + NTHR * i;
      if (BLOCKS % NTHR && b >= BLOCKS) break;
#pragma unroll
      for (int j = 0; j < 4; j++)
        if (!((ok >> (4 * i + j)) & 1)) x[i][j] = u32x4{0u, 0u, 0u, 0u};
      const int dg = b % DG, rq = b / DG;
      const int p = kpos(4 * rq);  // a multiple of 4: the 4 rows stay consecutive
#pragma unroll
      for (int e = 0; e < 8; e++) {
        const int q = e >> 1;
        uint32_t lo, hi;
        if ((e & 1) == 0) {
          lo = (x[i][0][q] & 0xFFFFu) | (x[i][1][q] << 16);
          hi = (x[i][2][q] & 0xFFFFu) | (x[i][3][q] << 16);
        } else {
          lo = (x[i][0][q] >> 16) | (x[i][1][q] & 0xFFFF0000u);
          hi = (x[i][2][q] >> 16) | (x[i][3][q] & 0xFFFF0000u);
        }
        *reinterpret_cast<u32x2*>(S + loff<TILE>(8 * dg + e, p >> 3) + (p & 7)) = u32x2{lo, hi};
      }
    }
  }
};

template <int HSP, typename P>
GPT2_DEVICE_INLINE void tile_rows(uint16_t* S, const P* base, long long ld, int row0, int T,
                                  int hs, int tid) {
  RowsTile<HSP> t;
  t.load(base, ld, row0, T, hs, tid);
  t.store(S, tid);
}

template <int HSP, typename P>
GPT2_DEVICE_INLINE void tile_cols(uint16_t* S, const P* base, long long ld, int row0, int T,
                                  int hs, int tid) {
  ColsTile<HSP> t;
  t.load(base, ld, row0, T, hs, tid);
  t.store(S, tid);
}

GPT2_DEVICE_INLINE void tile_of_block(int ntiles, int NH, int* tile, int* head, int* b) {
  const int lid = xcd_logical_block(blockIdx.x, gridDim.x);
  *tile = lid % ntiles;
  const int bh = lid / ntiles;
  *head = bh % NH;
  *b = bh / NH;
}

// ---------------------------------------------------------------------------------------
// forward: a workgroup owns 64 queries (32 per wave) of one (batch, head)
// ---------------------------------------------------------------------------------------
template <int HSP, typename TS>
__global__ __launch_bounds__(NTHR) void attn_fwd_mma16_kernel(TS* __restrict__ out,
                                                              float* __restrict__ lse,
                                                              const TS* __restrict__ qkv, int T,
                                                              int C, int NH, int hs,
                                                              float scale_log2) {
  constexpr int KS = HSP / 16, ND = HSP / 32;
  __shared__ __attribute__((aligned(16))) uint16_t Ks[TILE * HSP];   // [key][d]
  __shared__ __attribute__((aligned(16))) uint16_t Vt[HSP * TILE];   // [d][kpos(key)]

  const int nqt = (T + TILE - 1) / TILE;
  int qt, head, b;
  tile_of_block(nqt, NH, &qt, &head, &b);
  qt = nqt - 1 - qt;  // longest rows first
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r = lane & 31, lh = lane >> 5;
  const long long C3 = 3LL * C;
  const TS* base = qkv + (long long)b * T * C3 + (long long)head * hs;
  const int q = qt * TILE + wave * 32 + r;
  const int qm = min(q, T - 1);  // lanes past the end mask as the last row; never stored

  // this lane's query, d = 16ks + 8lh .. +7 for each k step
  bf16x8 qf[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ks++)
    qf[ks] = __builtin_bit_cast(bf16x8, load8(base, C3, qm, 16 * ks + 8 * lh, T, hs));

  f32x16 oacc[ND];
#pragma unroll
  for (int db = 0; db < ND; db++)
#pragma unroll
    for (int i = 0; i < 16; i++) oacc[db][i] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;  // in units of the scaled log2 domain

  const int ntiles = (min(T, (qt + 1) * TILE) + TILE - 1) / TILE;
  // the next key tile is loaded into registers while this one is used
  RowsTile<HSP> kn;
  ColsTile<HSP> vn;
  kn.load(base + C, C3, 0, T, hs, tid);
  vn.load(base + 2 * C, C3, 0, T, hs, tid);
  for (int kt = 0; kt < ntiles; kt++) {
    const int key0 = kt * TILE;
    __syncthreads();
    kn.store(Ks, tid);
    vn.store(Vt, tid);
    __syncthreads();
    if (kt + 1 < ntiles) {
      kn.load(base + C, C3, key0 + TILE, T, hs, tid);
      vn.load(base + 2 * C, C3, key0 + TILE, T, hs, tid);
    }

    // S^T for 2 x 32 keys: s[kb][i] = score of key 32kb + 8(i/4) + 4lh + i%4
    f32x16 s[2];
#pragma unroll
    for (int kb = 0; kb < 2; kb++) {
#pragma unroll
      for (int i = 0; i < 16; i++) s[kb][i] = 0.f;
#pragma unroll
      for (int ks = 0; ks < KS; ks++) {
        const bf16x8 kf =
            *reinterpret_cast<const bf16x8*>(&Ks[loff<HSP>(32 * kb + r, 2 * ks + lh)]);
        s[kb] = mfma16<TS>(kf, qf[ks], s[kb]);
      }
    }
    if (key0 + TILE > qt * TILE) {  // the diagonal tile (uniform): mask keys after the query
#pragma unroll
      for (int kb = 0; kb < 2; kb++)
#pragma unroll
        for (int i = 0; i < 16; i++) {
          const int key = key0 + 32 * kb + 8 * (i / 4) + 4 * lh + (i % 4);
          if (key > qm) s[kb][i] = -INFINITY;
        }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; kb++)
#pragma unroll
      for (int i = 0; i < 16; i++) mx = fmaxf(mx, s[kb][i]);
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64)) * scale_log2;
    // the running max moves only by more than 8 (see attention.hip): most tiles skip the
    // rescale; the first always moves it (key 0 <= qm is never masked)
    if (__any(mx > m_run + 8.f)) {
      const float m_new = fmaxf(m_run, mx);
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < ND; db++)
#pragma unroll
        for (int i = 0; i < 16; i++) oacc[db][i] *= alpha;
      m_run = m_new;
    }
    bf16x8 pf[2][2];  // P as the B operand of k step (kb, h)
#pragma unroll
    for (int kb = 0; kb < 2; kb++)
#pragma unroll
      for (int hh = 0; hh < 2; hh++) {
        u32x4 w;
#pragma unroll
        for (int j = 0; j < 4; j++) {
          const float p0 = __builtin_amdgcn_exp2f(fmaf(s[kb][8 * hh + 2 * j], scale_log2, -m_run));
          const float p1 = __builtin_amdgcn_exp2f(fmaf(s[kb][8 * hh + 2 * j + 1], scale_log2, -m_run));
          l_run += p0 + p1;
          w[j] = Half16<TS>::pack2(p0, p1);
        }
        pf[kb][hh] = __builtin_bit_cast(bf16x8, w);
      }
    // O^T[d][q] += V^T[d][key] P^T[key][q]
#pragma unroll
    for (int db = 0; db < ND; db++)
#pragma unroll
      for (int kb = 0; kb < 2; kb++)
#pragma unroll
        for (int hh = 0; hh < 2; hh++) {
          const bf16x8 vf = *reinterpret_cast<const bf16x8*>(
              &Vt[loff<TILE>(32 * db + r, 4 * kb + 2 * hh + lh)]);
          oacc[db] = mfma16<TS>(vf, pf[kb][hh], oacc[db]);
        }
  }

  const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
  const float inv = 1.0f / l_tot;
  if (q < T) {
    TS* o = out + ((long long)b * T + q) * C + (long long)head * hs;
#pragma unroll
    for (int db = 0; db < ND; db++)
#pragma unroll
      for (int ig = 0; ig < 4; ig++) {
        const int d = 32 * db + 8 * ig + 4 * lh;
        if (d < hs)
          st4(o + d, f32x4{oacc[db][4 * ig] * inv, oacc[db][4 * ig + 1] * inv,
                           oacc[db][4 * ig + 2] * inv, oacc[db][4 * ig + 3] * inv});
      }
    if (lh == 0) lse[((long long)b * NH + head) * T + q] = (m_run + log2f(l_tot)) * kLn2;
  }
}

// ---------------------------------------------------------------------------------------
// forward on fp32 tensors with split-operand products: each fp32 value of Q, K, V and P is
// split exactly into three bf16 parts (split8, x = hi + mid + lo, |mid| <= 2^-8 |x|,
// |lo| <= 2^-16 |x|) and every fp32 product becomes the six bf16 MFMA products of parts at
// or above 2^-16 of it (within 2^-23 of the exact product), accumulated in fp32. The
// structure is that of attn_fwd_bf16mma_kernel, with three LDS planes per K and V tile.
// ---------------------------------------------------------------------------------------
// acc += the six products of a (ah, am, al) x b (bh, bm, bl), smaller terms first
GPT2_DEVICE_INLINE f32x16 mfma_x6(bf16x8 ah, bf16x8 am, bf16x8 al, bf16x8 bh, bf16x8 bm,
                                  bf16x8 bl, f32x16 acc) {
  acc = mfma_bf16(am, bm, acc);
  acc = mfma_bf16(al, bh, acc);
  acc = mfma_bf16(ah, bl, acc);
  acc = mfma_bf16(am, bh, acc);
  acc = mfma_bf16(ah, bm, acc);
  return mfma_bf16(ah, bh, acc);
}

// 8 fp32 values of row t, columns d..d+7 (hs a multiple of 8); rows past T and columns
// past hs read as zero (addresses clamped into the tensor)
GPT2_DEVICE_INLINE void load8f(const float* base, long long ld, int t, int d, int T, int hs,
                               f32x4& x, f32x4& y) {
  const int tc = min(t, T - 1), dc = min(d, hs - 8);
  const float* p = base + (long long)tc * ld + dc;
  x = *reinterpret_cast<const f32x4*>(p);
  y = *reinterpret_cast<const f32x4*>(p + 4);
  if (!(t < T && d < hs)) {
    x = f32x4{0.f, 0.f, 0.f, 0.f};
    y = x;
  }
}

// The same load with the zeroing left to the caller: returns whether row t, columns d..d+7
// hold values (else the caller replaces x, y by zeros when it uses them). Staging code
// applies it when it stores, so the loads of the next tile stay in flight meanwhile (a
// select right after the load would make the compiler wait for them there).
GPT2_DEVICE_INLINE bool load8f_raw(const float* base, long long ld, int t, int d, int T, int hs,
                                   f32x4& x, f32x4& y) {
  const int tc = min(t, T - 1), dc = min(d, hs - 8);
  const float* p = base + (long long)tc * ld + dc;
  x = *reinterpret_cast<const f32x4*>(p);
  y = *reinterpret_cast<const f32x4*>(p + 4);
  return t < T && d < hs;
}
GPT2_DEVICE_INLINE void zero_unless(bool ok, f32x4& x, f32x4& y) {
  if (!ok) {
    x = f32x4{0.f, 0.f, 0.f, 0.f};
    y = x;
  }
}

// Natural tile of fp32 rows -> three bf16 planes S[p][row][d] (HSP columns each, loff
// layout), staged by NT threads
template <int HSP, int NT>
struct RowsTileX6 {
  static constexpr int CPR = HSP / 8, NI = TILE * CPR / NT;
  static_assert(NI * NT == TILE * CPR, "whole chunks per thread");
  f32x4 v[NI][2];
  uint32_t ok;  // bit i: chunk i holds values (else it is stored as zeros)
  __device__ __forceinline__ void load(const float* base, long long ld, int row0, int T,
                                       int hs, int tid) {
    ok = 0;
#pragma unroll
    for (int i = 0; i < NI; i++) {
      const int f = tid + NT * i;
      ok |= (uint32_t)load8f_raw(base, ld, row0 + f / CPR, 8 * (f % CPR), T, hs, v[i][0],
                                 v[i][1]) << i;
    }
  }
  __device__ __forceinline__ void store(bf16_t* S, int tid) {
#pragma unroll
    for (int i = 0; i < NI; i++) {
      const int f = tid + NT * i;
      zero_unless((ok >> i) & 1, v[i][0], v[i][1]);
      u32x4 h, m, l;
      split8(v[i][0], v[i][1], h, m, l);
      const int o = loff<HSP>(f / CPR, f % CPR);
      *reinterpret_cast<u32x4*>(S + o) = h;
      *reinterpret_cast<u32x4*>(S + TILE * HSP + o) = m;
      *reinterpret_cast<u32x4*>(S + 2 * TILE * HSP + o) = l;
    }
  }
};

// Transposed tile of fp32 rows -> three bf16 planes S[p][d][kpos(row)] (64 columns each; with
// KPOS false S[p][d][row]): a thread (of NT) moves blocks of 4 rows x 8 columns, split per
// row, then transposed per plane. Block b takes head dims 8 (b % DG) and the row run
// rq = run(b / DG): with kpos, run swaps bits 0 and 1, so the 16 lanes that write together
// pair runs 4 positions apart (the two 8-byte halves of a 16-byte chunk) rather than runs
// one chunk apart, whose writes to rows of one parity met in the same banks.
template <int HSP, int NT, bool KPOS = true>
struct ColsTileX6 {
  static constexpr int DG = HSP / 8;
  static constexpr int BLOCKS = (TILE / 4) * DG;
  static constexpr int NI = (BLOCKS + NT - 1) / NT;
  static __device__ __forceinline__ int run(int j) {
    return KPOS ? (j & ~3) | ((j & 1) << 1) | ((j >> 1) & 1) : j;
  }
  f32x4 v[NI][4][2];
  uint32_t ok;  // bit 4 i + j: row j of block i holds values (else it is stored as zeros)
  __device__ __forceinline__ void load(const float* base, long long ld, int row0, int T,
                                       int hs, int tid) {
    ok = 0;
#pragma unroll
    for (int i = 0; i < NI; i++) {
      const int b = tid + NT * i;
      if (BLOCKS % NT && b >= BLOCKS) break;
      const int dg = b % DG, rq = run(b / DG);
#pragma unroll
      for (int j = 0; j < 4; j++)
        ok |= (uint32_t)load8f_raw(base, ld, row0 + 4 * rq + j, 8 * dg, T, hs, v[i][j][0],
                                   v[i][j][1]) << (4 * i + j);
    }
  }
  __device__ __forceinline__ void store(bf16_t* S, int tid) {
#pragma unroll
    for (int i = 0; i < NI; i++) {
      const int b = tid + NT * i;
      if (BLOCKS % NT && b >= BLOCKS) break;
      const int dg = b % DG, rq = run(b / DG);
      const int p = KPOS ? kpos(4 * rq) : 4 * rq;
      u32x4 x[3][4];  // [plane][row]
#pragma unroll
      for (int j = 0; j < 4; j++) {
        zero_unless((ok >> (4 * i + j)) & 1, v[i][j][0], v[i][j][1]);
        split8(v[i][j][0], v[i][j][1], x[0][j], x[1][j], x[2][j]);
      }
#pragma unroll
      for (int pl = 0; pl < 3; pl++)
#pragma unroll
        for (int e = 0; e < 8; e++) {
          const int q = e >> 1;
          uint32_t lo, hi;
          if ((e & 1) == 0) {
            lo = (x[pl][0][q] & 0xFFFFu) | (x[pl][1][q] << 16);
            hi = (x[pl][2][q] & 0xFFFFu) | (x[pl][3][q] << 16);
          } else {
            lo = (x[pl][0][q] >> 16) | (x[pl][1][q] & 0xFFFF0000u);
            hi = (x[pl][2][q] >> 16) | (x[pl][3][q] & 0xFFFF0000u);
          }
          *reinterpret_cast<u32x2*>(S + pl * HSP * TILE + loff<TILE>(8 * dg + e, p >> 3) +
                                    (p & 7)) = u32x2{lo, hi};
        }
    }
  }
};

// A workgroup owns X6_QT = 128 queries (four waves of 32), so each split K and V tile
// serves four waves.
constexpr int X6_NW = 4, X6_NT = 64 * X6_NW, X6_QT = 32 * X6_NW;
template <int HSP>
__global__ __launch_bounds__(X6_NT, 2) void attn_fwd_x6_kernel(float* __restrict__ out,
                                                               float* __restrict__ lse,
                                                               const float* __restrict__ qkv,
                                                               int T, int C, int NH, int hs,
                                                               float scale_log2) {
  constexpr int KS = HSP / 16, ND = HSP / 32;
  constexpr int PK = TILE * HSP, PV = HSP * TILE;  // elements of one plane
  __shared__ __attribute__((aligned(16))) bf16_t Ks[3 * PK];  // [plane][key][d]
  __shared__ __attribute__((aligned(16))) bf16_t Vt[3 * PV];  // [plane][d][kpos(key)]

  const int nqt = (T + X6_QT - 1) / X6_QT;
  int qt, head, b;
  tile_of_block(nqt, NH, &qt, &head, &b);
  qt = nqt - 1 - qt;  // longest rows first
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r = lane & 31, lh = lane >> 5;
  const long long C3 = 3LL * C;
  const float* base = qkv + (long long)b * T * C3 + (long long)head * hs;
  const int q = qt * X6_QT + wave * 32 + r;
  const int qm = min(q, T - 1);  // lanes past the end mask as the last row; never stored
  const int wq_last = min(qt * X6_QT + wave * 32 + 31, T - 1);  // this wave's last query

  // this lane's query, d = 16ks + 8lh .. +7 for each k step, as three parts
  bf16x8 qh[KS], qmid[KS], ql[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ks++) {
    f32x4 x, y;
    load8f(base, C3, qm, 16 * ks + 8 * lh, T, hs, x, y);
    u32x4 h, m, l;
    split8(x, y, h, m, l);
    qh[ks] = __builtin_bit_cast(bf16x8, h);
    qmid[ks] = __builtin_bit_cast(bf16x8, m);
    ql[ks] = __builtin_bit_cast(bf16x8, l);
  }

  f32x16 oacc[ND];
#pragma unroll
  for (int db = 0; db < ND; db++)
#pragma unroll
    for (int i = 0; i < 16; i++) oacc[db][i] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;  // in units of the scaled log2 domain

  const int ntiles = (min(T, (qt + 1) * X6_QT) + TILE - 1) / TILE;
  RowsTileX6<HSP, X6_NT / 2> kn;
  ColsTileX6<HSP, X6_NT / 2> vn;
  // waves 2-3 stage K (four row chunks a thread), waves 0-1 stage V (one 4 x 8 block a
  // thread, transposed): the same load and split work on every wave (2.4% faster than all
  // waves staging both, where V's 128 blocks left half the threads idle)
  const bool kw = tid >= X6_NT / 2;
  const int t2 = tid & (X6_NT / 2 - 1);
  if (kw) kn.load(base + C, C3, 0, T, hs, t2);
  else vn.load(base + 2 * C, C3, 0, T, hs, t2);
  for (int kt = 0; kt < ntiles; kt++) {
    const int key0 = kt * TILE;
    __syncthreads();
    if (kw) kn.store(Ks, t2);
    else vn.store(Vt, t2);
    __syncthreads();
    if (kt + 1 < ntiles) {
      if (kw) kn.load(base + C, C3, key0 + TILE, T, hs, t2);
      else vn.load(base + 2 * C, C3, key0 + TILE, T, hs, t2);
    }
    if (key0 > wq_last) continue;  // every key of the tile follows this wave's queries

    // S^T for 2 x 32 keys: s[kb][i] = score of key 32kb + 8(i/4) + 4lh + i%4
    f32x16 s[2];
#pragma unroll
    for (int kb = 0; kb < 2; kb++) {
#pragma unroll
      for (int i = 0; i < 16; i++) s[kb][i] = 0.f;
#pragma unroll
      for (int ks = 0; ks < KS; ks++) {
        const int o = loff<HSP>(32 * kb + r, 2 * ks + lh);
        s[kb] = mfma_x6(*reinterpret_cast<const bf16x8*>(&Ks[o]),
                        *reinterpret_cast<const bf16x8*>(&Ks[PK + o]),
                        *reinterpret_cast<const bf16x8*>(&Ks[2 * PK + o]), qh[ks], qmid[ks],
                        ql[ks], s[kb]);
      }
    }
    if (key0 + TILE > qt * X6_QT + wave * 32) {  // a diagonal tile (uniform): mask later keys
#pragma unroll
      for (int kb = 0; kb < 2; kb++)
#pragma unroll
        for (int i = 0; i < 16; i++) {
          const int key = key0 + 32 * kb + 8 * (i / 4) + 4 * lh + (i % 4);
          if (key > qm) s[kb][i] = -INFINITY;
        }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; kb++)
#pragma unroll
      for (int i = 0; i < 16; i++) mx = fmaxf(mx, s[kb][i]);
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64)) * scale_log2;
    // the running max moves only by more than 8 (see attention.hip): most tiles skip the
    // rescale; the first always moves it (key 0 <= qm is never masked)
    if (__any(mx > m_run + 8.f)) {
      const float m_new = fmaxf(m_run, mx);
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < ND; db++)
#pragma unroll
        for (int i = 0; i < 16; i++) oacc[db][i] *= alpha;
      m_run = m_new;
    }
    // P as the B operand of k step (kb, hh), in three parts
    bf16x8 ph[2][2], pm[2][2], pl[2][2];
#pragma unroll
    for (int kb = 0; kb < 2; kb++)
#pragma unroll
      for (int hh = 0; hh < 2; hh++) {
        float pv[8];
#pragma unroll
        for (int j = 0; j < 8; j++) {
          pv[j] = __builtin_amdgcn_exp2f(fmaf(s[kb][8 * hh + j], scale_log2, -m_run));
          l_run += pv[j];
        }
        u32x4 wh, wm, wl;
        split8(f32x4{pv[0], pv[1], pv[2], pv[3]}, f32x4{pv[4], pv[5], pv[6], pv[7]}, wh, wm, wl);
        ph[kb][hh] = __builtin_bit_cast(bf16x8, wh);
        pm[kb][hh] = __builtin_bit_cast(bf16x8, wm);
        pl[kb][hh] = __builtin_bit_cast(bf16x8, wl);
      }
    // O^T[d][q] += V^T[d][key] P^T[key][q]
#pragma unroll
    for (int db = 0; db < ND; db++)
#pragma unroll
      for (int kb = 0; kb < 2; kb++)
#pragma unroll
        for (int hh = 0; hh < 2; hh++) {
          const int o = loff<TILE>(32 * db + r, 4 * kb + 2 * hh + lh);
          oacc[db] = mfma_x6(*reinterpret_cast<const bf16x8*>(&Vt[o]),
                             *reinterpret_cast<const bf16x8*>(&Vt[PV + o]),
                             *reinterpret_cast<const bf16x8*>(&Vt[2 * PV + o]), ph[kb][hh],
                             pm[kb][hh], pl[kb][hh], oacc[db]);
        }
  }

  const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
  const float inv = 1.0f / l_tot;
  if (q < T) {
    float* o = out + ((long long)b * T + q) * C + (long long)head * hs;
#pragma unroll
    for (int db = 0; db < ND; db++)
#pragma unroll
      for (int ig = 0; ig < 4; ig++) {
        const int d = 32 * db + 8 * ig + 4 * lh;
        if (d < hs)
          st4(o + d, f32x4{oacc[db][4 * ig] * inv, oacc[db][4 * ig + 1] * inv,
                           oacc[db][4 * ig + 2] * inv, oacc[db][4 * ig + 3] * inv});
      }
    if (lh == 0) lse[((long long)b * NH + head) * T + q] = (m_run + log2f(l_tot)) * kLn2;
  }
}

// causal 64x64 tiles (qt, kt <= qt) of one (batch, head), stored in row order
GPT2_DEVICE_INLINE long long tri_index(int qt, int kt) { return (long long)qt * (qt + 1) / 2 + kt; }
GPT2_DEVICE_INLINE long long tri_tiles(int n) { return (long long)n * (n + 1) / 2; }

// ---------------------------------------------------------------------------------------
// dQ = dS K on fp32 tensors with split-operand products (as attn_fwd_x6_kernel): a workgroup
// owns 128 queries (four waves of 32) and walks the 64-key tiles up to its diagonal; the
// fp32 dS tiles written by attn_bwd_dkdv_kernel ([query][key], 64 x 64 per causal tile) and
// the K tile are split into three bf16 planes each (dS [q][key], K transposed [d][key]).
// dQ^T[d][q] accumulates so a lane stores four consecutive head dims of its query.
// ---------------------------------------------------------------------------------------
template <int HSP>
__global__ __launch_bounds__(X6_NT, 2) void attn_bwd_dq_x6_kernel(float* __restrict__ dqkv,
                                                                  const float* __restrict__ qkv,
                                                                  const float* __restrict__ dsbuf,
                                                                  int T, int C, int NH, int hs,
                                                                  float scale) {
  constexpr int ND = HSP / 32, KS = TILE / 16;
  constexpr int PK = HSP * TILE, PS = X6_QT * TILE;  // elements of one plane
  __shared__ __attribute__((aligned(16))) bf16_t Kt[3 * PK];  // [plane][d][key]
  __shared__ __attribute__((aligned(16))) bf16_t Ss[3 * PS];  // [plane][q][key]

  const int nq64 = (T + TILE - 1) / TILE;  // 64-query tiles of the dS store
  const int nqt = (T + X6_QT - 1) / X6_QT;
  int qt, head, b;
  tile_of_block(nqt, NH, &qt, &head, &b);
  qt = nqt - 1 - qt;  // longest rows first
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r = lane & 31, lh = lane >> 5;
  const long long C3 = 3LL * C;
  const float* kbase = qkv + (long long)b * T * C3 + (long long)head * hs + C;
  const float* sbase = dsbuf + ((long long)b * NH + head) * tri_tiles(nq64) * (TILE * TILE);
  const int wq_last = min(qt * X6_QT + wave * 32 + 31, T - 1);

  f32x16 acc[ND];
#pragma unroll
  for (int db = 0; db < ND; db++)
#pragma unroll
    for (int i = 0; i < 16; i++) acc[db][i] = 0.f;

  // dS staging: 128 rows x 64 keys, chunks of 8 keys. Waves 0-1 take chunks t, t + 128, ...
  // (six each), waves 2-3 the last 256 (two each) and also stage the K tile, so the load and
  // split work is close to even over the waves (4% faster than every wave taking four dS
  // chunks while only waves 0-1 staged K)
  const bool kw = tid >= X6_NT / 2;
  const int t2 = tid & (X6_NT / 2 - 1);
  constexpr int CH_LO = 6, CH_HI = 2;  // chunks a thread: 128 x 6 + 128 x 2 = 1024
  static_assert((X6_NT / 2) * (CH_LO + CH_HI) == X6_QT * TILE / 8, "dS chunks");
  f32x4 sv6[CH_LO][2];
  auto chunk_of = [&](int i) { return kw ? (X6_NT / 2) * CH_LO + t2 + (X6_NT / 2) * i
                                         : t2 + (X6_NT / 2) * i; };
  auto load_ds = [&](int kt) {
#pragma unroll
    for (int i = 0; i < CH_LO; i++) {
      if (kw && i >= CH_HI) break;
      const int f = chunk_of(i), row = f / (TILE / 8), c = f % (TILE / 8);
      const int q64 = (X6_QT / TILE) * qt + row / TILE;  // the 64-query tile of this row
      if (q64 < nq64 && kt <= q64) {  // the causal tile (q64, kt) exists
        const float* p = sbase + tri_index(q64, kt) * (TILE * TILE) + (row % TILE) * TILE + 8 * c;
        sv6[i][0] = *reinterpret_cast<const f32x4*>(p);
        sv6[i][1] = *reinterpret_cast<const f32x4*>(p + 4);
      } else {
        sv6[i][0] = f32x4{0.f, 0.f, 0.f, 0.f};
        sv6[i][1] = sv6[i][0];
      }
    }
  };
  auto store_ds = [&]() {
#pragma unroll
    for (int i = 0; i < CH_LO; i++) {
      if (kw && i >= CH_HI) break;
      const int f = chunk_of(i), row = f / (TILE / 8), c = f % (TILE / 8);
      u32x4 h, m, l;
      split8(sv6[i][0], sv6[i][1], h, m, l);
      const int o = loff<TILE>(row, c);
      *reinterpret_cast<u32x4*>(Ss + o) = h;
      *reinterpret_cast<u32x4*>(Ss + PS + o) = m;
      *reinterpret_cast<u32x4*>(Ss + 2 * PS + o) = l;
    }
  };

  const int nkt = (min(T, (qt + 1) * X6_QT) + TILE - 1) / TILE;
  ColsTileX6<HSP, X6_NT / 2, false> kn;
  if (kw) kn.load(kbase, C3, 0, T, hs, t2);
  load_ds(0);
  for (int kt = 0; kt < nkt; kt++) {
    __syncthreads();
    if (kw) kn.store(Kt, t2);
    store_ds();
    __syncthreads();
    if (kt + 1 < nkt) {
      if (kw) kn.load(kbase, C3, (kt + 1) * TILE, T, hs, t2);
      load_ds(kt + 1);
    }
    if (kt * TILE > wq_last) continue;  // the tile lies wholly after this wave's queries
#pragma unroll
    for (int ks = 0; ks < KS; ks++) {
      const int os = loff<TILE>(32 * wave + r, 2 * ks + lh);
      const bf16x8 sh = *reinterpret_cast<const bf16x8*>(&Ss[os]);
      const bf16x8 sm = *reinterpret_cast<const bf16x8*>(&Ss[PS + os]);
      const bf16x8 sl = *reinterpret_cast<const bf16x8*>(&Ss[2 * PS + os]);
#pragma unroll
      for (int db = 0; db < ND; db++) {
        const int ok = loff<TILE>(32 * db + r, 2 * ks + lh);
        acc[db] = mfma_x6(*reinterpret_cast<const bf16x8*>(&Kt[ok]),
                          *reinterpret_cast<const bf16x8*>(&Kt[PK + ok]),
                          *reinterpret_cast<const bf16x8*>(&Kt[2 * PK + ok]), sh, sm, sl, acc[db]);
      }
    }
  }
  // acc[db][i]: head dim 32db + 8(i/4) + 4lh + i%4 of query 32 wave + r of the tile
  const int q = qt * X6_QT + 32 * wave + r;
  if (q < T) {
    float* dq = dqkv + ((long long)b * T + q) * C3 + (long long)head * hs;
#pragma unroll
    for (int db = 0; db < ND; db++)
#pragma unroll
      for (int ig = 0; ig < 4; ig++) {
        const int d = 32 * db + 8 * ig + 4 * lh;
        if (d < hs)
          st4(dq + d, f32x4{acc[db][4 * ig] * scale, acc[db][4 * ig + 1] * scale,
                            acc[db][4 * ig + 2] * scale, acc[db][4 * ig + 3] * scale});
      }
  }
}

// ---------------------------------------------------------------------------------------
// dK, dV on fp32 tensors with split-operand products. A workgroup owns DX6_KEYS = 128 keys
// (four waves of 32) of one (batch, head) and walks the 64-query tiles from its diagonal
// down. K and V of the lane's key are split once into registers; each query tile of Q and
// dO is split into three bf16 planes per tensor, [query][d] in LDS with the 16-byte chunk c
// of row q at chunk c ^ qswz(q). That one layout serves both uses:
//   S = Q K^T and dP = dO V^T take Q and dO as the A operand, a lane reading 8 consecutive
//   head dims of its query (16-byte reads);
//   dV^T = dO^T P and dK^T = Q^T dS take dO^T and Q^T as the A operand, read with
//   transposing reads (ds_read_b64_tr_b16): lanes 4j .. 4j+3 of a 16-lane group read 16
//   head dims of query row j of a run of four, and lane i receives head dim i of the four
//   rows. The two reads of a fragment take the query runs 16h + 4lh and 16h + 8 + 4lh, the
//   order in which the S / dP accumulators hold a lane's queries, so P and dS (split in
//   registers) are the B operands as they stand.
// qswz is linear in the bits of q (bits 0..3 map to 2, 6, 3, 4) and makes both read
// patterns conflict-free on the 64 four-byte banks of gfx950's LDS (and on 32): a row is
// 128 bytes, so even rows fill banks 0-31 and odd rows 32-63, and the 16 rows of a 16-lane
// row read take 8 different chunks among the even rows and 8 among the odd ones (a swizzle
// of bits 0..2 alone repeats every 8 rows: two-way conflicts, counted by
// SQ_LDS_BANK_CONFLICT); each transposing read of 32 lanes (either grouping of the four
// 16-lane groups) touches every bank once. Since qswz(q + 8) = qswz(q) ^ 4, the second read
// of head-dim block db (8 rows on) sits at the first read's offset for block db ^ 1.
// The fp32 dS of each causal 64x64 tile is written ([query][key]) for the dQ kernel, as
// attn_bwd_dkdv_kernel does.
// ---------------------------------------------------------------------------------------
constexpr int DX6_KEYS = X6_QT;
GPT2_DEVICE_INLINE int qswz(int q) {
  return ((q & 1) * 2) ^ (((q >> 1) & 1) * 6) ^ (((q >> 2) & 1) * 3) ^ (((q >> 3) & 1) * 4);
}
// element offset of head dims 8c .. 8c+7 of row q in a 64-wide plane
GPT2_DEVICE_INLINE int qoff(int q, int c) { return q * 64 + ((c ^ qswz(q)) << 3); }

template <int HSP>
__global__ __launch_bounds__(X6_NT, 2) void attn_bwd_dkdv_x6_kernel(
    float* __restrict__ dqkv, float* __restrict__ dsbuf, const float* __restrict__ dout,
    const float* __restrict__ qkv, const float* __restrict__ lse,
    const float* __restrict__ Drow, int T, int C, int NH, int hs, float scale,
    float scale_log2) {
  static_assert(HSP == 64, "64-wide planes");
  constexpr int KS = HSP / 16, ND = HSP / 32, CPR = HSP / 8;
  constexpr int PQ = TILE * HSP;  // elements of one plane
  __shared__ __attribute__((aligned(16))) bf16_t Qp[3 * PQ];  // [plane][q][d]
  __shared__ __attribute__((aligned(16))) bf16_t Op[3 * PQ];  // dO, same layout
  __shared__ __attribute__((aligned(16))) float Ls[TILE];
  __shared__ __attribute__((aligned(16))) float Ds[TILE];

  const int nkb = (T + DX6_KEYS - 1) / DX6_KEYS;
  int kb, head, b;
  key_block_of(nkb, NH, &kb, &head, &b);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r = lane & 31, lh = lane >> 5;
  const int i16 = lane & 15, g1 = (lane >> 4) & 1;  // lane in its 16-lane group, group parity
  const long long C3 = 3LL * C;
  const float* base = qkv + (long long)b * T * C3 + (long long)head * hs;
  const float* dobase = dout + (long long)b * T * C + (long long)head * hs;
  const float* lrow = lse + ((long long)b * NH + head) * T;
  const float* drow = Drow + ((long long)b * NH + head) * T;
  const int key0 = kb * DX6_KEYS + wave * 32;  // first key of this wave
  const int key = key0 + r;
  const int km = min(key, T - 1);
  const int kt = key0 / TILE;             // this wave's 64-key tile in the dS layout
  const int kcol = key0 - kt * TILE + r;  // this lane's column in that tile

  // this lane's key and value, d = 16ks + 8lh .. +7, as three parts each
  bf16x8 kh[KS], kmd[KS], kl[KS], vh[KS], vmd[KS], vl[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ks++) {
    f32x4 x, y;
    u32x4 h, m, l;
    load8f(base + C, C3, km, 16 * ks + 8 * lh, T, hs, x, y);
    split8(x, y, h, m, l);
    kh[ks] = __builtin_bit_cast(bf16x8, h);
    kmd[ks] = __builtin_bit_cast(bf16x8, m);
    kl[ks] = __builtin_bit_cast(bf16x8, l);
    load8f(base + 2 * C, C3, km, 16 * ks + 8 * lh, T, hs, x, y);
    split8(x, y, h, m, l);
    vh[ks] = __builtin_bit_cast(bf16x8, h);
    vmd[ks] = __builtin_bit_cast(bf16x8, m);
    vl[ks] = __builtin_bit_cast(bf16x8, l);
  }
  f32x16 dvacc[ND], dkacc[ND];  // [d][key]
#pragma unroll
  for (int db = 0; db < ND; db++)
#pragma unroll
    for (int i = 0; i < 16; i++) {
      dvacc[db][i] = 0.f;
      dkacc[db][i] = 0.f;
    }

  // transposing-read address of this lane for k step hh of sub-block qb, head-dim block db
  // (the first of the two reads, rows with bit 3 clear; the second, 8 rows on, is at
  // tr_off(qb, hh, db ^ 1) + 8 HSP)
  auto tr_off = [&](int qb, int hh, int db) {
    const int q = 32 * qb + 16 * hh + 4 * lh + (i16 >> 2);
    const int d = 32 * db + 16 * g1 + 4 * (i16 & 3);
    return qoff(q, d >> 3) + (d & 7);
  };
  auto frag_tr8 = [&](const bf16_t* p, const bf16_t* p8) -> bf16x8 {
    const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(p));
    const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(p8 + 8 * HSP));
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  };

  const int nqt = (T + TILE - 1) / TILE;
  for (int qt = kb * DX6_KEYS / TILE; qt < nqt; qt++) {
    const int q0 = qt * TILE;
    __syncthreads();
    // Q and dO rows q0 .. q0+63 -> three planes each; chunk f: row f / 8, head dims 8 (f % 8)
#pragma unroll
    for (int i = 0; i < TILE * CPR / X6_NT; i++) {
      const int f = tid + X6_NT * i, row = f / CPR, c = f % CPR;
      const int o = qoff(row, c);
      f32x4 x, y;
      u32x4 h, m, l;
      load8f(base, C3, q0 + row, 8 * c, T, hs, x, y);
      split8(x, y, h, m, l);
      *reinterpret_cast<u32x4*>(Qp + o) = h;
      *reinterpret_cast<u32x4*>(Qp + PQ + o) = m;
      *reinterpret_cast<u32x4*>(Qp + 2 * PQ + o) = l;
      load8f(dobase, C, q0 + row, 8 * c, T, hs, x, y);
      split8(x, y, h, m, l);
      *reinterpret_cast<u32x4*>(Op + o) = h;
      *reinterpret_cast<u32x4*>(Op + PQ + o) = m;
      *reinterpret_cast<u32x4*>(Op + 2 * PQ + o) = l;
    }
    if (tid < TILE) {
      const bool ok = q0 + tid < T;
      const int t = min(q0 + tid, T - 1);
      Ls[tid] = ok ? lrow[t] * kLog2e : 0.f;
      Ds[tid] = ok ? drow[t] : 0.f;
    }
    __syncthreads();
    if (q0 + TILE <= key0) continue;  // every query of the tile precedes this wave's keys
    // dS tile (qt, kt) of this (b, head): 64 x 64 floats, [query][key]; this lane writes
    // column kcol of rows 4lh + (32qb + 8(i/4) + i%4)
    float* dst = dsbuf + (((long long)b * NH + head) * tri_tiles(nqt) + tri_index(qt, kt)) *
                             (TILE * TILE) + 4 * lh * TILE + kcol;
#pragma unroll 1
    for (int qb = 0; qb < 2; qb++) {
      if (q0 + 32 * qb + 32 <= key0) {  // every query of the sub-block precedes the keys
#pragma unroll
        for (int i = 0; i < 16; i++) dst[(32 * qb + 8 * (i / 4) + (i % 4)) * TILE] = 0.f;
        continue;
      }
      f32x16 s, dp;
#pragma unroll
      for (int i = 0; i < 16; i++) {
        s[i] = 0.f;
        dp[i] = 0.f;
      }
#pragma unroll
      for (int ks = 0; ks < KS; ks++) {
        const int o = qoff(32 * qb + r, 2 * ks + lh);
        s = mfma_x6(*reinterpret_cast<const bf16x8*>(&Qp[o]),
                    *reinterpret_cast<const bf16x8*>(&Qp[PQ + o]),
                    *reinterpret_cast<const bf16x8*>(&Qp[2 * PQ + o]), kh[ks], kmd[ks], kl[ks], s);
        dp = mfma_x6(*reinterpret_cast<const bf16x8*>(&Op[o]),
                     *reinterpret_cast<const bf16x8*>(&Op[PQ + o]),
                     *reinterpret_cast<const bf16x8*>(&Op[2 * PQ + o]), vh[ks], vmd[ks], vl[ks],
                     dp);
      }
      // s[i], dp[i]: query 32qb + 8(i/4) + 4lh + i%4 of the tile, key = this lane's. The
      // lane's 16 row statistics are four runs of four consecutive rows, read as 16-byte
      // vectors; the exponential is taken for every entry and masked after (no branch per
      // entry). A sub-block whose 32 queries all follow the wave's 32 keys and lie before T
      // needs no mask (uniform test).
      const bool nomask = q0 + 32 * qb >= key0 + 31 && q0 + 32 * qb + 32 <= T;
#pragma unroll
      for (int g4 = 0; g4 < 4; g4++) {
        const int qo = 32 * qb + 8 * g4 + 4 * lh;  // first of the run
        const f32x4 lq = *reinterpret_cast<const f32x4*>(&Ls[qo]);
        const f32x4 dq = *reinterpret_cast<const f32x4*>(&Ds[qo]);
        float pv[4];
#pragma unroll
        for (int j = 0; j < 4; j++) pv[j] = __builtin_amdgcn_exp2f(fmaf(s[4 * g4 + j], scale_log2, -lq[j]));
        if (!nomask) {
#pragma unroll
          for (int j = 0; j < 4; j++) {
            const int qa = q0 + qo + j;
            if (!(qa < T && qa >= key)) pv[j] = 0.f;
          }
        }
#pragma unroll
        for (int j = 0; j < 4; j++) {
          const int i = 4 * g4 + j;
          s[i] = pv[j];
          dp[i] = pv[j] * (dp[i] - dq[j]);
          dst[(qo - 4 * lh + j) * TILE] = dp[i];  // 32 lanes store 32 consecutive keys
        }
      }
      // dV^T[d][key] += dO^T[d][q] P[q][key], dK^T[d][key] += Q^T[d][q] dS[q][key]; k step
      // hh takes accumulator entries 8hh .. 8hh+7 (queries 16hh + 4lh + {0..3, 8..11})
#pragma unroll
      for (int hh = 0; hh < 2; hh++) {
        u32x4 ph, pm, pl, sh, sm, sl;
        split8(f32x4{s[8 * hh], s[8 * hh + 1], s[8 * hh + 2], s[8 * hh + 3]},
               f32x4{s[8 * hh + 4], s[8 * hh + 5], s[8 * hh + 6], s[8 * hh + 7]}, ph, pm, pl);
        split8(f32x4{dp[8 * hh], dp[8 * hh + 1], dp[8 * hh + 2], dp[8 * hh + 3]},
               f32x4{dp[8 * hh + 4], dp[8 * hh + 5], dp[8 * hh + 6], dp[8 * hh + 7]}, sh, sm, sl);
#pragma unroll
        for (int db = 0; db < ND; db++) {
          const int o = tr_off(qb, hh, db), o8 = tr_off(qb, hh, db ^ 1);
          dvacc[db] = mfma_x6(frag_tr8(Op + o, Op + o8), frag_tr8(Op + PQ + o, Op + PQ + o8),
                              frag_tr8(Op + 2 * PQ + o, Op + 2 * PQ + o8),
                              __builtin_bit_cast(bf16x8, ph), __builtin_bit_cast(bf16x8, pm),
                              __builtin_bit_cast(bf16x8, pl), dvacc[db]);
          dkacc[db] = mfma_x6(frag_tr8(Qp + o, Qp + o8), frag_tr8(Qp + PQ + o, Qp + PQ + o8),
                              frag_tr8(Qp + 2 * PQ + o, Qp + 2 * PQ + o8),
                              __builtin_bit_cast(bf16x8, sh), __builtin_bit_cast(bf16x8, sm),
                              __builtin_bit_cast(bf16x8, sl), dkacc[db]);
        }
      }
    }
  }
  if (key < T) {
    float* dk = dqkv + ((long long)b * T + key) * C3 + C + (long long)head * hs;
    float* dv = dk + C;
#pragma unroll
    for (int db = 0; db < ND; db++)
#pragma unroll
      for (int ig = 0; ig < 4; ig++) {
        const int d = 32 * db + 8 * ig + 4 * lh;
        if (d < hs) {
          st4(dk + d, f32x4{dkacc[db][4 * ig] * scale, dkacc[db][4 * ig + 1] * scale,
                            dkacc[db][4 * ig + 2] * scale, dkacc[db][4 * ig + 3] * scale});
          st4(dv + d, f32x4{dvacc[db][4 * ig], dvacc[db][4 * ig + 1], dvacc[db][4 * ig + 2],
                            dvacc[db][4 * ig + 3]});
        }
      }
  }
}


// ---------------------------------------------------------------------------------------
// backward
// ---------------------------------------------------------------------------------------

// dK, dV for 64 keys (32 per wave), over the query tiles from the diagonal down. Per query
// tile, S and dP are computed with queries down the rows and this lane's key as the column;
// P and dS are then the B operands of dV^T = dO^T P and dK^T = Q^T dS, whose A operands are
// the transposed tiles dO^T and Q^T in LDS. dS^T of each causal 64x64 tile is written (TS,
// [key][query]) for the dQ kernel.
template <int HSP, typename TS>
__global__ __launch_bounds__(NTHR, 2) void attn_bwd_dkdv_mma16_kernel(
    TS* __restrict__ dqkv, uint16_t* __restrict__ dsbuf, const TS* __restrict__ dout,
    const TS* __restrict__ qkv, const float* __restrict__ lse,
    const float* __restrict__ Drow, int T, int C, int NH, int hs, float scale,
    float scale_log2) {
  constexpr int KS = HSP / 16, ND = HSP / 32;
  __shared__ __attribute__((aligned(16))) uint16_t Qs[TILE * HSP];   // [q][d]
  __shared__ __attribute__((aligned(16))) uint16_t Qt[HSP * TILE];   // [d][kpos(q)]
  __shared__ __attribute__((aligned(16))) uint16_t dOs[TILE * HSP];  // [q][d]
  __shared__ __attribute__((aligned(16))) uint16_t dOt[HSP * TILE];  // [d][kpos(q)]
  __shared__ __attribute__((aligned(16))) float Ls[TILE];
  __shared__ __attribute__((aligned(16))) float Ds[TILE];

  const int nkt = (T + TILE - 1) / TILE;
  int kt, head, b;
  tile_of_block(nkt, NH, &kt, &head, &b);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r = lane & 31, lh = lane >> 5;
  const long long C3 = 3LL * C;
  const TS* base = qkv + (long long)b * T * C3 + (long long)head * hs;
  const TS* dobase = dout + (long long)b * T * C + (long long)head * hs;
  const float* lrow = lse + ((long long)b * NH + head) * T;
  const float* drow = Drow + ((long long)b * NH + head) * T;
  const int key = kt * TILE + wave * 32 + r;
  const int km = min(key, T - 1);

  bf16x8 kf[KS], vf[KS];  // this lane's key and value, d = 16ks + 8lh .. +7
#pragma unroll
  for (int ks = 0; ks < KS; ks++) {
    kf[ks] = __builtin_bit_cast(bf16x8, load8(base + C, C3, km, 16 * ks + 8 * lh, T, hs));
    vf[ks] = __builtin_bit_cast(bf16x8, load8(base + 2 * C, C3, km, 16 * ks + 8 * lh, T, hs));
  }
  f32x16 dvacc[ND], dkacc[ND];  // [d][key]
#pragma unroll
  for (int db = 0; db < ND; db++)
#pragma unroll
    for (int i = 0; i < 16; i++) {
      dvacc[db][i] = 0.f;
      dkacc[db][i] = 0.f;
    }

  const int nqt = nkt;
  for (int qt = kt; qt < nqt; qt++) {
    const int q0 = qt * TILE;
    __syncthreads();
    tile_rows<HSP>(Qs, base, C3, q0, T, hs, tid);
    tile_cols<HSP>(Qt, base, C3, q0, T, hs, tid);
    tile_rows<HSP>(dOs, dobase, C, q0, T, hs, tid);
    tile_cols<HSP>(dOt, dobase, C, q0, T, hs, tid);
    if (tid < TILE) {
      const int t = q0 + tid;
      Ls[tid] = t < T ? lrow[t] * kLog2e : 0.f;
      Ds[tid] = t < T ? drow[t] : 0.f;
    }
    __syncthreads();
    // dS^T tile (kt, qt) of this (b, head): [key][query], 64 x 64 TS
    uint16_t* dst = dsbuf + (((long long)b * NH + head) * tri_tiles(nqt) + tri_index(qt, kt)) *
                              (TILE * TILE) + (long long)(wave * 32 + r) * TILE;
#pragma unroll
    for (int qb = 0; qb < 2; qb++) {
      // the lse and D of this lane's 16 queries (four runs of four consecutive rows), read
      // before the products so their latency is hidden
      f32x4 lq[4], dq[4];
#pragma unroll
      for (int g4 = 0; g4 < 4; g4++) {
        lq[g4] = *reinterpret_cast<const f32x4*>(&Ls[32 * qb + 8 * g4 + 4 * lh]);
        dq[g4] = *reinterpret_cast<const f32x4*>(&Ds[32 * qb + 8 * g4 + 4 * lh]);
      }
      u32x4 pw[2], sw[2];  // P and dS (TS pairs) as B operands of k step h
      f32x16 s, dp;
#pragma unroll
      for (int i = 0; i < 16; i++) {
        s[i] = 0.f;
        dp[i] = 0.f;
      }
#pragma unroll
      for (int ks = 0; ks < KS; ks++) {
        const bf16x8 qa = *reinterpret_cast<const bf16x8*>(&Qs[loff<HSP>(32 * qb + r, 2 * ks + lh)]);
        const bf16x8 oa = *reinterpret_cast<const bf16x8*>(&dOs[loff<HSP>(32 * qb + r, 2 * ks + lh)]);
        s = mfma16<TS>(qa, kf[ks], s);
        dp = mfma16<TS>(oa, vf[ks], dp);
      }
      // s[i], dp[i]: query 32qb + 8(i/4) + 4lh + i%4 of the tile, key = this lane's. The
      // exponential is taken for every entry and masked after (no branch per entry); a
      // sub-block whose 32 queries all follow the wave's 32 keys and lie before T needs no
      // mask (uniform test).
      const bool nomask = q0 + 32 * qb >= kt * TILE + wave * 32 + 31 && q0 + 32 * qb + 32 <= T;
#pragma unroll
      for (int g4 = 0; g4 < 4; g4++) {
        float pv[4], dsv[4];
#pragma unroll
        for (int j = 0; j < 4; j++) {
          const int i = 4 * g4 + j;
          const float e = __builtin_amdgcn_exp2f(fmaf(s[i], scale_log2, -lq[g4][j]));
          pv[j] = e;
          dsv[j] = dp[i] - dq[g4][j];
        }
        if (!nomask) {
#pragma unroll
          for (int j = 0; j < 4; j++) {
            const int qa = q0 + 32 * qb + 8 * g4 + 4 * lh + j;
            if (!(qa < T && qa >= key)) pv[j] = 0.f;
          }
        }
#pragma unroll
        for (int j = 0; j < 4; j++) dsv[j] *= pv[j];
        const int hh = g4 >> 1, w = 2 * (g4 & 1);  // acc entries 8hh .. 8hh+7 form k step hh
        pw[hh][w] = Half16<TS>::pack2(pv[0], pv[1]);
        pw[hh][w + 1] = Half16<TS>::pack2(pv[2], pv[3]);
        const uint32_t d01 = Half16<TS>::pack2(dsv[0], dsv[1]),
                       d23 = Half16<TS>::pack2(dsv[2], dsv[3]);
        sw[hh][w] = d01;
        sw[hh][w + 1] = d23;
        // 4 consecutive queries of this key: one 8-byte store
        *reinterpret_cast<u32x2*>(dst + 32 * qb + 8 * g4 + 4 * lh) = u32x2{d01, d23};
      }
#pragma unroll
      for (int db = 0; db < ND; db++)
#pragma unroll
        for (int hh = 0; hh < 2; hh++) {
          const int c = 4 * qb + 2 * hh + lh;
          const bf16x8 oa = *reinterpret_cast<const bf16x8*>(&dOt[loff<TILE>(32 * db + r, c)]);
          const bf16x8 qa = *reinterpret_cast<const bf16x8*>(&Qt[loff<TILE>(32 * db + r, c)]);
          dvacc[db] = mfma16<TS>(oa, __builtin_bit_cast(bf16x8, pw[hh]), dvacc[db]);
          dkacc[db] = mfma16<TS>(qa, __builtin_bit_cast(bf16x8, sw[hh]), dkacc[db]);
        }
    }
  }
  if (key < T) {
    TS* dk = dqkv + ((long long)b * T + key) * C3 + C + (long long)head * hs;
    TS* dv = dk + C;
#pragma unroll
    for (int db = 0; db < ND; db++)
#pragma unroll
      for (int ig = 0; ig < 4; ig++) {
        const int d = 32 * db + 8 * ig + 4 * lh;
        if (d < hs) {
          st4(dk + d, f32x4{dkacc[db][4 * ig] * scale, dkacc[db][4 * ig + 1] * scale,
                            dkacc[db][4 * ig + 2] * scale, dkacc[db][4 * ig + 3] * scale});
          st4(dv + d, f32x4{dvacc[db][4 * ig], dvacc[db][4 * ig + 1], dvacc[db][4 * ig + 2],
                            dvacc[db][4 * ig + 3]});
        }
      }
  }
}

// dQ^T[d][q] = scale * K^T[d][key] dS^T[key][q] for 64 queries (32 per wave), over key
// tiles 0 .. qt, reading the dS^T tiles of the dK/dV kernel transposed into LDS.
template <int HSP, typename TS>
__global__ __launch_bounds__(NTHR) void attn_bwd_dq_mma16_kernel(
    TS* __restrict__ dqkv, const TS* __restrict__ qkv, const uint16_t* __restrict__ dsbuf,
    int T, int C, int NH, int hs, float scale) {
  constexpr int ND = HSP / 32;
  __shared__ __attribute__((aligned(16))) uint16_t Kt[HSP * TILE];   // [d][kpos(key)]
  __shared__ __attribute__((aligned(16))) uint16_t Sq[TILE * TILE];  // [q][kpos(key)]

  const int nqt = (T + TILE - 1) / TILE;
  int qt, head, b;
  tile_of_block(nqt, NH, &qt, &head, &b);
  qt = nqt - 1 - qt;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r = lane & 31, lh = lane >> 5;
  const long long C3 = 3LL * C;
  const TS* kbase = qkv + (long long)b * T * C3 + (long long)head * hs + C;
  const uint16_t* src = dsbuf + (((long long)b * NH + head) * tri_tiles(nqt) + tri_index(qt, 0)) *
                                  (TILE * TILE);

  f32x16 acc[ND];
#pragma unroll
  for (int db = 0; db < ND; db++)
#pragma unroll
    for (int i = 0; i < 16; i++) acc[db][i] = 0.f;

  // the stored dS^T tile is [key][query] (64 x 64, rows of 64): as rows of a tensor with
  // T = 64 and hs = 64 it transposes into [query][kpos(key)]. The next key tile is loaded
  // into registers while this one is used.
  ColsTile<HSP> kn;
  ColsTile<TILE> sn;
  kn.load(kbase, C3, 0, T, hs, tid);
  sn.load(src, TILE, 0, TILE, TILE, tid);
  for (int kt = 0; kt <= qt; kt++) {
    __syncthreads();
    kn.store(Kt, tid);
    sn.store(Sq, tid);
    __syncthreads();
    if (kt < qt) {
      kn.load(kbase, C3, (kt + 1) * TILE, T, hs, tid);
      sn.load(src + (long long)(kt + 1) * TILE * TILE, TILE, 0, TILE, TILE, tid);
    }
#pragma unroll
    for (int db = 0; db < ND; db++)
#pragma unroll
      for (int kb = 0; kb < 2; kb++)
#pragma unroll
        for (int hh = 0; hh < 2; hh++) {
          const int c = 4 * kb + 2 * hh + lh;
          const bf16x8 ka = *reinterpret_cast<const bf16x8*>(&Kt[loff<TILE>(32 * db + r, c)]);
          const bf16x8 sb = *reinterpret_cast<const bf16x8*>(&Sq[loff<TILE>(32 * wave + r, c)]);
          acc[db] = mfma16<TS>(ka, sb, acc[db]);
        }
  }
  // acc[db][i]: d = 32db + 8(i/4) + 4lh + i%4, query 32 wave + r of the tile
  const int q = qt * TILE + 32 * wave + r;
  if (q < T) {
    TS* o = dqkv + ((long long)b * T + q) * C3 + (long long)head * hs;
#pragma unroll
    for (int db = 0; db < ND; db++)
#pragma unroll
      for (int ig = 0; ig < 4; ig++) {
        const int d = 32 * db + 8 * ig + 4 * lh;
        if (d < hs)
          st4(o + d, f32x4{acc[db][4 * ig] * scale, acc[db][4 * ig + 1] * scale,
                           acc[db][4 * ig + 2] * scale, acc[db][4 * ig + 3] * scale});
      }
  }
}

}  // namespace

int attention_forward_x6(float* out, float* lse, const float* qkv, int B, int T, int C, int NH,
                         hipStream_t stream) {
  if (B < 1 || T < 1 || NH < 1 || C % NH || !attention_bf16_mma_supported(C, NH)) {
    set_global_error("attention (split operands): unsupported shape B=%d T=%d C=%d NH=%d", B,
                     T, C, NH);
    return -1;
  }
  const int hs = C / NH;
  const float scale_log2 = kLog2e / sqrtf((float)hs);
  dim3 grid(((T + X6_QT - 1) / X6_QT) * NH * B);
  const double tri = (double)T * (T + 1) / 2.0;
  ProfScope ps("attn_fwd_x6_kernel", 4.0 * B * NH * hs * tri,
               4.0 * ((double)B * T * 3 * C + (double)B * T * C) + 4.0 * B * NH * T, stream);
  if (hs <= 32) attn_fwd_x6_kernel<32><<<grid, X6_NT, 0, stream>>>(out, lse, qkv, T, C, NH, hs, scale_log2);
  else if (hs <= 64) attn_fwd_x6_kernel<64><<<grid, X6_NT, 0, stream>>>(out, lse, qkv, T, C, NH, hs, scale_log2);
  else attn_fwd_x6_kernel<128><<<grid, X6_NT, 0, stream>>>(out, lse, qkv, T, C, NH, hs, scale_log2);
  GPT2_HIP_OK(hipGetLastError());
  return 0;
}

int attention_dq_x6(float* dqkv, const float* qkv, const float* ds_scratch, int B, int T, int C,
                    int NH, hipStream_t stream) {
  if (B < 1 || T < 1 || NH < 1 || C % NH || !attention_bf16_mma_supported(C, NH)) {
    set_global_error("attention dQ (split operands): unsupported shape B=%d T=%d C=%d NH=%d", B,
                     T, C, NH);
    return -1;
  }
  const int hs = C / NH;
  const float scale = 1.0f / sqrtf((float)hs);
  dim3 grid(((T + X6_QT - 1) / X6_QT) * NH * B);
  const double tri = (double)T * (T + 1) / 2.0;
  ProfScope ps("attn_bwd_dq_x6_kernel", 2.0 * B * NH * hs * tri,
               4.0 * B * NH * tri + 4.0 * 2.0 * B * T * C, stream);
  if (hs <= 32) attn_bwd_dq_x6_kernel<32><<<grid, X6_NT, 0, stream>>>(dqkv, qkv, ds_scratch, T, C, NH, hs, scale);
  else if (hs <= 64) attn_bwd_dq_x6_kernel<64><<<grid, X6_NT, 0, stream>>>(dqkv, qkv, ds_scratch, T, C, NH, hs, scale);
  else attn_bwd_dq_x6_kernel<128><<<grid, X6_NT, 0, stream>>>(dqkv, qkv, ds_scratch, T, C, NH, hs, scale);
  GPT2_HIP_OK(hipGetLastError());
  return 0;
}

int attention_dkdv_x6(float* dqkv, float* ds_scratch, const float* dout, const float* qkv,
                      const float* lse, const float* D, int B, int T, int C, int NH,
                      hipStream_t stream) {
  if (B < 1 || T < 1 || NH < 1 || C % NH || !attention_dkdv_x6_supported(C, NH)) {
    set_global_error("attention dK/dV (split operands): unsupported shape B=%d T=%d C=%d NH=%d",
                     B, T, C, NH);
    return -1;
  }
  const int hs = C / NH;
  const float scale = 1.0f / sqrtf((float)hs);
  dim3 grid(((T + DX6_KEYS - 1) / DX6_KEYS) * NH * B);
  const double tri = (double)T * (T + 1) / 2.0, BTC = (double)B * T * C;
  ProfScope ps("attn_bwd_dkdv_x6_kernel", 8.0 * B * NH * hs * tri,
               4.0 * (3.0 * BTC + BTC + 2.0 * BTC) + 4.0 * (2.0 * B * NH * T + B * NH * tri),
               stream);
  attn_bwd_dkdv_x6_kernel<64><<<grid, X6_NT, 0, stream>>>(dqkv, ds_scratch, dout, qkv, lse, D, T,
                                                          C, NH, hs, scale, scale * kLog2e);
  GPT2_HIP_OK(hipGetLastError());
  return 0;
}

bool attention_dkdv_x6_supported(int C, int NH) {
  const int hs = NH > 0 ? C / NH : 0;
  return NH > 0 && C % NH == 0 && hs % 8 == 0 && hs > 32 && hs <= 64;
}

bool attention_bf16_mma_supported(int C, int NH) {
  const int hs = C / NH;
  return hs % 8 == 0 && hs <= 128;
}

template <typename TS>
static int attention_forward_mma16(TS* out, float* lse, const TS* qkv, int B, int T, int C,
                                   int NH, hipStream_t stream) {
  constexpr bool F16 = std::is_same<TS, f16_t>::value;
  if (B < 1 || T < 1 || NH < 1 || C % NH || !attention_bf16_mma_supported(C, NH)) {
    set_global_error("attention (%s MFMA): unsupported shape B=%d T=%d C=%d NH=%d",
                     F16 ? "fp16" : "bf16", B, T, C, NH);
    return -1;
  }
  const int hs = C / NH;
  const float scale_log2 = kLog2e / sqrtf((float)hs);
  dim3 grid(((T + TILE - 1) / TILE) * NH * B);
  const double tri = (double)T * (T + 1) / 2.0;
  ProfScope ps(F16 ? "attn_fwd_f16mma_kernel" : "attn_fwd_bf16mma_kernel",
               4.0 * B * NH * hs * tri,
               2.0 * ((double)B * T * 3 * C + (double)B * T * C) + 4.0 * B * NH * T, stream);
  if (hs <= 32) attn_fwd_mma16_kernel<32, TS><<<grid, NTHR, 0, stream>>>(out, lse, qkv, T, C, NH, hs, scale_log2);
  else if (hs <= 64) attn_fwd_mma16_kernel<64, TS><<<grid, NTHR, 0, stream>>>(out, lse, qkv, T, C, NH, hs, scale_log2);
  else attn_fwd_mma16_kernel<128, TS><<<grid, NTHR, 0, stream>>>(out, lse, qkv, T, C, NH, hs, scale_log2);
  GPT2_HIP_OK(hipGetLastError());
  return 0;
}

int attention_forward_bf16_mma(bf16_t* out, float* lse, const bf16_t* qkv, int B, int T, int C,
                               int NH, hipStream_t stream) {
  return attention_forward_mma16(out, lse, qkv, B, T, C, NH, stream);
}
int attention_forward_f16_mma(f16_t* out, float* lse, const f16_t* qkv, int B, int T, int C,
                              int NH, hipStream_t stream) {
  return attention_forward_mma16(out, lse, qkv, B, T, C, NH, stream);
}

}  // namespace gpt2

namespace gpt2 {
template <typename TS>
static int attention_backward_mma16(TS* dqkv, const TS* dout, const TS* qkv, const TS* out,
                                    const float* lse, float* dscratch, float* ds_scratch, int B,
                                    int T, int C, int NH, hipStream_t stream) {
  constexpr bool F16 = std::is_same<TS, f16_t>::value;
  if (B < 1 || T < 1 || NH < 1 || C % NH || !attention_bf16_mma_supported(C, NH)) {
    set_global_error("attention (%s MFMA): unsupported shape B=%d T=%d C=%d NH=%d",
                     F16 ? "fp16" : "bf16", B, T, C, NH);
    return -1;
  }
  const int hs = C / NH;
  const float scale = 1.0f / sqrtf((float)hs);
  const float scale_log2 = scale * kLog2e;
  const double BTC = (double)B * T * C, tri = (double)T * (T + 1) / 2.0;
  const long long rows = (long long)B * NH * T;
  const int rc = attention_rowdot(dscratch, dout, out, B, T, C, NH, stream);
  if (rc) return rc;
  uint16_t* ds = reinterpret_cast<uint16_t*>(ds_scratch);
  dim3 grid(((T + TILE - 1) / TILE) * NH * B);
  {
    ProfScope ps(F16 ? "attn_bwd_dkdv_f16mma_kernel" : "attn_bwd_dkdv_bf16mma_kernel",
                 6.0 * B * NH * hs * tri,
                 2.0 * (3.0 * BTC + BTC + 2.0 * BTC) + 4.0 * 2.0 * rows + 2.0 * B * NH * tri,
                 stream);
    if (hs <= 32) attn_bwd_dkdv_mma16_kernel<32, TS><<<grid, NTHR, 0, stream>>>(dqkv, ds, dout, qkv, lse, dscratch, T, C, NH, hs, scale, scale_log2);
    else if (hs <= 64) attn_bwd_dkdv_mma16_kernel<64, TS><<<grid, NTHR, 0, stream>>>(dqkv, ds, dout, qkv, lse, dscratch, T, C, NH, hs, scale, scale_log2);
    else attn_bwd_dkdv_mma16_kernel<128, TS><<<grid, NTHR, 0, stream>>>(dqkv, ds, dout, qkv, lse, dscratch, T, C, NH, hs, scale, scale_log2);
  }
  {
    ProfScope ps(F16 ? "attn_bwd_dq_f16mma_kernel" : "attn_bwd_dq_bf16mma_kernel",
                 2.0 * B * NH * hs * tri, 2.0 * B * NH * tri + 2.0 * 2.0 * BTC, stream);
    if (hs <= 32) attn_bwd_dq_mma16_kernel<32, TS><<<grid, NTHR, 0, stream>>>(dqkv, qkv, ds, T, C, NH, hs, scale);
    else if (hs <= 64) attn_bwd_dq_mma16_kernel<64, TS><<<grid, NTHR, 0, stream>>>(dqkv, qkv, ds, T, C, NH, hs, scale);
    else attn_bwd_dq_mma16_kernel<128, TS><<<grid, NTHR, 0, stream>>>(dqkv, qkv, ds, T, C, NH, hs, scale);
  }
  GPT2_HIP_OK(hipGetLastError());
  return 0;
}

int attention_backward_bf16_mma(bf16_t* dqkv, const bf16_t* dout, const bf16_t* qkv,
                                const bf16_t* out, const float* lse, float* dscratch,
                                float* ds_scratch, int B, int T, int C, int NH,
                                hipStream_t stream) {
  return attention_backward_mma16(dqkv, dout, qkv, out, lse, dscratch, ds_scratch, B, T, C, NH,
                                  stream);
}
int attention_backward_f16_mma(f16_t* dqkv, const f16_t* dout, const f16_t* qkv,
                               const f16_t* out, const float* lse, float* dscratch,
                               float* ds_scratch, int B, int T, int C, int NH,
                               hipStream_t stream) {
  return attention_backward_mma16(dqkv, dout, qkv, out, lse, dscratch, ds_scratch, B, T, C, NH,
                                  stream);
}
}  // namespace gpt2
