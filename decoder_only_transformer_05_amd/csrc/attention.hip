// attention.hip -- causal multi-head self-attention, forward and backward, on gfx950 MFMA.
//
// What is computed is section 1.7 attention_forward and section 1.8 attention_backward of
// "llm.c 的中文注解-20240421" (and the Attention / causal mask sections of "高能技巧！60 行
// NumPy 代码实现一个 GPT"): per (batch b, head h), S = Q K^T / sqrt(hs) restricted to keys
// t2 <= t, P = row softmax of S, O = P V; backward dV = P^T dO, dP = dO V^T,
// dS = P * (dP - rowsum(P * dP)), dQ = dS K / sqrt(hs), dK = dS^T Q / sqrt(hs).
//
// How it differs from the pages' loops: the (B,NH,T,T) score and probability matrices
// are never stored. The forward keeps a running max and sum per query row over 64-key
// tiles (online softmax) and saves only the row log-sum-exp; the backward recomputes P
// from Q, K and that log-sum-exp, and uses rowsum(P*dP) = rowsum(dO*O) (precomputed per
// row). dK/dV come from one kernel per key tile, which also writes dS of each causal
// 64x64 tile to a scratch buffer; dQ = dS K is then a second kernel per query tile. Each
// kernel owns its outputs, so nothing is accumulated with atomics and results are
// deterministic.
//
// MFMA layout trick: S is computed transposed (keys down the rows, one query per lane
// column), so the softmax statistics of a query live in a single lane (plus its partner
// lane 32 away), and P^T is already in the register layout of the B operand of the next
// MFMA (O^T = V^T P^T). No shuffles or LDS round trips are needed between the two
// products. The head dimension is contracted in the permuted order
// d(s, half) = 8*(s/4) + 4*half + s%4, which lets one 16-byte LDS read feed four MFMAs;
// both operands use the same order, so the dot products are unchanged.
#include <cmath>
#include <cstdlib>
#include <cstring>

#include <type_traits>

#include "attn_order.h"
#include "kernels.h"

namespace gpt2 {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int TILE = 64;    // queries per workgroup / keys per LDS tile
constexpr int NTHR = 128;   // two waves, 32 queries (or keys) each

// Loads 4 floats of row t, columns d..d+3 (row stride ld) without a branch: the address is
// clamped into the tensor (t <= T-1, d <= hs-4) and out-of-range values are replaced by 0.
template <typename T>
GPT2_DEVICE_INLINE f32x4 load4_rowcol(const T* base, long long ld, int t, int d, int Tn,
                                      int hs) {
  const int tc = min(t, Tn - 1), dc = min(d, hs - 4);
  const f32x4 x = ld4(base + (long long)tc * ld + dc);
  return (t < Tn && d < hs) ? x : f32x4{0.f, 0.f, 0.f, 0.f};
}

// 1-D grid over (tile, head, batch) with the tile index fastest; logical ids are made
// XCD-local, so all tiles of one (batch, head) -- which share its K and V -- run on the same
// XCD and its L2.
GPT2_DEVICE_INLINE void tile_of_block(int ntiles, int NH, int* tile, int* head, int* b) {
  const int lid = xcd_logical_block(blockIdx.x, gridDim.x);
  *tile = lid % ntiles;
  const int bh = lid / ntiles;
  *head = bh % NH;
  *b = bh / NH;
}

// Cooperative load of `rows` x HSP values starting at row `row0` of a strided tensor
// (row stride `ld`, column offset already applied) into S[TILE][HSP+4]; rows >= T and
// columns >= hs are zero.
template <int HSP, typename TS>
GPT2_DEVICE_INLINE void load_tile(float (*S)[HSP + 4], const TS* base, long long ld,
                                  int row0, int T, int hs, int tid) {
  constexpr int F4 = HSP / 4;
#pragma unroll
  for (int i = 0; i < TILE * F4 / NTHR; i++) {
    const int f = tid + NTHR * i;
    const int row = f / F4, d = 4 * (f % F4);
    const int t = row0 + row;
    *reinterpret_cast<f32x4*>(&S[row][d]) = load4_rowcol(base, ld, t, d, T, hs);
  }
}

// ---------------------------------------------------------------------------------------
// forward
// ---------------------------------------------------------------------------------------
// 16 bytes from global memory straight into LDS: lane l writes lds + 16 l (the LDS address is
// the same for the whole wave). Kept out of the kernel bodies: clang's host pass drops the
// launch stub of a kernel that calls this builtin directly.
GPT2_DEVICE_INLINE void lds_copy16(const void* src, void* lds) {
  __builtin_amdgcn_global_load_lds(src, lds, 16, 0, 0);
}

// DIRECT (fp32 storage, hs == HSP == 64): the K and V tiles are copied from global memory
// straight into LDS (global_load_lds_dwordx4: no registers), one 1 KB run of four rows per
// wave instruction, so the tiles are unpadded; a key's 16-byte chunk c is stored at chunk
// c ^ (key & 15), chosen on the global side, which spreads the K reads over the banks.
template <int HSP, typename TS, bool DIRECT = false>
__global__ __launch_bounds__(NTHR) void attn_fwd_kernel(TS* __restrict__ out,
                                                        float* __restrict__ lse,
                                                        const TS* __restrict__ qkv, int T,
                                                        int C, int NH, int hs,
                                                        float scale_log2) {
  static_assert(!DIRECT || HSP == 64, "direct tile copies assume 64-dim rows");
  constexpr int LD = DIRECT ? HSP : HSP + 4, NS = HSP / 2, ND = HSP / 32;
  __shared__ __attribute__((aligned(16))) float Ks[TILE][LD];
  __shared__ __attribute__((aligned(16))) float Vs[TILE][LD];

  const int nqt = (T + TILE - 1) / TILE;
  int qt, head, b;
  tile_of_block(nqt, NH, &qt, &head, &b);
  qt = nqt - 1 - qt;  // longest rows first
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r = lane & 31, hf = lane >> 5;
  const long long C3 = 3LL * C;
  const TS* base = qkv + (long long)b * T * C3 + (long long)head * hs;
  const int q = qt * TILE + wave * 32 + r;
  const int qm = min(q, T - 1);  // lanes past the end mask as the last row; never stored

  float qf[NS];
#pragma unroll
  for (int g = 0; g < HSP / 8; g++) {
    const int d = 8 * g + 4 * hf;
    f32x4 v = load4_rowcol(base, C3, qm, d, T, hs);
#pragma unroll
    for (int j = 0; j < 4; j++) qf[4 * g + j] = v[j] * scale_log2;
  }

  f32x16 oacc[ND];
#pragma unroll
  for (int db = 0; db < ND; db++)
#pragma unroll
    for (int i = 0; i < 16; i++) oacc[db][i] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;

  const int kv_end = min(T, (qt + 1) * TILE);
  const int ntiles = (kv_end + TILE - 1) / TILE;
  for (int kt = 0; kt < ntiles; kt++) {
    const int key0 = kt * TILE;
    __syncthreads();
    if constexpr (DIRECT) {
      // 16 wave instructions per tile (two waves, eight each): lane l of instruction j
      // fills row 4j + l/16, stored chunk l%16; rows past T read the last row (those keys
      // are masked and their V rows weigh 0)
#pragma unroll
      for (int jj = 0; jj < TILE / 8; jj++) {
        const int j = 2 * jj + wave;
        const int row = 4 * j + (lane >> 4);
        const long long t = min(key0 + row, T - 1);
        const int cs = lane & 15;
        lds_copy16(base + C + t * C3 + 4 * (cs ^ (row & 15)), &Ks[4 * j][0]);
        lds_copy16(base + 2 * C + t * C3 + 4 * cs, &Vs[4 * j][0]);
      }
      __builtin_amdgcn_s_waitcnt(0);
    } else {
      load_tile<HSP>(Ks, base + C, C3, key0, T, hs, tid);
      load_tile<HSP>(Vs, base + 2 * C, C3, key0, T, hs, tid);
    }
    __syncthreads();

    f32x16 s[2];
#pragma unroll
    for (int kb = 0; kb < 2; kb++) {
#pragma unroll
      for (int i = 0; i < 16; i++) s[kb][i] = 0.f;
#pragma unroll
      for (int g = 0; g < HSP / 8; g++) {
        const int krow = 32 * kb + r, kc = 2 * g + hf;  // chunk of 4 head dims
        f32x4 kv = *reinterpret_cast<const f32x4*>(
            &Ks[krow][4 * (DIRECT ? kc ^ (krow & 15) : kc)]);
#pragma unroll
        for (int j = 0; j < 4; j++) s[kb] = mfma32x32x2(kv[j], qf[4 * g + j], s[kb]);
      }
    }
    if (key0 + TILE > qt * TILE) {  // the diagonal tile (uniform): mask keys after the query
#pragma unroll
      for (int kb = 0; kb < 2; kb++)
#pragma unroll
        for (int i = 0; i < 16; i++) {
          const int key = key0 + 32 * kb + 8 * (i / 4) + 4 * hf + (i % 4);
          if (key > qm) s[kb][i] = -INFINITY;
        }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; kb++)
#pragma unroll
      for (int i = 0; i < 16; i++) mx = fmaxf(mx, s[kb][i]);
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    // The running max only moves when a tile's max exceeds it by more than 8 (the
    // exponentials then stay below 2^8, harmless in fp32), so most tiles skip rescaling
    // oacc and l; O = oacc / l is unchanged by the choice of reference. The first tile
    // always moves it (m_run = -inf; key 0 <= qm is never masked, so mx is finite).
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
#pragma unroll
    for (int kb = 0; kb < 2; kb++)
#pragma unroll
      for (int i = 0; i < 16; i++) {
        const float p = __builtin_amdgcn_exp2f(s[kb][i] - m_run);
        s[kb][i] = p;
        l_run += p;
      }
#pragma unroll
    for (int db = 0; db < ND; db++)
#pragma unroll
      for (int st = 0; st < 32; st++) {
        const int kb = st / 16, i = st % 16;
        const int kl = 32 * kb + 8 * (i / 4) + 4 * hf + (i % 4);
        oacc[db] = mfma32x32x2(Vs[kl][32 * db + r], s[kb][i], oacc[db]);
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
        const int d = 32 * db + 8 * ig + 4 * hf;
        if (d < hs)
          st4(o + d, f32x4{oacc[db][4 * ig] * inv, oacc[db][4 * ig + 1] * inv,
                           oacc[db][4 * ig + 2] * inv, oacc[db][4 * ig + 3] * inv});
      }
    if (hf == 0) lse[((long long)b * NH + head) * T + q] = (m_run + log2f(l_tot)) * kLn2;
  }
}

// ---------------------------------------------------------------------------------------
// backward: D = rowsum(dO * O) per (b, head, query)
// ---------------------------------------------------------------------------------------
// Head sizes that are not 4 times a power of two: one thread per (b, q, head) segment.
template <typename TS>
__global__ void attn_bwd_rowdot_generic_kernel(float* __restrict__ D,
                                               const TS* __restrict__ dout,
                                               const TS* __restrict__ out, int B, int T,
                                               int C, int NH, int hs) {
  const long long idx = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (long long)B * NH * T) return;
  const int head = (int)(idx % NH);
  const long long bq = idx / NH;
  const int q = (int)(bq % T), b = (int)(bq / T);
  const long long off = bq * C + (long long)head * hs;
  float s = 0.f;
  for (int d = 0; d < hs; d += 4) {
    f32x4 a = ld4(dout + off + d);
    f32x4 o = ld4(out + off + d);
    s += a[0] * o[0] + a[1] * o[1] + a[2] * o[2] + a[3] * o[3];
  }
  D[((long long)b * NH + head) * T + q] = s;
}

// One float4 per thread, threads of a (b, q, head) segment adjacent: loads are contiguous
// across the wave, and the HS4 = hs/4 partial sums of a segment are combined with shuffles
// (HS4 a power of two up to 32). D is (B, NH, T).
template <int HS4, typename TS>
__global__ void attn_bwd_rowdot_kernel(float* __restrict__ D, const TS* __restrict__ dout,
                                       const TS* __restrict__ out, int B, int T, int C,
                                       int NH) {
  const long long idx = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  const long long n4 = (long long)B * T * (C / 4);
  const bool ok = idx < n4;
  const long long i4 = ok ? idx : 0;
  const f32x4 a = ld4(dout + 4 * i4);
  const f32x4 o = ld4(out + 4 * i4);
  float s = (a[0] * o[0] + a[1] * o[1]) + (a[2] * o[2] + a[3] * o[3]);
#pragma unroll
  for (int w = HS4 / 2; w > 0; w >>= 1) s += __shfl_xor(s, w, 64);
  if (ok && (threadIdx.x % HS4) == 0) {
    const long long bq = i4 / (C / 4);
    const int head = (int)((i4 % (C / 4)) / HS4);
    const int q = (int)(bq % T), b = (int)(bq / T);
    D[((long long)b * NH + head) * T + q] = s;
  }
}

// Causal 64x64 tiles (qt, kt), kt <= qt, of one (b, head), stored row after row:
// tile (qt, kt) is number qt(qt+1)/2 + kt.
GPT2_DEVICE_INLINE long long tri_index(int qt, int kt) { return (long long)qt * (qt + 1) / 2 + kt; }
GPT2_DEVICE_INLINE long long tri_tiles(int n) { return (long long)n * (n + 1) / 2; }

// dK, dV for a block of 128 keys (32 per wave, four waves), looping over 64-query tiles from
// the diagonal. It also writes dS = P * (dP - D) of every causal 64x64 tile it visits to
// `dsbuf`, from which attn_bwd_dq_kernel forms dQ = dS K without recomputing P and dP.
// The query tile is held in LDS twice: row-major for S = Q K^T and dP = dO V^T (a lane reads
// four consecutive head dims of its query), and transposed for dV^T = dO^T P^T and
// dK^T = Q^T dS^T (a lane reads four consecutive queries of its head dim), so every MFMA
// operand comes from a 16-byte LDS read. With 64-dim heads this fits two waves per SIMD.
constexpr int DK_KEYS = 128, DK_THR = 256;

template <int HSP, typename TS>
__global__ __launch_bounds__(DK_THR) __attribute__((amdgpu_waves_per_eu(HSP <= 64 ? 2 : 1)))
void attn_bwd_dkdv_kernel(TS* __restrict__ dqkv, float* __restrict__ dsbuf,
                          const TS* __restrict__ dout, const TS* __restrict__ qkv,
                          const float* __restrict__ lse, const float* __restrict__ Drow, int T,
                          int C, int NH, int hs, float scale, float scale_log2) {
  constexpr int LD = HSP + 4, LDT = TILE + 4, NS = HSP / 2, ND = HSP / 32;
  __shared__ float Qs[TILE][LD];
  __shared__ float dOs[TILE][LD];
  __shared__ float QT[HSP][LDT];
  __shared__ float dOT[HSP][LDT];
  __shared__ __attribute__((aligned(16))) float Ls[TILE];
  __shared__ __attribute__((aligned(16))) float Ds[TILE];

  const int nkb = (T + DK_KEYS - 1) / DK_KEYS;
  int kb, head, b;
  key_block_of(nkb, NH, &kb, &head, &b);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r = lane & 31, hf = lane >> 5;
  const long long C3 = 3LL * C;
  const TS* base = qkv + (long long)b * T * C3 + (long long)head * hs;
  const TS* dobase = dout + (long long)b * T * C + (long long)head * hs;
  const float* lrow = lse + ((long long)b * NH + head) * T;
  const float* drow = Drow + ((long long)b * NH + head) * T;
  const int key0 = kb * DK_KEYS + wave * 32;  // first key of this wave
  const int key = key0 + r;
  const int km = min(key, T - 1);
  const int kt = key0 / TILE;             // this wave's 64-key tile in the dS layout
  const int kcol = key0 - kt * TILE + r;  // this lane's column in that tile

  float kf[NS], vf[NS];
#pragma unroll
  for (int g = 0; g < HSP / 8; g++) {
    const int d = 8 * g + 4 * hf;
    f32x4 kv = load4_rowcol(base + C, C3, km, d, T, hs);
    f32x4 vv = load4_rowcol(base + 2 * C, C3, km, d, T, hs);
#pragma unroll
    for (int j = 0; j < 4; j++) {
      kf[4 * g + j] = kv[j];
      vf[4 * g + j] = vv[j];
    }
  }
  f32x16 dvacc[ND], dkacc[ND];
#pragma unroll
  for (int db = 0; db < ND; db++)
#pragma unroll
    for (int i = 0; i < 16; i++) {
      dvacc[db][i] = 0.f;
      dkacc[db][i] = 0.f;
    }

  const int nqt = (T + TILE - 1) / TILE;
  for (int qt = kb * DK_KEYS / TILE; qt < nqt; qt++) {
    const int q0 = qt * TILE;
    __syncthreads();
    // A thread takes a 4 x 4 block (rows 4a .. 4a+3, head dims 4dg .. 4dg+3), consecutive
    // threads consecutive row groups, and writes it row-major and, transposed in registers,
    // head-dim-major, all as 16-byte vectors: the transposed rows of eight consecutive
    // threads then fall on different banks, and the row-major rows are written in a
    // per-thread rotated order (row 4a + (w + a) % 4 at step w), which halves their
    // conflicts.
    constexpr int RG = TILE / 4, DG = HSP / 4;
#pragma unroll
    for (int blk = 0; blk < (RG * DG + DK_THR - 1) / DK_THR; blk++) {
      const int f = tid + DK_THR * blk;
      if (RG * DG % DK_THR != 0 && f >= RG * DG) break;
      const int a = f % RG, d = 4 * (f / RG);
      f32x4 qv[4], ov[4];
#pragma unroll
      for (int i = 0; i < 4; i++) {
        qv[i] = load4_rowcol(base, C3, q0 + 4 * a + i, d, T, hs);
        ov[i] = load4_rowcol(dobase, C, q0 + 4 * a + i, d, T, hs);
      }
#pragma unroll
      for (int w = 0; w < 4; w++) {
        const int i = (w + a) & 3;
        const f32x4 qr = i == 0 ? qv[0] : i == 1 ? qv[1] : i == 2 ? qv[2] : qv[3];
        const f32x4 orow = i == 0 ? ov[0] : i == 1 ? ov[1] : i == 2 ? ov[2] : ov[3];
        *reinterpret_cast<f32x4*>(&Qs[4 * a + i][d]) = qr;
        *reinterpret_cast<f32x4*>(&dOs[4 * a + i][d]) = orow;
      }
#pragma unroll
      for (int j = 0; j < 4; j++) {
        *reinterpret_cast<f32x4*>(&QT[d + j][4 * a]) = f32x4{qv[0][j], qv[1][j], qv[2][j], qv[3][j]};
        *reinterpret_cast<f32x4*>(&dOT[d + j][4 * a]) =
            f32x4{ov[0][j], ov[1][j], ov[2][j], ov[3][j]};
      }
    }
    if (tid < TILE) {
      const bool ok = q0 + tid < T;
      const int t = min(q0 + tid, T - 1);
      Ls[tid] = ok ? lrow[t] * kLog2e : 0.f;
      Ds[tid] = ok ? drow[t] : 0.f;
    }
    __syncthreads();
    if (qt < kt) continue;  // every query of this tile precedes this wave's keys
    // dS tile (qt, kt) of this (b, head): 64 x 64 floats, [query][key]; this lane writes
    // column kcol of rows 4hf + (32qb + 8(i/4) + i%4)
    float* dst = dsbuf + (((long long)b * NH + head) * tri_tiles(nqt) + tri_index(qt, kt)) *
                             (TILE * TILE) + 4 * hf * TILE + kcol;
#pragma unroll 1
    for (int qb = 0; qb < 2; qb++) {
      // the lse and D of this lane's 16 queries (four runs of four consecutive rows), read
      // before the products so their latency is hidden
      f32x4 lq[4], dq[4];
#pragma unroll
      for (int gq = 0; gq < 4; gq++) {
        lq[gq] = *reinterpret_cast<const f32x4*>(&Ls[32 * qb + 8 * gq + 4 * hf]);
        dq[gq] = *reinterpret_cast<const f32x4*>(&Ds[32 * qb + 8 * gq + 4 * hf]);
      }
      f32x16 s, dp;
#pragma unroll
      for (int i = 0; i < 16; i++) {
        s[i] = 0.f;
        dp[i] = 0.f;
      }
#pragma unroll
      for (int g = 0; g < HSP / 8; g++) {
        const f32x4 qv = *reinterpret_cast<const f32x4*>(&Qs[32 * qb + r][8 * g + 4 * hf]);
        const f32x4 ov = *reinterpret_cast<const f32x4*>(&dOs[32 * qb + r][8 * g + 4 * hf]);
#pragma unroll
        for (int j = 0; j < 4; j++) {
          s = mfma32x32x2(qv[j], kf[4 * g + j], s);
          dp = mfma32x32x2(ov[j], vf[4 * g + j], dp);
        }
      }
      // s[i], dp[i]: query ql = 32qb + 8(i/4) + 4hf + i%4, key = this lane's. The
      // exponential is taken for every entry and masked after (no branch per entry).
#pragma unroll
      for (int i = 0; i < 16; i++) {
        const int qo = 32 * qb + 8 * (i / 4) + (i % 4);  // ql - 4hf
        const int qa = q0 + qo + 4 * hf;
        const bool ok = qa < T && qa >= key;
        const float e = __builtin_amdgcn_exp2f(s[i] * scale_log2 - lq[i / 4][i % 4]);
        const float p = ok ? e : 0.f;
        s[i] = p;
        dp[i] = p * (dp[i] - dq[i / 4][i % 4]);
        dst[qo * TILE] = dp[i];  // 32 lanes store 32 consecutive keys
      }
      // dV^T[d][key] += dO[q][d] P[q][key] and dK^T[d][key] += Q[q][d] dS[q][key] over this
      // sub-block's queries; entries 4sg .. 4sg+3 of s and dp are four consecutive queries
#pragma unroll
      for (int db = 0; db < ND; db++)
#pragma unroll
        for (int sg = 0; sg < 4; sg++) {
          const int ql0 = 32 * qb + 8 * sg + 4 * hf;
          const f32x4 ot = *reinterpret_cast<const f32x4*>(&dOT[32 * db + r][ql0]);
          const f32x4 qt4 = *reinterpret_cast<const f32x4*>(&QT[32 * db + r][ql0]);
#pragma unroll
          for (int j = 0; j < 4; j++) {
            dvacc[db] = mfma32x32x2(ot[j], s[4 * sg + j], dvacc[db]);
            dkacc[db] = mfma32x32x2(qt4[j], dp[4 * sg + j], dkacc[db]);
          }
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
        const int d = 32 * db + 8 * ig + 4 * hf;
        if (d < hs) {
          st4(dk + d, f32x4{dkacc[db][4 * ig] * scale, dkacc[db][4 * ig + 1] * scale,
                            dkacc[db][4 * ig + 2] * scale, dkacc[db][4 * ig + 3] * scale});
          st4(dv + d, f32x4{dvacc[db][4 * ig], dvacc[db][4 * ig + 1], dvacc[db][4 * ig + 2],
                            dvacc[db][4 * ig + 3]});
        }
      }
  }
}

// dQ = scale * dS K for a tile of 64 queries (32 per wave), over key tiles 0 .. qt, reading
// the dS tiles written by attn_bwd_dkdv_kernel. M = queries, N = head dim, K = keys.
template <int HSP, typename TS>
__global__ __launch_bounds__(NTHR) void attn_bwd_dq_kernel(TS* __restrict__ dqkv,
                                                           const TS* __restrict__ qkv,
                                                           const float* __restrict__ dsbuf, int T,
                                                           int C, int NH, int hs, float scale) {
  constexpr int LD = HSP + 4, ND = HSP / 32, LDSS = TILE + 4;
  __shared__ float Ks[TILE][LD];
  __shared__ float Ss[TILE][LDSS];

  const int nqt = (T + TILE - 1) / TILE;
  int qt, head, b;
  tile_of_block(nqt, NH, &qt, &head, &b);
  qt = nqt - 1 - qt;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r = lane & 31, hf = lane >> 5;
  const long long C3 = 3LL * C;
  const TS* kbase = qkv + (long long)b * T * C3 + (long long)head * hs + C;
  const float* src = dsbuf + (((long long)b * NH + head) * tri_tiles(nqt) + tri_index(qt, 0)) *
                                 (TILE * TILE);

  f32x16 acc[ND];
#pragma unroll
  for (int db = 0; db < ND; db++)
#pragma unroll
    for (int i = 0; i < 16; i++) acc[db][i] = 0.f;

  // the next key tile's K and dS are loaded into registers while this one is used
  constexpr int F4 = HSP / 4, NK = TILE * F4 / NTHR, NS4 = TILE * TILE / 4 / NTHR;
  f32x4 pk[NK], ps[NS4];
  auto fetch = [&](int kt) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < NK; i++) {
      const int f = tid + NTHR * i;
      pk[i] = load4_rowcol(kbase, C3, kt * TILE + f / F4, 4 * (f % F4), T, hs);
    }
    const float* ts = src + (long long)kt * TILE * TILE;
#pragma unroll
    for (int i = 0; i < NS4; i++) {
      const int f = tid + NTHR * i;
      ps[i] = *reinterpret_cast<const f32x4*>(ts + 4 * f);
    }
  };
  fetch(0);
  for (int kt = 0; kt <= qt; kt++) {
    __syncthreads();
#pragma unroll
    for (int i = 0; i < NK; i++) {
      const int f = tid + NTHR * i;
      *reinterpret_cast<f32x4*>(&Ks[f / F4][4 * (f % F4)]) = pk[i];
    }
#pragma unroll
    for (int i = 0; i < NS4; i++) {
      const int f = tid + NTHR * i;
      *reinterpret_cast<f32x4*>(&Ss[f / (TILE / 4)][4 * (f % (TILE / 4))]) = ps[i];
    }
    __syncthreads();
    if (kt < qt) fetch(kt + 1);
    // 32 steps of two keys; at step s = 4g + j this half of the wave takes key 8g + 4hf + j
#pragma unroll
    for (int g = 0; g < TILE / 8; g++) {
      const f32x4 sv = *reinterpret_cast<const f32x4*>(&Ss[32 * wave + r][8 * g + 4 * hf]);
#pragma unroll
      for (int j = 0; j < 4; j++)
#pragma unroll
        for (int db = 0; db < ND; db++)
          acc[db] = mfma32x32x2(sv[j], Ks[8 * g + 4 * hf + j][32 * db + r], acc[db]);
    }
  }
  // acc[db][i]: query 32*wave + 8(i/4) + 4hf + i%4 of the tile, head dim 32*db + r
#pragma unroll
  for (int db = 0; db < ND; db++) {
    const int d = 32 * db + r;
    if (d >= hs) continue;
#pragma unroll
    for (int i = 0; i < 16; i++) {
      const int q = qt * TILE + 32 * wave + 8 * (i / 4) + 4 * hf + (i % 4);
      if (q < T) st1(dqkv + ((long long)b * T + q) * C3 + (long long)head * hs + d, acc[db][i] * scale);
    }
  }
}

template <typename TS>
constexpr bool is_f16() {
  return std::is_same<TS, f16_t>::value;
}

bool check_shape(int B, int T, int C, int NH, int* hsp) {
  if (B < 1 || T < 1 || C < 1 || NH < 1 || C % NH) return false;
  const int hs = C / NH;
  if (hs % 4 || C % 4) return false;
  if (hs <= 32) *hsp = 32;
  else if (hs <= 64) *hsp = 64;
  else if (hs <= 128) *hsp = 128;
  else return false;
  return true;
}


// the direct-to-LDS forward exists for fp32 storage only
template <typename TS>
bool launch_fwd_direct(dim3, hipStream_t, TS*, float*, const TS*, int, int, int, int, float) {
  return false;
}
template <>
bool launch_fwd_direct<float>(dim3 grid, hipStream_t stream, float* out, float* lse,
                              const float* qkv, int T, int C, int NH, int hs, float scale_log2) {
  attn_fwd_kernel<64, float, true><<<grid, NTHR, 0, stream>>>(out, lse, qkv, T, C, NH, hs,
                                                               scale_log2);
  return true;
}

template <typename TS>
int attention_forward_t(TS* out, float* lse, const TS* qkv, int B, int T, int C, int NH,
                        hipStream_t stream) {
  int hsp;
  if (!check_shape(B, T, C, NH, &hsp)) {
    set_global_error("attention: unsupported shape B=%d T=%d C=%d NH=%d", B, T, C, NH);
    return -1;
  }
  const int hs = C / NH;
  const float scale_log2 = kLog2e / sqrtf((float)hs);
  dim3 grid(((T + TILE - 1) / TILE) * NH * B);
  const double tri = (double)T * (T + 1) / 2.0;  // causal (query, key) pairs per head
  const double es = sizeof(TS);
  ProfScope ps(sizeof(TS) == 4 ? "attn_fwd_kernel" : is_f16<TS>() ? "attn_fwd_f16_kernel"
                                                                   : "attn_fwd_bf16_kernel",
               4.0 * B * NH * hs * tri,
               es * ((double)B * T * 3 * C + (double)B * T * C) + 4.0 * B * NH * T, stream);
  if (hsp == 64 && hs == 64 && launch_fwd_direct(grid, stream, out, lse, qkv, T, C, NH, hs, scale_log2)) {
  } else if (hsp == 32) attn_fwd_kernel<32, TS><<<grid, NTHR, 0, stream>>>(out, lse, qkv, T, C, NH, hs, scale_log2);
  else if (hsp == 64) attn_fwd_kernel<64, TS><<<grid, NTHR, 0, stream>>>(out, lse, qkv, T, C, NH, hs, scale_log2);
  else attn_fwd_kernel<128, TS><<<grid, NTHR, 0, stream>>>(out, lse, qkv, T, C, NH, hs, scale_log2);
  GPT2_HIP_OK(hipGetLastError());
  return 0;
}

}  // namespace

size_t attention_ds_scratch_floats(int B, int T, int NH) {
  const long long nt = (T + TILE - 1) / TILE;
  return (size_t)B * NH * (nt * (nt + 1) / 2) * TILE * TILE;
}

namespace {
// D = rowsum(dout * out) per (b, head, query), fp32, into D (B, NH, T)
template <typename TS>
int rowdot_t(float* D, const TS* dout, const TS* out, int B, int T, int C, int NH,
             hipStream_t stream) {
  const int hs = C / NH;
  const long long rows = (long long)B * NH * T;
  const double BTC = (double)B * T * C;
  ProfScope ps(sizeof(TS) == 4   ? "attn_bwd_rowdot_kernel"
               : is_f16<TS>() ? "attn_bwd_rowdot_f16_kernel"
                              : "attn_bwd_rowdot_bf16_kernel",
               2.0 * BTC, (double)sizeof(TS) * 2.0 * BTC + 4.0 * rows, stream);
  const long long n4 = (long long)B * T * (C / 4);
  const unsigned blocks = (unsigned)((n4 + 255) / 256);
  switch (hs / 4) {
    case 1: attn_bwd_rowdot_kernel<1, TS><<<blocks, 256, 0, stream>>>(D, dout, out, B, T, C, NH); break;
    case 2: attn_bwd_rowdot_kernel<2, TS><<<blocks, 256, 0, stream>>>(D, dout, out, B, T, C, NH); break;
    case 4: attn_bwd_rowdot_kernel<4, TS><<<blocks, 256, 0, stream>>>(D, dout, out, B, T, C, NH); break;
    case 8: attn_bwd_rowdot_kernel<8, TS><<<blocks, 256, 0, stream>>>(D, dout, out, B, T, C, NH); break;
    case 16: attn_bwd_rowdot_kernel<16, TS><<<blocks, 256, 0, stream>>>(D, dout, out, B, T, C, NH); break;
    case 32: attn_bwd_rowdot_kernel<32, TS><<<blocks, 256, 0, stream>>>(D, dout, out, B, T, C, NH); break;
    default:
      attn_bwd_rowdot_generic_kernel<TS><<<(unsigned)((rows + 255) / 256), 256, 0, stream>>>(
          D, dout, out, B, T, C, NH, hs);
  }
  GPT2_HIP_OK(hipGetLastError());
  return 0;
}

// fp32 attention with head sizes that are multiples of 8 forms its forward and dQ products
// from split operands on bf16 MFMA unless GPT2_ATTN_F32_PRODUCTS is "fp32"; other head sizes
// (and that setting) multiply on fp32 MFMA
bool attn_x6(int C, int NH) {
  const char* e = getenv("GPT2_ATTN_F32_PRODUCTS");
  return !(e && strcmp(e, "fp32") == 0) && NH > 0 && C % NH == 0 &&
         attention_bf16_mma_supported(C, NH);
}

template <typename TS>
int attention_backward_t(TS* dqkv, const TS* dout, const TS* qkv, const TS* out,
                         const float* lse, float* dscratch, float* ds_scratch, int B, int T,
                         int C, int NH, hipStream_t stream) {
  int hsp;
  if (!check_shape(B, T, C, NH, &hsp)) {
    set_global_error("attention: unsupported shape B=%d T=%d C=%d NH=%d", B, T, C, NH);
    return -1;
  }
  const bool f32 = sizeof(TS) == 4;
  const double es = sizeof(TS);
  const int hs = C / NH;
  const float scale = 1.0f / sqrtf((float)hs);
  const float scale_log2 = scale * kLog2e;
  const long long rows = (long long)B * NH * T;
  const double BTC = (double)B * T * C, tri = (double)T * (T + 1) / 2.0;
  const int rc = rowdot_t(dscratch, dout, out, B, T, C, NH, stream);
  if (rc) return rc;
  dim3 grid(((T + TILE - 1) / TILE) * NH * B);
  if (f32 && attn_x6(C, NH) && attention_dkdv_x6_supported(C, NH)) {
    const int rk = attention_dkdv_x6(reinterpret_cast<float*>(dqkv), ds_scratch,
                                     reinterpret_cast<const float*>(dout),
                                     reinterpret_cast<const float*>(qkv), lse, dscratch, B, T, C,
                                     NH, stream);
    if (rk) return rk;
  } else {  // dK, dV: the products dV = P^T dO and dK = dS^T Q (plus the dP = dO V^T they need)
    ProfScope ps(f32 ? "attn_bwd_dkdv_kernel"
                     : is_f16<TS>() ? "attn_bwd_dkdv_f16_kernel" : "attn_bwd_dkdv_bf16_kernel",
                 6.0 * B * NH * hs * tri,
                 es * (3.0 * BTC + BTC + 2.0 * BTC) + 4.0 * (2.0 * rows + B * NH * tri), stream);
    const dim3 gk(((T + DK_KEYS - 1) / DK_KEYS) * NH * B);
    if (hsp == 32) attn_bwd_dkdv_kernel<32, TS><<<gk, DK_THR, 0, stream>>>(dqkv, ds_scratch, dout, qkv, lse, dscratch, T, C, NH, hs, scale, scale_log2);
    else if (hsp == 64) attn_bwd_dkdv_kernel<64, TS><<<gk, DK_THR, 0, stream>>>(dqkv, ds_scratch, dout, qkv, lse, dscratch, T, C, NH, hs, scale, scale_log2);
    else attn_bwd_dkdv_kernel<128, TS><<<gk, DK_THR, 0, stream>>>(dqkv, ds_scratch, dout, qkv, lse, dscratch, T, C, NH, hs, scale, scale_log2);
  }
  if (f32 && attn_x6(C, NH)) {  // dQ = dS K with split-operand products
    const int rq = attention_dq_x6(reinterpret_cast<float*>(dqkv),
                                   reinterpret_cast<const float*>(qkv), ds_scratch, B, T, C, NH,
                                   stream);
    if (rq) return rq;
  } else {  // dQ = dS K
    ProfScope ps(f32 ? "attn_bwd_dq_kernel"
                     : is_f16<TS>() ? "attn_bwd_dq_f16_kernel" : "attn_bwd_dq_bf16_kernel",
                 2.0 * B * NH * hs * tri,
                 4.0 * B * NH * tri + es * 2.0 * BTC, stream);
    if (hsp == 32) attn_bwd_dq_kernel<32, TS><<<grid, NTHR, 0, stream>>>(dqkv, qkv, ds_scratch, T, C, NH, hs, scale);
    else if (hsp == 64) attn_bwd_dq_kernel<64, TS><<<grid, NTHR, 0, stream>>>(dqkv, qkv, ds_scratch, T, C, NH, hs, scale);
    else attn_bwd_dq_kernel<128, TS><<<grid, NTHR, 0, stream>>>(dqkv, qkv, ds_scratch, T, C, NH, hs, scale);
  }
  GPT2_HIP_OK(hipGetLastError());
  return 0;
}

}  // namespace

int attention_forward(float* out, float* lse, const float* qkv, int B, int T, int C, int NH,
                      hipStream_t stream) {
  if (attn_x6(C, NH)) return attention_forward_x6(out, lse, qkv, B, T, C, NH, stream);
  return attention_forward_t(out, lse, qkv, B, T, C, NH, stream);
}
int attention_forward(bf16_t* out, float* lse, const bf16_t* qkv, int B, int T, int C, int NH,
                      hipStream_t stream) {
  // head sizes that are multiples of 8 use the bf16-MFMA kernel; others multiply in fp32
  if (C % NH == 0 && attention_bf16_mma_supported(C, NH))
    return attention_forward_bf16_mma(out, lse, qkv, B, T, C, NH, stream);
  return attention_forward_t(out, lse, qkv, B, T, C, NH, stream);
}
int attention_backward(float* dqkv, const float* dout, const float* qkv, const float* out,
                       const float* lse, float* dscratch, float* ds_scratch, int B, int T, int C,
                       int NH, hipStream_t stream) {
  return attention_backward_t(dqkv, dout, qkv, out, lse, dscratch, ds_scratch, B, T, C, NH,
                              stream);
}
int attention_backward(bf16_t* dqkv, const bf16_t* dout, const bf16_t* qkv, const bf16_t* out,
                       const float* lse, float* dscratch, float* ds_scratch, int B, int T, int C,
                       int NH, hipStream_t stream) {
  if (C % NH == 0 && attention_bf16_mma_supported(C, NH))
    return attention_backward_bf16_mma(dqkv, dout, qkv, out, lse, dscratch, ds_scratch, B, T, C,
                                       NH, stream);
  return attention_backward_t(dqkv, dout, qkv, out, lse, dscratch, ds_scratch, B, T, C, NH,
                              stream);
}
int attention_rowdot(float* D, const bf16_t* dout, const bf16_t* out, int B, int T, int C,
                     int NH, hipStream_t stream) {
  return rowdot_t(D, dout, out, B, T, C, NH, stream);
}
int attention_forward(f16_t* out, float* lse, const f16_t* qkv, int B, int T, int C, int NH,
                      hipStream_t stream) {
  // head sizes that are multiples of 8 use the fp16-MFMA kernel; others multiply in fp32
  if (C % NH == 0 && attention_bf16_mma_supported(C, NH))
    return attention_forward_f16_mma(out, lse, qkv, B, T, C, NH, stream);
  return attention_forward_t(out, lse, qkv, B, T, C, NH, stream);
}
int attention_backward(f16_t* dqkv, const f16_t* dout, const f16_t* qkv, const f16_t* out,
                       const float* lse, float* dscratch, float* ds_scratch, int B, int T, int C,
                       int NH, hipStream_t stream) {
  if (C % NH == 0 && attention_bf16_mma_supported(C, NH))
    return attention_backward_f16_mma(dqkv, dout, qkv, out, lse, dscratch, ds_scratch, B, T, C,
                                      NH, stream);
  return attention_backward_t(dqkv, dout, qkv, out, lse, dscratch, ds_scratch, B, T, C, NH,
                              stream);
}
int attention_rowdot(float* D, const f16_t* dout, const f16_t* out, int B, int T, int C,
                     int NH, hipStream_t stream) {
  return rowdot_t(D, dout, out, B, T, C, NH, stream);
}

}  // namespace gpt2
