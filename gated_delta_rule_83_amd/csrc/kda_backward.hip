// Chunked backward pass of the KDA recurrence (decay, delta read, rank-1
// write, readout) for training: the gradients of the activations q^, k^, v^,
// the log-decay g, beta and the entering state S0, given the gradients dO of
// the readouts and dST of the final state. gfx950, wave64, fp32 arithmetic
// throughout (bf16 activations are widened on load).
//
// Forward form per chunk of n tokens (the chunkwise-parallel form of
// "为什么 Kimi K3 敢把 KV Cache 扔掉？…", sections 5-7), entering state S0:
//   Gam = in-chunk prefix sum of g, Q~ = e^Gam q^, K~ = e^Gam k^,
//   K^d = e^{Gam_n - Gam} k^, E_rjc = e^{Gam_rc - Gam_jc} (j <= r),
//   A_rj = sum_c k^_rc k^_jc E_rjc (j < r), P_rj = sum_c q^_rc k^_jc E_rjc (j <= r),
//   X = (I + diag(beta) A)^-1, W = X diag(beta) K~, U' = X diag(beta) V^,
//   U = U' - W S0, O = Q~ S0 + P U, S1 = Diag(e^{Gam_n}) S0 + K^d^T U.
// Backward, by reverse-mode differentiation of these products:
//   reverse chain (sequential over chunks, last first), dS1 the gradient
//   that reaches the chunk's leaving state:
//     dU = P^T dO + K^d dS1,  dS0 = Diag(e^{Gam_n}) dS1 + Q~^T dO - W^T dU;
//   per chunk, in parallel:
//     dQ~ = dO S0^T, dP = (dO U^T) on j <= r, dK^d = U dS1^T,
//     d e^{Gam_n} = rowsum(dS1 * S0), dW = -dU S0^T,
//     Y = X^T dW, Z = X^T dU: dK~ = beta Y, dV^ = beta Z, dbeta += K~.Y + V^.Z,
//     dX = dW (beta K~)^T + dU (beta V^)^T, dM = -X^T dX X^T (strictly lower),
//     dA = beta dM, dbeta += A.dM,
//     then back through the decayed Grams A and P, the scalings Q~, K~, K^d,
//     and dg as the reverse in-chunk prefix sum of dGam.
//
// Launches: prep (per chunk-head) -> state chain (per head and 32-column
// block, keeps the entering state of every chunk) -> reverse chain (same
// grid, keeps the leaving-state gradient of every chunk and dU) -> dense
// gradients (per chunk-head) -> inverse and beta gradients (per chunk-head)
// -> decayed-Gram gradients and dg (per chunk-head). Any finite g <= 0 is
// accepted: a chunk whose total decay stays within a limit forms its decayed
// pair terms as MFMA products of e^{Gam}- and e^{-Gam}-scaled rows, any other
// chunk one exponential of a non-positive difference per pair.
#include <algorithm>
#include <type_traits>

#include "kda_common.h"

namespace kda {
namespace {

constexpr int kBT = 256;  // threads per workgroup
constexpr int CM = 64;    // largest chunk

// Per-(chunk, sequence, head) scratch block, in floats; rows of token
// arrays are [CM][DK] / [CM][DV] row-major, C x C arrays [CM][CM].
template <int DK, int DV>
struct BwL {
  static constexpr long oQt = 0;                 // Q~
  static constexpr long oKt = oQt + CM * DK;     // K~
  static constexpr long oKd = oKt + CM * DK;     // K^d
  static constexpr long oW = oKd + CM * DK;      // W
  static constexpr long oG = oW + CM * DK;       // Gam
  static constexpr long odq = oG + CM * DK;      // dq^ (dense part)
  static constexpr long odk = odq + CM * DK;     // dk^ (dense part)
  static constexpr long odG = odk + CM * DK;     // dGam (dense part, then total)
  static constexpr long odW = odG + CM * DK;     // dW
  static constexpr long oU = odW + CM * DK;      // U', then U
  static constexpr long odU = oU + CM * DV;      // dU
  static constexpr long oP = odU + CM * DV;      // P
  static constexpr long oX = oP + CM * CM;       // X
  static constexpr long oA = oX + CM * CM;       // A
  static constexpr long odA = oA + CM * CM;      // dA
  static constexpr long odP = odA + CM * CM;     // dP
  static constexpr long oEn = odP + CM * CM;     // e^{Gam_n} [DK]
  static constexpr long n = oEn + DK;
};

__device__ __forceinline__ long tok(const BackwardArgs& a, int b, int t, int h) {
  return ((long)b * a.T + t) * a.H + h;
}

struct Item {
  int c, b, h, bh, t0, n;
};

__device__ __forceinline__ Item item_of(const BackwardArgs& a, long it) {
  Item r;
  const int BH = a.B * a.H;
  r.c = a.c0 + (int)(it / BH);  // blocks index the launch's chunks from c0
  r.bh = (int)(it % BH);
  r.b = r.bh / a.H;
  r.h = r.bh % a.H;
  r.t0 = r.c * a.chunk;
  r.n = min(a.chunk, a.T - r.t0);
  return r;
}

// 16 x 16 tile on fp32 MFMA (v_mfma_f32_16x16x4_f32): acc += A B over k in
// [0, K), K a multiple of 4, with a(i, k) = A[tile row i][k] and
// b(k, j) = B[k][tile column j]. Lane l supplies A[l % 16][k + l / 16] and
// B[k + l / 16][l % 16]; element e of the result is tile row 4 (l / 16) + e,
// column l % 16.
template <class FA, class FB>
__device__ __forceinline__ f32x4 mma_tile(f32x4 acc, int K, FA&& a, FB&& b) {
  const int l = threadIdx.x % kWave, i = l % 16, kk = l / 16;
#pragma unroll 4
  for (int k = 0; k < K; k += 4)
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a(i, k + kk), b(k + kk, i), acc, 0, 0, 0);
  return acc;
}

// Sum over the 16 lanes of a row group (lanes with equal l / 16).
__device__ __forceinline__ float sum16(float x) {
#pragma unroll
  for (int off = 1; off < 16; off <<= 1) x += __shfl_xor(x, off, kWave);
  return x;
}

constexpr f32x4 kZero4 = {0.f, 0.f, 0.f, 0.f};

typedef float f32x2 __attribute__((ext_vector_type(2)));

// Four consecutive elements as fp32 (one 16- or 8-byte load).
__device__ __forceinline__ f32x4 ld4f(const float* p) { return *reinterpret_cast<const f32x4*>(p); }
__device__ __forceinline__ f32x4 ld4f(const bf16* p) {
  const bf16x4 v = *reinterpret_cast<const bf16x4*>(p);
  return f32x4{(float)v[0], (float)v[1], (float)v[2], (float)v[3]};
}

// A thread's 16-byte pieces of a ROWS x COLS block, loaded into registers by
// get_rows and written to LDS by put_rows: between the two calls the loads
// stay in flight, so a block for a later step can be fetched while the
// current one is in use.
template <int NT, int ROWS, int COLS>
struct Pieces {
  static_assert(COLS % 4 == 0, "16-byte pieces");
  static constexpr int Q = COLS / 4, TOT = ROWS * Q, PER = (TOT + NT - 1) / NT;
  f32x4 v[PER];
};

// ld4(r, c) gives row r, columns c..c+3 for r < live; rows at or past `live`
// are zeros.
template <int NT, int ROWS, int COLS, class F>
__device__ __forceinline__ void get_rows(Pieces<NT, ROWS, COLS>& b, int live, F&& ld4) {
  using P = Pieces<NT, ROWS, COLS>;
#pragma unroll
  for (int p = 0; p < P::PER; ++p) {
    const int i = (int)threadIdx.x + p * NT, r = i / P::Q, c = 4 * (i % P::Q);
    b.v[p] = (i < P::TOT && r < live) ? ld4(r, c) : kZero4;
  }
}

// LDS destination rows of LD floats (LD a multiple of 4, 16-byte aligned rows).
template <int LD, int NT, int ROWS, int COLS>
__device__ __forceinline__ void put_rows(const Pieces<NT, ROWS, COLS>& b, float* dst) {
  using P = Pieces<NT, ROWS, COLS>;
  static_assert(LD % 4 == 0, "16-byte rows");
#pragma unroll
  for (int p = 0; p < P::PER; ++p) {
    const int i = (int)threadIdx.x + p * NT, r = i / P::Q, c = 4 * (i % P::Q);
    if (i < P::TOT) *reinterpret_cast<f32x4*>(dst + r * LD + c) = b.v[p];
  }
}

// Stages ROWS x COLS values into LDS (row stride LD floats): get_rows then
// put_rows, every load of a thread issued before its stores.
template <int NT, int ROWS, int COLS, int LD, class F>
__device__ __forceinline__ void stage_rows(float* dst, int live, F&& ld4) {
  Pieces<NT, ROWS, COLS> b;
  get_rows(b, live, ld4);
  put_rows<LD>(b, dst);
}

// put_rows into LDS rows of LD bf16 (LD a multiple of 4: 8-byte pieces),
// each value rounded to the nearest bf16.
template <int LD, int NT, int ROWS, int COLS>
__device__ __forceinline__ void put_rows_bf16(const Pieces<NT, ROWS, COLS>& b, bf16* dst) {
  using P = Pieces<NT, ROWS, COLS>;
  static_assert(LD % 4 == 0, "8-byte rows");
#pragma unroll
  for (int p = 0; p < P::PER; ++p) {
    const int i = (int)threadIdx.x + p * NT, r = i / P::Q, c = 4 * (i % P::Q);
    if (i < P::TOT)
      *reinterpret_cast<bf16x4*>(dst + r * LD + c) =
          bf16x4{(bf16)b.v[p][0], (bf16)b.v[p][1], (bf16)b.v[p][2], (bf16)b.v[p][3]};
  }
}
constexpr int kBP = 1024;  // threads of the per-chunk kernels with scalar loops

// Decay factors e^{Gam_r - Gam_j} (j <= r) of a chunk may be formed as the
// product e^{Gam_r} e^{-Gam_j} when every channel's total in-chunk decay
// -Gam_{n-1} is at most this (e^60 ~ 1e26 keeps every factor, and its
// products with the unit-norm activations and their gradients, well inside
// fp32); the pair sums then become matrix products. Chunks that decay faster
// take the explicit per-pair exponentials.
constexpr float kFactorMaxDecay = 60.f;

// true when -Gam[n-1][c] <= kFactorMaxDecay for every channel c (all
// threads of the workgroup take part; the result is uniform).
template <int NT, int DK, int LD>
__device__ __forceinline__ bool chunk_factorable(const float (*sG)[LD], int n, int* flag) {
  if (threadIdx.x == 0) *flag = 1;
  __syncthreads();
  for (int c = threadIdx.x; c < DK; c += NT)
    if (!(-sG[n - 1][c] <= kFactorMaxDecay)) *flag = 0;
  __syncthreads();
  const bool ok = *flag != 0;
  __syncthreads();
  return ok;
}
constexpr int kBS = 512;   // threads of the solve-gradient kernel

// ---- 1. per chunk-head: Gam, A, P, X, Q~, K~, K^d, W, U' --------------------
template <int DK, int DV, typename IO>
__global__ __launch_bounds__(kBP) void bw_prep_kernel(BackwardArgs a) {
  using L = BwL<DK, DV>;
  constexpr int PK = DK + 4, PKV = (DK > DV ? DK : DV) + 4;
  constexpr int NW = kBP / kWave;
  __shared__ __attribute__((aligned(16))) float sK[CM][PKV], sQ[CM][PK], sG[CM][PK];
  __shared__ __attribute__((aligned(16))) float sM[CM][CM + 1], sX[CM][CM + 4];
  __shared__ float sb[CM];  // sK later holds beta V^
  const Item it = item_of(a, blockIdx.x);
  const int n = it.n, n4 = (n + 3) & ~3;
  float* blk = a.scratch + (long)blockIdx.x * L::n;
  const int tid = threadIdx.x, lane = tid % kWave, wv = tid / kWave;
  const int l16 = lane % 16, r4 = 4 * (lane / 16);
  const IO* q = static_cast<const IO*>(a.q);
  const IO* k = static_cast<const IO*>(a.k);
  const IO* v = static_cast<const IO*>(a.v);
  const long row0 = tok(a, it.b, it.t0, it.h), rs = (long)a.H;  // token row r: row0 + r * rs
  // every input load issued before the first LDS store; V^ stays in registers
  // until its rows of LDS are free
  Pieces<kBP, CM, DK> pk, pq, pg;
  Pieces<kBP, CM, DV> pv;
  get_rows(pk, n, [&](int r, int c) { return ld4f(k + (row0 + r * rs) * DK + c); });
  get_rows(pq, n, [&](int r, int c) { return ld4f(q + (row0 + r * rs) * DK + c); });
  get_rows(pg, n, [&](int r, int c) { return ld4f(a.g + (row0 + r * rs) * DK + c); });
  get_rows(pv, n, [&](int r, int c) { return ld4f(v + (row0 + r * rs) * DV + c); });
  const float bt = tid < n ? a.beta[row0 + tid * rs] : 0.f;
  for (int i = tid; i < CM * CM; i += kBP) sX[i / CM][i % CM] = 0.f;
  put_rows<PKV>(pk, &sK[0][0]);
  put_rows<PK>(pq, &sQ[0][0]);
  put_rows<PK>(pg, &sG[0][0]);
  if (tid < CM) sb[tid] = bt;
  __syncthreads();
  if (tid < DK) {
    float s = 0.f;
    for (int r = 0; r < n; ++r) {
      s += sG[r][tid];
      sG[r][tid] = s;
    }
  }
  __syncthreads();
  __shared__ int sflag;
  if (chunk_factorable<kBP, DK, PK>(sG, n, &sflag)) {
    // A = K~ K-^T (strictly lower), P = Q~ K-^T (lower), with K~ = k^ e^{Gam},
    // Q~ = q^ e^{Gam}, K- = k^ e^{-Gam} formed per operand element: one 16 x 16
    // tile of the C x C matrices per wave (tiles right of the diagonal are zero)
    static_assert((CM / 16) * (CM / 16) == NW, "one C x C tile per wave");
    const int rt = wv / (CM / 16), ct = wv % (CM / 16);
    f32x4 ta = kZero4, tp = kZero4;
    if (16 * rt < n && ct <= rt) {
      auto kminus = [&](int kx, int j) { return sK[16 * ct + j][kx] * __expf(-sG[16 * ct + j][kx]); };
      ta = mma_tile(kZero4, DK, [&](int i, int kx) {
        return sK[16 * rt + i][kx] * __expf(sG[16 * rt + i][kx]);
      }, kminus);
      tp = mma_tile(kZero4, DK, [&](int i, int kx) {
        return sQ[16 * rt + i][kx] * __expf(sG[16 * rt + i][kx]);
      }, kminus);
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int r = 16 * rt + r4 + e, j = 16 * ct + l16;
      if (r >= n) continue;
      blk[L::oP + r * CM + j] = j <= r ? tp[e] : 0.f;
      blk[L::oA + r * CM + j] = j < r ? ta[e] : 0.f;
      sM[r][j] = j < r ? sb[r] * ta[e] : 0.f;
    }
  } else {
    // A (strictly lower) and P (lower), every exponent Gam_r - Gam_j (j <= r)
    // <= 0. Wave w takes the row pairs (r, CM-1-r), r = w, w+NW, ...: lanes
    // l < r hold row r, column l; the other lanes row CM-1-r, column l - r (its
    // diagonal included), so all 64 lanes work. The diagonal of row r and the
    // zeros right of every diagonal come from the pass after.
    for (int r = wv; r < CM / 2 && r < n; r += NW) {
      const bool first = lane < r;
      const int row = first ? r : CM - 1 - r, j = first ? lane : lane - r;
      if (row >= n) continue;
      float accA = 0.f, accP = 0.f;
  #pragma unroll 2
      for (int cc = 0; cc < DK; cc += 4) {
        const f32x4 kj = *reinterpret_cast<const f32x4*>(&sK[j][cc]);
        const f32x4 gj = *reinterpret_cast<const f32x4*>(&sG[j][cc]);
        const f32x4 kr = *reinterpret_cast<const f32x4*>(&sK[row][cc]);
        const f32x4 qr = *reinterpret_cast<const f32x4*>(&sQ[row][cc]);
        const f32x4 gr = *reinterpret_cast<const f32x4*>(&sG[row][cc]);
  #pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float ke = kj[e] * __expf(gr[e] - gj[e]);
          accA += kr[e] * ke;
          accP += qr[e] * ke;
        }
      }
      blk[L::oP + row * CM + j] = accP;
      blk[L::oA + row * CM + j] = j < row ? accA : 0.f;
      sM[row][j] = j < row ? sb[row] * accA : 0.f;
    }
    for (int i = tid; i < n * CM; i += kBP) {
      const int row = i / CM, j = i % CM;
      if (j < row || (j == row && row >= CM / 2)) continue;
      float p = 0.f;
      if (j == row)
        for (int cc = 0; cc < DK; ++cc) p += sQ[row][cc] * sK[row][cc];
      blk[L::oP + i] = p;
      blk[L::oA + i] = 0.f;
      sM[row][j] = 0.f;
    }
  }
  // rows of M past the chunk's last token were not written: zeros, so that
  // no product below meets a stale value (0 * NaN)
  for (int i = n * CM + tid; i < CM * CM; i += kBP) sM[i / CM][i % CM] = 0.f;
  __syncthreads();
  // X = (I + diag(beta) A)^-1 = (I + M)^-1, unit lower triangular, by 16-row
  // blocks (rows >= n stay zero):
  // - each diagonal block X_ii = (I + M_ii)^-1 by forward substitution, wave
  //   i for block i, four lanes per column splitting each row's dot product
  //   (a row's value is written by lane group 0 and read by the other groups
  //   of the same wave in the next row: LDS accesses of one wave complete in
  //   order);
  // - then the blocks below the diagonal, one block diagonal d = i - j at a
  //   time: X_ij = -X_ii (M_ij X_jj + M_i,j+1 X_j+1,j + ... + M_i,i-1 X_i-1,j),
  //   as 16 x 16 fp32 MFMA products, wave j for block (j + d, j).
  static_assert(CM == 64, "four 16-row blocks");
  if (wv < 4) {
    const int b0 = 16 * wv, j = b0 + l16, p = lane / 16;
    for (int r = b0; r < b0 + 16; ++r) {
      float acc = 0.f;
      for (int m = b0 + p; m < r; m += 4) acc += sM[r][m] * sX[m][j];
      acc += __shfl_xor(acc, 16, kWave);
      acc += __shfl_xor(acc, 32, kWave);
      if (p == 0) sX[r][j] = r >= n ? 0.f : (r > j ? -acc : (r == j ? 1.f : 0.f));
    }
  }
  __shared__ float sY[3][16][17];  // the sums of the current block diagonal
  for (int d = 1; d < 4; ++d) {
    __syncthreads();  // the previous block diagonal (or the diagonal blocks) is in sX
    const int jb = wv, ib = wv + d;
    if (wv < 4 - d) {
      f32x4 y = kZero4;
      for (int kb = jb; kb < ib; ++kb)
        y = mma_tile(y, 16, [&](int i, int kx) { return sM[16 * ib + i][16 * kb + kx]; },
                     [&](int kx, int jj) { return sX[16 * kb + kx][16 * jb + jj]; });
#pragma unroll
      for (int e = 0; e < 4; ++e) sY[wv][r4 + e][l16] = y[e];
    }
    __syncthreads();
    if (wv < 4 - d) {
      const f32x4 x = mma_tile(kZero4, 16, [&](int i, int kx) { return sX[16 * ib + i][16 * ib + kx]; },
                               [&](int kx, int jj) { return sY[wv][kx][jj]; });
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int row = 16 * ib + r4 + e;
        sX[row][16 * jb + l16] = row < n ? -x[e] : 0.f;
      }
    }
  }
  __syncthreads();
  for (int i = tid; i < n * CM; i += kBP) blk[L::oX + i] = sX[i / CM][i % CM];
  for (int i = tid; i < n * DK; i += kBP) {
    const int r = i / DK, cc = i % DK;
    const float G = sG[r][cc], eg = __expf(G), kt = eg * sK[r][cc];
    blk[L::oQt + i] = eg * sQ[r][cc];
    blk[L::oKt + i] = kt;
    blk[L::oKd + i] = __expf(sG[n - 1][cc] - G) * sK[r][cc];
    blk[L::oG + i] = G;
    sQ[r][cc] = sb[r] * kt;  // beta K~ (each element read by its writer only)
  }
  for (int i = n * DK + tid; i < CM * DK; i += kBP) sQ[i / DK][i % DK] = 0.f;
  if (tid < DK) blk[L::oEn + tid] = __expf(sG[n - 1][tid]);
  __syncthreads();
  // beta V^ over the (now unused) k rows
  {
    using P = Pieces<kBP, CM, DV>;
#pragma unroll
    for (int p = 0; p < P::PER; ++p) {
      const int i = tid + p * kBP, r = i / P::Q, c = 4 * (i % P::Q);
      if (i < P::TOT) *reinterpret_cast<f32x4*>(&sK[r][c]) = r < n ? sb[r] * pv.v[p] : kZero4;
    }
  }
  // W = X (beta K~): 16 x 16 tiles over the waves
  constexpr int TW = (CM / 16) * (DK / 16);
  for (int t = wv; t < TW; t += NW) {
    const int rt = t / (DK / 16), ct = t % (DK / 16);
    if (16 * rt >= n) continue;
    const f32x4 acc = mma_tile(kZero4, n4, [&](int i, int kx) { return sX[16 * rt + i][kx]; },
                               [&](int kx, int j) { return sQ[kx][16 * ct + j]; });
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int row = 16 * rt + r4 + e;
      if (row < n) blk[L::oW + (long)row * DK + 16 * ct + l16] = acc[e];
    }
  }
  __syncthreads();
  // U' = X (beta V^)
  constexpr int TU = (CM / 16) * (DV / 16);
  for (int t = wv; t < TU; t += NW) {
    const int rt = t / (DV / 16), ct = t % (DV / 16);
    if (16 * rt >= n) continue;
    const f32x4 acc = mma_tile(kZero4, n4, [&](int i, int kx) { return sX[16 * rt + i][kx]; },
                               [&](int kx, int j) { return sK[kx][16 * ct + j]; });
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int row = 16 * rt + r4 + e;
      if (row < n) blk[L::oU + (long)row * DV + 16 * ct + l16] = acc[e];
    }
  }
}

template <int DV, int W>
constexpr int bw_dvb() {
  return DV < W ? DV : W;
}

// Column-block widths of the two chains, measured on MI355X at T = 4096, 96
// heads of 128 x 128: the state chain takes 507 us with 16 columns against
// 557 with 32 and 793 with 64; the reverse chain 1007 us with 32 against
// 1207 with 16 and 1632 with 64.
constexpr int kStateChainW = 16, kReverseChainW = 32;
// threads of the reverse chain's workgroups: sixteen waves, one state tile
// each, so a chunk's latency-bound step is short (measured at T = 4096, 96
// heads of 128 x 128: 851 us against 946 with eight waves and 1008 with four;
// the results are the same bit for bit)
constexpr int kRevNT = 1024;
// threads of the state chain's workgroups: four waves (measured at T = 4096,
// 96 heads of 128 x 128: 509 us against 600 with eight waves and 587 with
// sixteen; a 16-column block holds only eight 16 x 16 state tiles, so more
// waves sit idle for most of a step and only add to its barriers' cost)
constexpr int kStateNT = 256;

// Tiling of a chain: a workgroup holds a DK x DVB block of the state (or of
// its gradient) as 16 x 16 MFMA accumulators, tile t = w + 4 m of wave w; the
// token-row blocks (U, dU, dO) are CM x DVB.
template <int DK, int DV, int W, int NW = 4>
struct ChainTiles {
  static constexpr int DVB = bw_dvb<DV, W>(), NB = DV / DVB, NCT = DVB / 16;
  static constexpr int SPB = DVB + 4, SPO = (DK > CM ? DK : CM) + 4;
  static constexpr int NST = (DK / 16) * NCT, SPW = (NST + NW - 1) / NW;
  static constexpr int NUT = (CM / 16) * NCT, UPW = (NUT + NW - 1) / NW;
};

// Workgroup L -> (column block cbk, sequence-head bh). Workgroups are dealt
// to the 8 XCDs in turn; when the sequence-head count allows, the NB column
// blocks of one sequence-head go to the same XCD, so the operands they share
// (W, K^d, Q~, P) are fetched into that XCD's L2 once.
__device__ __forceinline__ void chain_map(int L, int NB, int BH, int& cbk, int& bh) {
  if (BH % 8 == 0) {
    const int xcd = L % 8, s = L / 8;
    cbk = s % NB;
    bh = (s / NB) * 8 + xcd;
  } else {
    cbk = L % NB;
    bh = L / NB;
  }
}

// ---- 2. forward state chain: entering state of every chunk, U ---------------
// One workgroup per (16-column block, head, sequence). Per chunk: keep S,
// U = U' - W S (over U' in the scratch), S = Diag(e^{Gam_n}) S + K^d^T U.
template <int DK, int DV>
__global__ __launch_bounds__(kStateNT) void bw_state_chain_kernel(BackwardArgs a) {
  using L = BwL<DK, DV>;
  constexpr int NW = kStateNT / kWave;
  using CT = ChainTiles<DK, DV, kStateChainW, NW>;
  constexpr int NCT = CT::NCT, SPW = CT::SPW, UPW = CT::UPW, NST = CT::NST, NUT = CT::NUT;
  __shared__ float sS[DK][CT::SPB];
  __shared__ float sU[CM][CT::SPB];
  __shared__ __attribute__((aligned(16))) float sO[CM][CT::SPO];
  __shared__ __attribute__((aligned(16))) float sEn[DK];
  const int BH = a.B * a.H, c0 = a.c0, c1 = a.c1;
  int cbk, bh;
  chain_map(blockIdx.x, CT::NB, BH, cbk, bh);
  const int cb0 = cbk * CT::DVB;
  const int tid = threadIdx.x, lane = tid % kWave, wv = tid / kWave;
  const int l16 = lane % 16, r4 = 4 * (lane / 16);
  f32x4 accS[SPW];
#pragma unroll
  for (int m = 0; m < SPW; ++m) {
    const int t = wv + NW * m, rt = t / NCT, ct = t % NCT;
#pragma unroll
    for (int e = 0; e < 4; ++e)
      accS[m][e] = (t < NST && a.S0)
                       ? a.S0[((long)bh * DK + 16 * rt + r4 + e) * DV + cb0 + 16 * ct + l16]
                       : 0.f;
  }
  // operands of a chunk: W, then K^d (through one register set), e^{Gam_n}
  auto blk_of = [&](int c) { return a.scratch + ((long)(c - c0) * BH + bh) * L::n; };
  auto n_of = [&](int c) { return min(a.chunk, a.T - c * a.chunk); };
  Pieces<kStateNT, CM, DK> pk;
  Pieces<kStateNT, 1, DK> pe;
  if (c0 < c1) {
    const float* b0 = blk_of(c0);
    get_rows(pk, n_of(c0), [&](int r, int cx) { return ld4f(b0 + L::oW + r * DK + cx); });
    get_rows(pe, 1, [&](int, int cx) { return ld4f(b0 + L::oEn + cx); });
  }
  for (int c = c0; c < c1; ++c) {
    const int n = n_of(c), n4 = (n + 3) & ~3;
    float* blk = blk_of(c);
    float* Sk = a.S0s + ((long)(c - c0) * BH + bh) * DK * DV;
    __syncthreads();  // the previous chunk is done with sS, sU, sO, sEn
#pragma unroll
    for (int m = 0; m < SPW; ++m) {
      const int t = wv + NW * m, rt = t / NCT, ct = t % NCT;
      if (t < NST) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int row = 16 * rt + r4 + e, col = 16 * ct + l16;
          Sk[(long)row * DV + cb0 + col] = accS[m][e];
          sS[row][col] = accS[m][e];
        }
      }
    }
    put_rows<CT::SPO>(pk, &sO[0][0]);  // W
    put_rows<DK>(pe, sEn);
    get_rows(pk, n, [&](int r, int cx) { return ld4f(blk + L::oKd + r * DK + cx); });
    float up[UPW][4];  // U' of this thread's elements, loaded before the products
#pragma unroll
    for (int m = 0; m < UPW; ++m) {
      const int t = wv + NW * m, rt = t / NCT, ct = t % NCT;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int row = 16 * rt + r4 + e, col = 16 * ct + l16;
        up[m][e] = (t < NUT && row < n) ? blk[L::oU + (long)row * DV + cb0 + col] : 0.f;
      }
    }
    __syncthreads();
#pragma unroll
    for (int m = 0; m < UPW; ++m) {  // U = U' - W S
      const int t = wv + NW * m, rt = t / NCT, ct = t % NCT;
      if (t < NUT) {
        const f32x4 ws = mma_tile(kZero4, DK, [&](int i, int kx) { return sO[16 * rt + i][kx]; },
                                  [&](int kx, int j) { return sS[kx][16 * ct + j]; });
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int row = 16 * rt + r4 + e, col = 16 * ct + l16;
          const float u = row < n ? up[m][e] - ws[e] : 0.f;
          if (row < n) blk[L::oU + (long)row * DV + cb0 + col] = u;
          sU[row][col] = u;
        }
      }
    }
    __syncthreads();
    put_rows<CT::SPO>(pk, &sO[0][0]);  // K^d
    if (c + 1 < c1) {
      const float* bn = blk_of(c + 1);
      get_rows(pk, n_of(c + 1), [&](int r, int cx) { return ld4f(bn + L::oW + r * DK + cx); });
      get_rows(pe, 1, [&](int, int cx) { return ld4f(bn + L::oEn + cx); });
    }
    __syncthreads();
#pragma unroll
    for (int m = 0; m < SPW; ++m) {  // S = Diag(e^{Gam_n}) S + K^d^T U
      const int t = wv + NW * m, rt = t / NCT, ct = t % NCT;
      if (t < NST) {
#pragma unroll
        for (int e = 0; e < 4; ++e) accS[m][e] *= sEn[16 * rt + r4 + e];
        accS[m] = mma_tile(accS[m], n4, [&](int i, int kx) { return sO[kx][16 * rt + i]; },
                           [&](int kx, int j) { return sU[kx][16 * ct + j]; });
      }
    }
  }
  if (a.S_out) {  // the state leaving chunk c1 - 1: where the next chunk range starts
#pragma unroll
    for (int m = 0; m < SPW; ++m) {
      const int t = wv + NW * m, rt = t / NCT, ct = t % NCT;
      if (t < NST) {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          a.S_out[((long)bh * DK + 16 * rt + r4 + e) * DV + cb0 + 16 * ct + l16] = accS[m][e];
      }
    }
  }
}

// ---- 3. reverse chain: dS1 of every chunk, dU, and dS0 ----------------------
// Same grid and tiling as the state chain, chunks from the last to the
// first; one staging buffer holds P, K^d, Q~ and W in turn.
template <int DK, int DV, typename IO>
__global__ __launch_bounds__(kRevNT) void bw_reverse_chain_kernel(BackwardArgs a) {
  using L = BwL<DK, DV>;
  constexpr int NW = kRevNT / kWave;
  using CT = ChainTiles<DK, DV, kReverseChainW, NW>;
  constexpr int NCT = CT::NCT, SPW = CT::SPW, UPW = CT::UPW, NST = CT::NST, NUT = CT::NUT;
  constexpr int DVB = CT::DVB;
  __shared__ float sdS[DK][CT::SPB];
  __shared__ __attribute__((aligned(16))) float sdO[CM][CT::SPB];
  __shared__ float sdU[CM][CT::SPB];
  __shared__ __attribute__((aligned(16))) float sO[CM][CT::SPO];
  __shared__ __attribute__((aligned(16))) float sEn[DK];
  const int BH = a.B * a.H, c0 = a.c0, c1 = a.c1;
  int cbk, bh;
  chain_map(blockIdx.x, CT::NB, BH, cbk, bh);
  const int cb0 = cbk * DVB, b = bh / a.H, h = bh % a.H;
  const int tid = threadIdx.x, lane = tid % kWave, wv = tid / kWave;
  const int l16 = lane % 16, r4 = 4 * (lane / 16);
  const IO* dO = static_cast<const IO*>(a.dO);
  f32x4 accS[SPW];
#pragma unroll
  for (int m = 0; m < SPW; ++m) {
    const int t = wv + NW * m, rt = t / NCT, ct = t % NCT;
#pragma unroll
    for (int e = 0; e < 4; ++e)
      accS[m][e] = (t < NST && a.dST)
                       ? a.dST[((long)bh * DK + 16 * rt + r4 + e) * DV + cb0 + 16 * ct + l16]
                       : 0.f;
  }
  // Operands of a chunk, through register sets loaded one stage ahead: P,
  // dO and e^{Gam_n} (prefetched during the previous chunk's last stage),
  // then K^d, Q~ and W in turn through one set. Rows at or past the chunk's
  // last token are zeros (P is zero right of its diagonal, so its columns
  // past the last token are zero as stored).
  auto blk_of = [&](int c) { return a.scratch + ((long)(c - c0) * BH + bh) * L::n; };
  auto n_of = [&](int c) { return min(a.chunk, a.T - c * a.chunk); };
  Pieces<kRevNT, CM, CM> pp;
  Pieces<kRevNT, CM, DVB> pd;
  Pieces<kRevNT, 1, DK> pe;
  Pieces<kRevNT, CM, DK> pk;
  auto get_first = [&](int c) {  // P, dO, e^{Gam_n} of chunk c
    const float* bc = blk_of(c);
    const int nn = n_of(c);
    const long drow0 = tok(a, b, c * a.chunk, h);
    get_rows(pp, nn, [&](int r, int cx) { return ld4f(bc + L::oP + r * CM + cx); });
    get_rows(pd, nn, [&](int r, int cx) { return ld4f(dO + (drow0 + (long)r * a.H) * DV + cb0 + cx); });
    get_rows(pe, 1, [&](int, int cx) { return ld4f(bc + L::oEn + cx); });
  };
  if (c1 > c0) get_first(c1 - 1);
  for (int c = c1 - 1; c >= c0; --c) {
    const int n = n_of(c), n4 = (n + 3) & ~3;
    float* blk = blk_of(c);
    float* dSk = a.dS1s + ((long)(c - c0) * BH + bh) * DK * DV;
    auto get_k = [&](long off) {
      get_rows(pk, n, [&](int r, int cx) { return ld4f(blk + off + r * DK + cx); });
    };
    __syncthreads();  // the previous chunk is done with every buffer
#pragma unroll
    for (int m = 0; m < SPW; ++m) {
      const int t = wv + NW * m, rt = t / NCT, ct = t % NCT;
      if (t < NST) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int row = 16 * rt + r4 + e, col = 16 * ct + l16;
          dSk[(long)row * DV + cb0 + col] = accS[m][e];
          sdS[row][col] = accS[m][e];
        }
      }
    }
    put_rows<CT::SPO>(pp, &sO[0][0]);
    put_rows<CT::SPB>(pd, &sdO[0][0]);
    put_rows<DK>(pe, sEn);
    get_k(L::oKd);
    __syncthreads();
    f32x4 accU[UPW];
#pragma unroll
    for (int m = 0; m < UPW; ++m) {  // P^T dO
      const int t = wv + NW * m, rt = t / NCT, ct = t % NCT;
      accU[m] = kZero4;
      if (t < NUT)
        accU[m] = mma_tile(kZero4, n4, [&](int i, int kx) { return sO[kx][16 * rt + i]; },
                           [&](int kx, int j) { return sdO[kx][16 * ct + j]; });
    }
    __syncthreads();
    put_rows<CT::SPO>(pk, &sO[0][0]);  // K^d
    get_k(L::oQt);
    __syncthreads();
#pragma unroll
    for (int m = 0; m < UPW; ++m) {  // + K^d dS
      const int t = wv + NW * m, rt = t / NCT, ct = t % NCT;
      if (t < NUT) {
        accU[m] = mma_tile(accU[m], DK, [&](int i, int kx) { return sO[16 * rt + i][kx]; },
                           [&](int kx, int j) { return sdS[kx][16 * ct + j]; });
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int row = 16 * rt + r4 + e, col = 16 * ct + l16;
          const float u = row < n ? accU[m][e] : 0.f;
          sdU[row][col] = u;
          if (row < n) blk[L::odU + (long)row * DV + cb0 + col] = u;
        }
      }
    }
    __syncthreads();
    put_rows<CT::SPO>(pk, &sO[0][0]);  // Q~
    get_k(L::oW);
    __syncthreads();
#pragma unroll
    for (int m = 0; m < SPW; ++m) {  // dS = Diag(e^{Gam_n}) dS + Q~^T dO
      const int t = wv + NW * m, rt = t / NCT, ct = t % NCT;
      if (t < NST) {
#pragma unroll
        for (int e = 0; e < 4; ++e) accS[m][e] *= sEn[16 * rt + r4 + e];
        accS[m] = mma_tile(accS[m], n4, [&](int i, int kx) { return sO[kx][16 * rt + i]; },
                           [&](int kx, int j) { return sdO[kx][16 * ct + j]; });
      }
    }
    __syncthreads();
    put_rows<CT::SPO>(pk, &sO[0][0]);  // W
    if (c > c0) get_first(c - 1);
    __syncthreads();
#pragma unroll
    for (int m = 0; m < SPW; ++m) {  // - W^T dU
      const int t = wv + NW * m, rt = t / NCT, ct = t % NCT;
      if (t < NST)
        accS[m] = mma_tile(accS[m], n4, [&](int i, int kx) { return -sO[kx][16 * rt + i]; },
                           [&](int kx, int j) { return sdU[kx][16 * ct + j]; });
    }
  }
  if (a.dS0) {
#pragma unroll
    for (int m = 0; m < SPW; ++m) {
      const int t = wv + NW * m, rt = t / NCT, ct = t % NCT;
      if (t < NST) {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          a.dS0[((long)bh * DK + 16 * rt + r4 + e) * DV + cb0 + 16 * ct + l16] = accS[m][e];
      }
    }
  }
}

// ---- 4. per chunk-head: the products with S0 and dS1, and dP -----------------
// Contractions over d_v in slabs of 32 columns staged in LDS; wave w owns the
// column tiles w, w+4, ... of dQ~, dW and dK^d (all row tiles) and column
// tile w of dP.
template <int DK, int DV, typename IO>
__global__ __launch_bounds__(kBT, 2) void bw_grad_dense_kernel(BackwardArgs a) {
  using L = BwL<DK, DV>;
  constexpr int SL = DV < 32 ? DV : 32, SLP = SL + 4;
  constexpr int CTN = DK / 16, CPW = (CTN + 3) / 4, RT = CM / 16;
  __shared__ __attribute__((aligned(16))) float sS0[DK][SLP], sdS1[DK][SLP];
  __shared__ __attribute__((aligned(16))) float sdO[CM][SLP], sdU[CM][SLP], sU[CM][SLP];
  __shared__ float sdD[DK];
  const Item it = item_of(a, blockIdx.x);
  const int n = it.n;
  float* blk = a.scratch + (long)blockIdx.x * L::n;
  const float* S0 = a.S0s + (long)blockIdx.x * DK * DV;
  const float* dS1 = a.dS1s + (long)blockIdx.x * DK * DV;
  const int tid = threadIdx.x, lane = tid % kWave, wv = tid / kWave;
  const int l16 = lane % 16, r4 = 4 * (lane / 16);
  const IO* dO = static_cast<const IO*>(a.dO);
  const long row0 = tok(a, it.b, it.t0, it.h);
  f32x4 aQ[CPW][RT], aW[CPW][RT], aK[CPW][RT], aP[RT];
#pragma unroll
  for (int m = 0; m < CPW; ++m)
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) aQ[m][rt] = aW[m][rt] = aK[m][rt] = kZero4;
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) aP[rt] = kZero4;
  float dd = 0.f;
  for (int l0 = 0; l0 < DV; l0 += SL) {
    __syncthreads();
    stage_rows<kBT, DK, SL, SLP>(&sS0[0][0], DK,
                                 [&](int r, int c) { return ld4f(S0 + (long)r * DV + l0 + c); });
    stage_rows<kBT, DK, SL, SLP>(&sdS1[0][0], DK,
                                 [&](int r, int c) { return ld4f(dS1 + (long)r * DV + l0 + c); });
    stage_rows<kBT, CM, SL, SLP>(&sdO[0][0], n, [&](int r, int c) {
      return ld4f(dO + (row0 + (long)r * a.H) * DV + l0 + c);
    });
    stage_rows<kBT, CM, SL, SLP>(&sdU[0][0], n,
                                 [&](int r, int c) { return ld4f(blk + L::odU + r * DV + l0 + c); });
    stage_rows<kBT, CM, SL, SLP>(&sU[0][0], n,
                                 [&](int r, int c) { return ld4f(blk + L::oU + r * DV + l0 + c); });
    __syncthreads();
    if (tid < DK)
      for (int j = 0; j < SL; ++j) dd += sS0[tid][j] * sdS1[tid][j];
#pragma unroll
    for (int m = 0; m < CPW; ++m) {
      const int ct = wv + 4 * m;
      if (ct < CTN) {
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
          auto s0t = [&](int kx, int j) { return sS0[16 * ct + j][kx]; };
          aQ[m][rt] = mma_tile(aQ[m][rt], SL, [&](int i, int kx) { return sdO[16 * rt + i][kx]; },
                               s0t);
          aW[m][rt] = mma_tile(aW[m][rt], SL, [&](int i, int kx) { return sdU[16 * rt + i][kx]; },
                               s0t);
          aK[m][rt] = mma_tile(aK[m][rt], SL, [&](int i, int kx) { return sU[16 * rt + i][kx]; },
                               [&](int kx, int j) { return sdS1[16 * ct + j][kx]; });
        }
      }
    }
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
      aP[rt] = mma_tile(aP[rt], SL, [&](int i, int kx) { return sdO[16 * rt + i][kx]; },
                        [&](int kx, int j) { return sU[16 * wv + j][kx]; });
  }
  if (tid < DK) sdD[tid] = dd;
  __syncthreads();
#pragma unroll
  for (int m = 0; m < CPW; ++m) {
    const int ct = wv + 4 * m;
    if (ct >= CTN) continue;
    const int cc = 16 * ct + l16;
    // the tile's operands loaded before its first store, all in flight together
    float vG[RT][4], vkd[RT][4], vqt[RT][4];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int row = 16 * rt + r4 + e;
        const long i = (long)row * DK + cc;
        vG[rt][e] = row < n ? blk[L::oG + i] : 0.f;
        vkd[rt][e] = row < n ? blk[L::oKd + i] : 0.f;
        vqt[rt][e] = row < n ? blk[L::oQt + i] : 0.f;
      }
    const float Gn = blk[L::oG + (long)(n - 1) * DK + cc];
    const float En = blk[L::oEn + cc];
    float col = 0.f;  // sum over the rows of K^d * dK^d in this column
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int row = 16 * rt + r4 + e;
        if (row < n) col += vkd[rt][e] * aK[m][rt][e];
      }
    col += __shfl_xor(col, 16, kWave);
    col += __shfl_xor(col, 32, kWave);
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int row = 16 * rt + r4 + e;
        if (row >= n) continue;
        const long i = (long)row * DK + cc;
        const float G = vG[rt][e], kd = vkd[rt][e], qt = vqt[rt][e];
        const float dq = aQ[m][rt][e], dkd = aK[m][rt][e];
        float dG = qt * dq - kd * dkd;
        if (row == n - 1) dG += col + En * sdD[cc];
        blk[L::odq + i] = __expf(G) * dq;
        blk[L::odk + i] = __expf(Gn - G) * dkd;
        blk[L::odG + i] = dG;
        blk[L::odW + i] = -aW[m][rt][e];
      }
  }
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)  // dP = (dO U^T) on j <= r
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int row = 16 * rt + r4 + e, j = 16 * wv + l16;
      if (row < n) blk[L::odP + row * CM + j] = j <= row ? aP[rt][e] : 0.f;
    }
}

// The same products for bf16 I/O (d_v >= 32), with bf16 MFMA operands as in
// the forward (v_mfma_f32_16x16x32_bf16; fp32 accumulation): each 32-column
// slab of S0, dS1, dO, dU and U is staged in LDS as bf16 rows, and one MFMA
// per output tile and slab takes 8 consecutive elements per lane from two
// 16-byte LDS reads. The row sums of dS1 * S0 are taken in fp32 from the
// values as loaded, before rounding.
template <int DK, int DV>
__global__ __launch_bounds__(kBT, 2) void bw_grad_dense_bf16_kernel(BackwardArgs a) {
  using L = BwL<DK, DV>;
  constexpr int SL = 32, SLB = SL + 8;  // slab width; bf16 row stride (16-byte rows)
  constexpr int CTN = DK / 16, CPW = (CTN + 3) / 4, RT = CM / 16;
  constexpr int Q4 = SL / 4;                  // float4 pieces per slab row
  constexpr int SP = (DK * Q4 + kBT - 1) / kBT;  // S0 / dS1 pieces per thread
  constexpr int TP = (CM * Q4 + kBT - 1) / kBT;  // dO / dU / U pieces per thread
  static_assert(DV % SL == 0 && kBT % Q4 == 0, "dense bf16 tiling");
  __shared__ __attribute__((aligned(16))) bf16 sS0[DK][SLB], sdS1[DK][SLB];
  __shared__ __attribute__((aligned(16))) bf16 sdO[CM][SLB], sdU[CM][SLB], sU[CM][SLB];
  __shared__ float sdD[DK];
  const Item it = item_of(a, blockIdx.x);
  const int n = it.n;
  float* blk = a.scratch + (long)blockIdx.x * L::n;
  const float* S0 = a.S0s + (long)blockIdx.x * DK * DV;
  const float* dS1 = a.dS1s + (long)blockIdx.x * DK * DV;
  const int tid = threadIdx.x, lane = tid % kWave, wv = tid / kWave;
  const int l16 = lane % 16, r4 = 4 * (lane / 16), koff = 8 * (lane / 16);
  const bf16* dO = static_cast<const bf16*>(a.dO);
  const long row0 = tok(a, it.b, it.t0, it.h);
  f32x4 aQ[CPW][RT], aW[CPW][RT], aK[CPW][RT], aP[RT];
#pragma unroll
  for (int m = 0; m < CPW; ++m)
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) aQ[m][rt] = aW[m][rt] = aK[m][rt] = kZero4;
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) aP[rt] = kZero4;
  float dd[SP];  // row sums of dS1 * S0 for rows (tid + kBT p) / Q4, in lanes with tid % Q4 == 0
#pragma unroll
  for (int p = 0; p < SP; ++p) dd[p] = 0.f;
  auto cvt = [](f32x4 v) { return bf16x4{(bf16)v[0], (bf16)v[1], (bf16)v[2], (bf16)v[3]}; };
  // A slab's S0 and dS1 pieces are loaded as soon as the previous slab is in
  // LDS, so they are in flight during that slab's products.
  f32x4 vs[SP], vd[SP];
  auto load_state = [&](int l0) {
#pragma unroll
    for (int p = 0; p < SP; ++p) {
      const int idx = tid + kBT * p, r = idx / Q4, c = 4 * (idx % Q4);
      const bool live = idx < DK * Q4;
      vs[p] = live ? ld4f(S0 + (long)r * DV + l0 + c) : kZero4;
      vd[p] = live ? ld4f(dS1 + (long)r * DV + l0 + c) : kZero4;
    }
  };
  load_state(0);
  for (int l0 = 0; l0 < DV; l0 += SL) {
    f32x4 vo[TP], vdu[TP], vu[TP];
#pragma unroll
    for (int p = 0; p < TP; ++p) {
      const int idx = tid + kBT * p, r = idx / Q4, c = 4 * (idx % Q4);
      const bool live = idx < CM * Q4 && r < n;
      vo[p] = live ? ld4f(dO + (row0 + (long)r * a.H) * DV + l0 + c) : kZero4;
      vdu[p] = live ? ld4f(blk + L::odU + r * DV + l0 + c) : kZero4;
      vu[p] = live ? ld4f(blk + L::oU + r * DV + l0 + c) : kZero4;
    }
    __syncthreads();  // the previous slab's products are done with the LDS rows
#pragma unroll
    for (int p = 0; p < SP; ++p) {
      const int idx = tid + kBT * p, r = idx / Q4, c = 4 * (idx % Q4);
      float part = vs[p][0] * vd[p][0] + vs[p][1] * vd[p][1] + vs[p][2] * vd[p][2] +
                   vs[p][3] * vd[p][3];
#pragma unroll
      for (int off = 1; off < Q4; off <<= 1) part += __shfl_xor(part, off, kWave);
      dd[p] += part;
      if (idx < DK * Q4) {
        *reinterpret_cast<bf16x4*>(&sS0[r][c]) = cvt(vs[p]);
        *reinterpret_cast<bf16x4*>(&sdS1[r][c]) = cvt(vd[p]);
      }
    }
#pragma unroll
    for (int p = 0; p < TP; ++p) {
      const int idx = tid + kBT * p, r = idx / Q4, c = 4 * (idx % Q4);
      if (idx < CM * Q4) {
        *reinterpret_cast<bf16x4*>(&sdO[r][c]) = cvt(vo[p]);
        *reinterpret_cast<bf16x4*>(&sdU[r][c]) = cvt(vdu[p]);
        *reinterpret_cast<bf16x4*>(&sU[r][c]) = cvt(vu[p]);
      }
    }
    __syncthreads();
    if (l0 + SL < DV) load_state(l0 + SL);
#pragma unroll
    for (int m = 0; m < CPW; ++m) {
      const int ct = wv + 4 * m;
      if (ct < CTN) {
        const bf16x8 fs0 = *reinterpret_cast<const bf16x8*>(&sS0[16 * ct + l16][koff]);
        const bf16x8 fds1 = *reinterpret_cast<const bf16x8*>(&sdS1[16 * ct + l16][koff]);
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
          const bf16x8 fo = *reinterpret_cast<const bf16x8*>(&sdO[16 * rt + l16][koff]);
          const bf16x8 fdu = *reinterpret_cast<const bf16x8*>(&sdU[16 * rt + l16][koff]);
          const bf16x8 fu = *reinterpret_cast<const bf16x8*>(&sU[16 * rt + l16][koff]);
          aQ[m][rt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fo, fs0, aQ[m][rt], 0, 0, 0);
          aW[m][rt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fdu, fs0, aW[m][rt], 0, 0, 0);
          aK[m][rt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fu, fds1, aK[m][rt], 0, 0, 0);
        }
      }
    }
    {
      const bf16x8 fuj = *reinterpret_cast<const bf16x8*>(&sU[16 * wv + l16][koff]);
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        const bf16x8 fo = *reinterpret_cast<const bf16x8*>(&sdO[16 * rt + l16][koff]);
        aP[rt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fo, fuj, aP[rt], 0, 0, 0);
      }
    }
  }
#pragma unroll
  for (int p = 0; p < SP; ++p)
    if (tid % Q4 == 0 && tid + kBT * p < DK * Q4) sdD[(tid + kBT * p) / Q4] = dd[p];
  __syncthreads();
#pragma unroll
  for (int m = 0; m < CPW; ++m) {
    const int ct = wv + 4 * m;
    if (ct >= CTN) continue;
    const int cc = 16 * ct + l16;
    // the tile's operands loaded before its first store, all in flight together
    float vG[RT][4], vkd[RT][4], vqt[RT][4];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int row = 16 * rt + r4 + e;
        const long i = (long)row * DK + cc;
        vG[rt][e] = row < n ? blk[L::oG + i] : 0.f;
        vkd[rt][e] = row < n ? blk[L::oKd + i] : 0.f;
        vqt[rt][e] = row < n ? blk[L::oQt + i] : 0.f;
      }
    const float Gn = blk[L::oG + (long)(n - 1) * DK + cc];
    const float En = blk[L::oEn + cc];
    float col = 0.f;  // sum over the rows of K^d * dK^d in this column
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int row = 16 * rt + r4 + e;
        if (row < n) col += vkd[rt][e] * aK[m][rt][e];
      }
    col += __shfl_xor(col, 16, kWave);
    col += __shfl_xor(col, 32, kWave);
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int row = 16 * rt + r4 + e;
        if (row >= n) continue;
        const long i = (long)row * DK + cc;
        const float G = vG[rt][e], kd = vkd[rt][e], qt = vqt[rt][e];
        const float dq = aQ[m][rt][e], dkd = aK[m][rt][e];
        float dG = qt * dq - kd * dkd;
        if (row == n - 1) dG += col + En * sdD[cc];
        blk[L::odq + i] = __expf(G) * dq;
        blk[L::odk + i] = __expf(Gn - G) * dkd;
        blk[L::odG + i] = dG;
        blk[L::odW + i] = -aW[m][rt][e];
      }
  }
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)  // dP = (dO U^T) on j <= r
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int row = 16 * rt + r4 + e, j = 16 * wv + l16;
      if (row < n) blk[L::odP + row * CM + j] = j <= row ? aP[rt][e] : 0.f;
    }
}

// ---- 5. per chunk-head: through W, U' and the inverse; dv and dbeta --------
// LDS holds X and, in a first phase, dW, dU, K~, V^; in a second phase the
// same space holds dX and T1 = dX X^T.
template <int DK, int DV, typename IO>
__global__ __launch_bounds__(kBS) void bw_grad_solve_kernel(BackwardArgs a) {
  using L = BwL<DK, DV>;
  constexpr int PX = CM + 4, PK = DK + 4, PV = DV + 4, RT = CM / 16, NW = kBS / kWave;
  constexpr int XPW = RT * RT / NW;  // C x C tiles per wave
  constexpr int PH1 = 2 * CM * PK + 2 * CM * PV, PH2 = 2 * CM * PX;
  __shared__ __attribute__((aligned(16))) float sX[CM][PX];
  __shared__ __attribute__((aligned(16))) float sBuf[PH1 > PH2 ? PH1 : PH2];
  // dbeta partials, one slot per (product, column tile), summed in a fixed
  // order at the end (deterministic, unlike float atomics)
  constexpr int SY = 0, SZ = DK / 16, SM = SZ + DV / 16, NSLOT = SM + RT;
  __shared__ float sbt[CM], sdb[NSLOT][CM];
  float(*sdW)[PK] = reinterpret_cast<float(*)[PK]>(sBuf);
  float(*sKt)[PK] = reinterpret_cast<float(*)[PK]>(sBuf + CM * PK);
  float(*sdU)[PV] = reinterpret_cast<float(*)[PV]>(sBuf + 2 * CM * PK);
  float(*sV)[PV] = reinterpret_cast<float(*)[PV]>(sBuf + 2 * CM * PK + CM * PV);
  float(*sdX)[PX] = reinterpret_cast<float(*)[PX]>(sBuf);
  float(*sT)[PX] = reinterpret_cast<float(*)[PX]>(sBuf + CM * PX);
  const Item it = item_of(a, blockIdx.x);
  const int n = it.n, n4 = (n + 3) & ~3;
  float* blk = a.scratch + (long)blockIdx.x * L::n;
  const int tid = threadIdx.x, lane = tid % kWave, wv = tid / kWave;
  const int l16 = lane % 16, r4 = 4 * (lane / 16);
  const IO* v = static_cast<const IO*>(a.v);
  IO* dv = static_cast<IO*>(a.dv);
  const long row0 = tok(a, it.b, it.t0, it.h);
  stage_rows<kBS, CM, CM, PX>(&sX[0][0], n, [&](int r, int c) { return ld4f(blk + L::oX + r * CM + c); });
  stage_rows<kBS, CM, DK, PK>(&sdW[0][0], n, [&](int r, int c) { return ld4f(blk + L::odW + r * DK + c); });
  stage_rows<kBS, CM, DK, PK>(&sKt[0][0], n, [&](int r, int c) { return ld4f(blk + L::oKt + r * DK + c); });
  stage_rows<kBS, CM, DV, PV>(&sdU[0][0], n, [&](int r, int c) { return ld4f(blk + L::odU + r * DV + c); });
  stage_rows<kBS, CM, DV, PV>(&sV[0][0], n, [&](int r, int c) {
    return ld4f(v + (row0 + (long)r * a.H) * DV + c);
  });
  if (tid < CM) sbt[tid] = tid < n ? a.beta[tok(a, it.b, it.t0 + tid, it.h)] : 0.f;
  for (int i = tid; i < NSLOT * CM; i += kBS) sdb[i / CM][i % CM] = 0.f;
  __syncthreads();
  // Y = X^T dW: dk^ += e^Gam beta Y, dGam += K~ beta Y, dbeta += K~ . Y
  // Each tile's dk^, dGam partials and Gam are loaded one tile ahead, before
  // the stores of the tile before it.
  constexpr int TY = RT * (DK / 16);
  auto load_y = [&](int t, float* pk, float* pg, float* gg) {
    const int rt = t % RT, ct = t / RT;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int row = 16 * rt + r4 + e;
      const bool live = t < TY && row < n;
      const long o = (long)row * DK + 16 * ct + l16;
      pk[e] = live ? blk[L::odk + o] : 0.f;
      pg[e] = live ? blk[L::odG + o] : 0.f;
      gg[e] = live ? blk[L::oG + o] : 0.f;
    }
  };
  float pk[4], pg[4], gg[4];
  load_y(wv, pk, pg, gg);
  for (int t = wv; t < TY; t += NW) {
    const int rt = t % RT, ct = t / RT;
    float nk[4], ng[4], ngg[4];
    load_y(t + NW, nk, ng, ngg);
    if (16 * rt < n) {
      const f32x4 y = mma_tile(kZero4, n4, [&](int i, int kx) { return sX[kx][16 * rt + i]; },
                               [&](int kx, int j) { return sdW[kx][16 * ct + j]; });
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int row = 16 * rt + r4 + e, cc = 16 * ct + l16;
        float part = 0.f;
        if (row < n) {
          const long o = (long)row * DK + cc;
          const float br = sbt[row], kt = sKt[row][cc];
          blk[L::odk + o] = pk[e] + __expf(gg[e]) * br * y[e];
          blk[L::odG + o] = pg[e] + kt * br * y[e];
          part = kt * y[e];
        }
        part = sum16(part);
        if (l16 == 0 && row < n) sdb[SY + ct][row] = part;
      }
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      pk[e] = nk[e];
      pg[e] = ng[e];
      gg[e] = ngg[e];
    }
  }
  // Z = X^T dU: dv^ = beta Z, dbeta += V^ . Z
  for (int t = wv; t < RT * (DV / 16); t += NW) {
    const int rt = t % RT, ct = t / RT;
    if (16 * rt >= n) continue;
    const f32x4 z = mma_tile(kZero4, n4, [&](int i, int kx) { return sX[kx][16 * rt + i]; },
                             [&](int kx, int j) { return sdU[kx][16 * ct + j]; });
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int row = 16 * rt + r4 + e, l = 16 * ct + l16;
      float part = 0.f;
      if (row < n) {
        dv[tok(a, it.b, it.t0 + row, it.h) * DV + l] = from_f32<IO>(sbt[row] * z[e]);
        part = sV[row][l] * z[e];
      }
      part = sum16(part);
      if (l16 == 0 && row < n) sdb[SZ + ct][row] = part;
    }
  }
  // dX = (dW K~^T + dU V^^T) diag(beta), strictly lower; C x C tile
  // u = w + NW m of wave w is (row tile u / RT, column tile u % RT)
  f32x4 aX[XPW];
#pragma unroll
  for (int m = 0; m < XPW; ++m) {
    const int u = wv + NW * m, rt = u / RT, ct = u % RT;
    f32x4 acc = kZero4;
    if (16 * rt < n) {
      acc = mma_tile(acc, DK, [&](int i, int kx) { return sdW[16 * rt + i][kx]; },
                     [&](int kx, int j) { return sKt[16 * ct + j][kx]; });
      acc = mma_tile(acc, DV, [&](int i, int kx) { return sdU[16 * rt + i][kx]; },
                     [&](int kx, int j) { return sV[16 * ct + j][kx]; });
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int row = 16 * rt + r4 + e, col = 16 * ct + l16;
      acc[e] = col < row ? sbt[col] * acc[e] : 0.f;
    }
    aX[m] = acc;
  }
  __syncthreads();  // phase-1 operands are dead from here
#pragma unroll
  for (int m = 0; m < XPW; ++m) {
    const int u = wv + NW * m, rt = u / RT, ct = u % RT;
#pragma unroll
    for (int e = 0; e < 4; ++e) sdX[16 * rt + r4 + e][16 * ct + l16] = aX[m][e];
  }
  __syncthreads();
  // A for dbeta below, loaded before the first store of dA
  float vA[XPW][4];
#pragma unroll
  for (int m = 0; m < XPW; ++m) {
    const int u = wv + NW * m, rt = u / RT, ct = u % RT;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int row = 16 * rt + r4 + e, j = 16 * ct + l16;
      vA[m][e] = row < n && j < row ? blk[L::oA + row * CM + j] : 0.f;
    }
  }
  // T1 = dX X^T
#pragma unroll
  for (int m = 0; m < XPW; ++m) {
    const int u = wv + NW * m, rt = u / RT, ct = u % RT;
    f32x4 acc = kZero4;
    if (16 * rt < n)
      acc = mma_tile(acc, n4, [&](int i, int kx) { return sdX[16 * rt + i][kx]; },
                     [&](int kx, int j) { return sX[16 * ct + j][kx]; });
#pragma unroll
    for (int e = 0; e < 4; ++e) sT[16 * rt + r4 + e][16 * ct + l16] = acc[e];
  }
  __syncthreads();
  // dM = -X^T T1 (strictly lower): dA = beta dM, dbeta += A . dM
#pragma unroll
  for (int m = 0; m < XPW; ++m) {
    const int u = wv + NW * m, rt = u / RT, ct = u % RT;
    if (16 * rt >= n) continue;
    const f32x4 acc = mma_tile(kZero4, n4, [&](int i, int kx) { return sX[kx][16 * rt + i]; },
                               [&](int kx, int j) { return sT[kx][16 * ct + j]; });
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int row = 16 * rt + r4 + e, j = 16 * ct + l16;
      float part = 0.f;
      if (row < n) {
        const float dm = j < row ? -acc[e] : 0.f;
        blk[L::odA + row * CM + j] = sbt[row] * dm;
        part = j < row ? vA[m][e] * dm : 0.f;
      }
      part = sum16(part);
      if (l16 == 0 && row < n) sdb[SM + ct][row] = part;
    }
  }
  __syncthreads();
  if (tid < n) {
    float db = 0.f;
    for (int sl = 0; sl < NSLOT; ++sl) db += sdb[sl][tid];
    a.dbeta[tok(a, it.b, it.t0 + tid, it.h)] = db;
  }
}

// The same for bf16 I/O with a third of the LDS, so that two workgroups share
// a CU: dW and K~, then dU and V^, are held as bf16 rows (the operand
// rounding of the forward), in two phases through one buffer; X, dX and T1
// stay fp32. The products are the fp32 MFMAs of the kernel above on the
// rounded values, in the same order.
template <int DK, int DV>
__global__ __launch_bounds__(kBS, 2) void bw_grad_solve_bf16_kernel(BackwardArgs a) {
  using L = BwL<DK, DV>;
  constexpr int PX = CM + 4, PW = (DK > DV ? DK : DV) + 4, RT = CM / 16, NW = kBS / kWave;
  constexpr int XPW = RT * RT / NW;  // C x C tiles per wave
  constexpr int PH1 = 2 * CM * PW * 2, PH2 = 2 * CM * PX * 4;  // bytes
  __shared__ __attribute__((aligned(16))) float sX[CM][PX];
  __shared__ __attribute__((aligned(16))) uint8_t sBuf[PH1 > PH2 ? PH1 : PH2];
  constexpr int SY = 0, SZ = DK / 16, SM = SZ + DV / 16, NSLOT = SM + RT;
  __shared__ float sbt[CM], sdb[NSLOT][CM];
  bf16(*sA)[PW] = reinterpret_cast<bf16(*)[PW]>(sBuf);                   // dW, then dU
  bf16(*sB)[PW] = reinterpret_cast<bf16(*)[PW]>(sBuf + CM * PW * 2);     // K~, then V^
  float(*sdX)[PX] = reinterpret_cast<float(*)[PX]>(sBuf);
  float(*sT)[PX] = reinterpret_cast<float(*)[PX]>(sBuf + CM * PX * 4);
  const Item it = item_of(a, blockIdx.x);
  const int n = it.n, n4 = (n + 3) & ~3;
  float* blk = a.scratch + (long)blockIdx.x * L::n;
  const int tid = threadIdx.x, lane = tid % kWave, wv = tid / kWave;
  const int l16 = lane % 16, r4 = 4 * (lane / 16);
  const bf16* v = static_cast<const bf16*>(a.v);
  bf16* dv = static_cast<bf16*>(a.dv);
  const long row0 = tok(a, it.b, it.t0, it.h);
  {
    Pieces<kBS, CM, DK> pw, pk;
    get_rows(pw, n, [&](int r, int c) { return ld4f(blk + L::odW + r * DK + c); });
    get_rows(pk, n, [&](int r, int c) { return ld4f(blk + L::oKt + r * DK + c); });
    stage_rows<kBS, CM, CM, PX>(&sX[0][0], n, [&](int r, int c) { return ld4f(blk + L::oX + r * CM + c); });
    put_rows_bf16<PW>(pw, &sA[0][0]);
    put_rows_bf16<PW>(pk, &sB[0][0]);
  }
  if (tid < CM) sbt[tid] = tid < n ? a.beta[tok(a, it.b, it.t0 + tid, it.h)] : 0.f;
  for (int i = tid; i < NSLOT * CM; i += kBS) sdb[i / CM][i % CM] = 0.f;
  // dU and V^ for the second phase, loaded now and written to LDS after it
  Pieces<kBS, CM, DV> pu, pv;
  get_rows(pu, n, [&](int r, int c) { return ld4f(blk + L::odU + r * DV + c); });
  get_rows(pv, n, [&](int r, int c) { return ld4f(v + (row0 + (long)r * a.H) * DV + c); });
  __syncthreads();
  // Y = X^T dW: dk^ += e^Gam beta Y, dGam += K~ beta Y, dbeta += K~ . Y
  // Each tile's dk^, dGam partials and Gam are loaded one tile ahead, before
  // the stores of the tile before it.
  constexpr int TY = RT * (DK / 16);
  auto load_y = [&](int t, float* pk, float* pg, float* gg) {
    const int rt = t % RT, ct = t / RT;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int row = 16 * rt + r4 + e;
      const bool live = t < TY && row < n;
      const long o = (long)row * DK + 16 * ct + l16;
      pk[e] = live ? blk[L::odk + o] : 0.f;
      pg[e] = live ? blk[L::odG + o] : 0.f;
      gg[e] = live ? blk[L::oG + o] : 0.f;
    }
  };
  float pk[4], pg[4], gg[4];
  load_y(wv, pk, pg, gg);
  for (int t = wv; t < TY; t += NW) {
    const int rt = t % RT, ct = t / RT;
    float nk[4], ng[4], ngg[4];
    load_y(t + NW, nk, ng, ngg);
    if (16 * rt < n) {
      const f32x4 y = mma_tile(kZero4, n4, [&](int i, int kx) { return sX[kx][16 * rt + i]; },
                               [&](int kx, int j) { return (float)sA[kx][16 * ct + j]; });
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int row = 16 * rt + r4 + e, cc = 16 * ct + l16;
        float part = 0.f;
        if (row < n) {
          const long o = (long)row * DK + cc;
          const float br = sbt[row], kt = (float)sB[row][cc];
          blk[L::odk + o] = pk[e] + __expf(gg[e]) * br * y[e];
          blk[L::odG + o] = pg[e] + kt * br * y[e];
          part = kt * y[e];
        }
        part = sum16(part);
        if (l16 == 0 && row < n) sdb[SY + ct][row] = part;
      }
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      pk[e] = nk[e];
      pg[e] = ng[e];
      gg[e] = ngg[e];
    }
  }
  // dX = (dW K~^T + dU V^^T) diag(beta), strictly lower: the dW K~^T part
  f32x4 aX[XPW];
#pragma unroll
  for (int m = 0; m < XPW; ++m) {
    const int u = wv + NW * m, rt = u / RT, ct = u % RT;
    aX[m] = kZero4;
    if (16 * rt < n)
      aX[m] = mma_tile(aX[m], DK, [&](int i, int kx) { return (float)sA[16 * rt + i][kx]; },
                       [&](int kx, int j) { return (float)sB[16 * ct + j][kx]; });
  }
  __syncthreads();  // dW and K~ are dead from here
  put_rows_bf16<PW>(pu, &sA[0][0]);
  put_rows_bf16<PW>(pv, &sB[0][0]);
  __syncthreads();
  // Z = X^T dU: dv^ = beta Z, dbeta += V^ . Z
  for (int t = wv; t < RT * (DV / 16); t += NW) {
    const int rt = t % RT, ct = t / RT;
    if (16 * rt >= n) continue;
    const f32x4 z = mma_tile(kZero4, n4, [&](int i, int kx) { return sX[kx][16 * rt + i]; },
                             [&](int kx, int j) { return (float)sA[kx][16 * ct + j]; });
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int row = 16 * rt + r4 + e, l = 16 * ct + l16;
      float part = 0.f;
      if (row < n) {
        dv[tok(a, it.b, it.t0 + row, it.h) * DV + l] = (bf16)(sbt[row] * z[e]);
        part = (float)sB[row][l] * z[e];
      }
      part = sum16(part);
      if (l16 == 0 && row < n) sdb[SZ + ct][row] = part;
    }
  }
#pragma unroll
  for (int m = 0; m < XPW; ++m) {  // + dU V^^T, then diag(beta) on the strict lower part
    const int u = wv + NW * m, rt = u / RT, ct = u % RT;
    f32x4 acc = aX[m];
    if (16 * rt < n)
      acc = mma_tile(acc, DV, [&](int i, int kx) { return (float)sA[16 * rt + i][kx]; },
                     [&](int kx, int j) { return (float)sB[16 * ct + j][kx]; });
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int row = 16 * rt + r4 + e, col = 16 * ct + l16;
      acc[e] = col < row ? sbt[col] * acc[e] : 0.f;
    }
    aX[m] = acc;
  }
  __syncthreads();  // dU and V^ are dead from here
#pragma unroll
  for (int m = 0; m < XPW; ++m) {
    const int u = wv + NW * m, rt = u / RT, ct = u % RT;
#pragma unroll
    for (int e = 0; e < 4; ++e) sdX[16 * rt + r4 + e][16 * ct + l16] = aX[m][e];
  }
  __syncthreads();
  // A for dbeta below, loaded before the first store of dA
  float vA[XPW][4];
#pragma unroll
  for (int m = 0; m < XPW; ++m) {
    const int u = wv + NW * m, rt = u / RT, ct = u % RT;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int row = 16 * rt + r4 + e, j = 16 * ct + l16;
      vA[m][e] = row < n && j < row ? blk[L::oA + row * CM + j] : 0.f;
    }
  }
  // T1 = dX X^T
#pragma unroll
  for (int m = 0; m < XPW; ++m) {
    const int u = wv + NW * m, rt = u / RT, ct = u % RT;
    f32x4 acc = kZero4;
    if (16 * rt < n)
      acc = mma_tile(acc, n4, [&](int i, int kx) { return sdX[16 * rt + i][kx]; },
                     [&](int kx, int j) { return sX[16 * ct + j][kx]; });
#pragma unroll
    for (int e = 0; e < 4; ++e) sT[16 * rt + r4 + e][16 * ct + l16] = acc[e];
  }
  __syncthreads();
  // dM = -X^T T1 (strictly lower): dA = beta dM, dbeta += A . dM
#pragma unroll
  for (int m = 0; m < XPW; ++m) {
    const int u = wv + NW * m, rt = u / RT, ct = u % RT;
    if (16 * rt >= n) continue;
    const f32x4 acc = mma_tile(kZero4, n4, [&](int i, int kx) { return sX[kx][16 * rt + i]; },
                               [&](int kx, int j) { return sT[kx][16 * ct + j]; });
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int row = 16 * rt + r4 + e, j = 16 * ct + l16;
      float part = 0.f;
      if (row < n) {
        const float dm = j < row ? -acc[e] : 0.f;
        blk[L::odA + row * CM + j] = sbt[row] * dm;
        part = j < row ? vA[m][e] * dm : 0.f;
      }
      part = sum16(part);
      if (l16 == 0 && row < n) sdb[SM + ct][row] = part;
    }
  }
  __syncthreads();
  if (tid < n) {
    float db = 0.f;
    for (int sl = 0; sl < NSLOT; ++sl) db += sdb[sl][tid];
    a.dbeta[tok(a, it.b, it.t0 + tid, it.h)] = db;
  }
}

// ---- 6. per chunk-head: through the decayed Grams; dq, dk, dg --------------
// Thread (channel c, row group): for each of its rows r the row-side sums
// over j <= r and the column-side sums over r2 >= r of the pair terms, each
// with its own exponential of a non-positive difference.
template <int DK, int DV, typename IO>
__global__ __launch_bounds__(kBP) void bw_grad_gram_kernel(BackwardArgs a) {
  using L = BwL<DK, DV>;
  constexpr int PK = DK + 4, PC = CM + 4, RG = kBP / (DK / 2);
  __shared__ __attribute__((aligned(16))) float sK[CM][PK], sQ[CM][PK], sG[CM][PK];
  // dA and dP, and once the products are done with them, the total dGam
  __shared__ __attribute__((aligned(16))) float sdAP[2 * CM * PC];
  static_assert(CM * PK <= 2 * CM * PC, "dGam fits where dA and dP were");
  float(*sdA)[PC] = reinterpret_cast<float(*)[PC]>(sdAP);
  float(*sdP)[PC] = reinterpret_cast<float(*)[PC]>(sdAP + CM * PC);
  float(*sdG)[PK] = reinterpret_cast<float(*)[PK]>(sdAP);
  const Item it = item_of(a, blockIdx.x);
  const int n = it.n;
  float* blk = a.scratch + (long)blockIdx.x * L::n;
  const int tid = threadIdx.x;
  const IO* q = static_cast<const IO*>(a.q);
  const IO* k = static_cast<const IO*>(a.k);
  IO* dq = static_cast<IO*>(a.dq);
  IO* dk = static_cast<IO*>(a.dk);
  const long row0 = tok(a, it.b, it.t0, it.h);
  {  // every load issued before the first LDS store
    Pieces<kBP, CM, DK> pk, pq, pg;
    Pieces<kBP, CM, CM> pa, pp;
    get_rows(pk, n, [&](int r, int c) { return ld4f(k + (row0 + (long)r * a.H) * DK + c); });
    get_rows(pq, n, [&](int r, int c) { return ld4f(q + (row0 + (long)r * a.H) * DK + c); });
    get_rows(pg, n, [&](int r, int c) { return ld4f(blk + L::oG + r * DK + c); });
    get_rows(pa, n, [&](int r, int c) { return ld4f(blk + L::odA + r * CM + c); });
    get_rows(pp, n, [&](int r, int c) { return ld4f(blk + L::odP + r * CM + c); });
    put_rows<PK>(pk, &sK[0][0]);
    put_rows<PK>(pq, &sQ[0][0]);
    put_rows<PK>(pg, &sG[0][0]);
    put_rows<PC>(pa, &sdA[0][0]);
    put_rows<PC>(pp, &sdP[0][0]);
  }
  __shared__ int sflag;
  __syncthreads();
  if (chunk_factorable<kBP, DK, PK>(sG, n, &sflag)) {
    // With e^{Gam_r - Gam_j} = e^{Gam_r} e^{-Gam_j}, per channel c:
    //   SA = e^{Gam} (dA K-), SP = e^{Gam} (dP K-), TT = e^{-Gam} (dA^T K~ + dP^T Q~)
    // with K- = k^ e^{-Gam}, K~ = k^ e^{Gam}, Q~ = q^ e^{Gam}: fp32 MFMA
    // tiles, the exponentials formed per operand element.
    const int lane = tid % kWave, wv = tid / kWave, l16 = lane % 16, r4 = 4 * (lane / 16);
    const int n4 = (n + 3) & ~3;
    constexpr int NW = kBP / kWave, NT16 = (CM / 16) * (DK / 16), TPW = (NT16 + NW - 1) / NW;
    f32x4 rsv[TPW], rpv[TPW], ctv[TPW];
#pragma unroll
    for (int m = 0; m < TPW; ++m) {
      const int t = wv + NW * m, rt = t / (DK / 16), ct = t % (DK / 16);
      rsv[m] = rpv[m] = ctv[m] = kZero4;
      if (t >= NT16 || 16 * rt >= n) continue;
      const int cb = 16 * ct;
      auto kminus = [&](int kx, int j) { return sK[kx][cb + j] * __expf(-sG[kx][cb + j]); };
      const f32x4 rs = mma_tile(kZero4, n4, [&](int i, int kx) { return sdA[16 * rt + i][kx]; },
                                kminus);
      const f32x4 rp = mma_tile(kZero4, n4, [&](int i, int kx) { return sdP[16 * rt + i][kx]; },
                                kminus);
      f32x4 ct4 = mma_tile(kZero4, n4, [&](int i, int kx) { return sdA[kx][16 * rt + i]; },
                           [&](int kx, int j) { return sK[kx][cb + j] * __expf(sG[kx][cb + j]); });
      ct4 = mma_tile(ct4, n4, [&](int i, int kx) { return sdP[kx][16 * rt + i]; },
                     [&](int kx, int j) { return sQ[kx][cb + j] * __expf(sG[kx][cb + j]); });
      rsv[m] = rs;
      rpv[m] = rp;
      ctv[m] = ct4;
    }
    // the dense parts of dq, dk and dGam loaded before the first store
    float vq[TPW][4], vk[TPW][4], vg[TPW][4];
#pragma unroll
    for (int m = 0; m < TPW; ++m) {
      const int t = wv + NW * m, rt = t / (DK / 16), ct = t % (DK / 16);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = 16 * rt + r4 + e;
        const bool live = t < NT16 && r < n;
        const long i = (long)r * DK + 16 * ct + l16;
        vq[m][e] = live ? blk[L::odq + i] : 0.f;
        vk[m][e] = live ? blk[L::odk + i] : 0.f;
        vg[m][e] = live ? blk[L::odG + i] : 0.f;
      }
    }
    __syncthreads();  // dA and dP are dead from here
#pragma unroll
    for (int m = 0; m < TPW; ++m) {
      const int t = wv + NW * m, rt = t / (DK / 16), ct = t % (DK / 16);
      if (t >= NT16 || 16 * rt >= n) continue;
      const int cb = 16 * ct;
      const f32x4 rs = rsv[m], rp = rpv[m], ct4 = ctv[m];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = 16 * rt + r4 + e, c = cb + l16;
        if (r >= n) continue;
        const float G = sG[r][c], eg = __expf(G);
        const float SA = eg * rs[e], SP = eg * rp[e], TT = ct4[e] * __expf(-G);
        const float kr = sK[r][c], qr = sQ[r][c];
        const long o = tok(a, it.b, it.t0 + r, it.h) * DK + c;
        dq[o] = from_f32<IO>(vq[m][e] + SP);
        dk[o] = from_f32<IO>(vk[m][e] + SA + TT);
        sdG[r][c] = vg[m][e] + (kr * SA + qr * SP - kr * TT);
      }
    }
  } else {
  // two channels per thread (8-byte LDS reads); rows r0, r0 + RG, ...
  constexpr int RPT = (CM + RG - 1) / RG;  // rows per thread
  const int c0 = 2 * (tid % (DK / 2));
  f32x2 SAv[RPT], SPv[RPT], TTv[RPT];
#pragma unroll
  for (int m = 0; m < RPT; ++m) {
    const int r = tid / (DK / 2) + RG * m;
    if (r >= n) continue;
    const f32x2 Gr = *reinterpret_cast<const f32x2*>(&sG[r][c0]);
    const f32x2 kr = *reinterpret_cast<const f32x2*>(&sK[r][c0]);
    const f32x2 qr = *reinterpret_cast<const f32x2*>(&sQ[r][c0]);
    f32x2 SA = {0.f, 0.f}, SP = {0.f, 0.f}, TT = {0.f, 0.f};
#pragma unroll 4
    for (int j = 0; j <= r; ++j) {
      const f32x2 kj = *reinterpret_cast<const f32x2*>(&sK[j][c0]);
      const f32x2 gj = *reinterpret_cast<const f32x2*>(&sG[j][c0]);
      const float da = sdA[r][j], dp = sdP[r][j];
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const float ke = kj[e] * __expf(Gr[e] - gj[e]);
        SA[e] += da * ke;
        SP[e] += dp * ke;
      }
    }
#pragma unroll 4
    for (int r2 = r; r2 < n; ++r2) {
      const f32x2 k2 = *reinterpret_cast<const f32x2*>(&sK[r2][c0]);
      const f32x2 q2 = *reinterpret_cast<const f32x2*>(&sQ[r2][c0]);
      const f32x2 g2 = *reinterpret_cast<const f32x2*>(&sG[r2][c0]);
      const float da = sdA[r2][r], dp = sdP[r2][r];
#pragma unroll
      for (int e = 0; e < 2; ++e) TT[e] += (da * k2[e] + dp * q2[e]) * __expf(g2[e] - Gr[e]);
    }
    SAv[m] = SA;
    SPv[m] = SP;
    TTv[m] = TT;
  }
  // the dense parts of dq, dk and dGam loaded before the first store
  f32x2 vq[RPT], vk[RPT], vg[RPT];
#pragma unroll
  for (int m = 0; m < RPT; ++m) {
    const int r = tid / (DK / 2) + RG * m;
    const long i = (long)r * DK + c0;
    vq[m] = r < n ? *reinterpret_cast<const f32x2*>(blk + L::odq + i) : f32x2{0.f, 0.f};
    vk[m] = r < n ? *reinterpret_cast<const f32x2*>(blk + L::odk + i) : f32x2{0.f, 0.f};
    vg[m] = r < n ? *reinterpret_cast<const f32x2*>(blk + L::odG + i) : f32x2{0.f, 0.f};
  }
  __syncthreads();  // dA and dP are dead from here
#pragma unroll
  for (int m = 0; m < RPT; ++m) {
    const int r = tid / (DK / 2) + RG * m;
    if (r >= n) continue;
    const f32x2 kr = *reinterpret_cast<const f32x2*>(&sK[r][c0]);
    const f32x2 qr = *reinterpret_cast<const f32x2*>(&sQ[r][c0]);
    const f32x2 SA = SAv[m], SP = SPv[m], TT = TTv[m];
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const long o = tok(a, it.b, it.t0 + r, it.h) * DK + c0 + e;
      dq[o] = from_f32<IO>(vq[m][e] + SP[e]);
      dk[o] = from_f32<IO>(vk[m][e] + SA[e] + TT[e]);
      sdG[r][c0 + e] = vg[m][e] + (kr[e] * SA[e] + qr[e] * SP[e] - kr[e] * TT[e]);
    }
  }
  }
  __syncthreads();
  if (tid < DK) {  // dg = reverse in-chunk prefix sum of dGam
    float s = 0.f;
    for (int r = n - 1; r >= 0; --r) {
      s += sdG[r][tid];
      a.dg[tok(a, it.b, it.t0 + r, it.h) * DK + tid] = s;
    }
  }
}

// Stages of one launch sequence over the chunk range [a.c0, a.c1).
enum : unsigned { kStPrep = 1, kStState = 2, kStReverse = 4, kStGrads = 8, kStAll = 15 };

template <int DK, int DV, typename IO>
hipError_t run_bw(const BackwardArgs& a, unsigned stages, hipStream_t st) {
  const long items = (long)(a.c1 - a.c0) * a.B * a.H;
  const unsigned chains_s = (unsigned)(DV / bw_dvb<DV, kStateChainW>() * a.B * a.H);
  const unsigned chains_r = (unsigned)(DV / bw_dvb<DV, kReverseChainW>() * a.B * a.H);
  if (items > 0 && (stages & kStPrep))
    hipLaunchKernelGGL((bw_prep_kernel<DK, DV, IO>), dim3((unsigned)items), dim3(kBP), 0, st, a);
  if (items > 0 && (stages & kStState))
    hipLaunchKernelGGL((bw_state_chain_kernel<DK, DV>), dim3(chains_s), dim3(kStateNT), 0, st, a);
  if (stages & kStReverse)
    hipLaunchKernelGGL((bw_reverse_chain_kernel<DK, DV, IO>), dim3(chains_r), dim3(kRevNT), 0, st,
                       a);
  if (items > 0 && (stages & kStGrads)) {
    if constexpr (std::is_same<IO, bf16>::value && DV >= 32)
      hipLaunchKernelGGL((bw_grad_dense_bf16_kernel<DK, DV>), dim3((unsigned)items), dim3(kBT), 0,
                         st, a);
    else
      hipLaunchKernelGGL((bw_grad_dense_kernel<DK, DV, IO>), dim3((unsigned)items), dim3(kBT), 0,
                         st, a);
    if constexpr (std::is_same<IO, bf16>::value)
      hipLaunchKernelGGL((bw_grad_solve_bf16_kernel<DK, DV>), dim3((unsigned)items), dim3(kBS), 0,
                         st, a);
    else
      hipLaunchKernelGGL((bw_grad_solve_kernel<DK, DV, IO>), dim3((unsigned)items), dim3(kBS), 0,
                         st, a);
    hipLaunchKernelGGL((bw_grad_gram_kernel<DK, DV, IO>), dim3((unsigned)items), dim3(kBP), 0,
                       st, a);
  }
  return hipGetLastError();
}

template <int DK, int DV>
hipError_t run_bw_io(const BackwardArgs& a, kda_dtype io, unsigned stages, hipStream_t st) {
  return io == KDA_BF16 ? run_bw<DK, DV, bf16>(a, stages, st)
                        : run_bw<DK, DV, float>(a, stages, st);
}

template <int DK>
hipError_t run_bw_dv(const BackwardArgs& a, kda_dtype io, unsigned stages, hipStream_t st) {
  switch (a.dvw) {
    case 16: return run_bw_io<DK, 16>(a, io, stages, st);
    case 32: return run_bw_io<DK, 32>(a, io, stages, st);
    case 64: return run_bw_io<DK, 64>(a, io, stages, st);
    case 128: return run_bw_io<DK, 128>(a, io, stages, st);
  }
  return hipErrorInvalidValue;
}

hipError_t run_bw_any(const BackwardArgs& a, kda_dtype io, unsigned stages, hipStream_t st) {
  switch (a.dkw) {
    case 16: return run_bw_dv<16>(a, io, stages, st);
    case 32: return run_bw_dv<32>(a, io, stages, st);
    case 64: return run_bw_dv<64>(a, io, stages, st);
    case 128: return run_bw_dv<128>(a, io, stages, st);
  }
  return hipErrorInvalidValue;
}

size_t scratch_floats(int dk, int dv) {
  switch (dk * 1000 + dv) {
#define KDA_BW_CASE(K, V) \
  case K * 1000 + V: return (size_t)BwL<K, V>::n;
    KDA_BW_CASE(16, 16) KDA_BW_CASE(16, 32) KDA_BW_CASE(16, 64) KDA_BW_CASE(16, 128)
    KDA_BW_CASE(32, 16) KDA_BW_CASE(32, 32) KDA_BW_CASE(32, 64) KDA_BW_CASE(32, 128)
    KDA_BW_CASE(64, 16) KDA_BW_CASE(64, 32) KDA_BW_CASE(64, 64) KDA_BW_CASE(64, 128)
    KDA_BW_CASE(128, 16) KDA_BW_CASE(128, 32) KDA_BW_CASE(128, 64) KDA_BW_CASE(128, 128)
#undef KDA_BW_CASE
  }
  return 0;
}

// Workspace bytes per chunk of all sequences and heads (its scratch blocks,
// entering states and leaving-state gradients) and per state [B][H][dk][dv].
struct BwSizes {
  size_t per_chunk, state;
};

BwSizes bw_sizes(int B, int H, int dk, int dv) {
  const size_t BH = (size_t)B * H, st = (size_t)dk * dv;
  return {BH * (scratch_floats(dk, dv) + 2 * st) * sizeof(float), BH * st * sizeof(float)};
}

// Bytes for ranges of L chunks out of nc: one range's blocks, plus, when
// there are several ranges, the state entering every range but the first
// and one carried state gradient.
size_t range_need(long nc, long L, const BwSizes& z) {
  if (L >= nc) return (size_t)nc * z.per_chunk;
  const long nseg = (nc + L - 1) / L;
  return (size_t)L * z.per_chunk + (size_t)nseg * z.state;
}

// The longest range that fits ws_bytes (nc when the one-shot layout fits,
// 0 when nothing does).
long range_chunks(long nc, size_t ws_bytes, const BwSizes& z) {
  if (range_need(nc, nc, z) <= ws_bytes) return nc;
  for (long L = std::min<long>(nc - 1, (long)(ws_bytes / z.per_chunk)); L >= 1; --L)
    if (range_need(nc, L, z) <= ws_bytes) return L;
  return 0;
}

}  // namespace

size_t backward_ws_bytes(int B, int T, int H, int dk, int dv, int chunk) {
  const long nc = ((long)T + chunk - 1) / chunk;
  return range_need(nc, nc, bw_sizes(B, H, dk, dv));
}

size_t backward_ws_min_bytes(int B, int T, int H, int dk, int dv, int chunk) {
  const long nc = ((long)T + chunk - 1) / chunk;
  const BwSizes z = bw_sizes(B, H, dk, dv);
  size_t best = range_need(nc, nc, z);
  // need(L) >= L * per_chunk, so no L past best / per_chunk can do better
  for (long L = 1; L < nc && (size_t)L * z.per_chunk < best; ++L)
    best = std::min(best, range_need(nc, L, z));
  return best;
}

// One-shot when the workspace holds every chunk's blocks; otherwise the
// chunks are taken in ranges of L (the longest that fits): a forward pass
// over the ranges keeps only the state entering each (prep + state chain),
// then, from the last range to the first, each range is prepared again, its
// state chain rerun from the kept state, its reverse chain started from the
// state gradient the later range handed back, and its per-chunk gradients
// formed. Every chunk sees the same fp32 values as in the one-shot call.
hipError_t launch_backward(BackwardArgs a, kda_dtype io, void* ws, size_t ws_bytes,
                           hipStream_t stream) {
  const long nc = ((long)a.T + a.chunk - 1) / a.chunk;
  const BwSizes z = bw_sizes(a.B, a.H, a.dkw, a.dvw);
  const long L = range_chunks(nc, ws_bytes, z);
  if (nc > 0 && L < 1) return hipErrorInvalidValue;
  const size_t BH = (size_t)a.B * a.H, st = (size_t)a.dkw * a.dvw;
  float* w = static_cast<float*>(ws);
  a.scratch = w;
  a.S0s = w + (size_t)L * BH * scratch_floats(a.dkw, a.dvw);
  a.dS1s = a.S0s + (size_t)L * BH * st;
  a.S_out = nullptr;
  if (L >= nc) {
    a.c0 = 0;
    a.c1 = (int)nc;
    return run_bw_any(a, io, kStAll, stream);
  }
  const long nseg = (nc + L - 1) / L;
  float* kept = a.dS1s + (size_t)L * BH * st;  // states entering ranges 1 .. nseg - 1
  float* carry = kept + (size_t)(nseg - 1) * BH * st;
  auto kept_of = [&](long s) { return kept + (size_t)(s - 1) * BH * st; };
  auto range = [&](long s) {
    BackwardArgs x = a;
    x.c0 = (int)(s * L);
    x.c1 = (int)std::min(nc, (s + 1) * L);
    x.S0 = s == 0 ? a.S0 : kept_of(s);
    return x;
  };
  for (long s = 0; s + 1 < nseg; ++s) {
    BackwardArgs x = range(s);
    x.S_out = kept_of(s + 1);
    const hipError_t e = run_bw_any(x, io, kStPrep | kStState, stream);
    if (e != hipSuccess) return e;
  }
  for (long s = nseg - 1; s >= 0; --s) {
    BackwardArgs x = range(s);
    x.dST = s == nseg - 1 ? a.dST : carry;
    x.dS0 = s == 0 ? a.dS0 : carry;  // read and written by the same thread, in place
    const hipError_t e = run_bw_any(x, io, kStAll, stream);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace kda
