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
// -> decayed-Gram gradients and dg (per chunk-head). The decay factors are
// formed as exponentials of non-positive differences, so any finite g <= 0
// is accepted.
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
  r.c = (int)(it / BH);
  r.bh = (int)(it % BH);
  r.b = r.bh / a.H;
  r.h = r.bh % a.H;
  r.t0 = r.c * a.chunk;
  r.n = min(a.chunk, a.T - r.t0);
  return r;
}

// ---- 1. per chunk-head: Gam, A, P, X, Q~, K~, K^d, W, U' --------------------
template <int DK, int DV, typename IO>
__global__ __launch_bounds__(kBT) void bw_prep_kernel(BackwardArgs a) {
  using L = BwL<DK, DV>;
  constexpr int PK = DK + 1;
  __shared__ float sK[CM][PK], sQ[CM][PK], sG[CM][PK];
  __shared__ float sM[CM][CM + 1], sX[CM][CM + 1];
  __shared__ float sb[CM];
  const Item it = item_of(a, blockIdx.x);
  const int n = it.n;
  float* blk = a.scratch + (long)blockIdx.x * L::n;
  const int tid = threadIdx.x, lane = tid % kWave, wv = tid / kWave;
  const IO* q = static_cast<const IO*>(a.q);
  const IO* k = static_cast<const IO*>(a.k);
  const IO* v = static_cast<const IO*>(a.v);
  for (int i = tid; i < n * DK; i += kBT) {
    const int r = i / DK, cc = i % DK;
    const long off = tok(a, it.b, it.t0 + r, it.h) * DK + cc;
    sK[r][cc] = to_f32(k[off]);
    sQ[r][cc] = to_f32(q[off]);
    sG[r][cc] = a.g[off];
  }
  if (tid < n) sb[tid] = a.beta[tok(a, it.b, it.t0 + tid, it.h)];
  __syncthreads();
  if (tid < DK) {
    float s = 0.f;
    for (int r = 0; r < n; ++r) {
      s += sG[r][tid];
      sG[r][tid] = s;
    }
  }
  __syncthreads();
  // A (strictly lower) and P (lower): wave w takes rows w, w+4, ..., lane j
  // the column; every exponent Gam_r - Gam_j (j <= r) is <= 0.
  for (int r = wv; r < n; r += 4) {
    const int j = lane;
    float accA = 0.f, accP = 0.f;
    if (j <= r) {
      for (int cc = 0; cc < DK; ++cc) {
        const float kj = sK[j][cc] * __expf(sG[r][cc] - sG[j][cc]);
        accA += sK[r][cc] * kj;
        accP += sQ[r][cc] * kj;
      }
    }
    blk[L::oP + r * CM + j] = j <= r ? accP : 0.f;
    blk[L::oA + r * CM + j] = j < r ? accA : 0.f;
    sM[r][j] = j < r ? sb[r] * accA : 0.f;
  }
  __syncthreads();
  // X = (I + diag(beta) A)^-1, unit lower triangular, by forward
  // substitution: lane j of wave 0 owns column j.
  if (wv == 0) {
    const int j = lane;
    for (int r = 0; r < n; ++r) {
      float acc = 0.f;
      for (int m = 0; m < r; ++m) acc += sM[r][m] * sX[m][j];
      sX[r][j] = r > j ? -acc : (r == j ? 1.f : 0.f);
    }
  }
  __syncthreads();
  for (int i = tid; i < n * CM; i += kBT) {
    const int r = i / CM, j = i % CM;
    blk[L::oX + i] = j < n ? sX[r][j] : 0.f;
  }
  for (int i = tid; i < n * DK; i += kBT) {
    const int r = i / DK, cc = i % DK;
    const float G = sG[r][cc], eg = __expf(G), kt = eg * sK[r][cc];
    blk[L::oQt + i] = eg * sQ[r][cc];
    blk[L::oKt + i] = kt;
    blk[L::oKd + i] = __expf(sG[n - 1][cc] - G) * sK[r][cc];
    blk[L::oG + i] = G;
    sQ[r][cc] = sb[r] * kt;  // beta K~ for W (each element read by its writer only)
  }
  if (tid < DK) blk[L::oEn + tid] = __expf(sG[n - 1][tid]);
  __syncthreads();
  for (int i = tid; i < n * DK; i += kBT) {  // W = X (beta K~)
    const int r = i / DK, cc = i % DK;
    float acc = 0.f;
    for (int j = 0; j <= r; ++j) acc += sX[r][j] * sQ[j][cc];
    blk[L::oW + i] = acc;
  }
  for (int i = tid; i < n * DV; i += kBT) {  // U' = X (beta V^)
    const int r = i / DV, l = i % DV;
    float acc = 0.f;
    for (int j = 0; j <= r; ++j)
      acc += sX[r][j] * sb[j] * to_f32(v[tok(a, it.b, it.t0 + j, it.h) * DV + l]);
    blk[L::oU + i] = acc;
  }
}

template <int DV>
constexpr int bw_dvb() {
  return DV < 32 ? DV : 32;
}

// ---- 2. forward state chain: entering state of every chunk, U ---------------
// One workgroup per (32-column block, head, sequence); the S block lives in
// LDS. Per chunk: keep S, U = U' - W S (over U' in the scratch), then
// S = Diag(e^{Gam_n}) S + K^d^T U.
template <int DK, int DV>
__global__ __launch_bounds__(kBT) void bw_state_chain_kernel(BackwardArgs a) {
  using L = BwL<DK, DV>;
  constexpr int DVB = bw_dvb<DV>(), NB = DV / DVB;
  __shared__ float sS[DK][DVB];
  __shared__ float sU[CM][DVB];
  __shared__ float sO[CM][DK + 1];
  const int cbk = blockIdx.x % NB, bh = blockIdx.x / NB, cb0 = cbk * DVB;
  const int BH = a.B * a.H, nc = (a.T + a.chunk - 1) / a.chunk;
  const int tid = threadIdx.x;
  for (int i = tid; i < DK * DVB; i += kBT) {
    const int r = i / DVB, j = i % DVB;
    sS[r][j] = a.S0 ? a.S0[((long)bh * DK + r) * DV + cb0 + j] : 0.f;
  }
  for (int c = 0; c < nc; ++c) {
    const int n = min(a.chunk, a.T - c * a.chunk);
    const long item = (long)c * BH + bh;
    float* blk = a.scratch + item * L::n;
    float* Sk = a.S0s + item * DK * DV;
    __syncthreads();  // S of this chunk complete
    for (int i = tid; i < DK * DVB; i += kBT) {
      const int r = i / DVB, j = i % DVB;
      Sk[(long)r * DV + cb0 + j] = sS[r][j];
    }
    for (int i = tid; i < n * DK; i += kBT) sO[i / DK][i % DK] = blk[L::oW + i];
    __syncthreads();
    for (int i = tid; i < n * DVB; i += kBT) {
      const int r = i / DVB, j = i % DVB;
      float acc = blk[L::oU + (long)r * DV + cb0 + j];
      for (int cc = 0; cc < DK; ++cc) acc -= sO[r][cc] * sS[cc][j];
      sU[r][j] = acc;
      blk[L::oU + (long)r * DV + cb0 + j] = acc;
    }
    __syncthreads();
    for (int i = tid; i < n * DK; i += kBT) sO[i / DK][i % DK] = blk[L::oKd + i];
    __syncthreads();
    for (int i = tid; i < DK * DVB; i += kBT) {
      const int cc = i / DVB, j = i % DVB;
      float acc = blk[L::oEn + cc] * sS[cc][j];
      for (int r = 0; r < n; ++r) acc += sO[r][cc] * sU[r][j];
      sS[cc][j] = acc;
    }
  }
}

// ---- 3. reverse chain: dS1 of every chunk, dU, and dS0 ----------------------
// Same grid as the state chain; chunks from the last to the first. The dS
// block lives in LDS; each thread keeps its elements of the update in
// registers across the two operand stages.
template <int DK, int DV, typename IO>
__global__ __launch_bounds__(kBT) void bw_reverse_chain_kernel(BackwardArgs a) {
  using L = BwL<DK, DV>;
  constexpr int DVB = bw_dvb<DV>(), NB = DV / DVB, PER = DK * DVB / kBT;
  static_assert(DK * DVB % kBT == 0, "dS block per thread");
  __shared__ float sdS[DK][DVB];
  __shared__ float sdO[CM][DVB];
  __shared__ float sdU[CM][DVB];
  __shared__ float sO[CM][DK + 1];
  const int cbk = blockIdx.x % NB, bh = blockIdx.x / NB, cb0 = cbk * DVB;
  const int b = bh / a.H, h = bh % a.H;
  const int BH = a.B * a.H, nc = (a.T + a.chunk - 1) / a.chunk;
  const int tid = threadIdx.x;
  const IO* dO = static_cast<const IO*>(a.dO);
  for (int i = tid; i < DK * DVB; i += kBT) {
    const int r = i / DVB, j = i % DVB;
    sdS[r][j] = a.dST ? a.dST[((long)bh * DK + r) * DV + cb0 + j] : 0.f;
  }
  for (int c = nc - 1; c >= 0; --c) {
    const int t0 = c * a.chunk, n = min(a.chunk, a.T - t0);
    const long item = (long)c * BH + bh;
    float* blk = a.scratch + item * L::n;
    float* dSk = a.dS1s + item * DK * DV;
    __syncthreads();  // dS of this chunk complete
    for (int i = tid; i < DK * DVB; i += kBT) {
      const int r = i / DVB, j = i % DVB;
      dSk[(long)r * DV + cb0 + j] = sdS[r][j];
    }
    for (int i = tid; i < n * DVB; i += kBT) {
      const int r = i / DVB, j = i % DVB;
      sdO[r][j] = to_f32(dO[tok(a, b, t0 + r, h) * DV + cb0 + j]);
    }
    for (int i = tid; i < n * DK; i += kBT) sO[i / DK][i % DK] = blk[L::oKd + i];
    __syncthreads();
    const float* P = blk + L::oP;
    for (int i = tid; i < n * DVB; i += kBT) {  // dU = P^T dO + K^d dS
      const int r = i / DVB, j = i % DVB;
      float acc = 0.f;
      for (int i2 = r; i2 < n; ++i2) acc += P[i2 * CM + r] * sdO[i2][j];
      for (int cc = 0; cc < DK; ++cc) acc += sO[r][cc] * sdS[cc][j];
      sdU[r][j] = acc;
      blk[L::odU + (long)r * DV + cb0 + j] = acc;
    }
    __syncthreads();
    for (int i = tid; i < n * DK; i += kBT) sO[i / DK][i % DK] = blk[L::oQt + i];
    __syncthreads();
    float acc[PER];
#pragma unroll
    for (int p = 0; p < PER; ++p) {  // Diag(e^{Gam_n}) dS + Q~^T dO
      const int i = tid + p * kBT, cc = i / DVB, j = i % DVB;
      float s = blk[L::oEn + cc] * sdS[cc][j];
      for (int r = 0; r < n; ++r) s += sO[r][cc] * sdO[r][j];
      acc[p] = s;
    }
    __syncthreads();
    for (int i = tid; i < n * DK; i += kBT) sO[i / DK][i % DK] = blk[L::oW + i];
    __syncthreads();
#pragma unroll
    for (int p = 0; p < PER; ++p) {  // - W^T dU
      const int i = tid + p * kBT, cc = i / DVB, j = i % DVB;
      float s = acc[p];
      for (int r = 0; r < n; ++r) s -= sO[r][cc] * sdU[r][j];
      sdS[cc][j] = s;
    }
  }
  __syncthreads();
  if (a.dS0) {
    for (int i = tid; i < DK * DVB; i += kBT) {
      const int r = i / DVB, j = i % DVB;
      a.dS0[((long)bh * DK + r) * DV + cb0 + j] = sdS[r][j];
    }
  }
}

// ---- 4. per chunk-head: the products with S0 and dS1, and dP -----------------
// Wave w takes channels w, w+4, ...; lane r is the token row, so the rows of
// S0 and dS1 are read as wave-uniform vectors.
template <int DK, int DV, typename IO>
__global__ __launch_bounds__(kBT) void bw_grad_dense_kernel(BackwardArgs a) {
  using L = BwL<DK, DV>;
  constexpr int PV = DV + 1;
  __shared__ float sdO[CM][PV], sdU[CM][PV], sU[CM][PV];
  const Item it = item_of(a, blockIdx.x);
  const int n = it.n;
  float* blk = a.scratch + (long)blockIdx.x * L::n;
  const float* S0 = a.S0s + (long)blockIdx.x * DK * DV;
  const float* dS1 = a.dS1s + (long)blockIdx.x * DK * DV;
  const int tid = threadIdx.x, lane = tid % kWave, wv = tid / kWave;
  const IO* dO = static_cast<const IO*>(a.dO);
  for (int i = tid; i < n * DV; i += kBT) {
    const int r = i / DV, l = i % DV;
    sdO[r][l] = to_f32(dO[tok(a, it.b, it.t0 + r, it.h) * DV + l]);
    sdU[r][l] = blk[L::odU + i];
    sU[r][l] = blk[L::oU + i];
  }
  __syncthreads();
  const int r = lane;
  const bool live = r < n;
  for (int cc = wv; cc < DK; cc += 4) {
    float dq = 0.f, dw = 0.f, dkd = 0.f, dd = 0.f;
    if (live) {
      for (int l = 0; l < DV; l += 4) {
        const f32x4 s = *reinterpret_cast<const f32x4*>(S0 + (long)cc * DV + l);
        const f32x4 ds = *reinterpret_cast<const f32x4*>(dS1 + (long)cc * DV + l);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          dq += sdO[r][l + e] * s[e];
          dw += sdU[r][l + e] * s[e];
          dkd += sU[r][l + e] * ds[e];
          dd += ds[e] * s[e];
        }
      }
    }
    const long i = (long)r * DK + cc;
    float kd = 0.f, G = 0.f, qt = 0.f;
    if (live) {
      kd = blk[L::oKd + i];
      G = blk[L::oG + i];
      qt = blk[L::oQt + i];
    }
    const float col = wave_sum(kd * dkd);  // sum over rows of K^d * dK^d
    if (live) {
      const float Gn = blk[L::oG + (long)(n - 1) * DK + cc];
      float dG = qt * dq - kd * dkd;
      if (r == n - 1) dG += col + blk[L::oEn + cc] * dd;
      blk[L::odq + i] = __expf(G) * dq;
      blk[L::odk + i] = __expf(Gn - G) * dkd;
      blk[L::odG + i] = dG;
      blk[L::odW + i] = -dw;
    }
  }
  // dP = (dO U^T) on j <= r: wave w takes rows w, w+4, ..., lane j the column
  for (int r2 = wv; r2 < n; r2 += 4) {
    const int j = lane;
    float acc = 0.f;
    if (j <= r2)
      for (int l = 0; l < DV; ++l) acc += sdO[r2][l] * sU[j][l];
    blk[L::odP + r2 * CM + j] = j <= r2 ? acc : 0.f;
  }
}

// ---- 5. per chunk-head: through W, U' and the inverse; dv and dbeta --------
template <int DK, int DV, typename IO>
__global__ __launch_bounds__(kBT) void bw_grad_solve_kernel(BackwardArgs a) {
  using L = BwL<DK, DV>;
  __shared__ float sX[CM][CM + 1], sKt[CM][DK + 1], sV[CM][DV + 1];
  __shared__ float sdX[CM][CM + 1], sT[CM][CM + 1];
  __shared__ float sbt[CM], sdb[CM];
  const Item it = item_of(a, blockIdx.x);
  const int n = it.n;
  float* blk = a.scratch + (long)blockIdx.x * L::n;
  const int tid = threadIdx.x, lane = tid % kWave, wv = tid / kWave;
  const IO* v = static_cast<const IO*>(a.v);
  IO* dv = static_cast<IO*>(a.dv);
  for (int i = tid; i < n * CM; i += kBT) sX[i / CM][i % CM] = blk[L::oX + i];
  for (int i = tid; i < n * DK; i += kBT) sKt[i / DK][i % DK] = blk[L::oKt + i];
  for (int i = tid; i < n * DV; i += kBT) {
    const int r = i / DV, l = i % DV;
    sV[r][l] = to_f32(v[tok(a, it.b, it.t0 + r, it.h) * DV + l]);
  }
  if (tid < n) sbt[tid] = a.beta[tok(a, it.b, it.t0 + tid, it.h)];
  __syncthreads();
  // Y = X^T dW and Z = X^T dU, row r per wave, channels across the lanes
  for (int r = wv; r < n; r += 4) {
    const float br = sbt[r];
    float db = 0.f;
    for (int cc = lane; cc < DK; cc += kWave) {
      float y = 0.f;
      for (int i = r; i < n; ++i) y += sX[i][r] * blk[L::odW + (long)i * DK + cc];
      db += sKt[r][cc] * y;
      const long o = (long)r * DK + cc;
      blk[L::odk + o] += __expf(blk[L::oG + o]) * br * y;
      blk[L::odG + o] += sKt[r][cc] * br * y;
    }
    for (int l = lane; l < DV; l += kWave) {
      float z = 0.f;
      for (int i = r; i < n; ++i) z += sX[i][r] * blk[L::odU + (long)i * DV + l];
      db += sV[r][l] * z;
      dv[tok(a, it.b, it.t0 + r, it.h) * DV + l] = from_f32<IO>(br * z);
    }
    db = wave_sum(db);
    if (lane == 0) sdb[r] = db;
  }
  // dX, strictly lower: dX[a][b] = beta_b (dW[a] . K~[b] + dU[a] . V^[b])
  for (int r = wv; r < n; r += 4) {
    const int j = lane;
    float acc = 0.f;
    if (j < r) {
      for (int cc = 0; cc < DK; ++cc) acc += blk[L::odW + (long)r * DK + cc] * sKt[j][cc];
      for (int l = 0; l < DV; ++l) acc += blk[L::odU + (long)r * DV + l] * sV[j][l];
      acc *= sbt[j];
    }
    sdX[r][j] = acc;
  }
  __syncthreads();
  // T1 = dX X^T on j < a (only those entries reach the strictly lower dM)
  for (int r = wv; r < n; r += 4) {
    const int j = lane;
    float acc = 0.f;
    if (j < r)
      for (int m = 0; m <= j; ++m) acc += sdX[r][m] * sX[j][m];
    sT[r][j] = acc;
  }
  __syncthreads();
  // dM = -X^T T1 (strictly lower); dA = beta dM; dbeta += A . dM
  for (int r = wv; r < n; r += 4) {
    const int j = lane;
    float dm = 0.f, arj = 0.f;
    if (j < r) {
      for (int m = r; m < n; ++m) dm -= sX[m][r] * sT[m][j];
      arj = blk[L::oA + r * CM + j];
    }
    blk[L::odA + r * CM + j] = j < r ? sbt[r] * dm : 0.f;
    const float part = wave_sum(arj * dm);
    if (lane == 0) sdb[r] += part;
  }
  __syncthreads();
  if (tid < n) a.dbeta[tok(a, it.b, it.t0 + tid, it.h)] = sdb[tid];
}

// ---- 6. per chunk-head: through the decayed Grams; dq, dk, dg --------------
// Thread (channel c, row group): for each of its rows r the row-side sums
// over j <= r and the column-side sums over r2 >= r of the pair terms, each
// with its own exponential of a non-positive difference.
template <int DK, int DV, typename IO>
__global__ __launch_bounds__(kBT) void bw_grad_gram_kernel(BackwardArgs a) {
  using L = BwL<DK, DV>;
  constexpr int PK = DK + 1, RG = kBT / DK;
  __shared__ float sK[CM][PK], sQ[CM][PK], sG[CM][PK];
  __shared__ float sdA[CM][CM + 1], sdP[CM][CM + 1];
  const Item it = item_of(a, blockIdx.x);
  const int n = it.n;
  float* blk = a.scratch + (long)blockIdx.x * L::n;
  const int tid = threadIdx.x;
  const IO* q = static_cast<const IO*>(a.q);
  const IO* k = static_cast<const IO*>(a.k);
  IO* dq = static_cast<IO*>(a.dq);
  IO* dk = static_cast<IO*>(a.dk);
  for (int i = tid; i < n * DK; i += kBT) {
    const int r = i / DK, cc = i % DK;
    const long off = tok(a, it.b, it.t0 + r, it.h) * DK + cc;
    sK[r][cc] = to_f32(k[off]);
    sQ[r][cc] = to_f32(q[off]);
    sG[r][cc] = blk[L::oG + i];
  }
  for (int i = tid; i < n * CM; i += kBT) {
    sdA[i / CM][i % CM] = blk[L::odA + i];
    sdP[i / CM][i % CM] = blk[L::odP + i];
  }
  __syncthreads();
  const int cc = tid % DK;
  for (int r = tid / DK; r < n; r += RG) {
    const float Gr = sG[r][cc], kr = sK[r][cc], qr = sQ[r][cc];
    float SA = 0.f, SP = 0.f, TT = 0.f;
    for (int j = 0; j <= r; ++j) {
      const float kje = sK[j][cc] * __expf(Gr - sG[j][cc]);
      SA += sdA[r][j] * kje;
      SP += sdP[r][j] * kje;
    }
    for (int r2 = r; r2 < n; ++r2)
      TT += (sdA[r2][r] * sK[r2][cc] + sdP[r2][r] * sQ[r2][cc]) * __expf(sG[r2][cc] - Gr);
    const long i = (long)r * DK + cc;
    const long o = tok(a, it.b, it.t0 + r, it.h) * DK + cc;
    dq[o] = from_f32<IO>(blk[L::odq + i] + SP);
    dk[o] = from_f32<IO>(blk[L::odk + i] + SA + TT);
    blk[L::odG + i] += kr * SA + qr * SP - kr * TT;
  }
  __syncthreads();
  if (tid < DK) {  // dg = reverse in-chunk prefix sum of dGam
    float s = 0.f;
    for (int r = n - 1; r >= 0; --r) {
      s += blk[L::odG + (long)r * DK + tid];
      a.dg[tok(a, it.b, it.t0 + r, it.h) * DK + tid] = s;
    }
  }
}

template <int DK, int DV, typename IO>
hipError_t run_bw(const BackwardArgs& a, hipStream_t st) {
  constexpr int NB = DV / bw_dvb<DV>();
  const int nc = (a.T + a.chunk - 1) / a.chunk;
  const long items = (long)nc * a.B * a.H;
  const unsigned chains = (unsigned)(NB * a.B * a.H);
  if (items > 0) {
    hipLaunchKernelGGL((bw_prep_kernel<DK, DV, IO>), dim3((unsigned)items), dim3(kBT), 0, st, a);
    hipLaunchKernelGGL((bw_state_chain_kernel<DK, DV>), dim3(chains), dim3(kBT), 0, st, a);
  }
  hipLaunchKernelGGL((bw_reverse_chain_kernel<DK, DV, IO>), dim3(chains), dim3(kBT), 0, st, a);
  if (items > 0) {
    hipLaunchKernelGGL((bw_grad_dense_kernel<DK, DV, IO>), dim3((unsigned)items), dim3(kBT), 0,
                       st, a);
    hipLaunchKernelGGL((bw_grad_solve_kernel<DK, DV, IO>), dim3((unsigned)items), dim3(kBT), 0,
                       st, a);
    hipLaunchKernelGGL((bw_grad_gram_kernel<DK, DV, IO>), dim3((unsigned)items), dim3(kBT), 0,
                       st, a);
  }
  return hipGetLastError();
}

template <int DK, int DV>
hipError_t run_bw_io(const BackwardArgs& a, kda_dtype io, hipStream_t st) {
  return io == KDA_BF16 ? run_bw<DK, DV, bf16>(a, st) : run_bw<DK, DV, float>(a, st);
}

template <int DK>
hipError_t run_bw_dv(const BackwardArgs& a, kda_dtype io, hipStream_t st) {
  switch (a.dvw) {
    case 16: return run_bw_io<DK, 16>(a, io, st);
    case 32: return run_bw_io<DK, 32>(a, io, st);
    case 64: return run_bw_io<DK, 64>(a, io, st);
    case 128: return run_bw_io<DK, 128>(a, io, st);
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

}  // namespace

size_t backward_ws_bytes(int B, int T, int H, int dk, int dv, int chunk) {
  const size_t nc = ((size_t)T + chunk - 1) / chunk;
  const size_t items = nc * B * H;
  return items * scratch_floats(dk, dv) * sizeof(float) +
         2 * items * (size_t)dk * dv * sizeof(float);
}

hipError_t launch_backward(BackwardArgs a, kda_dtype io, void* ws, hipStream_t stream) {
  const size_t nc = ((size_t)a.T + a.chunk - 1) / a.chunk;
  const size_t items = nc * a.B * a.H;
  float* w = static_cast<float*>(ws);
  a.scratch = w;
  a.S0s = w + items * scratch_floats(a.dkw, a.dvw);
  a.dS1s = a.S0s + items * (size_t)a.dkw * a.dvw;
  switch (a.dkw) {
    case 16: return run_bw_dv<16>(a, io, stream);
    case 32: return run_bw_dv<32>(a, io, stream);
    case 64: return run_bw_dv<64>(a, io, stream);
    case 128: return run_bw_dv<128>(a, io, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace kda
