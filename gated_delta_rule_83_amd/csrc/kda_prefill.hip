// Chunkwise-parallel KDA prefill ("为什么 Kimi K3 敢把 KV Cache 扔掉？一篇讲透
// GPT-2 到 K3 的架构进化", section 5: attention-like work inside a chunk, the
// previous chunk's final state handed on, the WY representation of the delta
// updates; section 6: cumulative decay inside a chunk; section 7: the
// per-channel Diag(alpha) of KDA).
//
// Per head, for a chunk of n <= C tokens entering with state S (dk x dv), with
// Gam_r = sum_{i<=r} g_i (per key channel, inside the chunk):
//   A_rj = sum_c k_r[c] k_j[c] e^{Gam_r[c]-Gam_j[c]}   (j < r)
//   P_rj = sum_c q_r[c] k_j[c] e^{Gam_r[c]-Gam_j[c]}   (j <= r)
//   X    = (I + diag(beta) A)^{-1}
//   W    = X diag(beta) (e^{Gam} * K),   U' = X diag(beta) V
//   U    = U' - W S
//   O    = (e^{Gam} * Q) S + P U
//   S   <- Diag(e^{Gam_n}) S + (e^{Gam_n - Gam} * K)^T U
// Everything except the last three lines is independent of S, so it runs in
// a fully parallel kernel over (chunk, head, sequence) ("prep") that writes
// -W, Q~ = e^{Gam}*Q, K^T = (e^{Gam_n-Gam}*K)^T, P, U' and e^{Gam_n} to a
// workspace. A second kernel ("chain") walks the chunks of each (sequence,
// head, dv-block) in order, keeping its block of S in MFMA accumulators.
//
// Overflow-safe Gram matrices: A and P are computed on MFMA as products of
// factors k_r e^{Gam_r - Gam_m} and k_j e^{Gam_m - Gam_j}, where m is the
// first row of the 16-row block of r. For j < m both exponents are <= 0; for
// j inside the diagonal block the second exponent is a sum of at most 15
// decays, which the documented precondition keeps inside the fp32 range.
#include "kda_common.h"

namespace kda {
namespace {

// v_mfma_f32_16x16x32_bf16: lane l holds A[l%16][8*(l/16) .. +7] and
// B[8*(l/16) .. +7][l%16]; the result D[4*(l/16) + e][l%16], e = 0..3.
struct MmaBf16 {
  using T = bf16;
  using frag = bf16x8;
  static constexpr int KS = 32, KPL = 8;
  __device__ static frag ld(const T* p) { return *reinterpret_cast<const frag*>(p); }
  __device__ static frag mk(const float* v) {
    frag f;
#pragma unroll
    for (int e = 0; e < 8; ++e) f[e] = (bf16)v[e];
    return f;
  }
  __device__ static f32x4 mma(frag a, frag b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
};

// v_mfma_f32_16x16x4_f32: lane l holds A[l%16][l/16] and B[l/16][l%16].
struct MmaF32 {
  using T = float;
  using frag = float;
  static constexpr int KS = 4, KPL = 1;
  __device__ static frag ld(const T* p) { return *p; }
  __device__ static frag mk(const float* v) { return v[0]; }
  __device__ static f32x4 mma(frag a, frag b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
  }
};

constexpr int rup(int x, int m) { return (x + m - 1) / m * m; }

// Workspace block of one (chunk, sequence, head). Offsets in elements of T.
template <int C, int DK, int DV, class M>
struct Ws {
  static constexpr int DKP = rup(DK, M::KS);  // K-dims padded to the MFMA depth
  static constexpr int CP = rup(C, M::KS);
  static constexpr size_t oW = 0;                          // -W    [C][DKP]
  static constexpr size_t oQ = oW + (size_t)C * DKP;       // Q~    [C][DKP]
  static constexpr size_t oK = oQ + (size_t)C * DKP;       // K^^T  [DK][CP]
  static constexpr size_t oP = oK + (size_t)DK * CP;       // P     [C][CP]
  static constexpr size_t oU = oP + (size_t)C * CP;        // U'    [C][DV]
  static constexpr size_t nT = oU + (size_t)C * DV;
  static constexpr size_t bytes = nT * sizeof(typename M::T) + DK * sizeof(float);  // + e^{Gam_n}
};

constexpr size_t ws_block_bytes(int C, int DK, int DV, int KS, size_t esz) {
  return ((size_t)C * rup(DK, KS) * 2 + (size_t)DK * rup(C, KS) + (size_t)C * rup(C, KS) +
          (size_t)C * DV) * esz + (size_t)DK * 4;
}

constexpr int kNT = 256;
constexpr int kNW = kNT / kWave;

template <typename IO>
struct Raw {
  const IO* x;      // [B][T][H][d]
  const IO* ring;   // this sequence's ring [3][ctot]
  long ctot;
  int T, H, d, b, h;
  // raw input of channel i (ring channel chan) at global token s
  __device__ float at(int i, long chan, int s) const {
    if (s >= 0) return to_f32(x[(((long)b * T + s) * H + h) * d + i]);
    return to_f32(ring[(long)(3 + s) * ctot + chan]);
  }
  __device__ float act(int i, long chan, f32x4 w, int t, bool conv) const {
    if (!conv) return at(i, chan, t);
    return silu(w.x * at(i, chan, t - 3) + w.y * at(i, chan, t - 2) +
                w.z * at(i, chan, t - 1) + w.w * at(i, chan, t));
  }
};

// ---------------------------------------------------------------------------
// prep: one workgroup per (chunk, head, sequence).
template <int C, int DK, int DV, typename IO, class M>
__global__ __launch_bounds__(kNT) void prefill_prep_kernel(PrefillArgs a, int t0, uint8_t* ws) {
  using L = Ws<C, DK, DV, M>;
  using MT = typename M::T;
  constexpr int LDX = DK + 4, LDL = C + 4;
  constexpr int DKP = L::DKP, CP = L::CP;
  __shared__ float sQ[C][LDX], sK[C][LDX], sG[C][LDX], sL[C][LDL], sBeta[C];

  const int cl = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid % kWave, wv = tid / kWave;
  const int H = a.H, T = a.T;
  const int tstart = t0 + cl * C;
  const int n = min(C, T - tstart);
  MT* blk = reinterpret_cast<MT*>(ws + ((size_t)cl * a.B * H + (size_t)b * H + h) * L::bytes);
  float* Dn = reinterpret_cast<float*>(blk + L::nT);
  const long ctot = (long)H * (2 * DK + DV);
  const bool do_conv = !(a.flags & KDA_F_SKIP_CONV);
  const bool do_l2 = !(a.flags & KDA_F_SKIP_L2);
  const IO* ring = static_cast<const IO*>(a.ring) + (long)b * 3 * ctot;
  const Raw<IO> rq{static_cast<const IO*>(a.q), ring, ctot, T, H, DK, b, h};
  const Raw<IO> rk{static_cast<const IO*>(a.k), ring, ctot, T, H, DK, b, h};
  const Raw<IO> rv{static_cast<const IO*>(a.v), ring, ctot, T, H, DV, b, h};

  // (1) q^, k^ of every token of the chunk (zero rows past n)
  {
    constexpr int U = (DK + kWave - 1) / kWave;
    f32x4 wq[U], wk[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int i = lane + u * kWave;
      wq[u] = wk[u] = f32x4{0.f, 0.f, 0.f, 0.f};
      if (do_conv && i < DK) {
        wq[u] = *reinterpret_cast<const f32x4*>(a.conv_w + 4 * ((long)h * DK + i));
        wk[u] = *reinterpret_cast<const f32x4*>(a.conv_w + 4 * ((long)H * DK + (long)h * DK + i));
      }
    }
    for (int r = wv; r < C; r += kNW) {
      float qv[U], kv[U];
      float ssq = 0.f, ssk = 0.f;
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int i = lane + u * kWave;
        qv[u] = kv[u] = 0.f;
        if (r < n && i < DK) {
          qv[u] = rq.act(i, (long)h * DK + i, wq[u], tstart + r, do_conv);
          kv[u] = rk.act(i, (long)H * DK + (long)h * DK + i, wk[u], tstart + r, do_conv);
        }
        ssq += qv[u] * qv[u];
        ssk += kv[u] * kv[u];
      }
      float iq = 1.f, ik = 1.f;
      if (do_l2) {
        iq = 1.0f / sqrtf(wave_sum(ssq) + kL2Eps);
        ik = 1.0f / sqrtf(wave_sum(ssk) + kL2Eps);
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int i = lane + u * kWave;
        if (i < DK) {
          sQ[r][i] = qv[u] * iq;
          sK[r][i] = kv[u] * ik;
        }
      }
    }
  }
  // (2) Gam = inclusive prefix sum of g inside the chunk; beta (0 past n)
  if (tid < DK) {
    const float* gp = a.g + (((long)b * T + tstart) * H + h) * DK + tid;
    float acc = 0.f;
#pragma unroll 8
    for (int r = 0; r < C; ++r) {
      if (r < n) acc += gp[(long)r * H * DK];
      sG[r][tid] = acc;
    }
  }
  if (tid >= kNT - C) {
    const int r = tid - (kNT - C);
    sBeta[r] = r < n ? a.beta[((long)b * T + tstart + r) * H + h] : 0.f;
  }
  __syncthreads();

  // (3) A (scaled by beta, strictly lower) to LDS, P (lower) to the workspace
  {
    constexpr int NRB = C / 16;
    constexpr int NKS = DKP / M::KS;
    const int l16 = lane % 16, koff = (lane / 16) * M::KPL;
    for (int arb = wv; arb < NRB; arb += kNW) {
      const int m = 16 * arb, r = m + l16;
      typename M::frag fk[NKS], fq[NKS];
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        float vk[M::KPL], vq[M::KPL];
#pragma unroll
        for (int e = 0; e < M::KPL; ++e) {
          const int c = ks * M::KS + koff + e;
          vk[e] = vq[e] = 0.f;
          if (c < DK) {
            const float ex = __expf(sG[r][c] - sG[m][c]);
            vk[e] = sK[r][c] * ex;
            vq[e] = sQ[r][c] * ex;
          }
        }
        fk[ks] = M::mk(vk);
        fq[ks] = M::mk(vq);
      }
      for (int bc = 0; bc < NRB; ++bc) {
        f32x4 accA = {0.f, 0.f, 0.f, 0.f}, accP = {0.f, 0.f, 0.f, 0.f};
        if (bc <= arb) {
          const int j = 16 * bc + l16;
#pragma unroll
          for (int ks = 0; ks < NKS; ++ks) {
            float vc[M::KPL];
#pragma unroll
            for (int e = 0; e < M::KPL; ++e) {
              const int c = ks * M::KS + koff + e;
              vc[e] = c < DK ? sK[j][c] * __expf(sG[m][c] - sG[j][c]) : 0.f;
            }
            const typename M::frag fc = M::mk(vc);
            accA = M::mma(fk[ks], fc, accA);
            accP = M::mma(fq[ks], fc, accP);
          }
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int rr = m + 4 * (lane / 16) + e, jj = 16 * bc + l16;
          sL[rr][jj] = jj < rr ? sBeta[rr] * accA[e] : 0.f;
          blk[L::oP + (size_t)rr * CP + jj] = (MT)(jj <= rr ? accP[e] : 0.f);
        }
      }
    }
    if constexpr (CP > C) {
      for (int idx = tid; idx < C * (CP - C); idx += kNT)
        blk[L::oP + (size_t)(idx / (CP - C)) * CP + C + idx % (CP - C)] = (MT)0.f;
    }
  }
  __syncthreads();

  // (4) W and U' by forward substitution, one column per thread:
  //     (I + L) x = beta * rhs,  L = diag(beta) strict_lower(A)
  for (int col = tid; col < DK + DV; col += kNT) {
    float x[C];
    if (col < DK) {
#pragma unroll
      for (int r = 0; r < C; ++r) x[r] = sBeta[r] * __expf(sG[r][col]) * sK[r][col];
    } else {
      const int jv = col - DK;
      const long chan = 2L * H * DK + (long)h * DV + jv;
      f32x4 w = {0.f, 0.f, 0.f, 1.f};
      float p0 = 0.f, p1 = 0.f, p2 = 0.f;  // raw tokens t-3, t-2, t-1
      if (do_conv) {
        w = *reinterpret_cast<const f32x4*>(a.conv_w + 4 * chan);
        p0 = rv.at(jv, chan, tstart - 3);
        p1 = rv.at(jv, chan, tstart - 2);
        p2 = rv.at(jv, chan, tstart - 1);
      }
#pragma unroll
      for (int r = 0; r < C; ++r) {
        const float xr = r < n ? rv.at(jv, chan, tstart + r) : 0.f;
        const float y = do_conv ? silu(w.x * p0 + w.y * p1 + w.z * p2 + w.w * xr) : xr;
        p0 = p1;
        p1 = p2;
        p2 = xr;
        x[r] = sBeta[r] * y;
      }
    }
#pragma unroll
    for (int r = 1; r < C; ++r) {
      float acc = x[r];
#pragma unroll
      for (int j = 0; j < r; ++j) acc -= sL[r][j] * x[j];
      x[r] = acc;
    }
    if (col < DK) {
#pragma unroll
      for (int r = 0; r < C; ++r) blk[L::oW + (size_t)r * DKP + col] = (MT)(-x[r]);
    } else {
#pragma unroll
      for (int r = 0; r < C; ++r) blk[L::oU + (size_t)r * DV + (col - DK)] = (MT)x[r];
    }
  }
  // (5) Q~ = e^{Gam} q^, K^^T = (e^{Gam_n - Gam} k^)^T, e^{Gam_n}; K-pads zeroed
  for (int idx = tid; idx < C * DKP; idx += kNT) {
    const int r = idx / DKP, c = idx % DKP;
    blk[L::oQ + idx] = (MT)(c < DK ? __expf(sG[r][c]) * sQ[r][c] : 0.f);
    if (c >= DK) blk[L::oW + idx] = (MT)0.f;
  }
  for (int idx = tid; idx < DK * CP; idx += kNT) {
    const int c = idx / CP, j = idx % CP;
    blk[L::oK + idx] = (MT)(j < C ? __expf(sG[C - 1][c] - sG[j][c]) * sK[j][c] : 0.f);
  }
  if (tid < DK) Dn[tid] = __expf(sG[C - 1][tid]);
}

// ---------------------------------------------------------------------------
// chain: one workgroup per (dv-block, head, sequence); walks the chunks.
template <int C, int DK, int DV, int DVB, typename IO, class M>
__global__ __launch_bounds__(kNT) void prefill_chain_kernel(PrefillArgs a, int t0, int ncs,
                                                            const uint8_t* ws) {
  using L = Ws<C, DK, DV, M>;
  using MT = typename M::T;
  constexpr int DKP = L::DKP, CP = L::CP;
  constexpr int NCB = DVB / 16;                 // 16-wide column tiles per block
  constexpr int NU = (C / 16) * NCB;            // tiles of U and O
  constexpr int NS = (DK / 16) * NCB;           // tiles of S
  constexpr int UPW = (NU + kNW - 1) / kNW, SPW = (NS + kNW - 1) / kNW;
  constexpr int PAD = 16 / (int)sizeof(MT);
  constexpr int LDST = DKP + PAD, LDUT = CP + PAD;
  __shared__ __attribute__((aligned(16))) MT sST[DVB][LDST];  // S^T (bf16 or fp32)
  __shared__ __attribute__((aligned(16))) MT sUT[DVB][LDUT];  // U^T

  const int H = a.H, T = a.T, B = a.B;
  constexpr int nblk = DV / DVB;
  // Workgroup -> (column block, head, sequence). Workgroups are dealt to the
  // 8 XCDs round-robin; when the (h, b) count allows it, the nblk column
  // blocks of one head land on the same XCD so they share its L2 copy of
  // the head's workspace.
  int cbk, hb;
  const int L1 = blockIdx.x;
  const int HB = H * B;
  if (HB % 8 == 0) {
    const int xcd = L1 % 8, s = L1 / 8;
    cbk = s % nblk;
    hb = (s / nblk) * 8 + xcd;
  } else {
    cbk = L1 % nblk;
    hb = L1 / nblk;
  }
  const int h = hb % H, b = hb / H;
  const int cb0 = cbk * DVB;
  const int tid = threadIdx.x, lane = tid % kWave, wv = tid / kWave;
  const int l16 = lane % 16, koff = (lane / 16) * M::KPL, r4 = 4 * (lane / 16);

  for (int idx = tid; idx < DVB * LDST; idx += kNT) (&sST[0][0])[idx] = (MT)0.f;
  for (int idx = tid; idx < DVB * LDUT; idx += kNT) (&sUT[0][0])[idx] = (MT)0.f;

  float* Sg = a.S + ((long)b * H + h) * DK * DV + cb0;
  f32x4 accS[SPW];
#pragma unroll
  for (int sl = 0; sl < SPW; ++sl) {
    const int s = wv + kNW * sl;
    accS[sl] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (s < NS) {
      const int i0 = 16 * (s / NCB) + r4, col = 16 * (s % NCB) + l16;
#pragma unroll
      for (int e = 0; e < 4; ++e) accS[sl][e] = Sg[(long)(i0 + e) * DV + col];
    }
  }
  __syncthreads();

  for (int cl = 0; cl < ncs; ++cl) {
    const MT* blk = reinterpret_cast<const MT*>(ws + ((size_t)cl * B * H + (size_t)b * H + h) * L::bytes);
    const float* Dn = reinterpret_cast<const float*>(blk + L::nT);
    const int tstart = t0 + cl * C;
    const int n = min(C, T - tstart);

    // (i) S -> LDS, transposed, in the MFMA operand type
#pragma unroll
    for (int sl = 0; sl < SPW; ++sl) {
      const int s = wv + kNW * sl;
      if (s < NS) {
        const int i0 = 16 * (s / NCB) + r4, col = 16 * (s % NCB) + l16;
#pragma unroll
        for (int e = 0; e < 4; ++e) sST[col][i0 + e] = (MT)accS[sl][e];
      }
    }
    __syncthreads();

    // (ii) U = U' - W S and O = Q~ S
    f32x4 accO[UPW];
#pragma unroll
    for (int sl = 0; sl < UPW; ++sl) {
      const int u = wv + kNW * sl;
      accO[sl] = f32x4{0.f, 0.f, 0.f, 0.f};
      if (u < NU) {
        const int rb = u / NCB, cbt = u % NCB;
        const int col = 16 * cbt + l16;
        f32x4 accU;
#pragma unroll
        for (int e = 0; e < 4; ++e)
          accU[e] = to_f32(blk[L::oU + (size_t)(16 * rb + r4 + e) * DV + cb0 + col]);
        const MT* wrow = blk + L::oW + (size_t)(16 * rb + l16) * DKP + koff;
        const MT* qrow = blk + L::oQ + (size_t)(16 * rb + l16) * DKP + koff;
        const MT* srow = &sST[col][koff];
#pragma unroll
        for (int ks = 0; ks < DKP / M::KS; ++ks) {
          const typename M::frag fs = M::ld(srow + ks * M::KS);
          accU = M::mma(M::ld(wrow + ks * M::KS), fs, accU);
          accO[sl] = M::mma(M::ld(qrow + ks * M::KS), fs, accO[sl]);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) sUT[col][16 * rb + r4 + e] = (MT)accU[e];
      }
    }
    __syncthreads();

    // (iii) O += P U (store), S = Diag(e^{Gam_n}) S + K^^T U
#pragma unroll
    for (int sl = 0; sl < UPW; ++sl) {
      const int u = wv + kNW * sl;
      if (u < NU) {
        const int rb = u / NCB, cbt = u % NCB;
        const int col = 16 * cbt + l16;
        const MT* prow = blk + L::oP + (size_t)(16 * rb + l16) * CP + koff;
        const MT* urow = &sUT[col][koff];
#pragma unroll
        for (int ks = 0; ks < CP / M::KS; ++ks)
          accO[sl] = M::mma(M::ld(prow + ks * M::KS), M::ld(urow + ks * M::KS), accO[sl]);
        IO* op = static_cast<IO*>(a.o) + (((long)b * T + tstart) * H + h) * DV + cb0 + col;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 16 * rb + r4 + e;
          if (r < n) op[(long)r * H * DV] = from_f32<IO>(accO[sl][e]);
        }
      }
    }
#pragma unroll
    for (int sl = 0; sl < SPW; ++sl) {
      const int s = wv + kNW * sl;
      if (s < NS) {
        const int rb = s / NCB, cbt = s % NCB;
        const int col = 16 * cbt + l16;
#pragma unroll
        for (int e = 0; e < 4; ++e) accS[sl][e] *= Dn[16 * rb + r4 + e];
        const MT* krow = blk + L::oK + (size_t)(16 * rb + l16) * CP + koff;
        const MT* urow = &sUT[col][koff];
#pragma unroll
        for (int ks = 0; ks < CP / M::KS; ++ks)
          accS[sl] = M::mma(M::ld(krow + ks * M::KS), M::ld(urow + ks * M::KS), accS[sl]);
      }
    }
  }

#pragma unroll
  for (int sl = 0; sl < SPW; ++sl) {
    const int s = wv + kNW * sl;
    if (s < NS) {
      const int i0 = 16 * (s / NCB) + r4, col = 16 * (s % NCB) + l16;
#pragma unroll
      for (int e = 0; e < 4; ++e) Sg[(long)(i0 + e) * DV + col] = accS[sl][e];
    }
  }
}

template <int C, int DK, int DV, typename IO, class M>
hipError_t run(const PrefillArgs& a, uint8_t* ws, size_t ws_bytes, hipStream_t st) {
  using L = Ws<C, DK, DV, M>;
  constexpr int DVB = DV < 32 ? DV : 32;
  const size_t per_chunk = L::bytes * a.B * a.H;
  const int nchunks = (a.T + C - 1) / C;
  int seg = (int)(ws_bytes / per_chunk);
  if (seg < 1) return hipErrorInvalidValue;
  if (seg > nchunks) seg = nchunks;
  for (int c0 = 0; c0 < nchunks; c0 += seg) {
    const int ncs = nchunks - c0 < seg ? nchunks - c0 : seg;
    const int t0 = c0 * C;
    hipLaunchKernelGGL((prefill_prep_kernel<C, DK, DV, IO, M>), dim3(ncs, a.H, a.B), dim3(kNT),
                       0, st, a, t0, ws);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((prefill_chain_kernel<C, DK, DV, DVB, IO, M>),
                       dim3((DV / DVB) * a.H * a.B), dim3(kNT), 0, st, a, t0, ncs,
                       (const uint8_t*)ws);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  return hipSuccess;
}

template <int C, int DK, int DV>
hipError_t run_io(const PrefillArgs& a, kda_dtype io, uint8_t* ws, size_t n, hipStream_t st) {
  if (io == KDA_BF16) return run<C, DK, DV, bf16, MmaBf16>(a, ws, n, st);
  return run<C, DK, DV, float, MmaF32>(a, ws, n, st);
}

template <int C, int DK>
hipError_t run_dv(const PrefillArgs& a, kda_dtype io, uint8_t* ws, size_t n, hipStream_t st) {
  switch (a.dv) {
    case 16: return run_io<C, DK, 16>(a, io, ws, n, st);
    case 32: return run_io<C, DK, 32>(a, io, ws, n, st);
    case 64: return run_io<C, DK, 64>(a, io, ws, n, st);
    case 128: return run_io<C, DK, 128>(a, io, ws, n, st);
  }
  return hipErrorInvalidValue;
}

template <int C>
hipError_t run_dk(const PrefillArgs& a, kda_dtype io, uint8_t* ws, size_t n, hipStream_t st) {
  switch (a.dk) {
    case 16: return run_dv<C, 16>(a, io, ws, n, st);
    case 32: return run_dv<C, 32>(a, io, ws, n, st);
    case 64: return run_dv<C, 64>(a, io, ws, n, st);
    case 128: return run_dv<C, 128>(a, io, ws, n, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace

size_t prefill_ws_bytes_per_chunk(int H, int B, int dk, int dv, int chunk, kda_dtype io) {
  const int ks = io == KDA_BF16 ? MmaBf16::KS : MmaF32::KS;
  const size_t esz = io == KDA_BF16 ? 2 : 4;
  return ws_block_bytes(chunk, dk, dv, ks, esz) * (size_t)H * (size_t)B;
}

hipError_t launch_prefill(const PrefillArgs& a, kda_dtype io, void* ws, size_t ws_bytes,
                          hipStream_t stream) {
  uint8_t* w = static_cast<uint8_t*>(ws);
  switch (a.chunk) {
    case 16: return run_dk<16>(a, io, w, ws_bytes, stream);
    case 32: return run_dk<32>(a, io, w, ws_bytes, stream);
    case 64: return run_dk<64>(a, io, w, ws_bytes, stream);
  }
  return hipErrorInvalidValue;
}

static_assert(Ws<64, 128, 128, MmaBf16>::bytes == ws_block_bytes(64, 128, 128, 32, 2), "");
static_assert(Ws<16, 16, 16, MmaBf16>::bytes == ws_block_bytes(16, 16, 16, 32, 2), "");
static_assert(Ws<16, 32, 64, MmaF32>::bytes == ws_block_bytes(16, 32, 64, 4, 4), "");

}  // namespace kda
