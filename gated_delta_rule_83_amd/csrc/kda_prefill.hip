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
// Overflow-safe Gram matrices, for any g <= 0 (-inf included): no factor is
// the exponential of a positive number. For j in an earlier 16-token block b
// than r's block a, e^{Gam_r - Gam_j} is the product of the row factor
// e^{Gam_r - Gam_m(a)}, the block factor e^{Gam_m(a) - Gam_e(b)} and the
// column factor e^{Gam_e(b) - Gam_j} (m = a block's first token, e = its
// last), each <= 1, and those tiles run on MFMA. Pairs inside one block are
// formed explicitly as sums over channels of k_r k_j (or q_r k_j) times the
// product of e^{g} over tokens j+1 .. r. Every exponent is a sum of decays of
// one sign, so a very large decay costs no precision through cancellation.
#include "kda_prefill.h"

namespace kda {
namespace {

// ---------------------------------------------------------------------------
// prep: one workgroup of 512 threads per (chunk, head, sequence) item.
// (A persistent variant that loaded the next item's inputs into registers
// during the current item was measured: the loop-carried registers spill and
// the gain was small.)
constexpr int kPrepNT = 512;
constexpr int kPrepNW = kPrepNT / kWave;

// n consecutive fp32 LDS values (16-byte aligned when n is a multiple of 4)
template <int N>
__device__ __forceinline__ void lds_rd(const float* p, float (&v)[N]) {
  if constexpr (N % 4 == 0) {
#pragma unroll
    for (int i = 0; i < N / 4; ++i) {
      const f32x4 t = reinterpret_cast<const f32x4*>(p)[i];
      v[4 * i] = t[0]; v[4 * i + 1] = t[1]; v[4 * i + 2] = t[2]; v[4 * i + 3] = t[3];
    }
  } else {
#pragma unroll
    for (int i = 0; i < N; ++i) v[i] = p[i];
  }
}

// eight values to 16-byte aligned LDS in the operand type
__device__ __forceinline__ void st8(bf16* p, const float* v) {
  bf16x8 t;
#pragma unroll
  for (int e = 0; e < 8; ++e) t[e] = (bf16)v[e];
  *reinterpret_cast<bf16x8*>(p) = t;
}
__device__ __forceinline__ void st8(float* p, const float* v) {
  reinterpret_cast<f32x4*>(p)[0] = f32x4{v[0], v[1], v[2], v[3]};
  reinterpret_cast<f32x4*>(p)[1] = f32x4{v[4], v[5], v[6], v[7]};
}

// Eight values of one channel row of a transposed tile, held in registers in
// the operand type until written as one (bf16) or two (fp32) 16-byte pieces.
template <typename MT> struct VTile;
template <> struct VTile<bf16> {
  using type = bf16x8;
  __device__ static void set(type& t, int i, float v) { t[i] = (bf16)v; }
  __device__ static void store(bf16* p, const type& t) { *reinterpret_cast<bf16x8*>(p) = t; }
};
template <> struct VTile<float> {
  struct type { float v[8]; };
  __device__ static void set(type& t, int i, float v) { t.v[i] = v; }
  __device__ static void store(float* p, const type& t) { st8(p, t.v); }
};

// Eight consecutive token elements as 16-byte pieces: one for bf16, two for fp32.
template <typename IO> struct Tok8 {
  static constexpr int NP = sizeof(IO) == 2 ? 1 : 2;  // 16-byte pieces per 8 elements
  __device__ static void load(const IO* p, f32x4* dst) {
#pragma unroll
    for (int i = 0; i < NP; ++i) dst[i] = reinterpret_cast<const f32x4*>(p)[i];
  }
  __device__ static float get(const f32x4* src, int e) {
    if constexpr (sizeof(IO) == 2) {
      const bf16x8 v = __builtin_bit_cast(bf16x8, src[0]);
      return (float)v[e];
    } else {
      return src[e / 4][e % 4];
    }
  }
};

template <int C, int DK, int DV, typename IO, class M>
struct PrepSmem {
  using MT = typename M::T;
  static constexpr int DKP = rup(DK, M::KS), CP = rup(C, M::KS);
  static constexpr int NRB = C / 16;
  static constexpr int LDK = DK + 4, LDC = C + 4;                 // fp32 row strides
  static constexpr int LDT = CP + (sizeof(MT) == 2 ? 8 : 0);      // MT rows over tokens
  static constexpr size_t mx(size_t a, size_t b) { return a > b ? a : b; }
  // Q: q^ (fp32), later (beta e^Gam k^)^T as MT [DK][LDT]
  static constexpr size_t oQ = 0, nQ = mx((size_t)C * LDK * 4, (size_t)DK * LDT * sizeof(MT));
  // K: k^ (fp32), later -W staging as MT [C][LDW] (rows padded by 16 bytes so
  // that the 16 rows of a fragment read fall in different LDS banks)
  static constexpr int LDW = DKP + 16 / (int)sizeof(MT);
  static constexpr size_t oK = oQ + nQ, nK = mx((size_t)C * LDK * 4, (size_t)C * LDW * sizeof(MT));
  // R: the decays g (fp32), then k^ E with E = e^{Gam_e - Gam_r} (the column
  // factors), later X (fp32 [C][LDC]) then X as MT [C][LDT]
  static constexpr size_t oR = oK + nK;
  static constexpr size_t oXb = oR + (size_t)C * LDC * 4;
  static constexpr size_t nR = mx((size_t)C * LDK * 4, (size_t)C * LDC * 4 + (size_t)C * LDT * sizeof(MT));
  // L: beta * strict_lower(A) (fp32 [C][LDC]); before that, the g strip sums
  static constexpr size_t oL = oR + nR;
  static constexpr size_t nL = mx((size_t)C * LDC * 4, (size_t)2 * NRB * DK * 4);
  static constexpr size_t oV = oL + nL;                              // (beta v^)^T as MT [DV][LDT]
  static constexpr size_t oB = oV + (size_t)DV * LDT * sizeof(MT);   // beta [C]
  // block decays: EB[a] = e^{Gam_m(a)}, EN[a] = e^{Gam_{C-1} - Gam_e(a)},
  // BT[a][b] = e^{Gam_m(a) - Gam_e(b)} for b < a
  static constexpr size_t oE = oB + (size_t)C * 4;
  static constexpr int NBT = NRB * (NRB - 1) / 2;
  static constexpr size_t bytes = oE + (size_t)(2 * NRB + NBT) * DK * 4;
  static_assert(bytes <= 160 * 1024, "prep LDS exceeds 160 KiB");
};

// thread roles of the load/activation phase
template <int C, int DK, int DV, typename IO>
struct PrepRoles {
  static constexpr int QS = 8;                         // tokens per q/k/v strip
  static constexpr int NQ = (DK / 8) * (C / QS);       // q threads (8 channels x 8 tokens)
  static constexpr int NV = (DV / 8) * (C / QS);       // v threads
  static constexpr int GS = 16;                        // tokens per g strip (= one 16-row block)
  static constexpr int NG = (DK / 4) * (C / GS);       // g threads (4 channels x 16 tokens)
  static constexpr int QB = (QS + 3) * Tok8<IO>::NP;   // 16-byte pieces per q/k/v thread
  static constexpr int NBUF = QB > GS ? QB : GS;
  static_assert(2 * NQ + NV + NG <= kPrepNT, "not enough threads for the load roles");
};

// CONV: the short convolution is applied (a compile-time switch, so that the
// unrolled activation loop carries no branches).
template <int C, int DK, int DV, typename IO, class M, bool CONV>
__global__ __launch_bounds__(kPrepNT) void prefill_prep_kernel(PrefillArgs a, int t0, int ncs,
                                                               uint8_t* ws) {
  using L = Ws<C, DK, DV, M>;
  using SM = PrepSmem<C, DK, DV, IO, M>;
  using RO = PrepRoles<C, DK, DV, IO>;
  using MT = typename M::T;
  using frag = typename M::frag;
  constexpr int LDK = SM::LDK, LDC = SM::LDC, LDT = SM::LDT;
  constexpr int DKP = L::DKP, CP = L::CP;
  constexpr int NRB = C / 16;
  constexpr int KS = M::KS, KPL = M::KPL;
  constexpr int QS = RO::QS, GS = RO::GS, NQ = RO::NQ, NV = RO::NV, NG = RO::NG;
  __shared__ __attribute__((aligned(16))) uint8_t smem[SM::bytes];
  float (*sQ)[LDK] = reinterpret_cast<float (*)[LDK]>(smem + SM::oQ);
  MT (*sKT)[LDT] = reinterpret_cast<MT (*)[LDT]>(smem + SM::oQ);
  float (*sK)[LDK] = reinterpret_cast<float (*)[LDK]>(smem + SM::oK);
  MT (*sWst)[SM::LDW] = reinterpret_cast<MT (*)[SM::LDW]>(smem + SM::oK);
  float (*sR)[LDK] = reinterpret_cast<float (*)[LDK]>(smem + SM::oR);
  float (*sX)[LDC] = reinterpret_cast<float (*)[LDC]>(smem + SM::oR);
  MT (*sXb)[LDT] = reinterpret_cast<MT (*)[LDT]>(smem + SM::oXb);
  float (*sL)[LDC] = reinterpret_cast<float (*)[LDC]>(smem + SM::oL);
  float (*sTot)[DK] = reinterpret_cast<float (*)[DK]>(smem + SM::oL);
  float (*sFirst)[DK] = reinterpret_cast<float (*)[DK]>(smem + SM::oL + (size_t)NRB * DK * 4);
  MT (*sVT)[LDT] = reinterpret_cast<MT (*)[LDT]>(smem + SM::oV);
  float* sB = reinterpret_cast<float*>(smem + SM::oB);
  float (*sEB)[DK] = reinterpret_cast<float (*)[DK]>(smem + SM::oE);
  float (*sEN)[DK] = reinterpret_cast<float (*)[DK]>(smem + SM::oE + (size_t)NRB * DK * 4);
  float (*sBT)[DK] = reinterpret_cast<float (*)[DK]>(smem + SM::oE + (size_t)2 * NRB * DK * 4);

  const int tid = threadIdx.x, lane = tid % kWave, wv = tid / kWave;
  const int l16 = lane % 16, g16 = lane / 16;
  const int H = a.H, T = a.T;
  const long ctot = (long)H * (2 * DK + DV);
  const bool do_l2 = !(a.flags & KDA_F_SKIP_L2);
  const int nitems = ncs * H * a.B;

  // role of this thread in the load/activation phase
  // 0: q, 1: k, 2: v (8 channels x 8 tokens), 3: g (4 channels x 16 tokens), 4: none
  const int role = tid < NQ ? 0 : (tid < 2 * NQ ? 1 : (tid < 2 * NQ + NV ? 2 : (tid < 2 * NQ + NV + NG ? 3 : 4)));
  const int rt = tid - (role == 0 ? 0 : role == 1 ? NQ : role == 2 ? 2 * NQ : 2 * NQ + NV);
  // q, k: channel group fastest (the lanes of one token form a group for the
  // L2 shuffle); v: token strip fastest (the lanes of one channel row write
  // adjacent 16-byte pieces of the transposed tile)
  const int cgn = DK / 8, nst = C / QS;
  const int qc0 = role == 2 ? 8 * (rt / nst) : 8 * (rt % cgn);
  const int qr0 = role == 2 ? QS * (rt % nst) : QS * (rt / cgn);
  const int gc0 = 4 * (rt % (DK / 4)), gs = rt / (DK / 4);  // g: first channel, strip
  const int dproj = role == 2 ? DV : DK;
  const long chan0 = (role == 0 ? 0L : (role == 1 ? (long)H * DK : 2L * H * DK)) + qc0;
  const IO* xproj = static_cast<const IO*>(role == 0 ? a.q : (role == 1 ? a.k : a.v));

  // token-padding columns of the (beta v^)^T tile (when the chunk is shorter
  // than the MFMA depth) are never written per item: zero them once
  if constexpr (CP > C) {
    for (int idx = tid; idx < DV * (CP - C); idx += kPrepNT)
      sVT[idx / (CP - C)][C + idx % (CP - C)] = (MT)0.f;
  }

  f32x4 buf[RO::NBUF];  // raw inputs of the item being loaded
  auto issue_loads = [&](int item) {
    const int cl = item % ncs, h = (item / ncs) % H, b = item / (ncs * H);
    const int tstart = t0 + cl * C;
    if (role <= 2) {
      const IO* xc = xproj + ((long)b * T * H + h) * dproj + qc0;
      const long ts = (long)H * dproj;  // token stride
      const int tok0 = tstart + qr0 - 3;
      if (tok0 >= 0 && tok0 + QS + 2 < T) {  // the whole window is inside the inputs
        const IO* p = xc + (long)tok0 * ts;
#pragma unroll
        for (int i = 0; i < QS + 3; ++i, p += ts) Tok8<IO>::load(p, &buf[i * Tok8<IO>::NP]);
      } else {  // history from the ring before token 0; clamped reads past T
        const IO* ring = static_cast<const IO*>(a.ring) + (long)b * 3 * ctot + chan0 + (long)h * dproj;
#pragma unroll
        for (int i = 0; i < QS + 3; ++i) {
          const int tok = tok0 + i;
          const int tcl = tok < T ? tok : T - 1;
          const IO* src = tcl >= 0 ? xc + (long)tcl * ts
                                   : (CONV ? ring + (long)(3 + tcl) * ctot : xc);
          Tok8<IO>::load(src, &buf[i * Tok8<IO>::NP]);
        }
      }
    } else if (role == 3) {
      const long ts = (long)H * DK;
      const int tok0 = tstart + GS * gs;
      const float* gb = a.g + ((long)b * T * H + h) * DK + gc0;
      if (a.flags & KDA_F_SCALAR_G) {  // one decay for every key channel of the head
        const float* gh = a.g + (long)b * T * H + h;
#pragma unroll
        for (int r = 0; r < GS; ++r) {
          const float gv = gh[(long)min(tok0 + r, T - 1) * H];
          buf[r] = f32x4{gv, gv, gv, gv};
        }
      } else if (tok0 + GS - 1 < T) {
        const float* p = gb + (long)tok0 * ts;
#pragma unroll
        for (int r = 0; r < GS; ++r, p += ts) buf[r] = *reinterpret_cast<const f32x4*>(p);
      } else {
#pragma unroll
        for (int r = 0; r < GS; ++r)
          buf[r] = *reinterpret_cast<const f32x4*>(gb + (long)min(tok0 + r, T - 1) * ts);
      }
    }
  };

  {
    const int item = blockIdx.x;
    if (item >= nitems) return;
    issue_loads(item);
    const int cl = item % ncs, h = (item / ncs) % H, b = item / (ncs * H);
    const int tstart = t0 + cl * C;
    const int n = min(C, T - tstart);
    MT* blk = reinterpret_cast<MT*>(ws + ((size_t)cl * a.B * H + (size_t)b * H + h) * L::bytes);
    float* Dn = reinterpret_cast<float*>(blk + L::nT);

    // ---- 1a. activations from the raw inputs ---------------------------
    if (role <= 2) {
      f32x4 w[8];
#pragma unroll
      for (int e = 0; e < 8; ++e)
        w[e] = CONV ? *reinterpret_cast<const f32x4*>(a.conv_w + 4 * (chan0 + (long)h * dproj + e))
                       : f32x4{0.f, 0.f, 0.f, 1.f};
      float bv[QS];
      typename VTile<MT>::type vt[8];  // (beta v^) for 8 channels x 8 tokens
      if (role == 2) {
#pragma unroll
        for (int r = 0; r < QS; ++r)
          bv[r] = a.beta[((long)b * T + min(tstart + qr0 + r, T - 1)) * H + h];
        if (a.flags & KDA_F_RAW_GATES) {  // raw projection: beta formed here
#pragma unroll
          for (int r = 0; r < QS; ++r) bv[r] = sigmoid(bv[r]);
        }
      }
#pragma unroll
      for (int r = 0; r < QS; ++r) {
        const bool valid = qr0 + r < n;
        float y[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float x3 = Tok8<IO>::get(&buf[(r + 3) * Tok8<IO>::NP], e);
          const float v = CONV
              ? silu(w[e].x * Tok8<IO>::get(&buf[r * Tok8<IO>::NP], e) +
                     w[e].y * Tok8<IO>::get(&buf[(r + 1) * Tok8<IO>::NP], e) +
                     w[e].z * Tok8<IO>::get(&buf[(r + 2) * Tok8<IO>::NP], e) + w[e].w * x3)
              : x3;
          y[e] = valid ? v : 0.f;
        }
        if (role < 2) {
          float ss = 0.f;
#pragma unroll
          for (int e = 0; e < 8; ++e) ss += y[e] * y[e];
#pragma unroll
          for (int off = 1; off < DK / 8; off <<= 1) ss += __shfl_xor(ss, off, kWave);
          const float inv = do_l2 ? __builtin_amdgcn_rsqf(ss + kL2Eps) : 1.0f;
          float* dst = role == 0 ? &sQ[qr0 + r][qc0] : &sK[qr0 + r][qc0];
          reinterpret_cast<f32x4*>(dst)[0] = f32x4{y[0] * inv, y[1] * inv, y[2] * inv, y[3] * inv};
          reinterpret_cast<f32x4*>(dst)[1] = f32x4{y[4] * inv, y[5] * inv, y[6] * inv, y[7] * inv};
        } else {
          const float bb = valid ? bv[r] : 0.f;
#pragma unroll
          for (int e = 0; e < 8; ++e) VTile<MT>::set(vt[e], r, bb * y[e]);
          if (qc0 == 0) sB[qr0 + r] = bb;  // beta, once per token
        }
      }
      if (role == 2) {
        static_assert(QS == 8, "v rows are written as 8-token pieces");
#pragma unroll
        for (int e = 0; e < 8; ++e) VTile<MT>::store(&sVT[qc0 + e][qr0], vt[e]);
      }
    } else if (role == 3) {
      // the strip's decays (0 past the last token) to the R region; its
      // first decay and the sum of the other 15 to sFirst / sTot
      if (a.flags & KDA_F_RAW_GATES) {  // raw projections: the log-decay formed here
#pragma unroll
        for (int r = 0; r < GS; ++r)
          buf[r] = f32x4{log_sigmoid(buf[r].x), log_sigmoid(buf[r].y), log_sigmoid(buf[r].z),
                         log_sigmoid(buf[r].w)};
      }
      f32x4 rest = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int r = 0; r < GS; ++r) {
        const bool valid = GS * gs + r < n;
        const f32x4 gv = valid ? buf[r] : f32x4{0.f, 0.f, 0.f, 0.f};
        if (r == 0) *reinterpret_cast<f32x4*>(&sFirst[gs][gc0]) = gv;
        else rest += gv;
        *reinterpret_cast<f32x4*>(&sR[GS * gs + r][gc0]) = gv;
      }
      *reinterpret_cast<f32x4*>(&sTot[gs][gc0]) = rest;
    }
    __syncthreads();

    // ---- 1b. (g threads) block decays, each the exponential of a sum of
    //          decays over the tokens it spans (first, rest: a block's first
    //          decay and the sum of its other 15): EB[a] = e^{Gam_m(a)},
    //          EN[a] = e^{Gam_{C-1} - Gam_e(a)} over the later blocks,
    //          BT[a][b] = e^{Gam_m(a) - Gam_e(b)} over the gap (b < a), and
    //          e^{Gam_n} to the workspace.
    //          (all threads) the pair terms inside each diagonal 16 x 16 block
    //          explicitly: task (block a, row i, channel group cg) walks the
    //          distance d = 0..15 keeping G = prod of e^{g} over tokens
    //          r-d+1 .. r (r = 16a + i) for its channels cg + 16u, and the 16
    //          lanes of a row sum over channels; lane cg keeps distance cg.
    constexpr int NDT = (NRB * 256 + kPrepNT - 1) / kPrepNT;  // tasks per thread
    constexpr int NCPT = DK / 16;                             // channels per task
    float dA[NDT], dP[NDT];
    if (role == 3) {
      f32x4 fst[NRB], rst[NRB];
#pragma unroll
      for (int b2 = 0; b2 < NRB; ++b2) {
        fst[b2] = *reinterpret_cast<const f32x4*>(&sFirst[b2][gc0]);
        rst[b2] = *reinterpret_cast<const f32x4*>(&sTot[b2][gc0]);
      }
      f32x4 before = {0.f, 0.f, 0.f, 0.f}, after = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int b2 = 0; b2 < NRB; ++b2) {
        if (b2 < gs) before += fst[b2] + rst[b2];
        if (b2 > gs) after += fst[b2] + rst[b2];
      }
      f32x4 eb, en;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        eb[e] = __expf(before[e] + fst[gs][e]);
        en[e] = __expf(after[e]);
      }
      *reinterpret_cast<f32x4*>(&sEB[gs][gc0]) = eb;
      *reinterpret_cast<f32x4*>(&sEN[gs][gc0]) = en;
      f32x4 gap = fst[gs];
#pragma unroll
      for (int b2 = NRB - 1; b2 >= 0; --b2) {
        if (b2 < gs) {
          f32x4 bt;
#pragma unroll
          for (int e = 0; e < 4; ++e) bt[e] = __expf(gap[e]);
          *reinterpret_cast<f32x4*>(&sBT[gs * (gs - 1) / 2 + b2][gc0]) = bt;
          gap += rst[b2] + fst[b2];
        }
      }
      if (gs == 0) {
        f32x4 all = {0.f, 0.f, 0.f, 0.f}, dn;
#pragma unroll
        for (int b2 = 0; b2 < NRB; ++b2) all += fst[b2] + rst[b2];
#pragma unroll
        for (int e = 0; e < 4; ++e) dn[e] = __expf(all[e]);
        *reinterpret_cast<f32x4*>(Dn + gc0) = dn;
      }
    }
#pragma unroll
    for (int u = 0; u < NDT; ++u) {
      dA[u] = dP[u] = 0.f;
      const int task = tid + u * kPrepNT;
      if (task < NRB * 256) {  // whole waves take part or not
        const int ab = task / 256, i = (task / 16) % 16, cg = task % 16;
        const int r = 16 * ab + i;
        float kr[NCPT], qr[NCPT], G[NCPT];
#pragma unroll
        for (int w = 0; w < NCPT; ++w) {
          kr[w] = sK[r][cg + 16 * w];
          qr[w] = sQ[r][cg + 16 * w];
          G[w] = 1.f;
        }
        for (int d = 0; d < 16; ++d) {
          const int j = max(r - d, 16 * ab), jn = max(r - d + 1, 16 * ab + 1);
          float ta = 0.f, tp = 0.f;
#pragma unroll
          for (int w = 0; w < NCPT; ++w) {
            if (d > 0) G[w] *= __expf(sR[jn][cg + 16 * w]);
            const float kg = sK[j][cg + 16 * w] * G[w];
            ta += kr[w] * kg;
            tp += qr[w] * kg;
          }
#pragma unroll
          for (int off = 1; off < 16; off <<= 1) {
            ta += __shfl_xor(ta, off, kWave);
            tp += __shfl_xor(tp, off, kWave);
          }
          if (cg == d) {
            dA[u] = ta;
            dP[u] = tp;
          }
        }
      }
    }
    __syncthreads();

    // ---- 1c. (g threads) the row factors R = e^{Gam_r - Gam_m} and column
    //          factors E = e^{Gam_e - Gam_r} of the strip's tokens (m, e =
    //          the block's first and last token), as sums of the decays
    //          between, applied in place: q^ <- q^ R, k^ <- k^ R and the
    //          R region <- k^ E. (all threads) the diagonal blocks' pair
    //          terms: beta_r A_rj (j < r) to sL, P_rj (j <= r, zero above)
    //          to the workspace.
    if (role == 3) {
      f32x4 gv[GS];
#pragma unroll
      for (int r = 0; r < GS; ++r) gv[r] = *reinterpret_cast<const f32x4*>(&sR[GS * gs + r][gc0]);
      f32x4 run = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int r = 0; r < GS; ++r) {  // R: decays of tokens m+1 .. r
        if (r > 0) run += gv[r];
        f32x4 rv;
#pragma unroll
        for (int e = 0; e < 4; ++e) rv[e] = __expf(run[e]);
        f32x4* pq = reinterpret_cast<f32x4*>(&sQ[GS * gs + r][gc0]);
        f32x4* pk = reinterpret_cast<f32x4*>(&sK[GS * gs + r][gc0]);
        *pq = *pq * rv;
        gv[r] = *pk;             // k^ of token r, for E below
        *pk = gv[r] * rv;
      }
      run = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int r = GS - 1; r >= 0; --r) {  // E: decays of tokens r+1 .. e
        f32x4 ev;
#pragma unroll
        for (int e = 0; e < 4; ++e) ev[e] = __expf(run[e]);
        f32x4* pr = reinterpret_cast<f32x4*>(&sR[GS * gs + r][gc0]);
        run += *pr;              // the decay of token r (still in place)
        *pr = gv[r] * ev;
      }
    }
#pragma unroll
    for (int u = 0; u < NDT; ++u) {
      const int task = tid + u * kPrepNT;
      if (task < NRB * 256) {
        const int ab = task / 256, i = (task / 16) % 16, d = task % 16;
        const int r = 16 * ab + i;
        if (d <= i) {
          if (d > 0) sL[r][r - d] = sB[r] * dA[u];
          blk[L::oP + (size_t)r * CP + (r - d)] = (MT)dP[u];
        } else {
          blk[L::oP + (size_t)r * CP + (r + d - i)] = (MT)0.f;
        }
      }
    }
    __syncthreads();
    // from here on: sQ = q^ R, sK = k^ R, sR = k^ E

    // ---- 2. A (beta-scaled, strictly lower) to LDS and P (lower) to the
    //         workspace: the tiles (a, bc < a) on MFMA; row factors k^ R,
    //         q^ R, column factors k^ E scaled by BT[a][bc] = e^{Gam_m(a) - Gam_e(bc)}
    {
      constexpr int NKS = DKP / KS;
      constexpr int NTILE = NRB * (NRB - 1) / 2;
      for (int tile = wv; tile < NTILE; tile += kPrepNW) {
        int arb = 1, rem = tile;
        while (rem >= arb) { rem -= arb; ++arb; }
        const int bc = rem;
        const int r = 16 * arb + l16, j = 16 * bc + l16;
        const float* bt = &sBT[arb * (arb - 1) / 2 + bc][0];
        f32x4 accA = {0.f, 0.f, 0.f, 0.f}, accP = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
          const int c0 = ks * KS + g16 * KPL;
          float vk[KPL], vq[KPL], vc[KPL];
          if (c0 < DK) {
            lds_rd(&sK[r][c0], vk);
            lds_rd(&sQ[r][c0], vq);
            lds_rd(&sR[j][c0], vc);
            float bv[KPL];
            lds_rd(bt + c0, bv);
#pragma unroll
            for (int e = 0; e < KPL; ++e) vc[e] *= bv[e];
          } else {
#pragma unroll
            for (int e = 0; e < KPL; ++e) vk[e] = vq[e] = vc[e] = 0.f;
          }
          const frag fc = M::mk(vc);
          accA = M::mma(M::mk(vk), fc, accA);
          accP = M::mma(M::mk(vq), fc, accP);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int rr = 16 * arb + 4 * g16 + e, jj = 16 * bc + l16;
          sL[rr][jj] = jj < rr ? sB[rr] * accA[e] : 0.f;
          blk[L::oP + (size_t)rr * CP + jj] = (MT)(jj <= rr ? accP[e] : 0.f);
        }
      }
      for (int idx = tid; idx < C * CP; idx += kPrepNT) {
        const int rr = idx / CP, jj = idx % CP;
        if (jj >= C || jj / 16 > rr / 16) {
          blk[L::oP + idx] = (MT)0.f;
          if (jj < C) sL[rr][jj] = 0.f;
        }
      }
    }

    // ---- 3. Q~ = e^{Gam_m(a)} (q^ R) and K^^T = e^{Gam_n - Gam_e(a)} (k^ E)
    //         (fragment-major) to the workspace ------------------------
    {
      constexpr int NPQ = C * DKP / KPL;
#pragma unroll 1
      for (int pc = tid; pc < NPQ; pc += kPrepNT) {
        const int ln = pc % kWave, frg = pc / kWave;
        const int rb = frg / (DKP / KS), ks = frg % (DKP / KS);
        const int r = 16 * rb + ln % 16, c0 = ks * KS + (ln / 16) * KPL;
        float v[KPL];
        if (c0 < DK) {
          float eb[KPL];
          lds_rd(&sEB[rb][c0], eb);
          lds_rd(&sQ[r][c0], v);
#pragma unroll
          for (int e = 0; e < KPL; ++e) v[e] *= eb[e];
        } else {
#pragma unroll
          for (int e = 0; e < KPL; ++e) v[e] = 0.f;
        }
        M::st(blk + L::oQ + (size_t)pc * KPL, M::mk(v));
      }
      constexpr int NPK = DK * CP / KPL;
#pragma unroll 1
      for (int pc = tid; pc < NPK; pc += kPrepNT) {
        const int ln = pc % kWave, frg = pc / kWave;
        const int rb = frg / (CP / KS), ks = frg % (CP / KS);
        const int c = 16 * rb + ln % 16, j0 = ks * KS + (ln / 16) * KPL;
        float v[KPL];
#pragma unroll
        for (int e = 0; e < KPL; ++e) {
          const int jj = j0 + e;
          v[e] = jj < C ? sEN[jj / 16][c] * sR[jj][c] : 0.f;
        }
        M::st(blk + L::oK + (size_t)pc * KPL, M::mk(v));
      }
    }
    __syncthreads();
    // (beta e^{Gam} k^)^T = (beta e^{Gam_16a} (k^ R))^T into the q^ region
    for (int idx = tid; idx < DK * (CP / 8); idx += kPrepNT) {
      const int c = idx % DK, j0 = 8 * (idx / DK);  // lanes walk channels: no bank conflicts
      float v[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int jj = j0 + e;
        v[e] = jj < C ? sB[jj] * sEB[jj / 16][c] * sK[jj][c] : 0.f;
      }
      st8(&sKT[c][j0], v);
    }
    __syncthreads();

    // ---- 4. X = (I + L)^{-1} -------------------------------------------
    unit_lower_inverse<C, kPrepNT>(sL, sX, tid);
    for (int idx = tid; idx < C * (CP / 8); idx += kPrepNT) {
      const int r = idx / (CP / 8), j0 = 8 * (idx % (CP / 8));
      float v[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = j0 + e < C ? sX[r][j0 + e] : 0.f;
      st8(&sXb[r][j0], v);
    }
    __syncthreads();

    // ---- 5. W = X (beta e^Gam K) and U' = X (beta V) on MFMA ------------
    {
      constexpr int NCBW = DK / 16, NCBU = DV / 16;
      constexpr int NKC = CP / KS;
      frag xa[NRB][NKC];  // the rows of X as A operands, loaded once per wave
#pragma unroll
      for (int rb = 0; rb < NRB; ++rb)
#pragma unroll
        for (int ks = 0; ks < NKC; ++ks) xa[rb][ks] = M::ld(&sXb[16 * rb + l16][ks * KS + g16 * KPL]);
      for (int cbk = wv; cbk < NCBW + NCBU; cbk += kPrepNW) {
        const bool isw = cbk < NCBW;
        const int col = (isw ? cbk : cbk - NCBW) * 16 + l16;
        const MT* brow = isw ? &sKT[col][0] : &sVT[col][0];
        frag fb[NKC];
#pragma unroll
        for (int ks = 0; ks < NKC; ++ks) fb[ks] = M::ld(brow + ks * KS + g16 * KPL);
#pragma unroll
        for (int rb = 0; rb < NRB; ++rb) {
          f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int ks = 0; ks < NKC; ++ks) acc = M::mma(xa[rb][ks], fb[ks], acc);
          if (isw) {
#pragma unroll
            for (int e = 0; e < 4; ++e) sWst[16 * rb + 4 * g16 + e][col] = (MT)(-acc[e]);
          } else {
            MT* dst = blk + L::oU + ((size_t)(rb * NCBU + (cbk - NCBW)) * kWave + lane) * 4;
            M::st4(dst, acc);
          }
        }
      }
      if constexpr (DKP > DK) {
        for (int idx = tid; idx < C * (DKP - DK); idx += kPrepNT)
          sWst[idx / (DKP - DK)][DK + idx % (DKP - DK)] = (MT)0.f;
      }
    }
    __syncthreads();
    {
      constexpr int NPW = C * DKP / KPL;
#pragma unroll 1
      for (int pc = tid; pc < NPW; pc += kPrepNT) {
        const int ln = pc % kWave, frg = pc / kWave;
        const int rb = frg / (DKP / KS), ks = frg % (DKP / KS);
        const int r = 16 * rb + ln % 16, c0 = ks * KS + (ln / 16) * KPL;
        M::st(blk + L::oW + (size_t)pc * KPL, M::ld(&sWst[r][c0]));
      }
    }
  }
}

// ---------------------------------------------------------------------------
// chain: one workgroup of 64*NW threads per (block of DVB columns of S and O,
// head, sequence) walks the chunks in order, keeping its DK x DVB block of S
// in MFMA accumulators. U/O tiles are 16 tokens x 16 columns: when the waves
// divide evenly over the C/16 row blocks and their column tiles, wave w owns
// U/O row block w % (C/16) and a run of column tiles; otherwise row blocks
// w, w + NW, ... and all column tiles. S row blocks of 16 key channels go to
// waves w, w + NW, .... The
// workspace operands of the next PF chunks are in flight to registers while
// the current one runs.
template <int C, int DK, int DVB, int NW>
struct ChainTiling {
  static constexpr int NRU = C / 16, NCB = DVB / 16, NRS = DK / 16;
  // several waves per U/O row block, each with a run of column tiles
  static constexpr bool SPLIT = NW >= NRU && NW % NRU == 0 && NCB % (NW / NRU) == 0;
  static constexpr int RU = SPLIT ? 1 : (NRU + NW - 1) / NW;   // U/O row blocks per wave
  static constexpr int NCBW = SPLIT ? NCB / (NW / NRU) : NCB;  // U/O column tiles per wave
  static constexpr int RS = (NRS + NW - 1) / NW;               // S row blocks per wave
};

template <int C, int DK, int DV, int DVB, int NW, int PF, typename IO, class M>
__global__ __launch_bounds__(kWave * NW) void prefill_chain_kernel(PrefillArgs a, int t0, int ncs,
                                                                   const uint8_t* ws) {
  using L = Ws<C, DK, DV, M>;
  using TL = ChainTiling<C, DK, DVB, NW>;
  using MT = typename M::T;
  using frag = typename M::frag;
  constexpr int NT = kWave * NW;
  constexpr int DKP = L::DKP, CP = L::CP;
  constexpr int KS = M::KS, KPL = M::KPL;
  constexpr int NCB = TL::NCB, NRU = TL::NRU, NRS = TL::NRS;
  constexpr int RU = TL::RU, NCBW = TL::NCBW, RS = TL::RS;
  constexpr int NKS = DKP / KS, NKP = CP / KS;
  constexpr int PAD = 16 / (int)sizeof(MT);
  constexpr int LDST = DKP + PAD, LDUT = CP + PAD;
  __shared__ __attribute__((aligned(16))) MT sST[DVB][LDST];  // S^T
  __shared__ __attribute__((aligned(16))) MT sUT[DVB][LDUT];  // U^T

  const int H = a.H, T = a.T, B = a.B;
  constexpr int nblk = DV / DVB;
  // Workgroup -> (column block, head, sequence). Workgroups are dealt to the
  // 8 XCDs round-robin; when the (h, b) count allows it, the column blocks
  // of one head land on the same XCD and share its L2 copy of the workspace.
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
  const int l16 = lane % 16, koff = (lane / 16) * KPL, r4 = 4 * (lane / 16);
  const int ub0 = TL::SPLIT ? wv % NRU : wv;             // first U/O row block
  const int ct0 = TL::SPLIT ? (wv / NRU) * NCBW : 0;     // first U/O column tile
  auto urb = [&](int i) { return ub0 + (TL::SPLIT ? 0 : NW * i); };
  auto srb = [&](int i) { return wv + NW * i; };
  // row-block guards, compile-time true when the tiling divides
  auto u_ok = [&](int rb) { return TL::SPLIT || (NRU % NW == 0) || rb < NRU; };
  auto s_ok = [&](int rb) { return (NRS % NW == 0) || rb < NRS; };

  for (int idx = tid; idx < DVB * LDST; idx += NT) (&sST[0][0])[idx] = (MT)0.f;
  for (int idx = tid; idx < DVB * LDUT; idx += NT) (&sUT[0][0])[idx] = (MT)0.f;

  struct Frags {
    frag w[RU][NKS], q[RU][NKS], p[RU][NKP], k[RS][NKP];
    typename M::quad u[RU][NCBW];
    f32x4 dn[RS];
  };
  auto load = [&](Frags& f, int cl) {
    const MT* blk =
        reinterpret_cast<const MT*>(ws + ((size_t)cl * B * H + (size_t)b * H + h) * L::bytes);
    const float* Dn = reinterpret_cast<const float*>(blk + L::nT);
#pragma unroll
    for (int i = 0; i < RU; ++i) {
      const int rb = urb(i);
      if (u_ok(rb)) {
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
          f.w[i][ks] = M::ld(blk + L::oW + ((size_t)(rb * NKS + ks) * kWave + lane) * KPL);
          f.q[i][ks] = M::ld(blk + L::oQ + ((size_t)(rb * NKS + ks) * kWave + lane) * KPL);
        }
#pragma unroll
        for (int ks = 0; ks < NKP; ++ks)
          f.p[i][ks] = M::ld(blk + L::oP + (size_t)(16 * rb + l16) * CP + ks * KS + koff);
#pragma unroll
        for (int j = 0; j < NCBW; ++j)
          f.u[i][j] = M::ld4(blk + L::oU +
                             ((size_t)(rb * (DV / 16) + cb0 / 16 + ct0 + j) * kWave + lane) * 4);
      }
    }
#pragma unroll
    for (int i = 0; i < RS; ++i) {
      const int rb = srb(i);
      if (s_ok(rb)) {
#pragma unroll
        for (int ks = 0; ks < NKP; ++ks)
          f.k[i][ks] = M::ld(blk + L::oK + ((size_t)(rb * NKP + ks) * kWave + lane) * KPL);
        f.dn[i] = *reinterpret_cast<const f32x4*>(Dn + 16 * rb + r4);
      }
    }
  };

  float* Sg = a.S + ((long)b * H + h) * DK * DV + cb0;
  f32x4 accS[RS][NCB];
#pragma unroll
  for (int i = 0; i < RS; ++i) {
    const int rb = srb(i);
#pragma unroll
    for (int ct = 0; ct < NCB; ++ct) {
      accS[i][ct] = f32x4{0.f, 0.f, 0.f, 0.f};
      if (s_ok(rb)) {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          accS[i][ct][e] = Sg[(long)(16 * rb + r4 + e) * DV + 16 * ct + l16];
      }
    }
  }
  // One chunk of the chain with the operands in `cur`.
  auto step = [&](const Frags& cur, int cl) {
    const int tstart = t0 + cl * C;
    const int n = min(C, T - tstart);

    // (i) S -> LDS, transposed, in the MFMA operand type
#pragma unroll
    for (int i = 0; i < RS; ++i) {
      const int rb = srb(i);
      if (s_ok(rb)) {
#pragma unroll
        for (int ct = 0; ct < NCB; ++ct)
#pragma unroll
          for (int e = 0; e < 4; ++e) sST[16 * ct + l16][16 * rb + r4 + e] = (MT)accS[i][ct][e];
      }
    }
    __syncthreads();

    // (ii) U = U' - W S and O = Q~ S
    f32x4 accO[RU][NCBW];
#pragma unroll
    for (int i = 0; i < RU; ++i) {
      const int rb = urb(i);
#pragma unroll
      for (int j = 0; j < NCBW; ++j) {
        const int ct = ct0 + j;
        accO[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (!u_ok(rb)) continue;
        f32x4 accU = M::cvt4(cur.u[i][j]);
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
          const frag fs = M::ld(&sST[16 * ct + l16][ks * KS + koff]);
          accU = M::mma(cur.w[i][ks], fs, accU);
          accO[i][j] = M::mma(cur.q[i][ks], fs, accO[i][j]);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) sUT[16 * ct + l16][16 * rb + r4 + e] = (MT)accU[e];
      }
    }
    __syncthreads();

    // (iii) O += P U (stored), S = Diag(e^{Gam_n}) S + K^^T U. Rows past
    // the chunk's last token fall outside the store resource and are dropped.
    const __amdgpu_buffer_rsrc_t orsrc =
        make_rsrc(static_cast<IO*>(a.o) + (((long)b * T + tstart) * H + h) * DV + cb0,
                  n * H * DV * (int)sizeof(IO));
#pragma unroll
    for (int i = 0; i < RU; ++i) {
      const int rb = urb(i);
#pragma unroll
      for (int j = 0; j < NCBW; ++j) {
        const int ct = ct0 + j;
        if (!u_ok(rb)) continue;
#pragma unroll
        for (int ks = 0; ks < NKP; ++ks)
          accO[i][j] = M::mma(cur.p[i][ks], M::ld(&sUT[16 * ct + l16][ks * KS + koff]), accO[i][j]);
#pragma unroll
        for (int e = 0; e < 4; ++e)
          buf_store(orsrc, ((16 * rb + r4 + e) * H * DV + 16 * ct + l16) * (int)sizeof(IO),
                    accO[i][j][e], (IO*)nullptr);
      }
    }
#pragma unroll
    for (int i = 0; i < RS; ++i) {
      const int rb = srb(i);
      if (s_ok(rb)) {
#pragma unroll
        for (int ct = 0; ct < NCB; ++ct) {
#pragma unroll
          for (int e = 0; e < 4; ++e) accS[i][ct][e] *= cur.dn[i][e];
#pragma unroll
          for (int ks = 0; ks < NKP; ++ks)
            accS[i][ct] = M::mma(cur.k[i][ks], M::ld(&sUT[16 * ct + l16][ks * KS + koff]),
                                 accS[i][ct]);
        }
      }
    }
  };
  // PF + 1 named operand sets, rotated by a (PF + 1)x unrolled loop: the
  // loads of chunk c + PF are issued before chunk c runs and waited for only
  // at their first use (no register copies, no wait on the chunk's own
  // stores). Prefetch indices are clamped rather than branched on, so that
  // the loads are unconditional and the wait counts stay exact.
  static_assert(PF == 1 || PF == 2, "prefetch depth");
  Frags f0, f1, f2;
  load(f0, 0);
  if constexpr (PF == 1) {
    __syncthreads();
    for (int cl = 0; cl < ncs; cl += 2) {
      load(f1, min(cl + 1, ncs - 1));
      step(f0, cl);
      if (cl + 1 >= ncs) break;
      load(f0, min(cl + 2, ncs - 1));
      step(f1, cl + 1);
    }
  } else {
    load(f1, min(1, ncs - 1));
    __syncthreads();
    for (int cl = 0; cl < ncs; cl += 3) {
      load(f2, min(cl + 2, ncs - 1));
      step(f0, cl);
      if (cl + 1 >= ncs) break;
      load(f0, min(cl + 3, ncs - 1));
      step(f1, cl + 1);
      if (cl + 2 >= ncs) break;
      load(f1, min(cl + 4, ncs - 1));
      step(f2, cl + 2);
    }
  }

#pragma unroll
  for (int i = 0; i < RS; ++i) {
    const int rb = srb(i);
    if (s_ok(rb)) {
#pragma unroll
      for (int ct = 0; ct < NCB; ++ct)
#pragma unroll
        for (int e = 0; e < 4; ++e) Sg[(long)(16 * rb + r4 + e) * DV + 16 * ct + l16] = accS[i][ct][e];
    }
  }
}

// chain, role-split form for bf16 operands, chunk 64 and d_k, d_v multiples
// of 64: one workgroup of 8 waves per (64-column block, head, sequence).
// Waves 0..3 own U/O row block w (all four column tiles); waves 4..7 own the
// S row blocks w-4, w, w+4, ... (all column tiles). Every workspace operand
// is loaded by exactly one wave, each SIMD runs one wave of each role, and
// the operands of the next two chunks are in flight while a chunk runs.
// Per chunk: S waves write S^T (bf16) to LDS | U/O waves: U = U' - W S,
// O = Q~ S, U^T to LDS | U/O waves: O += P U, store O; S waves:
// S = Diag(e^{Gam_n}) S + K^^T U. Measured at T = 4096, 96 heads of 128x128:
// 134-143 us against 149-165 us for the generic form with 64-column blocks.
template <int DK, int DV, typename IO>
__global__ __launch_bounds__(512) void prefill_chain_roles_kernel(PrefillArgs a, int t0, int ncs,
                                                                  const uint8_t* ws) {
  constexpr int C = 64;
  using M = MmaBf16;
  using L = Ws<C, DK, DV, M>;
  using MT = bf16;
  using frag = bf16x8;
  constexpr int DVB = 64, NCB = DVB / 16, KS = M::KS, KPL = M::KPL;
  constexpr int NKS = DK / KS, NKP = C / KS, RS = DK / 64;
  constexpr int LDST = DK + 8, LDUT = C + 8;
  static_assert(DK % 64 == 0 && DV % 64 == 0 && L::DKP == DK && L::CP == C, "roles chain shape");
  __shared__ __attribute__((aligned(16))) MT sST[DVB][LDST];  // S^T
  __shared__ __attribute__((aligned(16))) MT sUT[DVB][LDUT];  // U^T
  const int H = a.H, T = a.T, B = a.B;
  constexpr int nblk = DV / DVB;
  // Workgroup -> (column block, head, sequence), the column blocks of one
  // head on one XCD when the (h, b) count allows it (as in the generic form).
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
  const int l16 = lane % 16, koff = (lane / 16) * KPL, r4 = 4 * (lane / 16);
  for (int idx = tid; idx < DVB * LDST; idx += 512) (&sST[0][0])[idx] = (MT)0.f;
  for (int idx = tid; idx < DVB * LDUT; idx += 512) (&sUT[0][0])[idx] = (MT)0.f;
  auto block = [&](int cl) {
    return reinterpret_cast<const MT*>(ws + ((size_t)cl * B * H + (size_t)b * H + h) * L::bytes);
  };
  // Three operand sets rotated by a 3x unrolled loop: the loads of chunk
  // c + 2 are issued before chunk c runs; indices are clamped, not branched
  // on, so the loads are unconditional and the wait counts stay exact. Both
  // roles pass the same two barriers per chunk.
  auto walk = [&](auto& f0, auto& f1, auto& f2, auto&& load, auto&& step) {
    load(f0, 0);
    load(f1, min(1, ncs - 1));
    for (int cl = 0; cl < ncs; cl += 3) {
      load(f2, min(cl + 2, ncs - 1));
      step(f0, cl);
      if (cl + 1 >= ncs) break;
      load(f0, min(cl + 3, ncs - 1));
      step(f1, cl + 1);
      if (cl + 2 >= ncs) break;
      load(f1, min(cl + 4, ncs - 1));
      step(f2, cl + 2);
    }
  };
  __syncthreads();
  if (wv < 4) {
    const int rb = wv;  // U/O row block
    struct F {
      frag w[NKS], q[NKS], p[NKP];
      bf16x4 u[NCB];
    };
    auto load = [&](F& f, int cl) {
      const MT* blk = block(cl);
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        f.w[ks] = M::ld(blk + L::oW + ((size_t)(rb * NKS + ks) * kWave + lane) * KPL);
        f.q[ks] = M::ld(blk + L::oQ + ((size_t)(rb * NKS + ks) * kWave + lane) * KPL);
      }
#pragma unroll
      for (int ks = 0; ks < NKP; ++ks)
        f.p[ks] = M::ld(blk + L::oP + (size_t)(16 * rb + l16) * C + ks * KS + koff);
#pragma unroll
      for (int j = 0; j < NCB; ++j)
        f.u[j] = M::ld4(blk + L::oU + ((size_t)(rb * (DV / 16) + cb0 / 16 + j) * kWave + lane) * 4);
    };
    auto step = [&](const F& cur, int cl) {
      const int tstart = t0 + cl * C;
      const int n = min(C, T - tstart);
      __syncthreads();  // S^T of this chunk is in LDS
      f32x4 accO[NCB];
#pragma unroll
      for (int j = 0; j < NCB; ++j) {
        accO[j] = f32x4{0.f, 0.f, 0.f, 0.f};
        f32x4 accU = M::cvt4(cur.u[j]);
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
          const frag fs = M::ld(&sST[16 * j + l16][ks * KS + koff]);
          accU = M::mma(cur.w[ks], fs, accU);
          accO[j] = M::mma(cur.q[ks], fs, accO[j]);
        }
        M::st4(&sUT[16 * j + l16][16 * rb + r4], accU);
      }
      __syncthreads();  // U^T in LDS
      // Rows past the chunk's last token fall outside the store resource.
      const __amdgpu_buffer_rsrc_t orsrc =
          make_rsrc(static_cast<IO*>(a.o) + (((long)b * T + tstart) * H + h) * DV + cb0,
                    n * H * DV * (int)sizeof(IO));
#pragma unroll
      for (int j = 0; j < NCB; ++j) {
#pragma unroll
        for (int ks = 0; ks < NKP; ++ks)
          accO[j] = M::mma(cur.p[ks], M::ld(&sUT[16 * j + l16][ks * KS + koff]), accO[j]);
#pragma unroll
        for (int e = 0; e < 4; ++e)
          buf_store(orsrc, ((16 * rb + r4 + e) * H * DV + 16 * j + l16) * (int)sizeof(IO),
                    accO[j][e], (IO*)nullptr);
      }
    };
    F f0, f1, f2;
    walk(f0, f1, f2, load, step);
  } else {
    const int sw = wv - 4;  // S row blocks sw + 4i
    struct F {
      frag k[RS][NKP];
      f32x4 dn[RS];
    };
    auto load = [&](F& f, int cl) {
      const MT* blk = block(cl);
      const float* Dn = reinterpret_cast<const float*>(blk + L::nT);
#pragma unroll
      for (int i = 0; i < RS; ++i) {
        const int rb = sw + 4 * i;
#pragma unroll
        for (int ks = 0; ks < NKP; ++ks)
          f.k[i][ks] = M::ld(blk + L::oK + ((size_t)(rb * NKP + ks) * kWave + lane) * KPL);
        f.dn[i] = *reinterpret_cast<const f32x4*>(Dn + 16 * rb + r4);
      }
    };
    float* Sg = a.S + ((long)b * H + h) * DK * DV + cb0;
    f32x4 accS[RS][NCB];
#pragma unroll
    for (int i = 0; i < RS; ++i)
#pragma unroll
      for (int ct = 0; ct < NCB; ++ct)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          accS[i][ct][e] = Sg[(long)(16 * (sw + 4 * i) + r4 + e) * DV + 16 * ct + l16];
    auto step = [&](const F& cur, int) {
#pragma unroll
      for (int i = 0; i < RS; ++i)
#pragma unroll
        for (int ct = 0; ct < NCB; ++ct)
          M::st4(&sST[16 * ct + l16][16 * (sw + 4 * i) + r4], accS[i][ct]);
      __syncthreads();  // S^T in LDS
      __syncthreads();  // U^T in LDS
#pragma unroll
      for (int i = 0; i < RS; ++i)
#pragma unroll
        for (int ct = 0; ct < NCB; ++ct) {
#pragma unroll
          for (int e = 0; e < 4; ++e) accS[i][ct][e] *= cur.dn[i][e];
#pragma unroll
          for (int ks = 0; ks < NKP; ++ks)
            accS[i][ct] = M::mma(cur.k[i][ks], M::ld(&sUT[16 * ct + l16][ks * KS + koff]),
                                 accS[i][ct]);
        }
    };
    F f0, f1, f2;
    walk(f0, f1, f2, load, step);
#pragma unroll
    for (int i = 0; i < RS; ++i)
#pragma unroll
      for (int ct = 0; ct < NCB; ++ct)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          Sg[(long)(16 * (sw + 4 * i) + r4 + e) * DV + 16 * ct + l16] = accS[i][ct][e];
  }
  // The conv ring of this head's channels takes the call's last three raw
  // tokens (older ring entries shift down when the call has fewer than three),
  // written by the launch that holds the last chunk, its column blocks
  // splitting the head's q | k | v channels. The preparation, which reads the
  // old ring for the first chunk's history, has finished before this launch.
  if (!(a.flags & KDA_F_SKIP_CONV) && t0 + ncs * C >= T) {
    constexpr int NCH = 2 * DK + DV, PER = (NCH + nblk - 1) / nblk;
    const long ctot = (long)H * NCH;
    MT* rb = static_cast<MT*>(a.ring) + (long)b * 3 * ctot;
    for (int u = tid; u < PER; u += 512) {
      const int ch = cbk * PER + u;
      if (ch >= NCH) break;
      const MT* x;
      int d;
      long c;  // ring channel
      if (ch < DK) {
        x = static_cast<const MT*>(a.q); d = DK; c = (long)h * DK + ch;
      } else if (ch < 2 * DK) {
        x = static_cast<const MT*>(a.k); d = DK; c = (long)H * DK + (long)h * DK + (ch - DK);
      } else {
        x = static_cast<const MT*>(a.v); d = DV; c = 2L * H * DK + (long)h * DV + (ch - 2 * DK);
      }
      const int hc = ch < 2 * DK ? (ch % DK) : ch - 2 * DK;
      MT nw[3];
#pragma unroll
      for (int tap = 0; tap < 3; ++tap) {
        const int s = T - 3 + tap;
        nw[tap] = s >= 0 ? x[(((long)b * T + s) * H + h) * d + hc] : rb[(long)(3 + s) * ctot + c];
      }
#pragma unroll
      for (int tap = 0; tap < 3; ++tap) rb[(long)tap * ctot + c] = nw[tap];
    }
  }
}

template <int C, int DK, int DV, typename IO, class M>
hipError_t run(const PrefillArgs& a, uint8_t* ws, size_t ws_bytes, hipStream_t st) {
  using L = Ws<C, DK, DV, M>;
  // Column block of the chain: 64 columns for bf16 operands (half the
  // re-reads of the shared W, Q~, P, K^^T of 32-column blocks, measured
  // 159 us against 192 us at T = 4096, 96 heads of 128 x 128); 32 for fp32.
  constexpr int DVB = DV < 32 ? DV : (sizeof(IO) == 2 && DV >= 64 ? 64 : 32);
  constexpr int CNW = 4;
  const size_t per_chunk = L::bytes * a.B * a.H;
  const int nchunks = (a.T + C - 1) / C;
  int seg = (int)(ws_bytes / per_chunk);
  if (seg < 1) return hipErrorInvalidValue;
  if (seg > nchunks) seg = nchunks;
  for (int c0 = 0; c0 < nchunks; c0 += seg) {
    const int ncs = nchunks - c0 < seg ? nchunks - c0 : seg;
    const int t0 = c0 * C;
    const long items = (long)ncs * a.H * a.B;
    hipError_t e;
    if (prep_rows_supported(C, DK, DV, sizeof(IO) == 2 ? KDA_BF16 : KDA_F32)) {
      e = launch_prep_rows(a, t0, ncs, ws, st);
    } else {
      if (a.flags & KDA_F_SKIP_CONV)
        hipLaunchKernelGGL((prefill_prep_kernel<C, DK, DV, IO, M, false>), dim3((unsigned)items),
                           dim3(kPrepNT), 0, st, a, t0, ncs, ws);
      else
        hipLaunchKernelGGL((prefill_prep_kernel<C, DK, DV, IO, M, true>), dim3((unsigned)items),
                           dim3(kPrepNT), 0, st, a, t0, ncs, ws);
      e = hipGetLastError();
    }
    if (e != hipSuccess) return e;
    if constexpr (sizeof(IO) == 2 && C == 64 && DK % 64 == 0 && DV % 64 == 0)
      hipLaunchKernelGGL((prefill_chain_roles_kernel<DK, DV, IO>), dim3((DV / 64) * a.H * a.B),
                         dim3(512), 0, st, a, t0, ncs, (const uint8_t*)ws);
    else
      hipLaunchKernelGGL((prefill_chain_kernel<C, DK, DV, DVB, CNW, 1, IO, M>),
                         dim3((DV / DVB) * a.H * a.B), dim3(kWave * CNW), 0, st, a, t0, ncs,
                         (const uint8_t*)ws);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  // the roles chain advances the ring in its last launch; otherwise a kernel of its own
  constexpr bool ring_in_chain = sizeof(IO) == 2 && C == 64 && DK % 64 == 0 && DV % 64 == 0;
  if (!ring_in_chain && !(a.flags & KDA_F_SKIP_CONV))
    return launch_ring_advance(a.q, a.k, a.v, a.ring, a.B, a.T, a.H, a.dk, a.dv,
                               sizeof(IO) == 2 ? KDA_BF16 : KDA_F32, st);
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
