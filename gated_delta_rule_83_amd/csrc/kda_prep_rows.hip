// Chunked-prefill preparation in the token-row layout, for bf16 inputs.
//
// Computes, per (chunk, head, sequence), the S-independent part of the chunk
// recurrence ("为什么 Kimi K3 敢把 KV Cache 扔掉？一篇讲透 GPT-2 到 K3 的架构进化",
// section 5 for the WY form, section 6 for the in-chunk cumulative decay,
// section 7 for KDA's per-channel decay) and writes the same workspace block
// as the general preparation kernel: -W, Q~, K^^T, P, U' and e^{Gam_n}.
//
// Layout. One workgroup of C/16 waves per item; wave w owns tokens
// 16w .. 16w+15 of the chunk, and lane l holds token 16w + l%16 for the
// channels 32s + 8(l/16) + e (e = 0..7) of every 32-channel slice s. A lane's
// eight channels of one slice are exactly its piece of a
// v_mfma_f32_16x16x32_bf16 operand (row l%16, depth 8(l/16)..+7), so the
// activations feed the Gram products from registers. Along a 16-lane DPP
// row the lanes are consecutive tokens, so
//   - the short convolution takes its three history taps with row shifts
//     (lanes 0..2 of a row take the three tokens before the block from LDS:
//     the previous block's last three, or those before the chunk), and
//   - the in-block prefix sums of g are a 4-step row scan.
// Transposes (token-contiguous operands for the contractions over tokens)
// go through MFMAs with a 0/1 selection matrix as B: the product returns
// four consecutive tokens of one channel per lane, exactly, and two lanes
// (l and l^16) pair up into one 16-byte fragment piece.
//
// Decayed pair terms without overflow, for any g <= 0 (-inf included). The
// factor e^{Gam_r - Gam_j} of a pair j <= r (r in 16-token block a, j in
// block b) is the product of a row factor R_r = e^{Gam_r - Gam_m(a)} <= 1
// (m = a block's first token, e = its last), a column factor and a block
// factor, chosen per column block b:
//   - narrow b (no key channel decays by more than kSpan over its last 15
//     tokens): column factor 1/R_j <= e^{kSpan}, block factor
//     e^{Gam_m(a) - Gam_m(b)} (b < a) or 1 (b = a);
//   - wide b: column factor E_j = e^{Gam_e(b) - Gam_j} <= 1 and block factor
//     e^{Gam_m(a) - Gam_e(b)} <= 1 (b < a); its diagonal tile is formed by
//     the block's wave in fp32, as sums over channels of k_r k_j (or q_r k_j)
//     times the running product of e^{g} over tokens j+1 .. r along the DPP
//     row.
// All factors stay within e^{+-kSpan}, and every exponent is a sum of decays
// of one sign, so no cancellation loses precision when one decay is large.
//
// LDS holds only what crosses waves (45 KiB at C = 64, d = 128, in three
// regions reused from phase to phase) and the kernel is held to 168 VGPRs,
// so three items share a CU and one item's loads overlap another's math.
#include "kda_prefill.h"

namespace kda {
namespace {

constexpr int kRowShr = 0x110;  // DPP row_shr:n is kRowShr + n
constexpr int kRowShl = 0x100;  // DPP row_shl:n is kRowShl + n

// Lane value from `CTRL`'s source lane inside the 16-lane row; lanes whose
// source falls outside the row keep `old`.
template <int CTRL>
__device__ __forceinline__ unsigned dpp(unsigned old, unsigned src) {
  return (unsigned)__builtin_amdgcn_update_dpp((int)old, (int)src, CTRL, 0xF, 0xF, false);
}
// Lane value from `CTRL`'s source lane inside the row; 0 where it falls outside.
template <int CTRL>
__device__ __forceinline__ unsigned dpp0(unsigned src) {
  return (unsigned)__builtin_amdgcn_mov_dpp((int)src, CTRL, 0xF, 0xF, true);
}
template <int CTRL>
__device__ __forceinline__ float dppf(float old, float src) {
  return __builtin_bit_cast(float, dpp<CTRL>(__builtin_bit_cast(unsigned, old),
                                             __builtin_bit_cast(unsigned, src)));
}
template <int CTRL>
__device__ __forceinline__ float dpp0f(float src) {
  return __builtin_bit_cast(float, dpp0<CTRL>(__builtin_bit_cast(unsigned, src)));
}

// Largest decay over a block's last 15 tokens (natural log) for which the
// block keeps the column factors 1/R (and its diagonal tile the factored MFMA
// product): the factors then stay within e^{+-kSpan}, far inside the bf16 /
// fp32 range.
constexpr float kSpan = 64.0f;

// Pair terms of a diagonal 16 x 16 tile for the eight channels of one
// slice, distances D0 .. min(D0 + 7, 15): lane i of a DPP row holds token i
// (k, the row-side operand x = k or q, and a = e^{g}). Stepping the distance
// D by one shifts two running values one lane along the row: kj becomes k of
// token i - D, and G = a_i * (G of lane i - 1) the product of a over tokens
// i - D + 1 .. i; sum_c x_i kj G is added to acc[D - D0]. Lanes i < D see
// zeros shifted in from outside the row; their sums are not used.
template <int D0, int NE>
__device__ __forceinline__ void diag_terms(const float* k, const float* x, const float* av,
                                           float (&acc)[8]) {
  float kj[NE], G[NE];
  if constexpr (D0 == 0) {
    float t = 0.f;
#pragma unroll
    for (int e = 0; e < NE; ++e) t += x[e] * k[e];
    acc[0] += t;
  }
#pragma unroll
  for (int e = 0; e < NE; ++e) kj[e] = k[e];
#pragma unroll
  for (int D = 1; D < 16 && D < D0 + 8; ++D) {
    float t = 0.f;
#pragma unroll
    for (int e = 0; e < NE; ++e) {
      kj[e] = dpp0f<kRowShr + 1>(kj[e]);
      G[e] = D == 1 ? av[e] : av[e] * dpp0f<kRowShr + 1>(G[e]);
      t += x[e] * (kj[e] * G[e]);
    }
    // one distance at a time: the sum is formed here and the running values
    // pass through, so no step's shifted copies stay live for later
#pragma unroll
    for (int e = 0; e < NE; ++e) asm volatile("" : "+v"(kj[e]), "+v"(G[e]));
    asm volatile("" : "+v"(t));
    if (D >= D0) acc[D - D0] += t;
  }
}

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

// element e of eight packed bf16 (exact)
__device__ __forceinline__ float bfe(const u32x4& w, int e) {
  const unsigned x = w[e / 2];
  return __builtin_bit_cast(float, (e & 1) ? (x & 0xffff0000u) : (x << 16));
}

__device__ __forceinline__ bf16x8 to_bf16x8(const float* v) {
  bf16x8 t;
#pragma unroll
  for (int e = 0; e < 8; ++e) t[e] = (bf16)v[e];
  return t;
}

template <int C, int DK, int DV>
struct RowsSmem {
  static constexpr int NRB = C / 16, NCH = 2 * DK + DV, NBT = NRB * (NRB - 1) / 2;
  static constexpr int LDC = C + 4, LDT = C + 8;
  static constexpr size_t mx(size_t a, size_t b) { return a > b ? a : b; }
  // A: g of each block's first token and block sums of the rest (fp32
  //    [NRB][DK] each) -> k^/R (fragment-major) -> X (fp32 [C][LDC]) ->
  //    (beta e^Gam k^)^T [DK][LDT]
  static constexpr size_t nA = mx(mx((size_t)2 * NRB * DK * 4, (size_t)C * DK * 2),
                                  mx((size_t)C * LDC * 4, (size_t)DK * LDT * 2));
  // B: conv weights (one 16-byte pad per 8 channels) -> beta A (fp32) -> (beta v^)^T
  static constexpr int NWQ = NCH + NCH / 8;
  static constexpr size_t nB =
      mx(mx((size_t)NWQ * 16, (size_t)C * LDC * 4), (size_t)DV * LDT * 2);
  // C: the raw inputs of the three tokens before each block ([NRB][3][NCH]
  //    bf16) -> block decays EB[a] = e^{Gam_m(a)}, EN[a] = e^{Gam_n - Gam_m(a)}
  //    (narrow a) or e^{Gam_n - Gam_e(a)} (wide a), BT[a][b] (b < a; row
  //    a(a-1)/2 + b) = e^{Gam_m(a) - Gam_m(b)} (narrow b) or
  //    e^{Gam_m(a) - Gam_e(b)} (wide b), fp32 [.][DK] -> X as bf16
  static constexpr size_t nC = mx(mx((size_t)NRB * 3 * NCH * 2, (size_t)(2 * NRB + NBT) * DK * 4),
                                  (size_t)C * LDT * 2);
  static constexpr size_t oB = nA, oC = oB + nB, oF = oC + nC;  // F: a wide flag per block
  static constexpr size_t bytes = oF + 16;
};

// (launch bounds: C/16 waves, at least three waves per SIMD, i.e. three
// items per CU). CONV: the inputs are raw projections (conv + SiLU here);
// SG: g holds one decay per (token, head), shared by all key channels.
// RAW: g and beta are raw projections; the gates are formed on load.
template <int C, int DK, int DV, bool CONV, bool SG, bool RAW>
__global__ __launch_bounds__(C * 4, 3) void prefill_prep_rows_kernel(PrefillArgs a, int t0, int ncs,
                                                                  uint8_t* ws) {
  using M = MmaBf16;
  using L = Ws<C, DK, DV, M>;
  using SM = RowsSmem<C, DK, DV>;
  constexpr int NRB = C / 16, NT = kWave * NRB;
  constexpr int NKS = DK / 32, NVS = DV / 32, NKC = C / 32;
  constexpr int LDC = SM::LDC, LDT = SM::LDT, CP = L::CP;
  static_assert(C % 32 == 0 && DK % 32 == 0 && DV % 32 == 0, "row layout needs 32 | C, dk, dv");
  static_assert(L::DKP == DK && CP == C, "no padding in the row layout");
  static_assert(SM::bytes <= 53 * 1024, "row-layout prep LDS budget (three items per CU)");

  __shared__ __attribute__((aligned(16))) uint8_t smem[SM::bytes];
  bf16* sKi = reinterpret_cast<bf16*>(smem);
  float (*sX)[LDC] = reinterpret_cast<float (*)[LDC]>(smem);
  bf16 (*sKT)[LDT] = reinterpret_cast<bf16 (*)[LDT]>(smem);
  f32x4* sW = reinterpret_cast<f32x4*>(smem + SM::oB);
  float (*sL)[LDC] = reinterpret_cast<float (*)[LDC]>(smem + SM::oB);
  bf16 (*sVT)[LDT] = reinterpret_cast<bf16 (*)[LDT]>(smem + SM::oB);
  bf16 (*sXb)[LDT] = reinterpret_cast<bf16 (*)[LDT]>(smem + SM::oC);
  float (*sFirst)[DK] = reinterpret_cast<float (*)[DK]>(smem);
  float (*sTot)[DK] = reinterpret_cast<float (*)[DK]>(smem + (size_t)NRB * DK * 4);
  bf16 (*sHist)[3][SM::NCH] = reinterpret_cast<bf16 (*)[3][SM::NCH]>(smem + SM::oC);
  float (*sEB)[DK] = reinterpret_cast<float (*)[DK]>(smem + SM::oC);
  float (*sEN)[DK] = reinterpret_cast<float (*)[DK]>(smem + SM::oC + (size_t)NRB * DK * 4);
  float (*sBT)[DK] = reinterpret_cast<float (*)[DK]>(smem + SM::oC + (size_t)2 * NRB * DK * 4);
  int* sWide = reinterpret_cast<int*>(smem + SM::oF);

  const int tid = threadIdx.x, lane = tid % kWave, rb = tid / kWave;
  const int i = lane % 16, gq = lane / 16;
  const int H = a.H, T = a.T;
  // Items run chunk-major from the last chunk to the first (all heads of a
  // chunk together), so that the workspace blocks of the first chunks, which
  // the chain reads first, are the most recently written ones and still sit
  // in the memory-side cache when the chain starts.
  const int item = blockIdx.x;
  const int hbi = item % (H * a.B);
  const int cl = ncs - 1 - item / (H * a.B), h = hbi % H, b = hbi / H;
  const int tstart = t0 + cl * C;
  const int n = min(C, T - tstart);
  const int r = 16 * rb + i;  // this lane's token in the chunk
  const bool valid = r < n;
  const int t = tstart + r;
  const long row = ((long)b * T + min(t, T - 1)) * H + h;  // (b, token, h), clamped
  const bool do_l2 = !(a.flags & KDA_F_SKIP_L2);
  // scale of the activations as computed (see the conv below) and the L2
  // epsilon in that scale: (z ln2) / sqrt(sum (z ln2)^2 + eps) = z / sqrt(sum z^2 + eps / ln2^2)
  constexpr float kLn2 = 0.69314718055994531f, kLog2e = 1.4426950408889634f;
  constexpr float kAct = CONV ? kLn2 : 1.0f;
  constexpr float kEps = CONV ? kL2Eps / (kLn2 * kLn2) : kL2Eps;
  bf16* blk = reinterpret_cast<bf16*>(ws + ((size_t)cl * a.B * H + (size_t)b * H + h) * L::bytes);
  float* Dn = reinterpret_cast<float*>(blk + L::nT);
  // the lane's eight log-decays of slice s as the recurrence applies them
  // (formed from the raw projection with RAW), 0 past the last token
  // (NE = 8: the slice's eight channels; NE = 4: channels 4 h4 .. 4 h4 + 3)
  auto load_decay = [&](int s, int h4, auto nec, float* x) __attribute__((always_inline)) {
    constexpr int NE = decltype(nec)::value;
    if constexpr (SG) {
      const float gv = a.g[row];
#pragma unroll
      for (int e = 0; e < NE; ++e) x[e] = gv;
    } else {
      const float* gp = a.g + row * DK + 32 * s + 8 * gq + 4 * h4;
#pragma unroll
      for (int u = 0; u < NE / 4; ++u) {
        const f32x4 w = *reinterpret_cast<const f32x4*>(gp + 4 * u);
#pragma unroll
        for (int e = 0; e < 4; ++e) x[4 * u + e] = w[e];
      }
    }
#pragma unroll
    for (int e = 0; e < NE; ++e) {
      if constexpr (RAW) x[e] = log_sigmoid(x[e]);
      x[e] = valid ? x[e] : 0.f;
    }
  };

  // ---- 0. loads: conv weights of the head (to LDS), then the lane's token
  //         (q, k, v, g, beta); the conv history of each block to LDS: the
  //         last three tokens of the block before it, or for block 0 the
  //         three tokens before the chunk (from the ring before token 0) -----
  constexpr int NWR = (SM::NCH + NT - 1) / NT;
  f32x4 wreg[NWR];
  if constexpr (CONV) {
#pragma unroll
    for (int u = 0; u < NWR; ++u) {
      const int idx = tid + u * NT;
      if (idx < SM::NCH) {
        const long chan = idx < DK ? (long)h * DK + idx
                        : idx < 2 * DK ? (long)H * DK + (long)h * DK + (idx - DK)
                                       : 2L * H * DK + (long)h * DV + (idx - 2 * DK);
        wreg[u] = *reinterpret_cast<const f32x4*>(a.conv_w + 4 * chan);
      }
    }
  }
  float betav = valid ? a.beta[row] : 0.f;
  const bf16* qsrc = static_cast<const bf16*>(a.q) + row * DK + 8 * gq;
  const bf16* ksrc = static_cast<const bf16*>(a.k) + row * DK + 8 * gq;
  const bf16* vsrc = static_cast<const bf16*>(a.v) + row * DV + 8 * gq;
  u32x4 xq[NKS], xk[NKS], xv[NVS];
  f32x4 gl[NKS][2];
#pragma unroll
  for (int s = 0; s < NKS; ++s) {
    xq[s] = *reinterpret_cast<const u32x4*>(qsrc + 32 * s);
    xk[s] = *reinterpret_cast<const u32x4*>(ksrc + 32 * s);
  }
#pragma unroll
  for (int s = 0; s < NVS; ++s) xv[s] = *reinterpret_cast<const u32x4*>(vsrc + 32 * s);
  if constexpr (SG) {  // one decay for every key channel of the head
    const float gv = a.g[row];
#pragma unroll
    for (int s = 0; s < NKS; ++s) gl[s][0] = gl[s][1] = f32x4{gv, gv, gv, gv};
  } else {
    const float* gsrc = a.g + row * DK + 8 * gq;
#pragma unroll
    for (int s = 0; s < NKS; ++s) {
      gl[s][0] = *reinterpret_cast<const f32x4*>(gsrc + 32 * s);
      gl[s][1] = *reinterpret_cast<const f32x4*>(gsrc + 32 * s + 4);
    }
  }
  if constexpr (CONV) {
    if (rb == 0 && i < 3) {
      const int t3 = tstart - 3 + i;
      const bf16 *q3, *k3, *v3;
      if (t3 >= 0) {
        const long row3 = ((long)b * T + t3) * H + h;
        q3 = static_cast<const bf16*>(a.q) + row3 * DK;
        k3 = static_cast<const bf16*>(a.k) + row3 * DK;
        v3 = static_cast<const bf16*>(a.v) + row3 * DV;
      } else {  // before the first token of the call: the ring, slot 3 + t3
        const long ctot = (long)H * SM::NCH;
        const bf16* ring = static_cast<const bf16*>(a.ring) + ((long)b * 3 + (3 + t3)) * ctot;
        q3 = ring + (long)h * DK;
        k3 = ring + (long)H * DK + (long)h * DK;
        v3 = ring + 2L * H * DK + (long)h * DV;
      }
#pragma unroll
      for (int s = 0; s < NKS; ++s) {
        *reinterpret_cast<u32x4*>(&sHist[0][i][32 * s + 8 * gq]) =
            *reinterpret_cast<const u32x4*>(q3 + 32 * s + 8 * gq);
        *reinterpret_cast<u32x4*>(&sHist[0][i][DK + 32 * s + 8 * gq]) =
            *reinterpret_cast<const u32x4*>(k3 + 32 * s + 8 * gq);
      }
#pragma unroll
      for (int s = 0; s < NVS; ++s)
        *reinterpret_cast<u32x4*>(&sHist[0][i][2 * DK + 32 * s + 8 * gq]) =
            *reinterpret_cast<const u32x4*>(v3 + 32 * s + 8 * gq);
    }
    if (rb + 1 < NRB && i >= 13) {
#pragma unroll
      for (int s = 0; s < NKS; ++s) {
        *reinterpret_cast<u32x4*>(&sHist[rb + 1][i - 13][32 * s + 8 * gq]) = xq[s];
        *reinterpret_cast<u32x4*>(&sHist[rb + 1][i - 13][DK + 32 * s + 8 * gq]) = xk[s];
      }
#pragma unroll
      for (int s = 0; s < NVS; ++s)
        *reinterpret_cast<u32x4*>(&sHist[rb + 1][i - 13][2 * DK + 32 * s + 8 * gq]) = xv[s];
    }
#pragma unroll
    for (int u = 0; u < NWR; ++u) {
      const int idx = tid + u * NT;
      if (idx < SM::NCH) sW[idx + idx / 8] = wreg[u] * kLog2e;
    }
  }

  // ---- 1a. g: in-block prefix sums (row scan) and R = e^{Gam_r - Gam_m},
  //          m = the block's first token; block first values and sums of
  //          the rest to LDS ------------------------------------------------
  if constexpr (RAW) betav = sigmoid(betav);  // raw projection: beta formed here
  float R[NKS][8];
  bool wide = false;
#pragma unroll
  for (int s = 0; s < NKS; ++s) {
    float p[8];
    if constexpr (RAW) {  // raw projections: the log-decay formed here
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float gv = valid ? log_sigmoid(gl[s][e / 4][e % 4]) : 0.f;
        gl[s][e / 4][e % 4] = gv;
        p[e] = i == 0 ? 0.f : gv;
      }
      if (i == 0) {
        *reinterpret_cast<f32x4*>(&sFirst[rb][32 * s + 8 * gq]) = gl[s][0];
        *reinterpret_cast<f32x4*>(&sFirst[rb][32 * s + 8 * gq + 4]) = gl[s][1];
      }
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float gv = valid ? gl[s][e / 4][e % 4] : 0.f;
        p[e] = i == 0 ? 0.f : gv;
        if (e % 4 == 3 && i == 0)
          *reinterpret_cast<f32x4*>(&sFirst[rb][32 * s + 8 * gq + e - 3]) =
              valid ? gl[s][e / 4] : f32x4{0.f, 0.f, 0.f, 0.f};
      }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      p[e] += dppf<kRowShr + 1>(0.f, p[e]);
      p[e] += dppf<kRowShr + 2>(0.f, p[e]);
      p[e] += dppf<kRowShr + 4>(0.f, p[e]);
      p[e] += dppf<kRowShr + 8>(0.f, p[e]);
      R[s][e] = __expf(p[e]);
    }
    if (i == 15) {
      *reinterpret_cast<f32x4*>(&sTot[rb][32 * s + 8 * gq]) = f32x4{p[0], p[1], p[2], p[3]};
      *reinterpret_cast<f32x4*>(&sTot[rb][32 * s + 8 * gq + 4]) = f32x4{p[4], p[5], p[6], p[7]};
#pragma unroll
      for (int e = 0; e < 8; ++e) wide |= !(p[e] >= -kSpan);
    }
  }
  // this wave's block decays by more than kSpan on some channel (or by -inf):
  // it is wide (wave-uniform; the other waves read it after the barrier)
  const bool explicit_diag = __builtin_amdgcn_ballot_w64(wide) != 0;
  if (lane == 0) sWide[rb] = explicit_diag;
  if constexpr (CONV) __syncthreads();  // conv weights and history visible

  // ---- 1a. q, k, v: short conv + SiLU (taps by row shifts), L2 of q, k ----
  // With y = w0 x_{t-3} + w1 x_{t-2} + w2 x_{t-1} + w3 x_t, SiLU(y) =
  // y / (1 + e^{-y}). The weights in LDS are pre-scaled by log2(e), so the
  // sum is u = y log2(e) and z = u / (1 + 2^{-u}) = SiLU(y) / ln 2; the 1/ln 2
  // is taken out again by the L2 step (whose epsilon is scaled to match) or
  // folded into beta for v. Tap x_{t-d} of lane j is x_t of lane j-d, or for
  // j < d the history token j+3-d of the block, which lane j+3-d (< 3)
  // reads from LDS.
  auto activate = [&](u32x4 x, int wbase, float* z) {
    if constexpr (CONV) {
      u32x4 y = *reinterpret_cast<const u32x4*>(&sHist[rb][i < 3 ? i : 2][wbase]);
      // pin the raw words here, so that the shifted copies are made slice by
      // slice and not all at once ahead of the weights' barrier
      asm volatile("" : "+v"(x), "+v"(y));
      u32x4 t1, t2, t3;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        t1[w] = dpp<kRowShr + 1>(dpp0<kRowShl + 2>(y[w]), x[w]);
        t2[w] = dpp<kRowShr + 2>(dpp0<kRowShl + 1>(y[w]), x[w]);
        t3[w] = dpp<kRowShr + 3>(y[w], x[w]);
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int wi = wbase + e;
        const f32x4 wt = sW[wi + wi / 8];
        const float u = wt.x * bfe(t3, e) + wt.y * bfe(t2, e) + wt.z * bfe(t1, e) + wt.w * bfe(x, e);
        z[e] = u * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-u));
      }
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) z[e] = bfe(x, e);
    }
  };
  bf16x8 vb[NVS];  // beta v^ (the B side of U' after a transpose)
#pragma unroll
  for (int s = 0; s < NVS; ++s) {
    float z[8];
    activate(xv[s], 2 * DK + 32 * s + 8 * gq, z);
#pragma unroll
    for (int e = 0; e < 8; ++e) z[e] *= betav * kAct;
    vb[s] = to_bf16x8(z);
    asm volatile("" : "+v"(vb[s]));
  }
  __builtin_amdgcn_sched_barrier(0);
  float qf[NKS][8], kf[NKS][8];
  {
    float sq = 0.f, sk = 0.f;
#pragma unroll
    for (int s = 0; s < NKS; ++s) {
      activate(xq[s], 32 * s + 8 * gq, qf[s]);
#pragma unroll
      for (int e = 0; e < 8; ++e) sq += qf[s][e] * qf[s][e];
      __builtin_amdgcn_sched_barrier(0);  // one slice's weights in flight at a time
    }
#pragma unroll
    for (int s = 0; s < NKS; ++s) {
      activate(xk[s], DK + 32 * s + 8 * gq, kf[s]);
#pragma unroll
      for (int e = 0; e < 8; ++e) sk += kf[s][e] * kf[s][e];
      __builtin_amdgcn_sched_barrier(0);
    }
    sq += __shfl_xor(sq, 16, kWave);
    sq += __shfl_xor(sq, 32, kWave);
    sk += __shfl_xor(sk, 16, kWave);
    sk += __shfl_xor(sk, 32, kWave);
    const float iq = !valid ? 0.f : do_l2 ? __builtin_amdgcn_rsqf(sq + kEps) : kAct;
    const float ik = !valid ? 0.f : do_l2 ? __builtin_amdgcn_rsqf(sk + kEps) : kAct;
#pragma unroll
    for (int s = 0; s < NKS; ++s)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        qf[s][e] *= iq;
        kf[s][e] *= ik;
      }
  }
  __syncthreads();

  // ---- 1b. block decays, each the exponential of a sum of decays over the
  //          tokens it spans (first[a] = g of block a's first token, rest[a]
  //          = the sum over its other 15): EB[a] = e^{Gam_m(a)}; EN[a] over
  //          the tokens after block a's first (narrow a) or last (wide a)
  //          token; BT[a][b] (b < a) over the tokens after block b's first
  //          (narrow b) or last (wide b) token up to block a's first;
  //          e^{Gam_n} to the workspace
  for (int c = tid; c < DK; c += NT) {
    float fst[NRB], rst[NRB];
    bool wd[NRB];
#pragma unroll
    for (int bb = 0; bb < NRB; ++bb) {
      fst[bb] = sFirst[bb][c];
      rst[bb] = sTot[bb][c];
      wd[bb] = sWide[bb] != 0;
    }
    float cum = 0.f;
#pragma unroll
    for (int bb = 0; bb < NRB; ++bb) {
      sEB[bb][c] = __expf(cum + fst[bb]);
      cum += fst[bb] + rst[bb];
    }
    Dn[c] = __expf(cum);
    float later = 0.f;
#pragma unroll
    for (int bb = NRB - 1; bb >= 0; --bb) {
      sEN[bb][c] = __expf(wd[bb] ? later : later + rst[bb]);
      later += fst[bb] + rst[bb];
    }
#pragma unroll
    for (int bb = 1; bb < NRB; ++bb) {
      float gap = fst[bb];
#pragma unroll
      for (int b2 = bb - 1; b2 >= 0; --b2) {
        sBT[bb * (bb - 1) / 2 + b2][c] = __expf(wd[b2] ? gap : gap + rst[b2]);
        gap += rst[b2] + fst[b2];
      }
    }
  }

  // ---- 1b'. a wave whose block decays past kSpan forms its diagonal tile
  //           here, in fp32, from the unscaled q^, k^ and e^{g} (reloaded):
  //           beta_r A_rj (j < r) to sL[r][j] and P_rj (j <= r) transposed to
  //           sL[j][r]; the inverse reads only the strictly lower part ------
  if (explicit_diag) {
    // Room for the passes below: R (as fp16) and the beta v^ pieces wait in
    // this wave's rows of the -W and U' blocks of the workspace, which only
    // this wave writes, and only in step 4 (4 * NKS and 4 * NVS dwords per lane).
    unsigned* rpark = reinterpret_cast<unsigned*>(blk + L::oW + (size_t)rb * NKS * kWave * 8) +
                      (size_t)lane * NKS * 4;
    unsigned* vpark = reinterpret_cast<unsigned*>(blk + L::oU + (size_t)rb * (DV / 16) * kWave * 4) +
                      (size_t)lane * NVS * 4;
#pragma unroll
    for (int s = 0; s < NKS; ++s) {
      u32x4 w;
#pragma unroll
      for (int u = 0; u < 4; ++u)
        w[u] = __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_pkrtz(R[s][2 * u], R[s][2 * u + 1]));
      reinterpret_cast<u32x4*>(rpark)[s] = w;
    }
#pragma unroll
    for (int s = 0; s < NVS; ++s) reinterpret_cast<u32x4*>(vpark)[s] = __builtin_bit_cast(u32x4, vb[s]);
    asm volatile("" ::: "memory");
    // four passes of eight distances (A: 1..8, 9..15; P: 0..7, 8..15), each
    // summed over the slices, reduced over the lane's four channel groups
    // and stored, so that only eight sums are live at a time
    auto pass = [&](auto d0c, auto isp) __attribute__((always_inline)) {
      constexpr int D0 = decltype(d0c)::value;
      constexpr bool ISP = decltype(isp)::value;
      float acc[8];
#pragma unroll
      for (int d = 0; d < 8; ++d) acc[d] = 0.f;
#pragma unroll
      for (int s = 0; s < NKS; ++s) {
#pragma unroll
        for (int h4 = 0; h4 < 2; ++h4) {  // four channels at a time
          // opaque copies, so that the passes do not share (and keep alive)
          // one another's shifted values
          float av[4], kk[4], xx[4];
          load_decay(s, h4, std::integral_constant<int, 4>{}, av);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            kk[e] = kf[s][4 * h4 + e];
            xx[e] = ISP ? qf[s][4 * h4 + e] : kf[s][4 * h4 + e];
            asm volatile("" : "+v"(av[e]), "+v"(kk[e]), "+v"(xx[e]));
            av[e] = __expf(av[e]);
          }
          diag_terms<D0, 4>(kk, xx, av, acc);
          __builtin_amdgcn_sched_barrier(0);
        }
        __builtin_amdgcn_sched_barrier(0);  // one slice's decays at a time
      }
#pragma unroll
      for (int dd = 0; dd < 8; ++dd) {
        acc[dd] += __shfl_xor(acc[dd], 16, kWave);
        acc[dd] += __shfl_xor(acc[dd], 32, kWave);
        const int d = D0 + dd;
        if (d < 16 && d % 4 == gq && d <= i) {
          if constexpr (ISP) sL[r - d][r] = acc[dd];
          else sL[r][r - d] = betav * acc[dd];
        }
      }
      __builtin_amdgcn_sched_barrier(0);  // passes one after the other
    };
    pass(std::integral_constant<int, 1>{}, std::false_type{});
    pass(std::integral_constant<int, 9>{}, std::false_type{});
    pass(std::integral_constant<int, 0>{}, std::true_type{});
    pass(std::integral_constant<int, 8>{}, std::true_type{});
    asm volatile("" ::: "memory");  // read back what was parked, not a forwarded copy
#pragma unroll
    for (int s = 0; s < NKS; ++s) {
      const u32x4 w = reinterpret_cast<const u32x4*>(rpark)[s];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const unsigned wu = w[u];  // (a bit_cast of the vector element itself reads element 0)
        const f16x2 hv = __builtin_bit_cast(f16x2, wu);
        R[s][2 * u] = (float)hv[0];
        R[s][2 * u + 1] = (float)hv[1];
      }
    }
#pragma unroll
    for (int s = 0; s < NVS; ++s) vb[s] = __builtin_bit_cast(bf16x8, reinterpret_cast<const u32x4*>(vpark)[s]);
  }
  __syncthreads();

  // selection matrices: B_hf[k][n] = (k == n + 16 hf) picks channel half hf
  bf16x8 sel[2];
#pragma unroll
  for (int hf = 0; hf < 2; ++hf)
#pragma unroll
    for (int e = 0; e < 8; ++e) sel[hf][e] = (bf16)(8 * gq + e == i + 16 * hf ? 1.f : 0.f);
  const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};

  // ---- 1c. per slice: the column factor E = 1/R (narrow block) or
  //          e^{Gam_e - Gam_r} from a row scan of the decays after the token
  //          (wide); Q~ = e^{Gam} q^ = EB (q^ R) and K^^T = e^{Gam_n - Gam} k^
  //          = EN (k^ E) to the workspace, k^ E to LDS; q^ <- q^ R and
  //          k^ <- k^ R (the Gram row factors). The barrier above also
  //          orders sKi after the block sums it overwrites -----------------
#pragma unroll
  for (int s = 0; s < NKS; ++s) {
    const f32x4* pb = reinterpret_cast<const f32x4*>(&sEB[rb][32 * s + 8 * gq]);
    const f32x4* pn = reinterpret_cast<const f32x4*>(&sEN[rb][32 * s + 8 * gq]);
    const f32x4 b0 = pb[0], b1 = pb[1], n0 = pn[0], n1 = pn[1];
    float E[8];
    if (explicit_diag) {
      float x[8];
      load_decay(s, 0, std::integral_constant<int, 8>{}, x);
#pragma unroll
      for (int e = 0; e < 8; ++e) {  // decays of tokens i+1 .. 15 of the block
        x[e] = dpp0f<kRowShl + 1>(x[e]);
        x[e] += dpp0f<kRowShl + 1>(x[e]);
        x[e] += dpp0f<kRowShl + 2>(x[e]);
        x[e] += dpp0f<kRowShl + 4>(x[e]);
        x[e] += dpp0f<kRowShl + 8>(x[e]);
        E[e] = __expf(x[e]);
      }
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) E[e] = __builtin_amdgcn_rcpf(R[s][e]);
    }
    float qt[8], ki[8], kh[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float eb = e < 4 ? b0[e] : b1[e - 4], en = e < 4 ? n0[e] : n1[e - 4];
      const float rr = R[s][e];
      const float qr = qf[s][e] * rr, kr = kf[s][e] * rr;
      ki[e] = kf[s][e] * E[e];
      qt[e] = eb * qr;
      kh[e] = en * ki[e];
      qf[s][e] = qr;
      kf[s][e] = kr;
    }
    *reinterpret_cast<bf16x8*>(blk + L::oQ + ((size_t)(rb * NKS + s) * kWave + lane) * 8) =
        to_bf16x8(qt);
    *reinterpret_cast<bf16x8*>(sKi + ((size_t)(rb * NKS + s) * kWave + lane) * 8) = to_bf16x8(ki);
    // K^^T: channel rows 32s + 16hf + i, tokens 16rb + 4gq + e per selection
    const bf16x8 khb = to_bf16x8(kh);
    const f32x4 d0 = M::mma(khb, sel[0], zero4), d1 = M::mma(khb, sel[1], zero4);
    const u32x4 pc = pair_piece(d0, d1, gq);
    const int cb = 2 * s + (gq & 1), lk = 16 * (2 * (rb % 2) + gq / 2) + i;
    *reinterpret_cast<u32x4*>(blk + L::oK + ((size_t)(cb * NKC + rb / 2) * kWave + lk) * 8) = pc;
    __builtin_amdgcn_sched_barrier(0);  // one slice at a time
  }
  __syncthreads();

  // ---- 2. Gram tiles of this wave's block row, transposed: the product of
  //         A operand k^ E of block bc (LDS) and B operand (k^ R), (q^ R) of
  //         this wave's tokens, scaled by BT[rb][bc] for bc < rb, is the
  //         tile (rows j of block bc, columns r of block rb) of A^T and P^T
  //         (the diagonal tile of a wide block comes from sL, formed in 1b').
  //         Lane (l%16, l/16) then holds A_rj, P_rj for r = 16rb + l%16 and
  //         j = 16bc + 4(l/16) + e: beta_r A_rj (strictly lower) goes to
  //         LDS as one 16-byte row piece, P (lower) to the workspace as
  //         16-byte pieces of 8 columns (two tiles paired). Then beta
  //         e^{Gam} k^ = beta EB[rb] (k^ R), the B side of W after a
  //         transpose. -------------------------------------------------------
  bf16x8 kb[NKS];
  {
    f32x4 pt[2];
#pragma unroll
    for (int bc = 0; bc < NRB; ++bc) {
      f32x4 accA = zero4, accP = zero4;
      if (bc <= rb) {
        f32x4 la;
        if (bc == rb && explicit_diag) {
          // reads of this wave's own 1b' values, before its stores below
          const f32x4 fa4 = *reinterpret_cast<const f32x4*>(&sL[r][16 * bc + 4 * gq]);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int jj = 16 * bc + 4 * gq + e;
            la[e] = jj < r ? fa4[e] : 0.f;
            accP[e] = jj <= r ? sL[jj][r] : 0.f;
          }
        } else {
#pragma unroll
          for (int s = 0; s < NKS; ++s) {
            const bf16x8 fa =
                *reinterpret_cast<const bf16x8*>(sKi + ((size_t)(bc * NKS + s) * kWave + lane) * 8);
            float bk[8], bqv[8];
            if (bc < rb) {
              const f32x4* pb = reinterpret_cast<const f32x4*>(
                  &sBT[rb * (rb - 1) / 2 + bc][32 * s + 8 * gq]);
              const f32x4 t0v = pb[0], t1v = pb[1];
#pragma unroll
              for (int e = 0; e < 8; ++e) {
                const float sc = e < 4 ? t0v[e] : t1v[e - 4];
                bk[e] = kf[s][e] * sc;
                bqv[e] = qf[s][e] * sc;
              }
            } else {
#pragma unroll
              for (int e = 0; e < 8; ++e) {
                bk[e] = kf[s][e];
                bqv[e] = qf[s][e];
              }
            }
            accA = M::mma(fa, to_bf16x8(bk), accA);
            accP = M::mma(fa, to_bf16x8(bqv), accP);
            __builtin_amdgcn_sched_barrier(0);
          }
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int jj = 16 * bc + 4 * gq + e;
            la[e] = jj < r ? betav * accA[e] : 0.f;
            accP[e] = jj <= r ? accP[e] : 0.f;
          }
        }
        *reinterpret_cast<f32x4*>(&sL[r][16 * bc + 4 * gq]) = la;
      }
      pt[bc % 2] = accP;
      if (bc % 2 == 1) {
        const u32x4 pc = pair_piece(pt[0], pt[1], gq);
        const int j0 = 16 * (bc - 1 + (gq & 1)) + 8 * (gq / 2);
        *reinterpret_cast<u32x4*>(blk + L::oP + (size_t)r * CP + j0) = pc;
      }
    }
#pragma unroll
    for (int s = 0; s < NKS; ++s) {
      const f32x4* pb = reinterpret_cast<const f32x4*>(&sEB[rb][32 * s + 8 * gq]);
      const f32x4 b0 = pb[0], b1 = pb[1];
      float v[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = betav * (e < 4 ? b0[e] : b1[e - 4]) * kf[s][e];
      kb[s] = to_bf16x8(v);
      asm volatile("" : "+v"(kb[s]));  // made here, so that k^ R dies here
    }
  }
  __syncthreads();

  // ---- 3. X = (I + beta A)^{-1}, then X as bf16 and (beta v^)^T ---------
  unit_lower_inverse<C, NT>(sL, sX, tid);
  for (int idx = tid; idx < C * (C / 8); idx += NT) {
    const int rr = idx / (C / 8), j0 = 8 * (idx % (C / 8));
    const f32x4 x0 = *reinterpret_cast<const f32x4*>(&sX[rr][j0]);
    const f32x4 x1 = *reinterpret_cast<const f32x4*>(&sX[rr][j0 + 4]);
    const float v[8] = {x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
    *reinterpret_cast<bf16x8*>(&sXb[rr][j0]) = to_bf16x8(v);
  }
#pragma unroll
  for (int s = 0; s < NVS; ++s) {
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      const f32x4 d = M::mma(vb[s], sel[hf], zero4);
      *reinterpret_cast<bf16x4*>(&sVT[32 * s + 16 * hf + i][16 * rb + 4 * gq]) = to_bf16x4(d);
    }
  }
  __syncthreads();
#pragma unroll
  for (int s = 0; s < NKS; ++s) {
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      const f32x4 d = M::mma(kb[s], sel[hf], zero4);
      *reinterpret_cast<bf16x4*>(&sKT[32 * s + 16 * hf + i][16 * rb + 4 * gq]) = to_bf16x4(d);
    }
  }
  __syncthreads();

  // ---- 4. U' = X (beta V) (accumulator layout) and W^T = (beta e^Gam K)^T
  //         X^T, stored as -W pieces (fragment-major) --------------------
  bf16x8 xb[NKC];
#pragma unroll
  for (int kc = 0; kc < NKC; ++kc) xb[kc] = *reinterpret_cast<const bf16x8*>(&sXb[r][32 * kc + 8 * gq]);
#pragma unroll
  for (int vt = 0; vt < DV / 16; ++vt) {
    f32x4 acc = zero4;
#pragma unroll
    for (int kc = 0; kc < NKC; ++kc)
      acc = M::mma(xb[kc], *reinterpret_cast<const bf16x8*>(&sVT[16 * vt + i][32 * kc + 8 * gq]), acc);
    *reinterpret_cast<bf16x4*>(blk + L::oU + ((size_t)(rb * (DV / 16) + vt) * kWave + lane) * 4) =
        to_bf16x4(acc);
  }
#pragma unroll
  for (int s = 0; s < NKS; ++s) {
    f32x4 d[2];
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      f32x4 acc = zero4;
#pragma unroll
      for (int kc = 0; kc < NKC; ++kc)
        acc = M::mma(*reinterpret_cast<const bf16x8*>(&sKT[32 * s + 16 * hf + i][32 * kc + 8 * gq]),
                     xb[kc], acc);
      d[hf] = -acc;
    }
    const u32x4 pc = pair_piece(d[0], d[1], gq);
    const int lw = 16 * (2 * (gq & 1) + gq / 2) + i;
    *reinterpret_cast<u32x4*>(blk + L::oW + ((size_t)(rb * NKS + s) * kWave + lw) * 8) = pc;
  }
}

template <int C, int DK, int DV, bool CONV, bool SG>
void launch_sg(const PrefillArgs& a, int t0, int ncs, uint8_t* ws, hipStream_t st) {
  const dim3 grid((unsigned)((long)ncs * a.H * a.B)), block(C * 4);
  if (a.flags & KDA_F_RAW_GATES)
    hipLaunchKernelGGL((prefill_prep_rows_kernel<C, DK, DV, CONV, SG, true>), grid, block, 0,
                       st, a, t0, ncs, ws);
  else
    hipLaunchKernelGGL((prefill_prep_rows_kernel<C, DK, DV, CONV, SG, false>), grid, block, 0,
                       st, a, t0, ncs, ws);
}

template <int C, int DK, int DV, bool CONV>
void launch_conv(const PrefillArgs& a, int t0, int ncs, uint8_t* ws, hipStream_t st) {
  if (a.flags & KDA_F_SCALAR_G)
    launch_sg<C, DK, DV, CONV, true>(a, t0, ncs, ws, st);
  else
    launch_sg<C, DK, DV, CONV, false>(a, t0, ncs, ws, st);
}

template <int C, int DK, int DV>
hipError_t launch_t(const PrefillArgs& a, int t0, int ncs, uint8_t* ws, hipStream_t st) {
  if (a.flags & KDA_F_SKIP_CONV)
    launch_conv<C, DK, DV, false>(a, t0, ncs, ws, st);
  else
    launch_conv<C, DK, DV, true>(a, t0, ncs, ws, st);
  return hipGetLastError();
}

template <int C, int DK>
hipError_t launch_dv(const PrefillArgs& a, int t0, int ncs, uint8_t* ws, hipStream_t st) {
  switch (a.dv) {
    case 32: return launch_t<C, DK, 32>(a, t0, ncs, ws, st);
    case 64: return launch_t<C, DK, 64>(a, t0, ncs, ws, st);
    case 128: return launch_t<C, DK, 128>(a, t0, ncs, ws, st);
  }
  return hipErrorInvalidValue;
}

template <int C>
hipError_t launch_dk(const PrefillArgs& a, int t0, int ncs, uint8_t* ws, hipStream_t st) {
  switch (a.dk) {
    case 32: return launch_dv<C, 32>(a, t0, ncs, ws, st);
    case 64: return launch_dv<C, 64>(a, t0, ncs, ws, st);
    case 128: return launch_dv<C, 128>(a, t0, ncs, ws, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace

bool prep_rows_supported(int chunk, int dk, int dv, kda_dtype io) {
  return io == KDA_BF16 && (chunk == 32 || chunk == 64) && dk >= 32 && dv >= 32;
}

hipError_t launch_prep_rows(const PrefillArgs& a, int t0, int ncs, void* ws, hipStream_t st) {
  if (!prep_rows_supported(a.chunk, a.dk, a.dv, KDA_BF16)) return hipErrorInvalidValue;
  uint8_t* w = static_cast<uint8_t*>(ws);
  return a.chunk == 32 ? launch_dk<32>(a, t0, ncs, w, st) : launch_dk<64>(a, t0, ncs, w, st);
}

}  // namespace kda
