// Fused KDA decode step: one pass over the fp32 state per token.
//
// Per (sequence b, head h) and token t ("KV缓存从11.25GB缩到0.21GB：WARP中Kimi
// Delta Attention线性注意力原理剖析", section "KDA 递推公式先衰减再差分"):
//   q~, k~, v~ = SiLU(conv4(raw, ring))      ring <- last three raw tokens
//   q^, k^     = q~ / |q~|, k~ / |k~|         (sqrt(sum x^2 + 1e-6))
//   S'         = Diag(exp g) S
//   delta      = beta (v~ - S'^T k^)
//   S          = S' + k^ delta^T
//   o          = S^T q^ = S'^T q^ + (k^ . q^) delta
// The last identity lets one read of S produce both reductions (S'^T k^ and
// S'^T q^), so S is read once and written once: the step streams 2*dk*dv*4
// bytes per head and is HBM-bound.
//
// Work decomposition (gfx950, wave64): one workgroup of NT threads per (b, h).
// A row of S (dv floats) is covered by LPR = dv/4 lanes holding one float4
// each, so one wave load instruction moves 1 KiB of contiguous state; each
// thread keeps J = dk*dv/(4*NT) float4 of S in registers between the read
// and the write. The column reductions over rows run in registers, then
// across lanes of a wave with xor shuffles, then across waves through LDS.
#include "kda_common.h"

namespace kda {
namespace {

// NTH: stream S with non-temporal loads and stores (it is read once and
// written once per step; keeping it out of the caches leaves them to the
// small per-token inputs). GATE: o receives the gated RMSNorm of the readout,
// o = r / sqrt(mean r^2 + eps) * w * sigmoid(z) over the head's dv values.
template <int DK, int DV, int NT, typename IO, bool NTH, bool GATE>
__global__ __launch_bounds__(NT) void decode_step_kernel(DecodeArgs a) {
  constexpr int LPR = DV / 4;         // lanes per state row
  constexpr int RPP = NT / LPR;       // state rows per load pass
  constexpr int J = DK / RPP;         // float4 of S per thread
  constexpr int NW = NT / kWave;      // waves per workgroup
  constexpr int NCH = 2 * DK + DV;    // conv channels of this head (q | k | v)
  constexpr int CPT = (NCH + NT - 1) / NT;
  static_assert(NT % LPR == 0 && DK % RPP == 0 && J >= 1, "bad tiling");
  static_assert(LPR <= kWave && NT % kWave == 0 && NT >= DV, "bad tiling");

  __shared__ float sq[DK], sk[DK], sv[DV], sdec[DK], sdel[DV];
  __shared__ float sred[NW][LPR][8];
  __shared__ float snorm[3];
  constexpr int NWD = (DV + kWave - 1) / kWave;  // waves that hold readout values
  __shared__ float sgate[NWD];

  const int h = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  const int H = a.H;
  const long bh = (long)b * H + h;
  const long ctot = (long)H * NCH;
  const int c4 = tid % LPR, rg = tid / LPR;
  const bool do_conv = !(a.flags & KDA_F_SKIP_CONV);
  const bool do_l2 = !(a.flags & KDA_F_SKIP_L2);
  IO* ring = static_cast<IO*>(a.ring) + (long)b * 3 * ctot;

  // ---- 1. token inputs into registers (issued before the state loads so
  //         that their wait does not also wait for the state) -------------
  float xr[CPT][4];
  float wr[CPT][4];
  long chan[CPT];
#pragma unroll
  for (int u = 0; u < CPT; ++u) {
    const int ch = tid + u * NT;
    chan[u] = -1;
    if (ch < NCH) {
      const IO* src;
      if (ch < DK) {
        src = static_cast<const IO*>(a.q) + bh * DK + ch;
        chan[u] = (long)h * DK + ch;
      } else if (ch < 2 * DK) {
        src = static_cast<const IO*>(a.k) + bh * DK + (ch - DK);
        chan[u] = (long)H * DK + (long)h * DK + (ch - DK);
      } else {
        src = static_cast<const IO*>(a.v) + bh * DV + (ch - 2 * DK);
        chan[u] = 2L * H * DK + (long)h * DV + (ch - 2 * DK);
      }
      xr[u][3] = to_f32(*src);
      if (do_conv) {
        xr[u][0] = to_f32(ring[0 * ctot + chan[u]]);
        xr[u][1] = to_f32(ring[1 * ctot + chan[u]]);
        xr[u][2] = to_f32(ring[2 * ctot + chan[u]]);
        const f32x4 w = *reinterpret_cast<const f32x4*>(a.conv_w + 4 * chan[u]);
        wr[u][0] = w.x; wr[u][1] = w.y; wr[u][2] = w.z; wr[u][3] = w.w;
      }
    }
  }
  constexpr int GPT = (DK + NT - 1) / NT;  // decay channels per thread
  float gval[GPT];
  if (a.flags & KDA_F_SCALAR_G) {  // one decay for every key channel of the head
    const float gs = a.g[bh];
#pragma unroll
    for (int u = 0; u < GPT; ++u) gval[u] = tid + u * NT < DK ? gs : 0.0f;
  } else {
#pragma unroll
    for (int u = 0; u < GPT; ++u) {
      const int i = tid + u * NT;
      gval[u] = i < DK ? a.g[bh * DK + i] : 0.0f;
    }
  }
  float betav = a.beta[bh];
  if (a.flags & KDA_F_RAW_GATES) {  // raw projections: form the gates here
#pragma unroll
    for (int u = 0; u < GPT; ++u) gval[u] = log_sigmoid(gval[u]);
    betav = sigmoid(betav);
  }
  float zg = 0.f, wg = 0.f;  // gate pre-activation and norm weight of column tid
  if constexpr (GATE) {
    if (tid < DV) {
      zg = to_f32(static_cast<const IO*>(a.gate)[bh * DV + tid]);
      wg = a.norm_w[tid];
    }
  }

  // ---- 2. the state: J float4 per thread, rows rg + RPP*jj ---------------
  float* Sbh = a.S + bh * DK * DV + 4 * c4;
  f32x4 s[J];
#pragma unroll
  for (int jj = 0; jj < J; ++jj) {
    const f32x4* src = reinterpret_cast<const f32x4*>(Sbh + (long)(rg + RPP * jj) * DV);
    s[jj] = NTH ? __builtin_nontemporal_load(src) : *src;
  }

  // ---- 3. short conv + SiLU, ring advance, decay factors ----------------
#pragma unroll
  for (int u = 0; u < CPT; ++u) {
    const int ch = tid + u * NT;
    if (ch < NCH) {
      float y = xr[u][3];
      if (do_conv) {
        y = silu(wr[u][0] * xr[u][0] + wr[u][1] * xr[u][1] + wr[u][2] * xr[u][2] +
                 wr[u][3] * xr[u][3]);
        // raw values are stored back unchanged (they came from IO)
        ring[0 * ctot + chan[u]] = from_f32<IO>(xr[u][1]);
        ring[1 * ctot + chan[u]] = from_f32<IO>(xr[u][2]);
        ring[2 * ctot + chan[u]] = from_f32<IO>(xr[u][3]);
      }
      if (ch < DK) sq[ch] = y;
      else if (ch < 2 * DK) sk[ch - DK] = y;
      else sv[ch - 2 * DK] = y;
    }
  }
#pragma unroll
  for (int u = 0; u < GPT; ++u) {
    const int i = tid + u * NT;
    if (i < DK) sdec[i] = __expf(gval[u]);
  }
  __syncthreads();

  // ---- 4. L2 norms of q~ and k~ and the scalar k^.q^ (wave 0) ----------
  if (tid < kWave) {
    float ssq = 0.f, ssk = 0.f, sqk = 0.f;
    for (int i = tid; i < DK; i += kWave) {
      const float qv = sq[i], kv = sk[i];
      ssq += qv * qv;
      ssk += kv * kv;
      sqk += qv * kv;
    }
    ssq = wave_sum(ssq);
    ssk = wave_sum(ssk);
    sqk = wave_sum(sqk);
    if (tid == 0) {
      const float iq = do_l2 ? 1.0f / sqrtf(ssq + kL2Eps) : 1.0f;
      const float ik = do_l2 ? 1.0f / sqrtf(ssk + kL2Eps) : 1.0f;
      snorm[0] = iq;
      snorm[1] = ik;
      snorm[2] = sqk * iq * ik;
    }
  }
  __syncthreads();
  const float iq = snorm[0], ik = snorm[1], qk = snorm[2];

  // ---- 5. decay and the two partial column reductions -------------------
  f32x4 ak = {0.f, 0.f, 0.f, 0.f}, aq = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int jj = 0; jj < J; ++jj) {
    const int i = rg + RPP * jj;
    s[jj] *= sdec[i];
    ak += s[jj] * (sk[i] * ik);
    aq += s[jj] * (sq[i] * iq);
  }
#pragma unroll
  for (int off = LPR; off < kWave; off <<= 1) {
    ak.x += __shfl_xor(ak.x, off, kWave);
    ak.y += __shfl_xor(ak.y, off, kWave);
    ak.z += __shfl_xor(ak.z, off, kWave);
    ak.w += __shfl_xor(ak.w, off, kWave);
    aq.x += __shfl_xor(aq.x, off, kWave);
    aq.y += __shfl_xor(aq.y, off, kWave);
    aq.z += __shfl_xor(aq.z, off, kWave);
    aq.w += __shfl_xor(aq.w, off, kWave);
  }
  const int lane = tid % kWave, wv = tid / kWave;
  if (lane < LPR) {
    *reinterpret_cast<f32x4*>(&sred[wv][lane][0]) = ak;
    *reinterpret_cast<f32x4*>(&sred[wv][lane][4]) = aq;
  }
  __syncthreads();

  // ---- 6. per column: delta and the readout -----------------------------
  float ov = 0.f;
  if (tid < DV) {
    const int cc = tid / 4, e = tid % 4;
    float rk = 0.f, rq = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      rk += sred[w][cc][e];
      rq += sred[w][cc][4 + e];
    }
    const float del = betav * (sv[tid] - rk);
    sdel[tid] = del;
    ov = rq + qk * del;
    if constexpr (!GATE) static_cast<IO*>(a.o)[bh * DV + tid] = from_f32<IO>(ov);
  }
  if constexpr (GATE) {
    if (wv < NWD) {  // wave-uniform: every lane of these waves takes part
      const float ss = wave_sum(tid < DV ? ov * ov : 0.f);
      if (lane == 0) sgate[wv] = ss;
    }
  }
  __syncthreads();
  if constexpr (GATE) {
    if (tid < DV) {
      float ss = 0.f;
#pragma unroll
      for (int w = 0; w < NWD; ++w) ss += sgate[w];
      const float inv = 1.0f / sqrtf(ss * (1.0f / DV) + a.norm_eps);
      const float sig = 1.0f / (1.0f + __expf(-zg));
      static_cast<IO*>(a.o)[bh * DV + tid] = from_f32<IO>(ov * inv * wg * sig);
    }
  }

  // ---- 7. rank-1 write and store -----------------------------------------
  const f32x4 dl = *reinterpret_cast<const f32x4*>(&sdel[4 * c4]);
#pragma unroll
  for (int jj = 0; jj < J; ++jj) {
    const int i = rg + RPP * jj;
    s[jj] += (sk[i] * ik) * dl;
    f32x4* dst = reinterpret_cast<f32x4*>(Sbh + (long)i * DV);
    if (NTH) __builtin_nontemporal_store(s[jj], dst);
    else *dst = s[jj];
  }
}

// Threads per head: 4 float4 of S per thread, at least one wave and at most
// 1024 threads. Measured on MI355X for 64 x 96 heads of 128 x 128: 16 float4
// per thread (256 threads) streams 5.1 TB/s, 8 (512 threads) 6.0 TB/s and
// 4 (1024 threads) 6.2 TB/s, with non-temporal loads and stores of S.
template <int DK, int DV>
constexpr int decode_threads() {
  constexpr int n = DK * DV / 16;
  return n < kWave ? kWave : (n > 1024 ? 1024 : n);
}

template <int DK, int DV, typename IO>
hipError_t launch_t(const DecodeArgs& a, hipStream_t stream) {
  constexpr int NT = decode_threads<DK, DV>();
  dim3 grid(a.H, a.B);
  if (a.gate)
    hipLaunchKernelGGL((decode_step_kernel<DK, DV, NT, IO, true, true>), grid, dim3(NT), 0,
                       stream, a);
  else
    hipLaunchKernelGGL((decode_step_kernel<DK, DV, NT, IO, true, false>), grid, dim3(NT), 0,
                       stream, a);
  return hipGetLastError();
}

template <int DK, typename IO>
hipError_t launch_dv(const DecodeArgs& a, hipStream_t stream) {
  switch (a.dv) {
    case 16: return launch_t<DK, 16, IO>(a, stream);
    case 32: return launch_t<DK, 32, IO>(a, stream);
    case 64: return launch_t<DK, 64, IO>(a, stream);
    case 128: return launch_t<DK, 128, IO>(a, stream);
  }
  return hipErrorInvalidValue;
}

template <typename IO>
hipError_t launch_dk(const DecodeArgs& a, hipStream_t stream) {
  switch (a.dk) {
    case 16: return launch_dv<16, IO>(a, stream);
    case 32: return launch_dv<32, IO>(a, stream);
    case 64: return launch_dv<64, IO>(a, stream);
    case 128: return launch_dv<128, IO>(a, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_decode(const DecodeArgs& a, kda_dtype io, hipStream_t stream) {
  return io == KDA_BF16 ? launch_dk<bf16>(a, stream) : launch_dk<float>(a, stream);
}

}  // namespace kda
