// Standalone prologue (short conv + SiLU + L2) over T tokens, the ring
// advance that follows a T-token block, and the zero-fill used by reset.
//
// Short conv: width 4, causal, depthwise, no bias, on every channel of q, k
// and v; SiLU after it; q and k are then L2-normalised per head over d_k
// ("KV缓存从11.25GB缩到0.21GB：WARP中Kimi Delta Attention线性注意力原理剖析",
// section "KDA 递推公式先衰减再差分"). Tokens are independent once their three
// raw predecessors are known (from the inputs, or from the ring before token
// 0), so every (b, t, h) is one wave and the whole call is one parallel launch.
// The ring is advanced by a second launch so that no workgroup overwrites
// history another one still reads.
#include "kda_common.h"

namespace kda {
namespace {

template <int DK, int DV, typename IO>
__global__ __launch_bounds__(256) void prologue_kernel(PrologueArgs a) {
  constexpr int UQ = (DK + kWave - 1) / kWave;
  constexpr int UV = (DV + kWave - 1) / kWave;
  const int lane = threadIdx.x % kWave;
  const long item = (long)blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave;
  const int H = a.H, T = a.T;
  if (item >= (long)a.B * T * H) return;  // whole wave leaves together
  const int h = (int)(item % H);
  const int t = (int)((item / H) % T);
  const int b = (int)(item / ((long)H * T));
  const long ctot = (long)H * (2 * DK + DV);
  const bool do_conv = !(a.flags & KDA_F_SKIP_CONV);
  const IO* ring = static_cast<const IO*>(a.ring) + (long)b * 3 * ctot;

  // raw value of channel (i of head h) of a projection, `back` tokens before t
  auto raw = [&](const IO* x, int d, int i, long chan, int back) -> float {
    const int s = t - back;
    if (s >= 0) return to_f32(x[(((long)b * T + s) * H + h) * d + i]);
    return to_f32(ring[(long)(3 + s) * ctot + chan]);
  };
  auto act = [&](const IO* x, int d, int i, long chan) -> float {
    if (!do_conv) return to_f32(x[(((long)b * T + t) * H + h) * d + i]);
    const f32x4 w = *reinterpret_cast<const f32x4*>(a.conv_w + 4 * chan);
    return silu(w.x * raw(x, d, i, chan, 3) + w.y * raw(x, d, i, chan, 2) +
                w.z * raw(x, d, i, chan, 1) + w.w * raw(x, d, i, chan, 0));
  };

  float qv[UQ], kv[UQ], vv[UV];
  float ssq = 0.f, ssk = 0.f;
#pragma unroll
  for (int u = 0; u < UQ; ++u) {
    const int i = lane + u * kWave;
    qv[u] = kv[u] = 0.f;
    if (i < DK) {
      qv[u] = act(static_cast<const IO*>(a.q), DK, i, (long)h * DK + i);
      kv[u] = act(static_cast<const IO*>(a.k), DK, i, (long)H * DK + (long)h * DK + i);
    }
    ssq += qv[u] * qv[u];
    ssk += kv[u] * kv[u];
  }
#pragma unroll
  for (int u = 0; u < UV; ++u) {
    const int j = lane + u * kWave;
    vv[u] = j < DV ? act(static_cast<const IO*>(a.v), DV, j, 2L * H * DK + (long)h * DV + j)
                   : 0.f;
  }
  float iq = 1.f, ik = 1.f;
  if (!(a.flags & KDA_F_SKIP_L2)) {
    iq = 1.0f / sqrtf(wave_sum(ssq) + kL2Eps);
    ik = 1.0f / sqrtf(wave_sum(ssk) + kL2Eps);
  }
  const long tok = ((long)b * T + t) * H + h;
#pragma unroll
  for (int u = 0; u < UQ; ++u) {
    const int i = lane + u * kWave;
    if (i < DK) {
      a.q_out[tok * DK + i] = qv[u] * iq;
      a.k_out[tok * DK + i] = kv[u] * ik;
    }
  }
#pragma unroll
  for (int u = 0; u < UV; ++u) {
    const int j = lane + u * kWave;
    if (j < DV) a.v_out[tok * DV + j] = vv[u];
  }
}

// ring[b][tap][c] <- raw token T-3+tap of channel c (from the old ring when
// T - 3 + tap < 0). One thread per (b, c) reads all three values first.
template <typename IO>
__global__ __launch_bounds__(256) void ring_advance_kernel(const IO* q, const IO* k,
                                                           const IO* v, IO* ring, int B,
                                                           int T, int H, int dk, int dv) {
  const long ctot = (long)H * (2 * dk + dv);
  const long idx = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (long)B * ctot) return;
  const int b = (int)(idx / ctot);
  const long c = idx % ctot;
  const IO* x;
  int d;
  long hc;  // h*d + i
  if (c < (long)H * dk) {
    x = q; d = dk; hc = c;
  } else if (c < 2L * H * dk) {
    x = k; d = dk; hc = c - (long)H * dk;
  } else {
    x = v; d = dv; hc = c - 2L * H * dk;
  }
  IO* rb = ring + (long)b * 3 * ctot;
  IO nw[3];
#pragma unroll
  for (int tap = 0; tap < 3; ++tap) {
    const int s = T - 3 + tap;
    nw[tap] = s >= 0 ? x[((long)b * T + s) * H * d + hc] : rb[(long)(3 + s) * ctot + c];
  }
#pragma unroll
  for (int tap = 0; tap < 3; ++tap) rb[(long)tap * ctot + c] = nw[tap];
}

__global__ __launch_bounds__(256) void fill_zero_kernel(uint8_t* p, size_t bytes) {
  const size_t n16 = bytes / 16;
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += stride)
    reinterpret_cast<uint4*>(p)[i] = make_uint4(0u, 0u, 0u, 0u);
  for (size_t i = n16 * 16 + (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < bytes;
       i += stride)
    p[i] = 0;
}

template <int DK, typename IO>
hipError_t prologue_dv(const PrologueArgs& a, hipStream_t st) {
  const long items = (long)a.B * a.T * a.H;
  const dim3 grid((unsigned)((items + 3) / 4));
  switch (a.dv) {
    case 16: hipLaunchKernelGGL((prologue_kernel<DK, 16, IO>), grid, dim3(256), 0, st, a); break;
    case 32: hipLaunchKernelGGL((prologue_kernel<DK, 32, IO>), grid, dim3(256), 0, st, a); break;
    case 64: hipLaunchKernelGGL((prologue_kernel<DK, 64, IO>), grid, dim3(256), 0, st, a); break;
    case 128: hipLaunchKernelGGL((prologue_kernel<DK, 128, IO>), grid, dim3(256), 0, st, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <typename IO>
hipError_t prologue_dk(const PrologueArgs& a, hipStream_t st) {
  switch (a.dk) {
    case 16: return prologue_dv<16, IO>(a, st);
    case 32: return prologue_dv<32, IO>(a, st);
    case 64: return prologue_dv<64, IO>(a, st);
    case 128: return prologue_dv<128, IO>(a, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_prologue(const PrologueArgs& a, kda_dtype io, hipStream_t stream) {
  if ((long)a.B * a.T * a.H == 0) return hipSuccess;
  return io == KDA_BF16 ? prologue_dk<bf16>(a, stream) : prologue_dk<float>(a, stream);
}

hipError_t launch_ring_advance(const void* q, const void* k, const void* v, void* ring, int B,
                               int T, int H, int dk, int dv, kda_dtype io,
                               hipStream_t stream) {
  const long n = (long)B * H * (2 * dk + dv);
  if (n == 0 || T == 0) return hipSuccess;
  const dim3 grid((unsigned)((n + 255) / 256));
  if (io == KDA_BF16)
    hipLaunchKernelGGL(ring_advance_kernel<bf16>, grid, dim3(256), 0, stream,
                       static_cast<const bf16*>(q), static_cast<const bf16*>(k),
                       static_cast<const bf16*>(v), static_cast<bf16*>(ring), B, T, H, dk, dv);
  else
    hipLaunchKernelGGL(ring_advance_kernel<float>, grid, dim3(256), 0, stream,
                       static_cast<const float*>(q), static_cast<const float*>(k),
                       static_cast<const float*>(v), static_cast<float*>(ring), B, T, H, dk,
                       dv);
  return hipGetLastError();
}

hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t stream) {
  if (bytes == 0) return hipSuccess;
  size_t blocks = (bytes / 16 + 255) / 256;
  if (blocks < 1) blocks = 1;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                     static_cast<uint8_t*>(p), bytes);
  return hipGetLastError();
}

}  // namespace kda
