// Gradient of the prologue (the width-4 causal short conv, SiLU, and the L2
// normalisation of q and k) for training: from the gradients of q^, k^, v^
// to those of the raw projections q, k, v, of the conv weights and of the
// ring history read before token 0. gfx950, wave64, fp32 arithmetic.
//
// Per channel c with raw values x_s (s < 0 from the ring), the forward is
// y_t = sum_j w[c][j] x_{t-3+j}, z_t = SiLU(y_t), q^ = z / sqrt(|z|^2 + eps)
// over the d_k channels of a (token, head) for q and k, v^ = z for v
// ("KV缓存从11.25GB缩到0.21GB：…", section "KDA 递推公式先衰减再差分").
// Reverse mode: dz = (dq^ - q^ (q^ . dq^)) / sqrt(|z|^2 + eps) (q, k) or
// dz = dv^ (v); dy = dz (s(y) + y s(y) (1 - s(y))), s the logistic sigmoid;
// dx_{t-3+j} += w[c][j] dy_t and dw[c][j] += dy_t x_{t-3+j}.
//
// One workgroup per (sequence, head, 32-token segment): the raw values of
// the segment and the 3 tokens before it are staged in LDS, dy is formed for
// the segment and the 3 tokens after it (wave per token, lanes over
// channels, the two L2 sums by wave reductions), then dx of the segment,
// the segment's share of dw (to a partial buffer) and, in the first segment,
// the ring's gradient. A second kernel adds the dw partials in a fixed order.
#include "kda_common.h"

namespace kda {
namespace {

constexpr int kSeg = 32;       // tokens per workgroup
// threads per workgroup: eight waves, four workgroups per CU (37 KB of LDS
// each). Measured on MI355X for the 4096-token, 96-head workload: 504 us,
// against 570 with 256 threads and 531 with 1024 (the results are the same
// bit for bit: each token's and channel's arithmetic stays in one wave or
// thread, in the same order).
constexpr int kPBT = 512;
constexpr int kHalo = 3;       // conv history

__device__ __forceinline__ f32x4 ld4x(const float* p) { return *reinterpret_cast<const f32x4*>(p); }
__device__ __forceinline__ f32x4 ld4x(const bf16* p) {
  const bf16x4 v = *reinterpret_cast<const bf16x4*>(p);
  return f32x4{(float)v[0], (float)v[1], (float)v[2], (float)v[3]};
}

// rows x N values into LDS rows of 128 floats, 4 per load, every load of a
// thread issued before its stores; src(u, c) gives the four values of row u
// from column c.
template <int N, int MAXROWS, class F>
__device__ __forceinline__ void stage(float (*dst)[128], int rows, F&& src) {
  constexpr int Q = N / 4, PER = (MAXROWS * Q + kPBT - 1) / kPBT;
  f32x4 buf[PER];
#pragma unroll
  for (int p = 0; p < PER; ++p) {
    const int i = (int)threadIdx.x + p * kPBT, u = i / Q, c = 4 * (i % Q);
    buf[p] = u < rows ? src(u, c) : f32x4{0.f, 0.f, 0.f, 0.f};
  }
#pragma unroll
  for (int p = 0; p < PER; ++p) {
    const int i = (int)threadIdx.x + p * kPBT, u = i / Q, c = 4 * (i % Q);
    if (u < rows) *reinterpret_cast<f32x4*>(&dst[u][c]) = buf[p];
  }
}

template <int N, bool L2, typename IO>
__device__ void proj_backward(const PrologueBwdArgs& a, int b, int h, int seg, long c0,
                              const IO* x, const IO* dxh, IO* dxo, float (*sx)[128],
                              float (*sdy)[128]) {
  const int T = a.T, t0 = seg * kSeg, t1 = min(t0 + kSeg, T), te = min(t0 + kSeg + kHalo, T);
  const int tid = threadIdx.x, lane = tid % kWave, wv = tid / kWave;
  const long st = (long)a.H * N;                          // token stride
  const long base = (long)b * T * st + (long)h * N;       // token 0 of (b, h)
  const long Ctot = (long)a.H * (2 * a.dk + a.dv);
  const IO* ring = static_cast<const IO*>(a.ring);
  // raw values of tokens t0-3 .. te-1 (row u is token t0 - 3 + u), and the
  // activation gradients of tokens t0 .. te-1 (sdy, replaced by dy in place)
  stage<N, kSeg + 2 * kHalo>(sx, te - t0 + kHalo, [&](int u, int c) {
    const int t = t0 - kHalo + u;
    if (t >= 0) return ld4x(x + base + (long)t * st + c);
    if (ring) return ld4x(ring + ((long)b * 3 + (3 + t)) * Ctot + c0 + c);
    return f32x4{0.f, 0.f, 0.f, 0.f};
  });
  stage<N, kSeg + kHalo>(sdy, te - t0,
                         [&](int u, int c) { return ld4x(dxh + base + (long)(t0 + u) * st + c); });
  __syncthreads();
  // dy of tokens t0 .. te-1: wave per token, lanes over channels
  constexpr int CPL = (N + kWave - 1) / kWave;
  f32x4 wl[CPL];
#pragma unroll
  for (int m = 0; m < CPL; ++m) {
    const int c = lane + kWave * m;
    wl[m] = c < N ? *reinterpret_cast<const f32x4*>(a.conv_w + 4 * (c0 + c))
                  : f32x4{0.f, 0.f, 0.f, 0.f};
  }
  for (int u = wv; u < te - t0; u += kPBT / kWave) {
    float yv[CPL], zv[CPL], gv[CPL], sv[CPL];
    float ss = 0.f, dot = 0.f;
#pragma unroll
    for (int m = 0; m < CPL; ++m) {
      const int c = lane + kWave * m;
      yv[m] = zv[m] = gv[m] = sv[m] = 0.f;
      if (c < N) {
        const f32x4 w = wl[m];
        yv[m] = w[0] * sx[u][c] + w[1] * sx[u + 1][c] + w[2] * sx[u + 2][c] + w[3] * sx[u + 3][c];
        // sigmoid by the hardware reciprocal (about 1 ulp), as in the forward's SiLU
        sv[m] = __builtin_amdgcn_rcpf(1.0f + __expf(-yv[m]));
        zv[m] = yv[m] * sv[m];
        gv[m] = sdy[u][c];
        ss += zv[m] * zv[m];
        dot += zv[m] * gv[m];
      }
    }
    float inv = 1.f;
    if constexpr (L2) {
      ss = wave_sum(ss);
      dot = wave_sum(dot);
      inv = __builtin_amdgcn_rsqf(ss + kL2Eps);
    }
#pragma unroll
    for (int m = 0; m < CPL; ++m) {
      const int c = lane + kWave * m;
      if (c < N) {
        // (dq^ - q^ (q^ . dq^)) / |z| with q^ = z / |z| and q^ . dq^ = (z . dq^) / |z|
        const float dz = L2 ? (gv[m] - zv[m] * dot * inv * inv) * inv : gv[m];
        const float sg = sv[m];
        sdy[u][c] = dz * (sg + yv[m] * sg * (1.0f - sg));
      }
    }
  }
  __syncthreads();
  // dx of the segment's tokens: dx_t = sum_j w[j] dy_{t+3-j} (t + 3 - j < T);
  // a thread's channel is the same in every iteration (N divides kPBT)
  static_assert(kPBT % N == 0, "channel per thread");
  {
    const int c = tid % N;
    const f32x4 w = *reinterpret_cast<const f32x4*>(a.conv_w + 4 * (c0 + c));
    for (int u = tid / N; u < t1 - t0; u += kPBT / N) {
      float acc = 0.f;
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (u + 3 - j < te - t0) acc += w[j] * sdy[u + 3 - j][c];
      dxo[base + (long)(t0 + u) * st + c] = from_f32<IO>(acc);
    }
  }
  // the segment's share of dw, and the ring's gradient in the first segment
  for (int c = tid; c < N; c += kPBT) {
    f32x4 dw = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
    for (int u = 0; u < t1 - t0; ++u) {
      const float d = sdy[u][c];
#pragma unroll
      for (int j = 0; j < 4; ++j) dw[j] += d * sx[u + j][c];
    }
    *reinterpret_cast<f32x4*>(a.wpart + (((long)b * a.nseg + seg) * Ctot + c0 + c) * 4) = dw;
    if (seg == 0 && a.dring) {
      const f32x4 w = *reinterpret_cast<const f32x4*>(a.conv_w + 4 * (c0 + c));
#pragma unroll
      for (int s = 0; s < 3; ++s) {  // ring slot s holds token s - 3
        float acc = 0.f;
#pragma unroll
        for (int j = 0; j < 4; ++j)
          if (s - j >= 0 && s - j < te) acc += w[j] * sdy[s - j][c];
        a.dring[((long)b * 3 + s) * Ctot + c0 + c] = acc;
      }
    }
  }
  __syncthreads();  // sx, sdy are reused by the next projection
}

template <int DK, int DV, typename IO>
__global__ __launch_bounds__(kPBT) void prologue_bwd_kernel(PrologueBwdArgs a) {
  __shared__ __attribute__((aligned(16))) float sx[kSeg + 2 * kHalo][128];
  __shared__ __attribute__((aligned(16))) float sdy[kSeg + kHalo][128];
  const int seg = blockIdx.x % a.nseg, bh = blockIdx.x / a.nseg;
  const int b = bh / a.H, h = bh % a.H;
  const IO* q = static_cast<const IO*>(a.q);
  const IO* k = static_cast<const IO*>(a.k);
  const IO* v = static_cast<const IO*>(a.v);
  proj_backward<DK, true, IO>(a, b, h, seg, (long)h * DK, q, static_cast<const IO*>(a.dqh),
                              static_cast<IO*>(a.dq_raw), sx, sdy);
  proj_backward<DK, true, IO>(a, b, h, seg, (long)a.H * DK + (long)h * DK, k,
                              static_cast<const IO*>(a.dkh), static_cast<IO*>(a.dk_raw), sx, sdy);
  proj_backward<DV, false, IO>(a, b, h, seg, 2L * a.H * DK + (long)h * DV, v,
                               static_cast<const IO*>(a.dvh), static_cast<IO*>(a.dv_raw), sx,
                               sdy);
}

// dconv_w[c] = the partials of every (sequence, segment), added in order.
__global__ __launch_bounds__(256) void conv_w_grad_kernel(const float* wpart, long parts,
                                                          long ctot, float* dconv_w) {
  const long c = (long)blockIdx.x * 256 + threadIdx.x;
  if (c >= ctot) return;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 8
  for (long p = 0; p < parts; ++p) acc += *reinterpret_cast<const f32x4*>(wpart + (p * ctot + c) * 4);
  *reinterpret_cast<f32x4*>(dconv_w + c * 4) = acc;
}

template <int DK, int DV>
hipError_t run_pb(const PrologueBwdArgs& a, kda_dtype io, hipStream_t st) {
  const unsigned grid = (unsigned)((long)a.B * a.H * a.nseg);
  if (grid == 0) return hipSuccess;  // no tokens
  if (io == KDA_BF16)
    hipLaunchKernelGGL((prologue_bwd_kernel<DK, DV, bf16>), dim3(grid), dim3(kPBT), 0, st, a);
  else
    hipLaunchKernelGGL((prologue_bwd_kernel<DK, DV, float>), dim3(grid), dim3(kPBT), 0, st, a);
  return hipGetLastError();
}

template <int DK>
hipError_t run_pb_dv(const PrologueBwdArgs& a, kda_dtype io, hipStream_t st) {
  switch (a.dv) {
    case 16: return run_pb<DK, 16>(a, io, st);
    case 32: return run_pb<DK, 32>(a, io, st);
    case 64: return run_pb<DK, 64>(a, io, st);
    case 128: return run_pb<DK, 128>(a, io, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace

int prologue_bwd_segments(int T) { return (T + kSeg - 1) / kSeg; }

hipError_t launch_prologue_backward(const PrologueBwdArgs& a, kda_dtype io, hipStream_t st) {
  hipError_t e = hipErrorInvalidValue;
  switch (a.dk) {
    case 16: e = run_pb_dv<16>(a, io, st); break;
    case 32: e = run_pb_dv<32>(a, io, st); break;
    case 64: e = run_pb_dv<64>(a, io, st); break;
    case 128: e = run_pb_dv<128>(a, io, st); break;
  }
  if (e != hipSuccess) return e;
  const long ctot = (long)a.H * (2 * a.dk + a.dv);
  hipLaunchKernelGGL(conv_w_grad_kernel, dim3((unsigned)((ctot + 255) / 256)), dim3(256), 0, st,
                     (const float*)a.wpart, (long)a.B * a.nseg, ctot, a.dconv_w);
  return hipGetLastError();
}

}  // namespace kda
