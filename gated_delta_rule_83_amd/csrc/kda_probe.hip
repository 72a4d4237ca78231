// The practical HBM ceiling of a state stream: an in-place read-modify-write
// of a buffer with the access pattern of the decode step (16-byte vectors,
// non-temporal loads and stores, every byte read once and written once).
#include "kda_common.h"

namespace kda {
namespace {

// One workgroup of 256 threads per 32 KiB block, eight 16-byte vectors per
// thread, all loads issued before the stores. Of the shapes measured on
// MI355X (256 x 4 .. 1024 x 4 vectors per thread, with and without a grid
// stride, with and without the non-temporal hint) this one is the fastest on
// both a 384 MiB and a 6 GiB buffer: 6.1-6.3 and 5.6 TB/s. Full blocks take
// a path without per-vector bounds checks: with a check on every access the
// compiler waits for each load before issuing the next (4.4 TB/s).
constexpr int kProbeNT = 256;
constexpr int kProbeU = 8;

__global__ __launch_bounds__(kProbeNT) void stream_rmw_kernel(f32x4* p, long n4, float scale) {
  const long blk = (long)blockIdx.x * kProbeNT * kProbeU;
  f32x4* q = p + blk + threadIdx.x;
  if (blk + kProbeNT * kProbeU <= n4) {
    // a whole block in bounds: every load in flight before the first store
    f32x4 v[kProbeU];
#pragma unroll
    for (int u = 0; u < kProbeU; ++u) v[u] = __builtin_nontemporal_load(q + u * kProbeNT);
#pragma unroll
    for (int u = 0; u < kProbeU; ++u) __builtin_nontemporal_store(v[u] * scale, q + u * kProbeNT);
  } else {
    for (int u = 0; u < kProbeU; ++u) {
      if (blk + threadIdx.x + (long)u * kProbeNT < n4) {
        const f32x4 v = __builtin_nontemporal_load(q + u * kProbeNT);
        __builtin_nontemporal_store(v * scale, q + u * kProbeNT);
      }
    }
  }
}

}  // namespace

hipError_t launch_stream_rmw(void* buf, size_t bytes, float scale, hipStream_t stream) {
  const long n4 = (long)(bytes / 16);
  const long blocks = (n4 + (long)kProbeNT * kProbeU - 1) / ((long)kProbeNT * kProbeU);
  if (blocks < 1) return hipSuccess;
  if (blocks > 0x7fffffffL) return hipErrorInvalidValue;
  hipLaunchKernelGGL(stream_rmw_kernel, dim3((unsigned)blocks), dim3(kProbeNT), 0, stream,
                     static_cast<f32x4*>(buf), n4, scale);
  return hipGetLastError();
}

}  // namespace kda
