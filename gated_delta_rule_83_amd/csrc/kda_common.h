// Shared device helpers and kernel launch declarations for the KDA kernels
// (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kda.h"

namespace kda {

using bf16 = __bf16;
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;
constexpr float kL2Eps = 1e-6f;

// Element loads/stores of the token I/O type. __bf16 -> float is exact;
// float -> __bf16 rounds to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16 x) { return (float)x; }
template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float x) { return (bf16)x; }

// Raw buffer stores: a store whose byte offset is at or past the resource's
// size is dropped by the hardware range check, so row tails need no branch.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(base, (short)0, bytes, 0x00020000);
}
__device__ __forceinline__ void buf_store(__amdgpu_buffer_rsrc_t r, int off, float v, float*) {
  __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(unsigned, v), r, off, 0, 0);
}
__device__ __forceinline__ void buf_store(__amdgpu_buffer_rsrc_t r, int off, float v, bf16*) {
  __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(unsigned short, (bf16)v), r, off, 0,
                                        0);
}

// SiLU(y) = y * sigmoid(y), with the hardware reciprocal (about 1 ulp) in place
// of an IEEE division; y -> -inf gives -0.
__device__ __forceinline__ float silu(float y) {
  return y * __builtin_amdgcn_rcpf(1.0f + __expf(-y));
}

// The gates formed from raw projections (KDA_F_RAW_GATES): the log-decay
// log(sigmoid(x)) = min(x, 0) - log(1 + e^{-|x|}), which does not overflow,
// with the hardware exp2/log2 (the log's argument lies in (1, 2], so the
// result is within about 1e-7 absolute), and the update strength sigmoid(x).
__device__ __forceinline__ float log_sigmoid(float x) {
  return fminf(x, 0.0f) - __logf(1.0f + __expf(-fabsf(x)));
}
__device__ __forceinline__ float sigmoid(float x) { return 1.0f / (1.0f + __expf(-x)); }

// Sum over the 64 lanes of a wave; every lane receives the total.
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off, kWave);
  return x;
}

// ---- launch helpers (defined in the .hip files) ---------------------------

struct DecodeArgs {
  float* S;              // [B][H][dk][dv]
  void* ring;            // [B][3][Ctot] io dtype
  const void* q;         // [B][H][dk]
  const void* k;         // [B][H][dk]
  const void* v;         // [B][H][dv]
  const float* g;        // [B][H][dk], or [B][H] with KDA_F_SCALAR_G
  const float* beta;     // [B][H]
  const float* conv_w;   // [Ctot][4]
  void* o;               // [B][H][dv]
  int B, H, dk, dv;
  uint32_t flags;
  // output gate fused into the readout (NULL gate: plain readout)
  const void* gate;      // [B][H][dv] io dtype, gate pre-activations
  const float* norm_w;   // [dv]
  float norm_eps;
};
hipError_t launch_decode(const DecodeArgs& a, kda_dtype io, hipStream_t stream);

// Gated RMSNorm of rows of dv values: y = x / sqrt(mean x^2 + eps) * w * sigmoid(z).
hipError_t launch_gated_rmsnorm(const void* x, const void* z, const float* w, float eps,
                                void* y, long rows, int dv, kda_dtype io, hipStream_t stream);

struct PrologueArgs {
  const void* q;  // [B][T][H][dk]
  const void* k;
  const void* v;  // [B][T][H][dv]
  const float* conv_w;
  void* ring;     // [B][3][Ctot]
  float* q_out;
  float* k_out;
  float* v_out;
  int B, T, H, dk, dv;
  uint32_t flags;
};
hipError_t launch_prologue(const PrologueArgs& a, kda_dtype io, hipStream_t stream);

// Ring advance after a T-token block: ring <- last 3 raw tokens of
// (ring, x_0..x_{T-1}). Reads x from the raw inputs [B][T][H][d].
hipError_t launch_ring_advance(const void* q, const void* k, const void* v, void* ring,
                               int B, int T, int H, int dk, int dv, kda_dtype io,
                               hipStream_t stream);

hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t stream);

// In-place non-temporal read-modify-write of bytes (a multiple of 16) at buf:
// buf *= scale, 16 bytes per access (the HBM ceiling of a state stream).
hipError_t launch_stream_rmw(void* buf, size_t bytes, float scale, hipStream_t stream);

struct PrefillArgs {
  float* S;            // [B][H][dk][dv]
  void* ring;          // [B][3][Ctot]
  const void* q;       // [B][T][H][dk]
  const void* k;
  const void* v;       // [B][T][H][dv]
  const float* g;      // [B][T][H][dk], or [B][T][H] with KDA_F_SCALAR_G
  const float* beta;   // [B][T][H]
  const float* conv_w; // [Ctot][4]
  void* o;             // [B][T][H][dv]
  int B, T, H, dk, dv, chunk;
  uint32_t flags;
};
size_t prefill_ws_bytes_per_chunk(int H, int B, int dk, int dv, int chunk, kda_dtype io);
hipError_t launch_prefill(const PrefillArgs& a, kda_dtype io, void* ws, size_t ws_bytes,
                          hipStream_t stream);

struct BackwardArgs {
  const void* q;        // [B][T][H][dk] q^ (io dtype), after conv, SiLU and L2
  const void* k;        // [B][T][H][dk] k^
  const void* v;        // [B][T][H][dv] v^
  const float* g;       // [B][T][H][dk]
  const float* beta;    // [B][T][H]
  const float* S0;      // [B][H][dk][dv] state entering chunk c0, or NULL (zero)
  const void* dO;       // [B][T][H][dv] (io dtype)
  const float* dST;     // [B][H][dk][dv] gradient of the state leaving chunk c1 - 1, or NULL
  void* dq;             // [B][T][H][dk] (io dtype)
  void* dk;
  void* dv;             // [B][T][H][dv] (io dtype)
  float* dg;            // [B][T][H][dk]
  float* dbeta;         // [B][T][H]
  float* dS0;           // [B][H][dk][dv] gradient of the state entering chunk c0, or NULL
  int B, T, H, dkw, dvw, chunk;  // widths d_k, d_v
  // set by launch_backward for each launch: the chunk range [c0, c1) and
  // the workspace regions (indexed from chunk c0)
  int c0, c1;
  float* S_out;         // [B][H][dk][dv] state leaving chunk c1 - 1, or NULL
  float* scratch;       // per (chunk, sequence, head) blocks
  float* S0s;           // entering state of every chunk [c1 - c0][B][H][dk][dv]
  float* dS1s;          // gradient reaching every chunk's leaving state
};
// Workspace of the one-shot call (every chunk's blocks at once), and the
// least any chunk-range split needs.
size_t backward_ws_bytes(int B, int T, int H, int dk, int dv, int chunk);
size_t backward_ws_min_bytes(int B, int T, int H, int dk, int dv, int chunk);
hipError_t launch_backward(BackwardArgs a, kda_dtype io, void* ws, size_t ws_bytes,
                           hipStream_t stream);

struct PrologueBwdArgs {
  const void* q;        // [B][T][H][dk] raw projections (io dtype)
  const void* k;
  const void* v;        // [B][T][H][dv]
  const float* conv_w;  // [Ctot][4]
  const void* ring;     // [B][3][Ctot] history before token 0 (io dtype), or NULL
  const void* dqh;      // [B][T][H][dk] gradient of q^ (io dtype)
  const void* dkh;
  const void* dvh;      // [B][T][H][dv]
  void* dq_raw;         // [B][T][H][dk] (io dtype)
  void* dk_raw;
  void* dv_raw;         // [B][T][H][dv]
  float* dconv_w;       // [Ctot][4]
  float* dring;         // [B][3][Ctot], or NULL
  float* wpart;         // [B][nseg][Ctot][4] per-segment weight gradients
  int B, T, H, dk, dv, nseg;
};
int prologue_bwd_segments(int T);
hipError_t launch_prologue_backward(const PrologueBwdArgs& a, kda_dtype io, hipStream_t stream);

}  // namespace kda
