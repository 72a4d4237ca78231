// Workspace layout, MFMA operand policies and the unit-lower-triangular
// inverse shared by the chunked-prefill kernels (gfx950, wave64).
#pragma once

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
  __device__ static void st(T* p, frag f) { *reinterpret_cast<frag*>(p) = f; }
  __device__ static void st4(T* p, f32x4 v) {
    *reinterpret_cast<bf16x4*>(p) = bf16x4{(bf16)v[0], (bf16)v[1], (bf16)v[2], (bf16)v[3]};
  }
  using quad = bf16x4;  // four elements as loaded (converted at first use)
  __device__ static quad ld4(const T* p) { return *reinterpret_cast<const quad*>(p); }
  __device__ static f32x4 cvt4(quad v) {
    return f32x4{(float)v[0], (float)v[1], (float)v[2], (float)v[3]};
  }
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
  __device__ static void st(T* p, frag f) { *p = f; }
  __device__ static void st4(T* p, f32x4 v) { *reinterpret_cast<f32x4*>(p) = v; }
  using quad = f32x4;
  __device__ static quad ld4(const T* p) { return *reinterpret_cast<const quad*>(p); }
  __device__ static f32x4 cvt4(quad v) { return v; }
  __device__ static frag mk(const float* v) { return v[0]; }
  __device__ static f32x4 mma(frag a, frag b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
  }
};

constexpr int rup(int x, int m) { return (x + m - 1) / m * m; }

__device__ __forceinline__ f32x4 mma_f32x4(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// Workspace block of one (chunk, sequence, head); offsets in elements of T.
// "Fragment-major" arrays hold an MFMA A-operand as it sits in the lanes:
// element ((rb * nks + ks) * 64 + lane) * KPL + e is row 16*rb + lane%16,
// column ks*KS + (lane/16)*KPL + e, so one lane loads one contiguous piece.
// U' is stored in the accumulator layout: element ((rb * DV/16 + cb) * 64 +
// lane) * 4 + e is row 16*rb + 4*(lane/16) + e, column 16*cb + lane%16.
template <int C, int DK, int DV, class M>
struct Ws {
  static constexpr int DKP = rup(DK, M::KS);  // K-dims padded to the MFMA depth
  static constexpr int CP = rup(C, M::KS);
  static constexpr size_t oW = 0;                          // -W    [C x DKP] fragment-major
  static constexpr size_t oQ = oW + (size_t)C * DKP;       // Q~    [C x DKP] fragment-major
  static constexpr size_t oK = oQ + (size_t)C * DKP;       // K^^T  [DK x CP] fragment-major
  static constexpr size_t oP = oK + (size_t)DK * CP;       // P     [C][CP] row-major
  static constexpr size_t oU = oP + (size_t)C * CP;        // U'    [C x DV] accumulator layout
  static constexpr size_t nT = oU + (size_t)C * DV;
  static constexpr size_t bytes = nT * sizeof(typename M::T) + DK * sizeof(float);  // + e^{Gam_n}
};

constexpr size_t ws_block_bytes(int C, int DK, int DV, int KS, size_t esz) {
  return ((size_t)C * rup(DK, KS) * 2 + (size_t)DK * rup(C, KS) + (size_t)C * rup(C, KS) +
          (size_t)C * DV) * esz + (size_t)DK * 4;
}

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ bf16x4 to_bf16x4(f32x4 v) {
  return bf16x4{(bf16)v[0], (bf16)v[1], (bf16)v[2], (bf16)v[3]};
}

// Two 16x16 tiles d0, d1 in the accumulator layout (lane: rows 4(l/16)+e,
// column l%16), to one 16-byte piece per lane of 8 consecutive rows: lanes
// with even l/16 take d0's rows 8(l/32)..+7, lanes with odd l/16 take d1's
// (the partner lane is l^16).
__device__ __forceinline__ u32x4 pair_piece(f32x4 d0, f32x4 d1, int gq) {
  const u32x2 v0 = __builtin_bit_cast(u32x2, to_bf16x4(d0));
  const u32x2 v1 = __builtin_bit_cast(u32x2, to_bf16x4(d1));
  const bool odd = gq & 1;
  const u32x2 send = odd ? v0 : v1;
  const u32x2 recv = {(unsigned)__shfl_xor((int)send[0], 16, kWave),
                      (unsigned)__shfl_xor((int)send[1], 16, kWave)};
  return odd ? u32x4{recv[0], recv[1], v1[0], v1[1]} : u32x4{v0[0], v0[1], recv[0], recv[1]};
}

// X = (I + L)^{-1} for a strictly lower C x C matrix L (fp32, row stride
// C + 4), by 16 x 16 blocks: forward substitution inside each diagonal block
// (16 lanes of wave a for block a), then the block rows below the diagonal
// by distance, X_ab = -X_aa * sum_{b <= c < a} L_ac X_cb, on fp32 MFMA. All
// NT threads of the workgroup call it; the blocks above the diagonal of X
// are zeroed, the part of L above the diagonal is never read. Ends with a
// barrier.
template <int C, int NT>
__device__ __forceinline__ void unit_lower_inverse(const float (*sL)[C + 4], float (*sX)[C + 4],
                                                   int tid) {
  constexpr int NRB = C / 16;
  const int lane = tid % kWave, wv = tid / kWave, l16 = lane % 16, g16 = lane / 16;
  for (int idx = tid; idx < C * C; idx += NT) {
    const int rr = idx / C, jj = idx % C;
    if (jj / 16 > rr / 16) sX[rr][jj] = 0.f;
  }
  if (wv < NRB && lane < 16) {
    const int m = 16 * wv, j = lane;
    float x[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float acc = r == j ? 1.f : 0.f;
#pragma unroll
      for (int i = 0; i < r; ++i) acc -= sL[m + r][m + i] * x[i];
      x[r] = acc;
      __builtin_amdgcn_sched_barrier(0);  // one row of L in flight at a time
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) sX[m + r][m + j] = x[r];
  }
  __syncthreads();
  for (int dist = 1; dist < NRB; ++dist) {
    if (wv < NRB - dist) {
      const int ab = wv + dist, bb = wv;
      f32x4 y = {0.f, 0.f, 0.f, 0.f};
      for (int cb = bb; cb < ab; ++cb) {
#pragma unroll
        for (int s = 0; s < 4; ++s)
          y = mma_f32x4(sL[16 * ab + l16][16 * cb + 4 * s + g16],
                        sX[16 * cb + 4 * s + g16][16 * bb + l16], y);
      }
      // X_aa * Y with the contraction index of step s taken as 4*(lane/16)+s:
      // Y's rows are then exactly the accumulator elements each lane holds.
      f32x4 x = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < 4; ++s) x = mma_f32x4(sX[16 * ab + l16][16 * ab + 4 * g16 + s], y[s], x);
#pragma unroll
      for (int e = 0; e < 4; ++e) sX[16 * ab + 4 * g16 + e][16 * bb + l16] = -x[e];
    }
    __syncthreads();
  }
}

}  // namespace

// Preparation pass in the token-row layout (bf16 inputs, chunk 32 or 64,
// d_k and d_v multiples of 32): writes the same workspace blocks as the
// general preparation kernel. Returns hipErrorInvalidValue for shapes it
// does not cover.
bool prep_rows_supported(int chunk, int dk, int dv, kda_dtype io);
hipError_t launch_prep_rows(const PrefillArgs& a, int t0, int ncs, void* ws, hipStream_t stream);

}  // namespace kda
