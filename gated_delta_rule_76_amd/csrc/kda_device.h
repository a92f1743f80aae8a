// Device-side helpers shared by the KDA kernels: element loads for the two
// q/k/v dtypes and the 16x16 MFMA tile products used by the prefill.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(__bf16 x) { return (float)x; }

// ---------------------------------------------------------------------------
// 16x16 output tiles on the matrix cores.
//
// Lane layout (wave64; lane = 16*g + m, g in 0..3, m in 0..15):
//   accumulator   lane holds C[4*g + i][m], i = 0..3
//   A operand     lane holds A[m][k] for 8 k-slots j = 0..7
//   B operand     lane holds B[k][m] for the same 8 k-slots
// A k-block is 32 wide; the k-slot (g, j) of a lane stands for column
// kb + 8*g + j of A and row kb + 8*g + j of B.  Any one-to-one assignment of
// k indices to (g, j) slots gives the same product as long as A and B use the
// same one; the kernels use this freedom to feed accumulators of one product
// straight into the next without moving data between lanes.
//
// Two precisions:
//   SplitBF16  each fp32 operand x is carried as hi = bf16(x) and
//              lo = bf16(x - hi) (both round-to-nearest-even), and a*b is
//              formed as hi*hi + hi*lo + lo*hi on v_mfma_f32_16x16x32_bf16
//              (about 16 significand bits per operand; the dropped lo*lo
//              term is below 2^-16 relative).
//   F32        plain fp32 operands on v_mfma_f32_16x16x4_f32 (8 issues per
//              32-wide k-block, each covering the k-slots j of all 4 lane
//              groups).
// ---------------------------------------------------------------------------

struct SplitBF16 {
  struct Frag {
    bf16x8 hi, lo;
  };
  static constexpr bool kSplit = true;

  __device__ __forceinline__ static Frag make(const float (&x)[8]) {
    Frag f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      __bf16 h = (__bf16)x[j];
      f.hi[j] = h;
      f.lo[j] = (__bf16)(x[j] - (float)h);
    }
    return f;
  }
  __device__ __forceinline__ static Frag zero() {
    Frag f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      f.hi[j] = (__bf16)0.0f;
      f.lo[j] = (__bf16)0.0f;
    }
    return f;
  }
  __device__ __forceinline__ static void mma(f32x4 &acc, const Frag &a, const Frag &b) {
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.hi, b.hi, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.hi, b.lo, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.lo, b.hi, acc, 0, 0, 0);
  }
};

struct F32 {
  struct Frag {
    float v[8];
  };
  static constexpr bool kSplit = false;

  __device__ __forceinline__ static Frag make(const float (&x)[8]) {
    Frag f;
#pragma unroll
    for (int j = 0; j < 8; ++j) f.v[j] = x[j];
    return f;
  }
  __device__ __forceinline__ static Frag zero() {
    Frag f;
#pragma unroll
    for (int j = 0; j < 8; ++j) f.v[j] = 0.0f;
    return f;
  }
  __device__ __forceinline__ static void mma(f32x4 &acc, const Frag &a, const Frag &b) {
#pragma unroll
    for (int j = 0; j < 8; ++j) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v[j], b.v[j], acc, 0, 0, 0);
  }
};

__device__ __forceinline__ f32x4 zero4() {
  f32x4 z;
  z[0] = z[1] = z[2] = z[3] = 0.0f;
  return z;
}

}  // namespace kda
