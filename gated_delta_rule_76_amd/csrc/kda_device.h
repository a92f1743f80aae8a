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

// Eight consecutive q/k/v elements as loaded from memory (one 16-byte load
// for bf16, two for fp32), kept packed in registers until converted.
template <typename T>
struct Raw8;

template <>
struct Raw8<__bf16> {
  uint4 u;
  __device__ __forceinline__ void load(const __bf16 *p) { u = *reinterpret_cast<const uint4 *>(p); }
  __device__ __forceinline__ void to_f32(float (&x)[8]) const {
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[2 * i] = __uint_as_float(w[i] << 16);
      x[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  }
};

template <>
struct Raw8<float> {
  float4 a, b;
  __device__ __forceinline__ void load(const float *p) {
    a = *reinterpret_cast<const float4 *>(p);
    b = *reinterpret_cast<const float4 *>(p + 4);
  }
  __device__ __forceinline__ void to_f32(float (&x)[8]) const {
    x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
    x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
  }
};

// Four consecutive elements (8 bytes for bf16, 16 for fp32).
template <typename T>
struct Raw4;

template <>
struct Raw4<__bf16> {
  uint2 u;
  __device__ __forceinline__ void load(const __bf16 *p) { u = *reinterpret_cast<const uint2 *>(p); }
  __device__ __forceinline__ void to_f32(float (&x)[4]) const {
    x[0] = __uint_as_float(u.x << 16);
    x[1] = __uint_as_float(u.x & 0xffff0000u);
    x[2] = __uint_as_float(u.y << 16);
    x[3] = __uint_as_float(u.y & 0xffff0000u);
  }
};

template <>
struct Raw4<float> {
  float4 a;
  __device__ __forceinline__ void load(const float *p) { a = *reinterpret_cast<const float4 *>(p); }
  __device__ __forceinline__ void to_f32(float (&x)[4]) const {
    x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
  }
};

// Two consecutive elements (4 bytes for bf16, 8 for fp32).
template <typename T>
struct Raw2;

template <>
struct Raw2<__bf16> {
  uint32_t u;
  __device__ __forceinline__ void load(const __bf16 *p) { u = *reinterpret_cast<const uint32_t *>(p); }
  __device__ __forceinline__ void to_f32(float (&x)[2]) const {
    x[0] = __uint_as_float(u << 16);
    x[1] = __uint_as_float(u & 0xffff0000u);
  }
};

template <>
struct Raw2<float> {
  float2 a;
  __device__ __forceinline__ void load(const float *p) { a = *reinterpret_cast<const float2 *>(p); }
  __device__ __forceinline__ void to_f32(float (&x)[2]) const {
    x[0] = a.x; x[1] = a.y;
  }
};

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
