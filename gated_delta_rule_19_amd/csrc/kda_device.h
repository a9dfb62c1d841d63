// Device-side building blocks shared by the KDA kernels (gfx950 / CDNA4).
//
// Matrix products run on the 16x16 MFMA tiles of CDNA4 with wave64:
//   bf16 : v_mfma_f32_16x16x32_bf16  (one instruction per K = 32 step)
//   fp32 : v_mfma_f32_16x16x4f32     (eight instructions per K = 32 step)
// A "fragment" is the 8 consecutive K-elements one lane contributes to one
// K = 32 step.  Lane l of a wave holds, for a 16 x 32 A tile, row (l % 16)
// and K-columns 8*(l/16) .. 8*(l/16)+7; for a 32 x 16 B tile, column (l % 16)
// and K-rows 8*(l/16) .. +7.  The 16 x 16 fp32 accumulator holds column
// (l % 16) and rows 4*(l/16) .. 4*(l/16)+3 in its four registers.
//
// The fp32 path feeds the same fragments to eight K = 4 instructions: in
// instruction j lane l supplies element j of its fragment as K-index (l/16).
// Summed over j that covers the same 32 K-indices, so both element types
// share one code path and one data layout.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kda_internal.h"

namespace kda {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

template <typename T> struct Frag;

template <> struct Frag<bf16> {
  bf16x8 v;
};

template <> struct Frag<float> {
  f32x4 lo, hi;
};

// Load 8 consecutive elements (16-byte aligned for bf16, 32 for fp32).
__device__ __forceinline__ Frag<bf16> load_frag(const bf16 *p) {
  Frag<bf16> f;
  f.v = *reinterpret_cast<const bf16x8 *>(p);
  return f;
}

__device__ __forceinline__ Frag<float> load_frag(const float *p) {
  Frag<float> f;
  f.lo = *reinterpret_cast<const f32x4 *>(p);
  f.hi = *reinterpret_cast<const f32x4 *>(p + 4);
  return f;
}

template <typename T> __device__ __forceinline__ Frag<T> frag_from_f32(const float (&x)[8]);

template <> __device__ __forceinline__ Frag<bf16> frag_from_f32<bf16>(const float (&x)[8]) {
  Frag<bf16> f;
#pragma unroll
  for (int j = 0; j < 8; ++j)
    f.v[j] = static_cast<bf16>(x[j]);
  return f;
}

template <> __device__ __forceinline__ Frag<float> frag_from_f32<float>(const float (&x)[8]) {
  Frag<float> f;
  f.lo = f32x4{x[0], x[1], x[2], x[3]};
  f.hi = f32x4{x[4], x[5], x[6], x[7]};
  return f;
}

__device__ __forceinline__ void frag_to_f32(const Frag<bf16> &f, float (&x)[8]) {
#pragma unroll
  for (int j = 0; j < 8; ++j)
    x[j] = static_cast<float>(f.v[j]);
}

__device__ __forceinline__ void frag_to_f32(const Frag<float> &f, float (&x)[8]) {
  x[0] = f.lo[0]; x[1] = f.lo[1]; x[2] = f.lo[2]; x[3] = f.lo[3];
  x[4] = f.hi[0]; x[5] = f.hi[1]; x[6] = f.hi[2]; x[7] = f.hi[3];
}

// acc(16x16) += A(16x32) * B(32x16)
__device__ __forceinline__ void mma(f32x4 &acc, const Frag<bf16> &a, const Frag<bf16> &b) {
  acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.v, b.v, acc, 0, 0, 0);
}

__device__ __forceinline__ void mma(f32x4 &acc, const Frag<float> &a, const Frag<float> &b) {
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.lo[0], b.lo[0], acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.lo[1], b.lo[1], acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.lo[2], b.lo[2], acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.lo[3], b.lo[3], acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.hi[0], b.hi[0], acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.hi[1], b.hi[1], acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.hi[2], b.hi[2], acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.hi[3], b.hi[3], acc, 0, 0, 0);
}

// Scalar element conversions.
__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16 x) { return static_cast<float>(x); }
template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float x) { return static_cast<bf16>(x); }

// Store 4 consecutive elements converted from fp32 (8-byte aligned for
// bf16, 16 for fp32).
__device__ __forceinline__ void store4(bf16 *p, float a, float b, float c, float d) {
  bf16x4 v;
  v[0] = static_cast<bf16>(a); v[1] = static_cast<bf16>(b);
  v[2] = static_cast<bf16>(c); v[3] = static_cast<bf16>(d);
  *reinterpret_cast<bf16x4 *>(p) = v;
}

__device__ __forceinline__ void store4(float *p, float a, float b, float c, float d) {
  *reinterpret_cast<f32x4 *>(p) = f32x4{a, b, c, d};
}

// Store 8 consecutive elements.
__device__ __forceinline__ void store8(bf16 *p, const float (&x)[8]) {
  bf16x8 v;
#pragma unroll
  for (int j = 0; j < 8; ++j)
    v[j] = static_cast<bf16>(x[j]);
  *reinterpret_cast<bf16x8 *>(p) = v;
}

__device__ __forceinline__ void store8(float *p, const float (&x)[8]) {
  *reinterpret_cast<f32x4 *>(p) = f32x4{x[0], x[1], x[2], x[3]};
  *reinterpret_cast<f32x4 *>(p + 4) = f32x4{x[4], x[5], x[6], x[7]};
}

} // namespace kda
