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

// Raw buffer resource over `bytes` bytes at p: loads past the end read 0,
// stores past the end are dropped, and offsets are 32-bit.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void *p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), 0, (int)bytes, 0x00020000);
}

// 16 bytes per lane from a buffer straight into LDS: lane l reads at byte
// voff (its own) and writes LDS bytes 16 l .. 16 l + 15 after the
// wave-uniform LDS base.
__device__ __forceinline__ void lds_load16(__amdgpu_buffer_rsrc_t r, int voff, uint8_t *lds_base) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(
      r, (__attribute__((address_space(3))) void *)lds_base, 16, voff, 0, 0, 0);
}

// One element to a buffer at byte voff + soff (soff wave-uniform).
__device__ __forceinline__ void buffer_store(__amdgpu_buffer_rsrc_t r, bf16 x, int voff, int soff) {
  __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(short, x), r, voff, soff, 0);
}
__device__ __forceinline__ void buffer_store(__amdgpu_buffer_rsrc_t r, float x, int voff, int soff) {
  __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(int, x), r, voff, soff, 0);
}

// 4 consecutive elements (8-byte aligned for bf16, 16 for fp32) from a
// buffer at byte voff, widened to fp32; past the end they read 0.
__device__ __forceinline__ void buffer_load4(__amdgpu_buffer_rsrc_t r, int voff, const bf16 *,
                                             float *x) {
  auto w = __builtin_amdgcn_raw_buffer_load_b64(r, voff, 0, 0);
  x[0] = __builtin_bit_cast(float, w[0] << 16);
  x[1] = __builtin_bit_cast(float, w[0] & 0xffff0000u);
  x[2] = __builtin_bit_cast(float, w[1] << 16);
  x[3] = __builtin_bit_cast(float, w[1] & 0xffff0000u);
}
// (the whole vector is bit-cast: this compiler mis-handles a bit-cast of a
// single vector element, reading element 0 whatever the index)
__device__ __forceinline__ void buffer_load4(__amdgpu_buffer_rsrc_t r, int voff, const float *,
                                             float *x) {
  const f32x4 v = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, 0, 0));
#pragma unroll
  for (int j = 0; j < 4; ++j)
    x[j] = v[j];
}
// One element from a buffer at byte voff, widened to fp32 (0 past the end).
__device__ __forceinline__ float buffer_load1(__amdgpu_buffer_rsrc_t r, int voff, const bf16 *) {
  const unsigned short w = __builtin_amdgcn_raw_buffer_load_b16(r, voff, 0, 0);
  return __builtin_bit_cast(float, (unsigned)w << 16);
}
__device__ __forceinline__ float buffer_load1(__amdgpu_buffer_rsrc_t r, int voff, const float *) {
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, voff, 0, 0));
}

// acc += A * B for 16 x 16 fp32 blocks on v_mfma_f32_16x16x4f32.  A is read
// from LDS (row-major, 16-byte aligned rows): lane (lr, lg) loads
// A[lr][4lg .. 4lg+3].  B is held in the MFMA accumulator layout (lane holds
// B[4lg + i][lr] in element i), which is also a valid B operand: in step i
// every lane supplies K-index 4lg + i on both sides.  So a product's result
// feeds the next product directly.  sign = -1 negates A.
// B is taken by value: acc and B may be the same variable (Y <- Y + A Y).
__device__ __forceinline__ void mm16_lds_acc(f32x4 &acc, const float *A, int lda, const f32x4 B,
                                             int lr, int lg, float sign = 1.f) {
  const f32x4 a = *reinterpret_cast<const f32x4 *>(A + lr * lda + 4 * lg) * sign;
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[0], B[0], acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[1], B[1], acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[2], B[2], acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[3], B[3], acc, 0, 0, 0);
}

// acc += A B for 16 x 16 fp32 blocks with both operands in registers.  A
// block is held either in the accumulator ("column") layout, lane (lr, lg)
// element i = X[4 lg + i][lr], or in the row layout, element i = X[lr][4 lg + i]
// (the column layout of X^T).  a is A in the row layout, b is B in the column
// layout; the result is in the column layout.  Passing (B column, A row)
// instead yields B^T A^T in the column layout, i.e. A B in the row layout.
__device__ __forceinline__ void mm16_rr(f32x4 &acc, const f32x4 a, const f32x4 b) {
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[0], b[0], acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[1], b[1], acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[2], b[2], acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[3], b[3], acc, 0, 0, 0);
}

// Store / load a 16 x 16 fp32 block in the accumulator layout.
__device__ __forceinline__ void acc_store(float *D, int ld, const f32x4 &x, int lr, int lg) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
    D[(4 * lg + i) * ld + lr] = x[i];
}
__device__ __forceinline__ f32x4 acc_load(const float *D, int ld, int lr, int lg) {
  f32x4 x;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    x[i] = D[(4 * lg + i) * ld + lr];
  return x;
}

// Workgroup barrier ordering LDS only; global loads stay in flight across it.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// The bounded log decay from a raw gate logit z, g_min * sigmoid(ea z), with
// ea = exp(A_h) the head's scale ("Kimi K3.1 Pro 架构完全拆解" §3.2).  Tends
// to 0 as ea z -> -inf (exp overflows to inf, its reciprocal is 0).
__device__ __forceinline__ float gate_log_decay(float z, float ea, float g_min) {
  return g_min * __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(-(ea * z) * 1.4426950408889634f));
}

// Lane index as an opaque value: lane-dependent addresses built on it are
// recomputed where they are used instead of being hoisted out of the chunk
// loop and kept alive (or spilled) across all of its stages.
__device__ __forceinline__ int opaque_lane() {
  int l;
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(l));
  return l;
}

// x plus its value in lane ^ 32, and in lane ^ 16: the gfx950 lane swaps
// (VALU, no LDS round trip) hand each lane its own value and its partner's,
// and the sum is the same in both lanes (fp32 addition commutes).
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ float add_xor32(float x) {
  const unsigned u = __builtin_bit_cast(unsigned, x);
  const f32x2_t r = __builtin_bit_cast(
      f32x2_t, (u32x2_t)__builtin_amdgcn_permlane32_swap(u, u, false, false));
  return r.x + r.y;
}
__device__ __forceinline__ float add_xor16(float x) {
  const unsigned u = __builtin_bit_cast(unsigned, x);
  const f32x2_t r = __builtin_bit_cast(
      f32x2_t, (u32x2_t)__builtin_amdgcn_permlane16_swap(u, u, false, false));
  return r.x + r.y;
}

// LDS writes of this wave are complete and visible to its own later reads.
__device__ __forceinline__ void wave_lds_fence() {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
}

__device__ __forceinline__ void wait_vmem_all() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// Sum of squares of 8 bf16 values held as 4 raw dwords, added to acc
// (v_dot2c_f32_bf16: the products are exact in fp32).  The pairs come out of
// a whole-vector bit-cast: a bit-cast of a single element r[j] would read
// element 0 whatever j.
__device__ __forceinline__ float sumsq8_bf16(const u32x4 &r, float acc) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  const bf16x8 v = __builtin_bit_cast(bf16x8, r);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(v, v, 0, 1),
                                        __builtin_shufflevector(v, v, 0, 1), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(v, v, 2, 3),
                                        __builtin_shufflevector(v, v, 2, 3), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(v, v, 4, 5),
                                        __builtin_shufflevector(v, v, 4, 5), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(v, v, 6, 7),
                                        __builtin_shufflevector(v, v, 6, 7), acc, false);
  return acc;
}

// 8 bf16 (raw dwords) -> fp32
__device__ __forceinline__ void widen8(u32x4 w, float *x) {
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    x[2 * d] = __builtin_bit_cast(float, w[d] << 16);
    x[2 * d + 1] = __builtin_bit_cast(float, w[d] & 0xffff0000u);
  }
}

// Inclusive prefix sum over the 16 lanes of each DPP row (row_shr with
// bound_ctrl: lanes before the row start contribute 0).
__device__ __forceinline__ float dpp_shr(float x, int n) {
  const int v = __builtin_bit_cast(int, x);
  int r;
  switch (n) {
  case 1: r = __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, true); break;
  case 2: r = __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, true); break;
  case 4: r = __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, true); break;
  default: r = __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, true); break;
  }
  return __builtin_bit_cast(float, r);
}
__device__ __forceinline__ float row_scan16(float x) {
  x += dpp_shr(x, 1);
  x += dpp_shr(x, 2);
  x += dpp_shr(x, 4);
  x += dpp_shr(x, 8);
  return x;
}

__device__ __forceinline__ Frag<bf16> pack8(const float *x) {
  Frag<bf16> f;
#pragma unroll
  for (int j = 0; j < 8; ++j)
    f.v[j] = static_cast<bf16>(x[j]);
  return f;
}

__device__ __forceinline__ Frag<bf16> pack_acc2(const f32x4 &lo, const f32x4 &hi) {
  Frag<bf16> f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f.v[i] = static_cast<bf16>(lo[i]);
    f.v[4 + i] = static_cast<bf16>(hi[i]);
  }
  return f;
}

__device__ __forceinline__ void load8f(const float *p, float *x) {
  const f32x4 a = *reinterpret_cast<const f32x4 *>(p);
  const f32x4 b = *reinterpret_cast<const f32x4 *>(p + 4);
  x[0] = a[0]; x[1] = a[1]; x[2] = a[2]; x[3] = a[3];
  x[4] = b[0]; x[5] = b[1]; x[6] = b[2]; x[7] = b[3];
}

} // namespace kda
