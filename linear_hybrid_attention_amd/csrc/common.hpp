// Device helpers shared by the gfx950 kernels: bf16 packing, MFMA wrappers,
// the 32x32 MFMA register layouts and LDS tile addressing.
//
// MFMA layouts used throughout (v_mfma_f32_32x32x16_bf16, wave64, lane l,
// g = l >> 5, c = l & 31):
//   A (32 x 16):  lane holds row c, k-slots 8g .. 8g+7
//   B (16 x 32):  lane holds column c, k-slots 8g .. 8g+7
//   C (32 x 32):  lane holds column c; register r holds row crow(l, r)
//                 = 8 (r >> 2) + 4 g + (r & 3)
// A contraction may visit its k index in any order as long as the A and B
// fragments agree. The kernels exploit this to feed a C tile straight back
// into the next MFMA as a B (or A) operand: register r of the C tile becomes
// k-slot r of the operand, so the other operand must hold, at slot 8g + i,
// the element whose index is crow(l, i). kperm() maps an index to the slot
// that holds it (a swap of bits 2 and 3, an involution).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ttr {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ int crow(int lane, int r) {
  return 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
}
__host__ __device__ __forceinline__ constexpr int kperm(int x) {
  return (x & ~12) | ((x & 4) << 1) | ((x & 8) >> 1);
}

__device__ __forceinline__ float bf2f(uint16_t h) { return __uint_as_float(uint32_t(h) << 16); }

// Round-to-nearest-even float -> bf16 (the gfx950 conversion instruction).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2 v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ uint16_t f2bf(float f) {
  return __builtin_bit_cast(uint16_t, (__bf16)f);
}

// elu(x) + 1 with alpha = 1: x + 1 for x > 0 and exp(x) for x <= 0. Written
// without a branch as max(x + 1, min(exp(x), 1)): for x > 0 the clamped
// exponential is 1 <= x + 1, and for x <= 0 exp(x) >= x + 1 (the tangent line
// at 0 lies below the exponential). exp uses the hardware base-2 exponential,
// exp(x) = 2^(x log2 e), and the clamp to [0, 1] folds into its output
// modifier where NaN semantics are not required (four instructions).
__device__ __forceinline__ float elu1(float x) {
  const float e = __builtin_amdgcn_exp2f(x * kLog2e);
  return fmaxf(x + 1.f, fminf(fmaxf(e, 0.f), 1.f));
}
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Feature maps of the linear branch ("NNT Define Linear Attention", section
// "The inputs": elu + 1 by default, also relu or softmax). The softmax runs
// over each token's features: phi_f = exp(z_f - m) / sum_f' exp(z_f' - m), with
// the token's feature maximum m and inverse sum inv_s found by the caller.
enum FeatureMap { kElu1 = 0, kRelu = 1, kSoftmax = 2 };

// Softmax statistics of one token whose features are spread over a group of
// lanes: each lane holds NV of them in z, and the group is the lanes reached
// by xor with the bits of XMASK (e.g. 7: 8 consecutive lanes; 32: the two
// halves of the wave). Every lane of the group must be active. Returns the
// group's maximum m and 1 / sum exp(z - m).
template <int NV, int XMASK>
__device__ __forceinline__ void softmax_stats(const float* z, float& m, float& inv_s) {
  m = z[0];
#pragma unroll
  for (int j = 1; j < NV; ++j) m = fmaxf(m, z[j]);
#pragma unroll
  for (int o = 1; o < 64; o <<= 1)
    if (XMASK & o) m = fmaxf(m, __shfl_xor(m, o));
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < NV; ++j) s += __builtin_amdgcn_exp2f((z[j] - m) * kLog2e);
#pragma unroll
  for (int o = 1; o < 64; o <<= 1)
    if (XMASK & o) s += __shfl_xor(s, o);
  inv_s = 1.f / s;
}
template <int MAP>
__device__ __forceinline__ float phi_of(float z, float m, float inv_s) {
  if constexpr (MAP == kElu1) return elu1(z);
  else if constexpr (MAP == kRelu) return fmaxf(z, 0.f);
  else return __builtin_amdgcn_exp2f((z - m) * kLog2e) * inv_s;
}

// ---------------------------------------------------------------- fragments
// Eight k-consecutive operand values of one lane, in the element type T of
// the MFMA (bf16: one 32x32x16 instruction; fp32: eight 32x32x2 instructions).
template <typename T> struct FragOf;
template <> struct FragOf<uint16_t> { using type = bf16x8; };
template <> struct FragOf<float> { using type = f32x8; };
template <typename T> using Frag = typename FragOf<T>::type;

__device__ __forceinline__ void mma(f32x16& c, const bf16x8& a, const bf16x8& b) {
  c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
// a . b + c into a new accumulator (c is only read: no copy of it is needed).
__device__ __forceinline__ f32x16 mma_from(const f32x16& c, const bf16x8& a, const bf16x8& b) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ void mma(f32x16& c, const f32x8& a, const f32x8& b) {
#pragma unroll
  for (int i = 0; i < 8; ++i) c = __builtin_amdgcn_mfma_f32_32x32x2f32(a[i], b[i], c, 0, 0, 0);
}

// Load 8 consecutive elements (16-byte aligned for bf16, 32-byte for fp32).
template <typename T> __device__ __forceinline__ Frag<T> ld_frag(const T* p);
template <> __device__ __forceinline__ bf16x8 ld_frag<uint16_t>(const uint16_t* p) {
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(p));
}
template <> __device__ __forceinline__ f32x8 ld_frag<float>(const float* p) {
  f32x4 lo = *reinterpret_cast<const f32x4*>(p);
  f32x4 hi = *reinterpret_cast<const f32x4*>(p + 4);
  f32x8 r;
  r[0] = lo[0]; r[1] = lo[1]; r[2] = lo[2]; r[3] = lo[3];
  r[4] = hi[0]; r[5] = hi[1]; r[6] = hi[2]; r[7] = hi[3];
  return r;
}
template <typename T> __device__ __forceinline__ Frag<T> zero_frag();
template <> __device__ __forceinline__ bf16x8 zero_frag<uint16_t>() {
  u32x4 z = {0u, 0u, 0u, 0u};
  return __builtin_bit_cast(bf16x8, z);
}
template <> __device__ __forceinline__ f32x8 zero_frag<float>() {
  f32x8 z = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  return z;
}

// Eight fp32 values -> operand fragment (bf16: round to nearest even).
template <typename T> __device__ __forceinline__ Frag<T> to_frag(const float* v);
template <> __device__ __forceinline__ bf16x8 to_frag<uint16_t>(const float* v) {
  u32x4 u;
  u[0] = pack_bf16x2(v[0], v[1]);
  u[1] = pack_bf16x2(v[2], v[3]);
  u[2] = pack_bf16x2(v[4], v[5]);
  u[3] = pack_bf16x2(v[6], v[7]);
  return __builtin_bit_cast(bf16x8, u);
}
template <> __device__ __forceinline__ f32x8 to_frag<float>(const float* v) {
  f32x8 r;
#pragma unroll
  for (int i = 0; i < 8; ++i) r[i] = v[i];
  return r;
}

// Fragment -> eight fp32 values.
__device__ __forceinline__ void frag_to_f32(const bf16x8& f, float* v) {
  u32x4 u = __builtin_bit_cast(u32x4, f);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = __uint_as_float(u[i] << 16);
    v[2 * i + 1] = __uint_as_float(u[i] & 0xffff0000u);
  }
}
__device__ __forceinline__ void frag_to_f32(const f32x8& f, float* v) {
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] = f[i];
}

// ---------------------------------------------------------------- element IO
template <typename T> __device__ __forceinline__ float to_f32(T x);
template <> __device__ __forceinline__ float to_f32<uint16_t>(uint16_t x) { return bf2f(x); }
template <> __device__ __forceinline__ float to_f32<float>(float x) { return x; }
template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ uint16_t from_f32<uint16_t>(float x) { return f2bf(x); }
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }

// Store four consecutive values (8 bytes for bf16, 16 bytes for fp32).
__device__ __forceinline__ void st4(uint16_t* p, float a, float b, float c, float d) {
  u32x2 u;
  u[0] = pack_bf16x2(a, b);
  u[1] = pack_bf16x2(c, d);
  *reinterpret_cast<u32x2*>(p) = u;
}
__device__ __forceinline__ void st4(float* p, float a, float b, float c, float d) {
  f32x4 v = {a, b, c, d};
  *reinterpret_cast<f32x4*>(p) = v;
}

// Store a pair of values at p (4 bytes for bf16, 8 bytes for fp32).
__device__ __forceinline__ void st_pair(uint16_t* p, uint16_t a, uint16_t b) {
  *reinterpret_cast<uint32_t*>(p) = uint32_t(a) | (uint32_t(b) << 16);
}
__device__ __forceinline__ void st_pair(float* p, float a, float b) {
  float2 v = {a, b};
  *reinterpret_cast<float2*>(p) = v;
}

// 8 consecutive elements as raw storage, loaded from global/LDS (aligned).
template <typename T> struct Vec8 { T v[8]; };
template <typename T> __device__ __forceinline__ Vec8<T> ld8(const T* p) {
  Vec8<T> r;
  if constexpr (sizeof(T) == 2) {
    u32x4 u = *reinterpret_cast<const u32x4*>(p);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      r.v[2 * i] = (T)(u[i] & 0xffffu);
      r.v[2 * i + 1] = (T)(u[i] >> 16);
    }
  } else {
    f32x4 lo = *reinterpret_cast<const f32x4*>(p);
    f32x4 hi = *reinterpret_cast<const f32x4*>(p + 4);
#pragma unroll
    for (int i = 0; i < 4; ++i) { r.v[i] = lo[i]; r.v[4 + i] = hi[i]; }
  }
  return r;
}
template <typename T> __device__ __forceinline__ void st8(T* p, const Vec8<T>& x) {
  if constexpr (sizeof(T) == 2) {
    u32x4 u;
#pragma unroll
    for (int i = 0; i < 4; ++i) u[i] = uint32_t(x.v[2 * i]) | (uint32_t(x.v[2 * i + 1]) << 16);
    *reinterpret_cast<u32x4*>(p) = u;
  } else {
    f32x4 lo = {x.v[0], x.v[1], x.v[2], x.v[3]};
    f32x4 hi = {x.v[4], x.v[5], x.v[6], x.v[7]};
    *reinterpret_cast<f32x4*>(p) = lo;
    *reinterpret_cast<f32x4*>(p + 4) = hi;
  }
}
template <typename T> __device__ __forceinline__ Vec8<T> zero8() {
  Vec8<T> r;
#pragma unroll
  for (int i = 0; i < 8; ++i) r.v[i] = (T)0;
  return r;
}

// LDS tile rows are padded by 16 bytes: a 16-byte read by 16 lanes of
// consecutive rows at one column then touches 16 disjoint bank groups.
template <typename T, int COLS> struct LdsRow {
  static constexpr int stride = COLS + 16 / (int)sizeof(T);
  static constexpr int bytes_per_row = stride * (int)sizeof(T);
};

__device__ __forceinline__ float shfl_xor32(float v) { return __shfl_xor(v, 32, 64); }

}  // namespace ttr
