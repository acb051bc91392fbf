// Device-side helpers shared by the gfx950 kernels: element types, 8-element
// operand chunks and the 32x32 MFMA step used by the GEMM and attention kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace wan {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// An operand chunk: 8 consecutive elements along the contraction axis, the
// per-lane operand of one 32x32x16 MFMA step.  bf16: 16 bytes, float: 32 bytes.
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// Chunks are moved with explicit vector loads and stores only (never struct
// assignment), so they stay in registers.
template <typename T> struct Chunk;
template <> struct Chunk<bf16> {
  u32x4 v;
  __device__ __forceinline__ void zero() { v = (u32x4){0u, 0u, 0u, 0u}; }
  __device__ __forceinline__ void load(const void* p) { v = *reinterpret_cast<const u32x4*>(p); }
  __device__ __forceinline__ void store(void* p) const { *reinterpret_cast<u32x4*>(p) = v; }
};
template <> struct Chunk<float> {
  f32x4 a, b;
  __device__ __forceinline__ void zero() {
    a = (f32x4){0.f, 0.f, 0.f, 0.f};
    b = a;
  }
  __device__ __forceinline__ void load(const void* p) {
    const f32x4* q = reinterpret_cast<const f32x4*>(p);
    a = q[0];
    b = q[1];
  }
  __device__ __forceinline__ void store(void* p) const {
    f32x4* q = reinterpret_cast<f32x4*>(p);
    q[0] = a;
    q[1] = b;
  }
};

__device__ __forceinline__ bf16x8 as_bf16x8(const u32x4& v) { return __builtin_bit_cast(bf16x8, v); }

// acc(32x32) += A(32x16) * B(16x32).  Lane l supplies A[l%32][8*(l/32) + e] and
// B[8*(l/32) + e][l%32] for e < 8; acc element r of lane l is row
// 8*(r/4) + 4*(l/32) + r%4, column l%32.  For float operands the same k-chunk
// is contracted by eight 32x32x2 steps, step e taking element e of each lane's
// chunk, so both element types share one operand layout.
__device__ __forceinline__ void mma32(f32x16& acc, const Chunk<bf16>& a, const Chunk<bf16>& b) {
  acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a.v), as_bf16x8(b.v), acc, 0, 0, 0);
}
__device__ __forceinline__ void mma32(f32x16& acc, const Chunk<float>& a, const Chunk<float>& b) {
#pragma unroll
  for (int e = 0; e < 4; ++e) acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a.a[e], b.a[e], acc, 0, 0, 0);
#pragma unroll
  for (int e = 0; e < 4; ++e) acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a.b[e], b.b[e], acc, 0, 0, 0);
}

// float -> bf16 with round-to-nearest-even (gfx950 converts in hardware).
__device__ __forceinline__ bf16 to_bf16(float x) { return (bf16)x; }
__device__ __forceinline__ float bf16_to_f(bf16 x) { return (float)x; }

template <typename T> __device__ __forceinline__ T from_f(float x);
template <> __device__ __forceinline__ bf16 from_f<bf16>(float x) { return to_bf16(x); }
template <> __device__ __forceinline__ float from_f<float>(float x) { return x; }

template <typename T> __device__ __forceinline__ float to_f(T x);
template <> __device__ __forceinline__ float to_f<bf16>(bf16 x) { return bf16_to_f(x); }
template <> __device__ __forceinline__ float to_f<float>(float x) { return x; }

// Two floats as bf16 (round to nearest even) in one 32-bit word, the first in the low half.
__device__ __forceinline__ unsigned pack_bf16x2(float lo, float hi) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  const bf16x2_t v = {to_bf16(lo), to_bf16(hi)};
  return __builtin_bit_cast(unsigned, v);
}

// Pack 8 floats into a chunk of T.
__device__ __forceinline__ void pack8(Chunk<bf16>& c, const float* f) {
  bf16x8 v;
#pragma unroll
  for (int e = 0; e < 8; ++e) v[e] = to_bf16(f[e]);
  c.v = __builtin_bit_cast(u32x4, v);
}
__device__ __forceinline__ void pack8(Chunk<float>& c, const float* f) {
  c.a = (f32x4){f[0], f[1], f[2], f[3]};
  c.b = (f32x4){f[4], f[5], f[6], f[7]};
}

// 8-bit operands: e4m3 values (bias 7, largest finite 448) with one power-of-two
// scale 2^e per block, kept as the byte e + 127.  e is the smallest exponent with
// max|block| / 2^e <= 448, clamped to [-127, 127], and 0 for an all-zero block:
// with max|block| = m 2^E, m in [1, 2), that is E - 8, plus one when m > 1.75.
__device__ __forceinline__ int e8_exponent(float amax) {
  const unsigned ab = __float_as_uint(amax);
  const int ef = (int)(ab >> 23);
  const int ex = ef == 0 ? (amax == 0.f ? 0 : -127) : ef - 135 + ((ab & 0x7FFFFFu) > 0x600000u ? 1 : 0);
  return ex < -127 ? -127 : ex;
}
// 8 values times inv (= 2^-e, an exact scaling) rounded to e4m3, nearest-even, 8 bytes
__device__ __forceinline__ uint2 e4m3_pack8(const float* v, float inv) {
  unsigned w0 = __builtin_amdgcn_cvt_pk_fp8_f32(v[0] * inv, v[1] * inv, 0u, false);
  w0 = __builtin_amdgcn_cvt_pk_fp8_f32(v[2] * inv, v[3] * inv, w0, true);
  unsigned w1 = __builtin_amdgcn_cvt_pk_fp8_f32(v[4] * inv, v[5] * inv, 0u, false);
  w1 = __builtin_amdgcn_cvt_pk_fp8_f32(v[6] * inv, v[7] * inv, w1, true);
  return make_uint2(w0, w1);
}

// Sum over each aligned group of 16 lanes, left in every lane of the group: four DPP
// adds on the vector ALU (quad swaps 1 and 2, then the half-row and row mirrors)
template <int CTRL>
__device__ __forceinline__ float dpp_f(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float row16_sum(float v) {
  v += dpp_f<0xB1>(v);   // quad_perm [1, 0, 3, 2]
  v += dpp_f<0x4E>(v);   // quad_perm [2, 3, 0, 1]
  v += dpp_f<0x141>(v);  // row_half_mirror
  v += dpp_f<0x140>(v);  // row_mirror
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// erf by the rational approximation 7.1.26 of Abramowitz & Stegun's Handbook of
// Mathematical Functions, |error| < 1.5e-7:
//   erf(x) = 1 - t (a1 + t (a2 + t (a3 + t (a4 + t a5)))) exp(-x^2),  t = 1 / (1 + p x),  x >= 0
__device__ __forceinline__ float erf_as26(float x) {
  const float ax = fabsf(x);
  const float t = __builtin_amdgcn_rcpf(__builtin_fmaf(0.3275911f, ax, 1.0f));
  float poly = __builtin_fmaf(1.061405429f, t, -1.453152027f);
  poly = __builtin_fmaf(poly, t, 1.421413741f);
  poly = __builtin_fmaf(poly, t, -0.284496736f);
  poly = __builtin_fmaf(poly, t, 0.254829592f);
  const float e = __builtin_amdgcn_exp2f(-ax * ax * 1.4426950408889634f);
  return copysignf(__builtin_fmaf(-poly * t, e, 1.0f), x);
}
// GELU(u) = u/2 (1 + erf(u / sqrt 2))
__device__ __forceinline__ float gelu_erf(float u) { return 0.5f * u * (1.0f + erf_as26(u * 0.70710678118654752f)); }
__device__ __forceinline__ float silu(float u) { return u / (1.0f + expf(-u)); }

// Workgroups are handed to the 8 XCDs round-robin; this maps the hardware
// order so that each XCD receives one contiguous range of logical ids.
__device__ __forceinline__ int xcd_remap(int id, int n) {
  const int nx = 8;
  int full = n - n % nx;
  if (id >= full) return id;
  return (id % nx) * (full / nx) + id / nx;
}

}  // namespace wan
