// Device-side helpers shared by the BRA kernels (gfx950, wave64).
//
// Layouts: Q, K, V, out are [B, H, W, C] channels-last.  A region r = (ry, rx)
// of the S x S grid covers rows ry*hs .. ry*hs+hs-1 and columns
// rx*ws .. rx*ws+ws-1; its pixel t (row-major inside the region) sits at
// (ry*hs + t / ws, rx*ws + t % ws).  This is the partition step of the
// cybasar.com BRA walk-through (§3), done by address arithmetic: nothing is
// copied into a region layout.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "bra_internal.h"
#include "fastdiv.h"

namespace bra {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef double f64x4 __attribute__((ext_vector_type(4)));

// Cache policy bits of the non-temporal output stores of the attention
// kernels that use them (gfx950 buffer stores: 1 = sc0, 2 = nt, 16 = sc1).
// Measured on MI355X: about 1 us less per launch for the whole-image and the
// dense-shape kernels, none for the stage-1 kernel, and 30-37% more HBM
// write bytes than the output (16-byte stores written through one by one).
#ifndef BRA_OUT_CPOL
#define BRA_OUT_CPOL 2
#endif

constexpr int kThreads = 256;   // 4 wavefronts of 64
constexpr int kWaves = 4;
constexpr int kXcds = 8;        // MI355X: workgroups go round-robin to 8 XCDs

__device__ __forceinline__ float bf16_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }

// Two floats -> two bfloat16 in one word (a low, b high), round to nearest
// even: a single v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  typedef float f2 __attribute__((ext_vector_type(2)));
  typedef __bf16 h2 __attribute__((ext_vector_type(2)));
  const f2 v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, h2));
}

// Butterfly partners across lane rows without LDS traffic (gfx950
// v_permlane16_swap / v_permlane32_swap): the value of lane l ^ 16 and of
// lane l ^ 32.
// GELU in its exact form, x Phi(x) = x/2 (1 + erf(x / sqrt 2)), with erf by
// Abramowitz & Stegun 7.1.26 (absolute error below 1.5e-7): for z >= 0,
// erfc(z) = t (a1 + t (a2 + t (a3 + t (a4 + t a5)))) exp(-z^2), t = 1 / (1 +
// p z).  Since 1 + erf(z) is 2 - erfc(z) for z >= 0 and erfc(-z) below,
// x Phi(x) = max(x, 0) - |x|/2 erfc(|x| / sqrt 2) for either sign; the 1/2
// is folded into the a_i and 1/sqrt 2 into p and the exponent.
__device__ __forceinline__ float gelu_as(float v) {
  const float av = fabsf(v);
  const float t = __builtin_amdgcn_rcpf(fmaf(0.3275911f * 0.70710678118654752f, av, 1.0f));
  float pz = fmaf(t, 0.5f * 1.061405429f, 0.5f * -1.453152027f);
  pz = fmaf(t, pz, 0.5f * 1.421413741f);
  pz = fmaf(t, pz, 0.5f * -0.284496736f);
  pz = fmaf(t, pz, 0.5f * 0.254829592f);
  // exp(-v^2 / 2) = 2^(v^2 * -log2(e) / 2)
  const float e = __builtin_amdgcn_exp2f(v * v * -0.72134752044448170f);
  return fmaf(-av, (t * pz) * e, fmaxf(v, 0.f));
}

__device__ __forceinline__ float xor16(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return (threadIdx.x & 16) ? __uint_as_float(r[0]) : __uint_as_float(r[1]);
}
__device__ __forceinline__ float xor32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return (threadIdx.x & 32) ? __uint_as_float(r[0]) : __uint_as_float(r[1]);
}

// Expand 16 bytes of elements into floats.  bf16: 8 values; f32: 4 values.
template <bool BF16>
__device__ __forceinline__ void unpack16(const uint4& u, float* f) {
  if constexpr (BF16) {
    f[0] = bf16_lo(u.x); f[1] = bf16_hi(u.x);
    f[2] = bf16_lo(u.y); f[3] = bf16_hi(u.y);
    f[4] = bf16_lo(u.z); f[5] = bf16_hi(u.z);
    f[6] = bf16_lo(u.w); f[7] = bf16_hi(u.w);
  } else {
    f[0] = __uint_as_float(u.x); f[1] = __uint_as_float(u.y);
    f[2] = __uint_as_float(u.z); f[3] = __uint_as_float(u.w);
  }
}

template <bool BF16>
struct Elem;
template <>
struct Elem<true> { using T = uint16_t; };
template <>
struct Elem<false> { using T = float; };

// 2 or 4 consecutive elements as floats (global memory or LDS)
template <bool BF16>
__device__ __forceinline__ void load2(const void* base, int off, float* f) {
  if constexpr (BF16) {
    const uint32_t u = *(const uint32_t*)((const uint16_t*)base + off);
    f[0] = bf16_lo(u); f[1] = bf16_hi(u);
  } else {
    const float2 u = *(const float2*)((const float*)base + off);
    f[0] = u.x; f[1] = u.y;
  }
}

template <bool BF16>
__device__ __forceinline__ void load4(const void* base, int off, float* f) {
  if constexpr (BF16) {
    const uint2 u = *(const uint2*)((const uint16_t*)base + off);
    f[0] = bf16_lo(u.x); f[1] = bf16_hi(u.x); f[2] = bf16_lo(u.y); f[3] = bf16_hi(u.y);
  } else {
    const float4 u = *(const float4*)((const float*)base + off);
    f[0] = u.x; f[1] = u.y; f[2] = u.z; f[3] = u.w;
  }
}

template <bool BF16>
__device__ __forceinline__ void store2(void* base, int off, float a, float b) {
  if constexpr (BF16) {
    *(uint32_t*)((uint16_t*)base + off) = pack_bf16x2(a, b);
  } else {
    *(float2*)((float*)base + off) = make_float2(a, b);
  }
}

template <bool BF16>
__device__ __forceinline__ void store4(void* base, int off, const float* f) {
  if constexpr (BF16) {
    uint2 u;
    u.x = pack_bf16x2(f[0], f[1]);
    u.y = pack_bf16x2(f[2], f[3]);
    *(uint2*)((uint16_t*)base + off) = u;
  } else {
    *(float4*)((float*)base + off) = make_float4(f[0], f[1], f[2], f[3]);
  }
}

}  // namespace bra
