// Shared device-side helpers for the gfx950 kernels: storage types, bf16
// conversion, MFMA wrappers and the activation functions used by epilogues.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tpcol {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------- bf16 storage
// bf16 values travel as raw uint16_t patterns.
__device__ __forceinline__ float bf2f(uint16_t h) { return __uint_as_float(((uint32_t)h) << 16); }

// float -> bf16, round to nearest even, by the gfx950 conversion instruction
// (v_cvt_pk_bf16_f32 converts two values per instruction; NaN stays NaN).
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf2(float lo, float hi) {
  const bf16x2_t v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ uint16_t f2bf(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }

template <typename T> struct Elem;
template <> struct Elem<uint16_t> {
  static constexpr int VW = 8;     // elements per 16-byte vector
  static constexpr int KP = 8;     // k values per lane in one MFMA operand
  static constexpr int KSTEP = 32; // k depth of one MFMA (16x16x32 bf16)
  __device__ static float to_f(uint16_t v) { return bf2f(v); }
  __device__ static uint16_t from_f(float v) { return f2bf(v); }
};
template <> struct Elem<float> {
  static constexpr int VW = 4;
  static constexpr int KP = 1;
  static constexpr int KSTEP = 4;  // 16x16x4 fp32
  __device__ static float to_f(float v) { return v; }
  __device__ static float from_f(float v) { return v; }
};

// ---------------------------------------------------------------- MFMA
// D[i][j] = sum_k A[i][k] B[k][j] + C for one 16x16 tile.  Lane l supplies
// row (A) / column (B) l%16 and k-slots (l/16)*KP .. +KP-1; the result lane l
// holds D[4*(l/16) + r][l%16], r = 0..3.
__device__ __forceinline__ f32x4_t mfma16(const uint4 &a, const uint4 &b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}
__device__ __forceinline__ f32x4_t mfma16(float a, float b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ uint32_t u4_word(const uint4 &v, int i) {
  return i == 0 ? v.x : (i == 1 ? v.y : (i == 2 ? v.z : v.w));
}

// ---------------------------------------------------------------- activations
// Standard normal CDF Phi(z) = (1 + erf(z / sqrt 2)) / 2 without branches,
// from the erf approximation of Abramowitz & Stegun, Handbook of
// Mathematical Functions, formula 7.1.26 (|error of erf| <= 1.5e-7):
//   erf(x) = 1 - (a1 t + a2 t^2 + a3 t^3 + a4 t^4 + a5 t^5) exp(-x^2),
//   t = 1 / (1 + p x),  x >= 0.
// For z < 0 the tail is taken directly (Phi(z) = q / 2), so there is no
// cancellation for large negative z.  exp(-x^2) comes back as well, for the
// density term of GELU'.
struct PhiResult {
  float phi_cdf;  // Phi(z)
  float pdf;      // standard normal density exp(-z^2 / 2) / sqrt(2 pi)
};
__device__ __forceinline__ PhiResult normal_cdf_pdf(float z) {
  const float x = fabsf(z) * 0.70710678118654752f;  // |z| / sqrt 2
  const float t = __builtin_amdgcn_rcpf(fmaf(0.3275911f, x, 1.0f));
  float poly = fmaf(t, 1.061405429f, -1.453152027f);
  poly = fmaf(t, poly, 1.421413741f);
  poly = fmaf(t, poly, -0.284496736f);
  poly = fmaf(t, poly, 0.254829592f);
  poly *= t;
  const float e = __builtin_amdgcn_exp2f(-x * x * 1.4426950408889634f);  // exp(-x^2)
  const float q = poly * e;                                               // erfc(x)
  PhiResult r;
  r.phi_cdf = z >= 0.0f ? fmaf(-0.5f, q, 1.0f) : 0.5f * q;
  r.pdf = 0.39894228040143268f * e;
  return r;
}

// Exact-form GELU z * Phi(z) ("张量并行", MLP 层的并行化): the same 7.1.26
// evaluation with its constants folded (1/sqrt 2 into p and into the
// exponent, the 1/2 of Phi into the polynomial), two VALU operations fewer
// per element than going through normal_cdf_pdf.
__device__ __forceinline__ float gelu_f(float z) {
  const float t = __builtin_amdgcn_rcpf(fmaf(0.3275911f * 0.70710678118654752f, fabsf(z), 1.0f));
  float hp = fmaf(t, 0.5f * 1.061405429f, 0.5f * -1.453152027f);
  hp = fmaf(t, hp, 0.5f * 1.421413741f);
  hp = fmaf(t, hp, 0.5f * -0.284496736f);
  hp = fmaf(t, hp, 0.5f * 0.254829592f);
  hp *= t;
  const float hq = hp * __builtin_amdgcn_exp2f(z * z * (-0.5f * 1.4426950408889634f));  // erfc(|z|/sqrt 2) / 2
  return z * (z >= 0.0f ? 1.0f - hq : hq);
}
// d/dz GELU = Phi(z) + z phi(z)
__device__ __forceinline__ float gelu_grad_f(float z) {
  const PhiResult r = normal_cdf_pdf(z);
  return fmaf(z, r.pdf, r.phi_cdf);
}
// sigmoid(z) = 1 / (1 + exp(-z)) with the hardware exp2 / reciprocal
__device__ __forceinline__ float sigmoid_f(float z) {
  return __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-z * 1.4426950408889634f));
}
__device__ __forceinline__ float silu_f(float z) { return z * sigmoid_f(z); }

}  // namespace tpcol
