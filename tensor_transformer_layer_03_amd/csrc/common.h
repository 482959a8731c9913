// Shared device-side helpers for the gfx950 kernels: storage types, bf16
// rounding, 16-byte vector access, and the MFMA step used by every dense
// contraction (GEMM and attention).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tpl {

typedef __bf16 bf16;
typedef float f32x4 __attribute__((__vector_size__(4 * sizeof(float))));
typedef float f32x16 __attribute__((__vector_size__(16 * sizeof(float))));
typedef __bf16 bf16x8 __attribute__((__vector_size__(8 * sizeof(__bf16))));
typedef uint32_t u32x4 __attribute__((__vector_size__(4 * sizeof(uint32_t))));
typedef uint32_t u32x2 __attribute__((__vector_size__(2 * sizeof(uint32_t))));

constexpr int kWave = 64;

// ---------------------------------------------------------------- conversions

__device__ __forceinline__ float to_f32(float v) { return v; }
__device__ __forceinline__ float to_f32(bf16 v) { return (float)v; }

template <typename T> __device__ __forceinline__ T from_f32(float v);
template <> __device__ __forceinline__ float from_f32<float>(float v) { return v; }
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float v) { return (bf16)v; }  // RNE

// 16-byte vector of storage elements (8 bf16 or 4 fp32).
template <typename T> struct Vec16 {
  static constexpr int N = 16 / sizeof(T);
  u32x4 raw;
  __device__ __forceinline__ T get(int i) const {
    T out;
    __builtin_memcpy(&out, reinterpret_cast<const char*>(&raw) + i * sizeof(T), sizeof(T));
    return out;
  }
  __device__ __forceinline__ void set(int i, T v) {
    __builtin_memcpy(reinterpret_cast<char*>(&raw) + i * sizeof(T), &v, sizeof(T));
  }
};

__device__ __forceinline__ u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
__device__ __forceinline__ void st16(void* p, u32x4 v) { *reinterpret_cast<u32x4*>(p) = v; }
__device__ __forceinline__ u32x2 ld8(const void* p) { return *reinterpret_cast<const u32x2*>(p); }
__device__ __forceinline__ void st8(void* p, u32x2 v) { *reinterpret_cast<u32x2*>(p) = v; }

// Pack 4 fp32 values into 4 storage elements (8 bytes for bf16, 16 for fp32).
__device__ __forceinline__ void store4(bf16* p, float a, float b, float c, float d) {
  bf16 v[4] = {(bf16)a, (bf16)b, (bf16)c, (bf16)d};
  u32x2 w;
  __builtin_memcpy(&w, v, 8);
  st8(p, w);
}
__device__ __forceinline__ void store4(float* p, float a, float b, float c, float d) {
  f32x4 v = {a, b, c, d};
  *reinterpret_cast<f32x4*>(p) = v;
}
__device__ __forceinline__ void load4(const bf16* p, float* o) {
  u32x2 w = ld8(p);
  bf16 v[4];
  __builtin_memcpy(v, &w, 8);
  o[0] = (float)v[0]; o[1] = (float)v[1]; o[2] = (float)v[2]; o[3] = (float)v[3];
}
__device__ __forceinline__ void load4(const float* p, float* o) {
  f32x4 v = *reinterpret_cast<const f32x4*>(p);
  o[0] = v[0]; o[1] = v[1]; o[2] = v[2]; o[3] = v[3];
}

// ---------------------------------------------------------------- MFMA step
// One "k16 step" of a 32x32 output tile: D[i][j] += sum_{k<16} A[i][k] B[k][j].
// Lane l supplies 8 k-values of row i = l%32 (A) and of column j = l%32 (B),
// lane group g = l/32 supplying the k-slots g*8..g*8+7. Any bijection between
// k-slots and true k indices is valid as long as A and B use the same one.
// Result layout: lane l holds D[8*(r/4) + 4*(l/32) + r%4][l%32] in acc[r].
//  bf16: one v_mfma_f32_32x32x16_bf16.
//  fp32: eight v_mfma_f32_32x32x2f32, the e-th consuming slot e of each group.
template <typename T> struct Frag8;
template <> struct Frag8<bf16> { bf16x8 v; };
template <> struct Frag8<float> { float v[8]; };

__device__ __forceinline__ void mfma_step(f32x16& acc, const Frag8<bf16>& a, const Frag8<bf16>& b) {
  acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a.v, b.v, acc, 0, 0, 0);
}
__device__ __forceinline__ void mfma_step(f32x16& acc, const Frag8<float>& a, const Frag8<float>& b) {
#pragma unroll
  for (int e = 0; e < 8; ++e) acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a.v[e], b.v[e], acc, 0, 0, 0);
}

// Load 8 consecutive storage elements (16 B bf16 / 32 B fp32) from LDS or global.
__device__ __forceinline__ void load_frag(Frag8<bf16>& f, const bf16* p) {
  u32x4 w = ld16(p);
  __builtin_memcpy(&f.v, &w, 16);
}
__device__ __forceinline__ void load_frag(Frag8<float>& f, const float* p) {
  u32x4 w0 = ld16(p), w1 = ld16(p + 4);
  __builtin_memcpy(&f.v[0], &w0, 16);
  __builtin_memcpy(&f.v[4], &w1, 16);
}
// Two 4-element halves from separate addresses (element offsets 0-3 and 4-7).
__device__ __forceinline__ void load_frag2(Frag8<bf16>& f, const bf16* p0, const bf16* p1) {
  u32x2 w0 = ld8(p0), w1 = ld8(p1);
  u32x4 w = {w0[0], w0[1], w1[0], w1[1]};
  __builtin_memcpy(&f.v, &w, 16);
}
__device__ __forceinline__ void load_frag2(Frag8<float>& f, const float* p0, const float* p1) {
  u32x4 w0 = ld16(p0), w1 = ld16(p1);
  __builtin_memcpy(&f.v[0], &w0, 16);
  __builtin_memcpy(&f.v[4], &w1, 16);
}
// Build a fragment from 8 fp32 values (rounded to the storage type).
__device__ __forceinline__ void frag_from_f32(Frag8<bf16>& f, const float* v) {
#pragma unroll
  for (int e = 0; e < 8; ++e) f.v[e] = (bf16)v[e];
}
__device__ __forceinline__ void frag_from_f32(Frag8<float>& f, const float* v) {
#pragma unroll
  for (int e = 0; e < 8; ++e) f.v[e] = v[e];
}

// ---------------------------------------------------------------- math

// Exact GeLU x*Phi(x) and its derivative Phi(x) + x*phi(x).
// Exact-erf GeLU (u * Phi(u)) and its derivative Phi(u) + u * phi(u), with the
// normal CDF from the complementary error function of Abramowitz & Stegun,
// Handbook of Mathematical Functions, 7.1.26: erfc(x) = t (a1 + t (a2 + ...))
// e^{-x^2}, t = 1 / (1 + p x), x >= 0, absolute error <= 1.5e-7. Taking erfc
// of |u| / sqrt(2) keeps the left tail free of cancellation, and e^{-u^2/2}
// is shared with the density.
__device__ __forceinline__ float normal_cdf_tail(float u, float& gauss) {
  const float x = fabsf(u) * 0.70710678118654752f;
  const float t = __builtin_amdgcn_rcpf(fmaf(0.3275911f, x, 1.0f));
  const float poly =
      t * fmaf(t, fmaf(t, fmaf(t, fmaf(t, 1.061405429f, -1.453152027f), 1.421413741f), -0.284496736f), 0.254829592f);
  gauss = __builtin_amdgcn_exp2f(-x * x * 1.4426950408889634f);   // e^{-u^2/2}; underflows to 0 in the far tail
  const float half_erfc = 0.5f * poly * gauss;
  return u >= 0.0f ? 1.0f - half_erfc : half_erfc;                 // Phi(u)
}
// GeLU(u) and GeLU'(u) from one evaluation of Phi and phi (the forward
// stores both: GeLU'(u) is what the backward needs of u).
__device__ __forceinline__ void gelu_and_grad(float x, float& gelu, float& grad) {
  float g;
  const float cdf = normal_cdf_tail(x, g);
  gelu = x * cdf;
  grad = fmaf(x * 0.39894228040143268f, g, cdf);
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}

}  // namespace tpl
