// Device-side building blocks shared by the fusedops kernels (gfx950 / CDNA4).
//
// Types, fp32 <-> bf16/fp16/fp8 conversions, OOB-safe buffer loads, wave
// reductions and the activation functions used by the epilogue and the
// LayerNorm+GELU row kernel.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/fusedops.h"

namespace fusedops {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) void lds_void;

constexpr int kWave = 64;
// Third dword of a raw buffer resource on gfx9-family parts (32-bit data
// format, no swizzle); reads at byte offsets >= num_records return zero.
constexpr int kBufferRsrcWord3 = 0x00020000;
// A voffset that is always out of range, so the buffer load returns zero.
constexpr uint32_t kOobOffset = 0x80000000u;
// Cache-policy operand of a buffer access asking for nontemporal (streaming) treatment:
// the `nt` bit on gfx94x / gfx950. Data read exactly once should not displace data
// that is reused.
constexpr int kNonTemporal = 2;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           kBufferRsrcWord3);
}

__device__ __forceinline__ u32x4 buffer_load_16B(__amdgpu_buffer_rsrc_t r, uint32_t voff) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, voff, 0, 0);
}

// Workgroup barrier that orders LDS use only: this wave's LDS reads and writes have completed,
// but its global stores may still be in flight (__syncthreads' release fence would also wait
// for those, s_waitcnt vmcnt(0)). For reusing an LDS buffer while earlier stores drain.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// ---------------------------------------------------------------------------
// conversions (round to nearest even everywhere)
// ---------------------------------------------------------------------------

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  __bf16 b = (__bf16)f;  // v_cvt_pk_bf16_f32: round to nearest even, NaN preserved
  return (uint32_t)__builtin_bit_cast(uint16_t, b);
}

__device__ __forceinline__ float f16_bits_to_f32(uint32_t b) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)b);
}

__device__ __forceinline__ uint32_t f32_to_f16_bits(float f) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)f);
}

// Two fp32 -> two bf16 / fp16 packed (low half = a), one v_cvt_pk_{bf16,f16}_f32 each
// (round to nearest even).
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  typedef __bf16 v2 __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, v2{(__bf16)a, (__bf16)b});
}
__device__ __forceinline__ uint32_t pack_f16x2(float a, float b) {
  typedef _Float16 v2 __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, v2{(_Float16)a, (_Float16)b});
}

// Two fp32 -> two OCP E4M3 codes (low byte = a); inputs must already be clamped to +-448.
__device__ __forceinline__ uint32_t pack_e4m3x2(float a, float b) {
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false) & 0xFFFFu;
}

// One element of a bf16 / fp16 / fp32 vector as fp32.
__device__ __forceinline__ float load1(const void* base, int dtype, int64_t idx) {
  if (dtype == FUSEDOPS_F32) return static_cast<const float*>(base)[idx];
  const uint32_t b = static_cast<const uint16_t*>(base)[idx];
  return dtype == FUSEDOPS_BF16 ? bf16_bits_to_f32(b) : f16_bits_to_f32(b);
}

// Load 4 consecutive elements of a 1-D / row vector with a runtime dtype, as fp32.
// `idx` must be a multiple of 4 (8-byte or 16-byte aligned access).
__device__ __forceinline__ f32x4 load4(const void* base, int dtype, int64_t idx) {
  f32x4 r;
  if (dtype == FUSEDOPS_F32) {
    r = *reinterpret_cast<const f32x4*>(static_cast<const float*>(base) + idx);
  } else {
    u32x2 v = *reinterpret_cast<const u32x2*>(static_cast<const uint16_t*>(base) + idx);
    if (dtype == FUSEDOPS_BF16) {
      r[0] = __uint_as_float(v[0] << 16);
      r[1] = __uint_as_float(v[0] & 0xFFFF0000u);
      r[2] = __uint_as_float(v[1] << 16);
      r[3] = __uint_as_float(v[1] & 0xFFFF0000u);
    } else {
      r[0] = f16_bits_to_f32(v[0] & 0xFFFF);
      r[1] = f16_bits_to_f32(v[0] >> 16);
      r[2] = f16_bits_to_f32(v[1] & 0xFFFF);
      r[3] = f16_bits_to_f32(v[1] >> 16);
    }
  }
  return r;
}

// Store 4 consecutive fp32 values as dtype (not fp8). `idx` multiple of 4.
__device__ __forceinline__ void store4(void* base, int dtype, int64_t idx, f32x4 v) {
  if (dtype == FUSEDOPS_F32) {
    *reinterpret_cast<f32x4*>(static_cast<float*>(base) + idx) = v;
  } else if (dtype == FUSEDOPS_BF16) {
    u32x2 o = {pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
    *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(base) + idx) = o;
  } else {
    u32x2 o = {pack_f16x2(v[0], v[1]), pack_f16x2(v[2], v[3])};
    *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(base) + idx) = o;
  }
}

// Store 2 consecutive fp32 values as dtype (not fp8). `idx` multiple of 2.
__device__ __forceinline__ void store2(void* base, int dtype, int64_t idx, float a, float b) {
  if (dtype == FUSEDOPS_F32) {
    float2 o = make_float2(a, b);
    *reinterpret_cast<float2*>(static_cast<float*>(base) + idx) = o;
  } else if (dtype == FUSEDOPS_BF16) {
    *reinterpret_cast<uint32_t*>(static_cast<uint16_t*>(base) + idx) = pack_bf16x2(a, b);
  } else {
    *reinterpret_cast<uint32_t*>(static_cast<uint16_t*>(base) + idx) = pack_f16x2(a, b);
  }
}

__device__ __forceinline__ int dtype_bytes(int dtype) {
  return dtype == FUSEDOPS_F32 ? 4 : (dtype == FUSEDOPS_F8E4M3 ? 1 : 2);
}

// Per-row factors of FP8 quantisation: q = clamp(v * pre * inv, +-448) stands for v / s. For
// s >= 2^-100 (every row whose absmax exceeds 448 * 2^-100 ~ 3.5e-28) pre = 1 and inv =
// fl(1 / s); for smaller s, 1 / s can overflow (s below 2^-128), so v is first scaled by the
// power of two 2^64 (exact: v <= 448 s is tiny) and inv = fl(1 / (s 2^64)). A zero row (s = 0)
// gets inv = 0 and all-zero codes.
struct Fp8RowFactor {
  float pre, inv;
};
__device__ __forceinline__ Fp8RowFactor fp8_row_factor(float s) {
  if (!(s > 0.f)) return {1.f, 0.f};
  if (s >= 0x1p-100f) return {1.f, __fdiv_rn(1.0f, s)};
  return {0x1p64f, __fdiv_rn(1.0f, s * 0x1p64f)};
}

// ---------------------------------------------------------------------------
// activations (fp32 in registers)
// ---------------------------------------------------------------------------

// GELU, erf form, for 16-bit and E4M3 outputs: 0.5 v (1 + erf(v / sqrt 2)) = v Phi(v). With
// h = 0.5 erfc(|v| / sqrt 2), Phi(v) = 1 - h for v >= 0 and h otherwise, so v Phi(v) =
// max(v, 0) - |v| h for either sign: no select, and for v < 0 the result is the product |v| h
// itself (no cancellation in the negative tail). h is computed with one transcendental as
// 2^p(a), where p is a degree-7 polynomial in a = min(|v|, 6) fitted to log2 h (Chebyshev least
// squares on [0, 6], coefficients rounded to fp32, evaluated by Horner in fp32): relative error
// of h at most 9.1e-6 on [0, 6], absolute error of the GELU value at most 4.6e-7 for |v| <= 6.
// Beyond, |v| h(6) (h(6) = 9.9e-10) stands for |v| h(|v|): the result is off by at most 9.9e-10 |v|,
// a relative 1e-9 of v for v > 6 and, for v < -6, a value below 1e-9 |v| where the exact one is
// below 1e-9 too. All of it is far below half a bf16 / fp16 / E4M3 ulp of the output's scale.
// 10 VALU operations and one v_exp_f32 per element.
__device__ __forceinline__ float gelu_erf_h(float x) {  // h for x = min(|v|, 6)
  constexpr float C0 = -9.999869466e-01f, C1 = -1.151324630e+00f, C2 = -4.582974911e-01f,
                  C3 = -5.411827192e-02f, C4 = 8.582354523e-03f, C5 = -9.488665964e-04f,
                  C6 = 6.386001041e-05f, C7 = -1.944896667e-06f;
  float p = __builtin_fmaf(C7, x, C6);
  p = __builtin_fmaf(p, x, C5);
  p = __builtin_fmaf(p, x, C4);
  p = __builtin_fmaf(p, x, C3);
  p = __builtin_fmaf(p, x, C2);
  p = __builtin_fmaf(p, x, C1);
  p = __builtin_fmaf(p, x, C0);
  return __builtin_amdgcn_exp2f(p);
}
// The same h to bf16 accuracy: a degree-6 polynomial (Chebyshev least squares on [0, 6],
// reweighted towards equal ripple) keeps h within 4.9e-5 of itself and the GELU value within
// 6.6e-6 for |v| <= 6, a small fraction of half a bf16 ulp (2^-9 of the value), for one FMA less.
__device__ __forceinline__ float gelu_erf_h_bf16(float x) {  // h for x = min(|v|, 6)
  constexpr float C0 = -1.000065804e+00f, C1 = -1.150170088e+00f, C2 = -4.612762332e-01f,
                  C3 = -5.118361115e-02f, C4 = 7.195291109e-03f, C5 = -6.110906834e-04f,
                  C6 = 2.299096741e-05f;
  float p = __builtin_fmaf(C6, x, C5);
  p = __builtin_fmaf(p, x, C4);
  p = __builtin_fmaf(p, x, C3);
  p = __builtin_fmaf(p, x, C2);
  p = __builtin_fmaf(p, x, C1);
  p = __builtin_fmaf(p, x, C0);
  return __builtin_amdgcn_exp2f(p);
}
// kBf16: the value is rounded to bf16 afterwards, so the degree-6 h suffices.
template <bool kBf16 = false>
__device__ __forceinline__ float gelu_erf_f32(float v) {
  const float a = fabsf(v);
  const float x = fminf(a, 6.0f);
  return __builtin_fmaf(-a, kBf16 ? gelu_erf_h_bf16(x) : gelu_erf_h(x), fmaxf(v, 0.f));
}
// The same for v read straight from an accumulator register: float min / max would first quiet
// such an operand (one more instruction per use, since the compiler cannot tell it is not a
// signalling NaN), so |v|, min(|v|, 6) and max(v, 0) are taken as integer operations on the bit
// pattern (non-negative floats order as their bit patterns). For v produced by arithmetic the
// float form above is shorter.
template <bool kBf16 = false>
__device__ __forceinline__ float gelu_erf_acc_f32(float v) {
  const uint32_t ub = __float_as_uint(v) & 0x7fffffffu;
  const float x = __uint_as_float(min(ub, 0x40c00000u));  // 0x40c00000 = 6.0f
  return __builtin_fmaf(-__uint_as_float(ub), kBf16 ? gelu_erf_h_bf16(x) : gelu_erf_h(x),
                        __int_as_float(max(__float_as_int(v), 0)));
}

// GELU, erf form, for fp32 outputs: the same v Phi(v) = max(v, 0) - |v| h with h = 0.5 erfc(|v| / sqrt 2)
// taken from the device math library's erfcf (a few ulp of relative error over its whole range),
// so the negative tail keeps fp32 relative accuracy (the 16-bit form above bounds the absolute
// error only). The rounding of |v| / sqrt 2 adds a relative error of about 2 (v^2 / 2) 2^-24 to
// h, 4e-6 at v = -8.
__device__ __forceinline__ float gelu_erf_precise_f32(float v) {
  const float a = fabsf(v);
  const float h = 0.5f * erfcf(a * 0.70710678118654752f);
  return __builtin_fmaf(-a, h, fmaxf(v, 0.f));
}

// GELU, tanh form. 0.5 v (1 + tanh u) equals v / (1 + e^{-2u}), which needs one exp
// and one reciprocal; u = sqrt(2/pi) (v + 0.044715 v^3). The constants -2 sqrt(2/pi) and
// log2(e) are folded so that e^{-2u} = 2^{v (A + B v^2)} with
// A = -2 sqrt(2/pi) log2(e) and B = 0.044715 A: three VALU ops and one v_exp_f32.
__device__ __forceinline__ float gelu_tanh_f32(float v) {
  constexpr double kA = -2.0 * 0.79788456080286536 * 1.4426950408889634;
  constexpr float A = (float)kA, B = (float)(kA * 0.044715);
  const float t = v * __builtin_fmaf(v * v, B, A);
  return v * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(t));
}

// silu(g) = g / (1 + e^-g) = g / (1 + 2^{-g log2 e}).
__device__ __forceinline__ float silu_f32(float g) {
  return g * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(g * -1.4426950408889634f));
}

// ---------------------------------------------------------------------------
// wave reductions
// ---------------------------------------------------------------------------

// DPP lane permutations within a 16-lane row (no LDS traffic): xor 1, xor 2 (quad
// permutes), i <-> 7-i (half mirror) and i <-> 15-i (mirror). Applied in that order with
// adds, every lane of a row ends with the sum of its 16 lanes.
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}
constexpr int kDppXor1 = 0xB1;        // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;        // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141; // row_half_mirror
constexpr int kDppMirror = 0x140;     // row_mirror

__device__ __forceinline__ float row16_sum(float v) {
  v += dpp_f32<kDppXor1>(v);
  v += dpp_f32<kDppXor2>(v);
  v += dpp_f32<kDppHalfMirror>(v);
  v += dpp_f32<kDppMirror>(v);
  return v;
}
__device__ __forceinline__ float row16_max(float v) {
  v = fmaxf(v, dpp_f32<kDppXor1>(v));
  v = fmaxf(v, dpp_f32<kDppXor2>(v));
  v = fmaxf(v, dpp_f32<kDppHalfMirror>(v));
  v = fmaxf(v, dpp_f32<kDppMirror>(v));
  return v;
}

// Sum over the whole wave, returned wave-uniform: 16-lane DPP sums, then the four row
// sums read with v_readlane.
__device__ __forceinline__ float wave_sum_uniform(float v) {
  v = row16_sum(v);
  const int b = __builtin_bit_cast(int, v);
  return (__builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 0)) +
          __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 16))) +
         (__builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 32)) +
          __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 48)));
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}

}  // namespace fusedops
