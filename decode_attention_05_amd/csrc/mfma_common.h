// MFMA operand helpers shared by the gfx950 decode and prefill kernels:
// fragment types, the 16x16x32 bf16 / fp16 MFMAs, packing, the
// half-argument GELU (fp32 and packed fp16) and the int4 decode.
#pragma once

#include "lowram_internal.h"

namespace lowram {
namespace mfma {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4 mfma_bf16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma_f16(f16x8 a, f16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) {
  bf16x8 r;
  __builtin_memcpy(&r, &v, 16);
  return r;
}
__device__ __forceinline__ f16x8 as_f16x8(uint4 v) {
  f16x8 r;
  __builtin_memcpy(&r, &v, 16);
  return r;
}

// fp32 -> bf16 with round-to-nearest-even: gfx950 converts in hardware
// (v_cvt_pk_bf16_f32)
__device__ __forceinline__ bf16x8 pack8_bf16(f32x4 a, f32x4 b) {
  bf16x8 r = {(__bf16)a[0], (__bf16)a[1], (__bf16)a[2], (__bf16)a[3],
              (__bf16)b[0], (__bf16)b[1], (__bf16)b[2], (__bf16)b[3]};
  return r;
}

// fp32 -> fp16 with round-to-nearest-even (v_cvt_pk_f16_f32)
__device__ __forceinline__ f16x8 pack8_f16(f32x4 a, f32x4 b) {
  f16x8 r = {(_Float16)a[0], (_Float16)a[1], (_Float16)a[2], (_Float16)a[3],
             (_Float16)b[0], (_Float16)b[1], (_Float16)b[2], (_Float16)b[3]};
  return r;
}

// GELU from half its argument, x2 = x / 2 (the MLP weights and bias are
// pre-halved, exactly, so the MFMA delivers x2).  With a = |x| and the normal
// upper tail 1 - Phi(a) = 0.5 exp(-f(a)) = q, GELU(x) = x Phi(x) =
// x2 + |x2| (1 - 2 q) for both signs of x.  f is a degree-4 polynomial on
// [0, 6] (Chebyshev fit by fit_gelu_tail.py), here rewritten in a2 = |x2|
// on [0, 3], pre-scaled by -log2(e) with the 0.5 folded in.  Max |error|
// 6.4e-6, max error / |x| 1.7e-4 against the exact erf form: far below the
// bf16 rounding (2^-9 relative) of the hidden activation that follows.
__device__ __forceinline__ float gelu_half(float x2) {
  const float a = __builtin_amdgcn_fmed3f(fabsf(x2), 0.0f, 3.0f);   // min(|x2|, 3) in one instruction
  const float e = -1.000479817e+00f + a * (-2.294740677e+00f + a * (-1.872075438e+00f +
                  a * (-3.526109159e-01f + a * 6.184971333e-02f)));
  const float q = __builtin_amdgcn_exp2f(e);       // 1 - Phi(|x|)
  return fmaf(fabsf(x2), fmaf(-2.0f, q, 1.0f), x2);
}

// gelu_half of two values at once in packed fp16 arithmetic, for an fp16
// MFMA operand: the same form and polynomial (coefficients rounded to fp16),
// each step one packed op on both values, the exponential by two v_exp_f16.
// The fp32 inputs are converted rounding toward zero, which saturates at the
// largest finite fp16 instead of overflowing, so the form never meets an
// infinity.  Max error / |x| 1.6e-3 and rms 3.1e-4 against the exact erf
// form (with a mean of -1.8e-4 from the truncation), against 3.9e-3 and
// 1.2e-3 for the fp32 form rounded to bf16.
__device__ __forceinline__ f16x2 gelu_half_pk(float x2a, float x2b) {
  const f16x2 h = __builtin_bit_cast(f16x2, __builtin_amdgcn_cvt_pkrtz(x2a, x2b));
  const f16x2 ah = __builtin_elementwise_abs(h);
  const f16x2 a = __builtin_elementwise_min(ah, f16x2{(_Float16)3.0f, (_Float16)3.0f});
  auto cst = [](float v) { return f16x2{(_Float16)v, (_Float16)v}; };
  f16x2 e = __builtin_elementwise_fma(a, cst(6.184971333e-02f), cst(-3.526109159e-01f));
  e = __builtin_elementwise_fma(e, a, cst(-1.872075438e+00f));
  e = __builtin_elementwise_fma(e, a, cst(-2.294740677e+00f));
  e = __builtin_elementwise_fma(e, a, cst(-1.000479817e+00f));
  const f16x2 q = __builtin_elementwise_exp2(e);
  return __builtin_elementwise_fma(ah, __builtin_elementwise_fma(q, cst(-2.0f), cst(1.0f)), h);
}

// int4 codes -> fp16 fragment, in rank order: code e of the word is the
// nibble at bits 4 e (two's complement).  XOR 8 makes it offset binary u;
// 0x6400 | u is the fp16 1024 + u, so subtracting 1032 leaves the code
// exactly, and one multiply by the fp16 group scale rounds code * scale to
// fp16 once (as the fp32 product converted to fp16 would).
__device__ __forceinline__ f16x8 dequant8(uint32_t w, uint32_t scale_bits) {
  typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
  const uint32_t x = w ^ 0x88888888u;
  _Float16 sc;
  const uint16_t sb = static_cast<uint16_t>(scale_bits);
  __builtin_memcpy(&sc, &sb, 2);
  const f16x2 bias = {(_Float16)1032.0f, (_Float16)1032.0f}, sv = {sc, sc};
  f16x8 r;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const uint32_t byte = (x >> (8 * q)) & 0xffu;
    const uint32_t m = (byte & 0xfu) | ((byte & 0xf0u) << 12) | 0x64006400u;   // codes 2q, 2q + 1
    f16x2 h;
    __builtin_memcpy(&h, &m, 4);
    h = (h - bias) * sv;
    r[2 * q] = h[0];
    r[2 * q + 1] = h[1];
  }
  return r;
}

}  // namespace mfma
}  // namespace lowram
