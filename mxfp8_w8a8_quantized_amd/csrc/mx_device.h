// Device-side MXFP8 helpers for gfx950: buffer resources, the per-group
// shared scale, and E4M3 encoding of 8 elements per lane with the four lanes
// of a DPP quad holding one group of 32.
//
// Format (model card "Wan2.2-I2V-A14B-Lightning · MXFP8 (AutoRound OptRTN)",
// section "Quantization Details"): E4M3 elements, one E8M0 scale per 32
// elements along K, symmetric. Shared exponent e = floor(log2 amax) - 8
// clamped to [-127, 127], elements E4M3(x * 2^-e) rounded to nearest even
// after saturation to +-448 (the E4M3 range of "Model Quantization
// Techniques", Conv3D mode table). A group holding NaN/Inf gets scale 0xFF
// and codes 0x7F.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mx {

typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
typedef short i16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short s16x2 __attribute__((ext_vector_type(2)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// Third dword of a gfx9 raw buffer descriptor (32-bit data format).
constexpr int kBufferFlags = 0x00020000;

// Raw buffer resource over `bytes` bytes from `base`. Loads past the end
// return zero and stores past the end are dropped, which is how ragged row
// tails are handled without branches.
__device__ inline __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, kBufferFlags);
}

// DPP quad permutations: swap with lane^1 and lane^2 inside groups of 4.
constexpr int kQuadXor1 = 0xB1;  // quad_perm [1,0,3,2]
constexpr int kQuadXor2 = 0x4E;  // quad_perm [2,3,0,1]

__device__ inline uint32_t quad_max_u32(uint32_t a) {
  a = max(a, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)a, kQuadXor1, 0xF, 0xF, false));
  a = max(a, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)a, kQuadXor2, 0xF, 0xF, false));
  return a;
}

// E8M0 code of a group's shared scale from the 8-bit biased exponent field
// E of its largest magnitude (bf16 and f32 share that field). For normal
// amax floor(log2 amax) = E - 127, so e = E - 135 and the code e + 127 is
// E - 8; E <= 8 (including subnormal and zero amax) clamps to code 0, i.e.
// e = -127. E = 255 means Inf or NaN: code 0xFF.
__device__ inline uint32_t scale_code_from_exponent(uint32_t E) {
  return E == 255u ? 0xFFu : (E > 8u ? E - 8u : 0u);
}

// 2^e as an f32 for scale code c = e + 127 (2^-127 is the subnormal 0x00400000).
__device__ inline float scale_value(uint32_t code) {
  return __uint_as_float(code ? (code << 23) : 0x00400000u);
}

// ---------------------------------------------------------------------------
// bf16 input: 8 elements per lane in 4 dwords (element 2d in the low half of
// dword d). The four lanes of a DPP quad must hold one 32-group and call this
// together. Produces 8 codes (byte i = element i) and the group's scale code.
//
// The gfx950 scaled convert v_cvt_scalef32_pk_fp8_bf16 divides by the scale
// and rounds to nearest even, but turns magnitudes from 464 * 2^e up into
// NaN instead of saturating; magnitudes are therefore clamped to 448 * 2^e in
// the bf16 domain first (two packed 16-bit minima: unsigned against
// 0x8000|lim clamps negatives, signed against lim clamps positives).
__device__ inline void quantize8_bf16(const uint32_t x[4], uint32_t out[2], uint32_t& scode) {
  u16x2 m0 = __builtin_bit_cast(u16x2, x[0] & 0x7FFF7FFFu);
  u16x2 m1 = __builtin_bit_cast(u16x2, x[1] & 0x7FFF7FFFu);
  u16x2 m2 = __builtin_bit_cast(u16x2, x[2] & 0x7FFF7FFFu);
  u16x2 m3 = __builtin_bit_cast(u16x2, x[3] & 0x7FFF7FFFu);
  u16x2 mm = __builtin_elementwise_max(__builtin_elementwise_max(m0, m1), __builtin_elementwise_max(m2, m3));
  uint32_t amax = quad_max_u32(max((uint32_t)mm[0], (uint32_t)mm[1]));
  scode = scale_code_from_exponent(amax >> 7);
  const float sv = scale_value(scode);
  const uint32_t lim = ((scode + 8u) << 7) | 0x60u;  // bf16 bits of 448 * 2^e
  const u16x2 lim_u = {(unsigned short)(lim | 0x8000u), (unsigned short)(lim | 0x8000u)};
  const i16x2 lim_i = {(short)lim, (short)lim};
  s16x2 r0 = {0, 0}, r1 = {0, 0};
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    u16x2 c = __builtin_elementwise_min(__builtin_bit_cast(u16x2, x[d]), lim_u);
    i16x2 c2 = __builtin_elementwise_min(__builtin_bit_cast(i16x2, c), lim_i);
    bf16x2 src = __builtin_bit_cast(bf16x2, c2);
    if (d == 0) r0 = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(r0, src, sv, false);
    if (d == 1) r0 = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(r0, src, sv, true);
    if (d == 2) r1 = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(r1, src, sv, false);
    if (d == 3) r1 = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(r1, src, sv, true);
  }
  out[0] = __builtin_bit_cast(uint32_t, r0);
  out[1] = __builtin_bit_cast(uint32_t, r1);
  if (scode == 0xFFu) {
    out[0] = 0x7F7F7F7Fu;
    out[1] = 0x7F7F7F7Fu;
  }
}

// ---------------------------------------------------------------------------
// f32 input (weights). Integer encoding of v = x * 2^-e into E4M3; |v| < 512
// always holds inside a group, and the power-of-two scaling is exact for
// every result at or above 2^-126 (anything smaller encodes to a signed zero).
__device__ inline uint32_t e4m3_from_scaled_f32(float v) {
  const uint32_t u = __float_as_uint(v);
  const uint32_t sign = (u >> 24) & 0x80u;
  const uint32_t a = u & 0x7FFFFFFFu;
  uint32_t c;
  if (a >= 0x43E00000u) {
    c = 0x7Eu;  // |v| >= 448 saturates
  } else if (a >= 0x3C800000u) {
    // |v| >= 2^-6: normal E4M3. Round the f32 mantissa to 3 bits, ties to
    // even (a carry moves into the exponent), then rebias 127 -> 7.
    c = ((a + 0x7FFFFu + ((a >> 20) & 1u)) >> 20) - ((127u - 7u) << 3);
  } else {
    // E4M3 subnormal range: a multiple of 2^-9, rounded to nearest even.
    c = (uint32_t)__builtin_rintf(__uint_as_float(a) * 512.0f);
  }
  return c | sign;
}

__device__ inline void quantize8_f32(const float x[8], uint32_t out[2], uint32_t& scode) {
  uint32_t m = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) m = max(m, __float_as_uint(x[i]) & 0x7FFFFFFFu);
  const uint32_t amax = quad_max_u32(m);
  scode = scale_code_from_exponent(amax >> 23);
  if (scode == 0xFFu) {
    out[0] = 0x7F7F7F7Fu;
    out[1] = 0x7F7F7F7Fu;
    return;
  }
  const float inv = __uint_as_float((254u - scode) << 23);  // 2^-e
  uint32_t c[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) c[i] = e4m3_from_scaled_f32(x[i] * inv);
  out[0] = c[0] | (c[1] << 8) | (c[2] << 16) | (c[3] << 24);
  out[1] = c[4] | (c[5] << 8) | (c[6] << 16) | (c[7] << 24);
}

// ---------------------------------------------------------------------------
// Epilogue of every GEMM kernel, applied to acc + bias before the bf16
// rounding: identity (EPI 0) or GELU-tanh (EPI 1, the activation of the Wan2.2
// feed-forward up-projection). Shared so that every kernel rounds the same
// values.
template <int EPI>
__device__ __forceinline__ float epilogue(float v) {
  if (EPI == 1) {
    // GELU, tanh form, as v * sigmoid(2u) = 0.5 v (1 + tanh(u)),
    // u = sqrt(2/pi) (v + 0.044715 v^3); this form has no cancellation.
    // exp(-2u) = exp2(v (c0 + c1 v^2)) with c0 = -2 sqrt(2/pi) / ln 2 and
    // c1 = 0.044715 c0, and the hardware exp2 and reciprocal (about 1 ulp
    // each) replace the IEEE division: 7 operations per output instead of
    // ~20 (the GELU linear 4.55 -> 4.16 ms at 75348x5120x13824). The result
    // is rounded to bf16 (2^-8) right after.
    const float t = __builtin_fmaf(v * v, -0.1029432395800235f, -2.302208198144325f);
    return v * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(v * t));
  }
  return v;
}

}  // namespace mx
