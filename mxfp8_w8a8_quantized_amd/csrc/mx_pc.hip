// Per-output-channel FP8 quantizer: one FP32 scale per row, E4M3 codes.
//
// Scheme ("Wan2.2 I2V A14B, four-step 720p: native LightX2V FP8 and NVFP4",
// section "Conversion and compatibility": E4M3 weights with per-output-
// channel FP32 scales, nearest rounding; "Model Quantization Techniques",
// mode table: channel-symmetric FP8 weights and channel-dynamic-symmetric FP8
// activations, row scale = max(abs(x)) / qmax, qmax 448 with FP32
// accumulation):
//   s    = fp32(max |x[r, :]|) / 448            (FP32 division, nearest even)
//   code = E4M3(fp32(x) / s)                   (FP32 division, then nearest
//                                               even, saturating at +-448)
//   s == 0: every code a signed zero; a row with NaN or Inf: s = NaN and
//   every code 0x7F.
//
// One wave per row, two passes over it: the row's largest magnitude (lanes
// hold 8 consecutive elements of each 512-element chunk; a wave-wide maximum
// of the magnitude bits), then the codes, written in the slab layout
// ([K/64][R][64], R = rows rounded up to 256) so that 8 lanes fill one
// 64-byte row segment of a slab. Pad rows get zero codes and scale 0. The
// second pass re-reads the row, which the first pass has just brought into
// the cache.
#include "mx_device.h"
#include "mx_internal.h"

namespace mx {
namespace {

constexpr int kRowsPerBlock = 4;  // one wave each

__device__ inline uint32_t wave_max_u32(uint32_t v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = max(v, (uint32_t)__shfl_xor((int)v, off, 64));
  return v;
}

// Eight consecutive elements of a row as f32 (zeros past the row's end).
template <bool F32>
__device__ inline void load8(const void* x, int64_t base, bool ok, float v[8]) {
  if (!ok) {
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = 0.f;
    return;
  }
  if constexpr (F32) {
    const float4* p = (const float4*)((const float*)x + base);
    const float4 a = p[0], b = p[1];
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  } else {
    const uint4 u = *(const uint4*)((const uint16_t*)x + base);
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(w[i] << 16);
      v[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
    }
  }
}

template <bool F32>
__global__ __launch_bounds__(64 * kRowsPerBlock) void pc_quantize_kernel(const void* __restrict__ x, int64_t rows,
                                                                       int K, int64_t ld, int64_t R,
                                                                       uint8_t* __restrict__ q, float* __restrict__ s) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6);
  if (row >= R) return;
  const bool real = row < rows;
  const int64_t rbase = real ? row * ld : 0;
  const int nchunk = (K + 511) / 512;

  uint32_t m = 0;
  for (int c = 0; c < nchunk; ++c) {
    const int k = c * 512 + 8 * lane;
    float v[8];
    load8<F32>(x, rbase + k, real && k < K, v);
#pragma unroll
    for (int i = 0; i < 8; ++i) m = max(m, __float_as_uint(v[i]) & 0x7FFFFFFFu);
  }
  m = wave_max_u32(m);
  const bool bad = m >= 0x7F800000u;                    // Inf or NaN in the row
  const float scale = __uint_as_float(m) / 448.0f;      // correctly rounded FP32 division
  if (lane == 0) s[row] = bad ? __uint_as_float(0x7FC00000u) : scale;

  for (int c = 0; c < nchunk; ++c) {
    const int k = c * 512 + 8 * lane;
    if (k >= K) break;
    float v[8];
    load8<F32>(x, rbase + k, real, v);
    uint32_t code[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float t = scale == 0.f ? __builtin_copysignf(0.f, v[i]) : v[i] / scale;
      code[i] = bad ? 0x7Fu : e4m3_from_scaled_f32(t);
    }
    const uint2 out = {code[0] | (code[1] << 8) | (code[2] << 16) | (code[3] << 24),
                       code[4] | (code[5] << 8) | (code[6] << 16) | (code[7] << 24)};
    *(uint2*)(q + ((int64_t)(k >> 6) * R + row) * 64 + (k & 63)) = out;
  }
}

}  // namespace

hipError_t launch_pc_quantize_slab(int kind, const void* x, int64_t rows, int64_t K, int64_t ld, uint8_t* q, float* s,
                                   hipStream_t stream) {
  const int64_t R = slab_rows(rows);
  const unsigned blocks = (unsigned)((R + kRowsPerBlock - 1) / kRowsPerBlock);
  if (kind == 1)
    hipLaunchKernelGGL(pc_quantize_kernel<true>, dim3(blocks), dim3(64 * kRowsPerBlock), 0, stream, x, rows, (int)K,
                       ld, R, q, s);
  else
    hipLaunchKernelGGL(pc_quantize_kernel<false>, dim3(blocks), dim3(64 * kRowsPerBlock), 0, stream, x, rows, (int)K,
                       ld, R, q, s);
  return hipGetLastError();
}

}  // namespace mx
