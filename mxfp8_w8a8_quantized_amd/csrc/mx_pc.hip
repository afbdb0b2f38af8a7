// Per-output-channel FP8 quantizer: one FP32 scale per row, E4M3 codes.
//
// Scheme ("Wan2.2 I2V A14B, four-step 720p: native LightX2V FP8 and NVFP4",
// section "Conversion and compatibility": E4M3 weight codes scaled by one
// FP32 factor per output channel, rounded to nearest; "Model Quantization
// Techniques", mode table: FP8 weights symmetric per channel, FP8
// activations symmetric per row and computed on the fly, row scale =
// max(abs(x)) / qmax, qmax 448, FP32 accumulation):
//   s    = fp32(max |x[r, :]|) / 448            (FP32 division, nearest even)
//   code = E4M3(fp32(x) / s)                   (FP32 division, then nearest
//                                               even, saturating at +-448)
//   s == 0: every code a signed zero; a row with NaN or Inf: s = NaN and
//   every code 0x7F.
//
// One wave per row: lanes hold 8 consecutive elements of each 512-element
// chunk; the row's largest magnitude is a wave-wide maximum of magnitude
// bits; the codes go to the slab layout ([K/64][R][64], R = rows rounded up
// to 256) so that 8 lanes fill one 64-byte row segment of a slab. bf16 rows
// of up to 28 chunks (K <= 14336) are held in registers and read once;
// longer rows and f32 weights take two passes. Pad rows get zero codes and
// scale 0.
#include "mx_device.h"
#include "mx_internal.h"

namespace mx {
namespace {

constexpr int kRowsPerBlock = 4;  // one wave each
constexpr int kUnroll = 8;        // 512-element chunks in flight per pass

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

// The correctly rounded FP32 quotient v / scale. For scale >= 2^-100 (rinv =
// RN(1 / scale) then finite and normal): q0 = RN(v rinv), then two FMA
// corrections q <- RN(q + RN(v - q scale) rinv) (the residual is exact by
// FMA). The first makes q faithful (within one ulp of v / scale); with rinv
// correctly rounded and q faithful, Markstein's theorem makes the second
// result RN(v / scale). The sign is put back from v, so -0 stays -0.
// Smaller scales take the full division. Five FMA-pipe operations per element
// instead of the division's scaled reciprocal iteration.
__device__ inline float quotient_fma(float v, float scale, float rinv) {
  float q = v * rinv;
  q = __builtin_fmaf(__builtin_fmaf(-q, scale, v), rinv, q);
  q = __builtin_fmaf(__builtin_fmaf(-q, scale, v), rinv, q);
  return __builtin_copysignf(q, v);
}

// Codes of 8 elements under the row's scale, packed 8 bytes. `fast` and
// `rinv` are the row's (scale >= 2^-100 and finite; RN(1 / scale)).
__device__ inline uint2 encode8(const float v[8], float scale, float rinv, bool fast, bool bad) {
  if (bad) return uint2{0x7F7F7F7Fu, 0x7F7F7F7Fu};
  float t[8];
  if (fast) {
#pragma unroll
    for (int i = 0; i < 8; ++i) t[i] = quotient_fma(v[i], scale, rinv);
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) t[i] = scale == 0.f ? __builtin_copysignf(0.f, v[i]) : v[i] / scale;
  }
  // The hardware conversion rounds to nearest even onto the E4M3 grid
  // (subnormals included, the sign of zero kept). Clamping to +-448 first
  // gives the saturated result: every value between 448 and 464 rounds to
  // 448 anyway, and 464 is a tie that goes to 448's even significand.
  int w[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    float c[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) c[i] = __builtin_amdgcn_fmed3f(t[4 * h + i], -448.0f, 448.0f);
    w[h] = __builtin_amdgcn_cvt_pk_fp8_f32(c[0], c[1], 0, false);
    w[h] = __builtin_amdgcn_cvt_pk_fp8_f32(c[2], c[3], w[h], true);
  }
  return uint2{(uint32_t)w[0], (uint32_t)w[1]};
}

// The row's scale from the lanes' partial maxima of magnitude bits.
__device__ inline float row_scale(uint32_t m, bool& bad) {
  m = wave_max_u32(m);
  bad = m >= 0x7F800000u;                // Inf or NaN in the row
  return __uint_as_float(m) / 448.0f;    // correctly rounded FP32 division
}

// NCH > 0: the whole row (at most NCH chunks of 512 elements) is loaded into
// registers at once and quantized from there: one read of the row. NCH == 0:
// two passes over any K, kUnroll chunks in flight, the second re-reading the
// row (the f32 weight path, quantized once, off the timed path).
template <bool F32, int NCH>
__global__ __launch_bounds__(64 * kRowsPerBlock) void pc_quantize_kernel(const void* __restrict__ x, int64_t rows,
                                                                       int K, int64_t ld, int64_t R,
                                                                       uint8_t* __restrict__ q, float* __restrict__ s) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6);
  if (row >= R) return;
  const bool real = row < rows;
  const int64_t rbase = real ? row * ld : 0;
  uint8_t* qrow = q + row * 64;
  bool bad;

  if constexpr (NCH > 0) {
    static_assert(!F32, "register-resident rows are bf16");
    uint4 raw[NCH];  // 8 bf16 per chunk, kept packed
    uint32_t m = 0;
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      const int k = c * 512 + 8 * lane;
      raw[c] = (real && k < K) ? *(const uint4*)((const uint16_t*)x + rbase + k) : uint4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      const uint32_t w[4] = {raw[c].x, raw[c].y, raw[c].z, raw[c].w};
#pragma unroll
      for (int i = 0; i < 4; ++i) m = max(m, max((w[i] << 16) & 0x7FFF0000u, w[i] & 0x7FFF0000u));
    }
    const float scale = row_scale(m, bad);
    if (lane == 0) s[row] = bad ? __uint_as_float(0x7FC00000u) : scale;
    const bool fast = scale >= 0x1p-100f && !bad;
    const float rinv = 1.0f / scale;
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      const int k = c * 512 + 8 * lane;
      if (k < K) {
        const uint32_t w[4] = {raw[c].x, raw[c].y, raw[c].z, raw[c].w};
        float v[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          v[2 * i] = __uint_as_float(w[i] << 16);
          v[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
        }
        *(uint2*)(qrow + (int64_t)(k >> 6) * R * 64 + (k & 63)) = encode8(v, scale, rinv, fast, bad);
      }
    }
  } else {
    const int nchunk = (K + 511) / 512;
    uint32_t m = 0;
    for (int c0 = 0; c0 < nchunk; c0 += kUnroll) {
      float v[kUnroll][8];  // kUnroll loads in flight before the first use
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const int k = (c0 + u) * 512 + 8 * lane;
        load8<F32>(x, rbase + k, real && k < K, v[u]);
      }
#pragma unroll
      for (int u = 0; u < kUnroll; ++u)
#pragma unroll
        for (int i = 0; i < 8; ++i) m = max(m, __float_as_uint(v[u][i]) & 0x7FFFFFFFu);
    }
    const float scale = row_scale(m, bad);
    if (lane == 0) s[row] = bad ? __uint_as_float(0x7FC00000u) : scale;
    const bool fast = scale >= 0x1p-100f && !bad;
    const float rinv = 1.0f / scale;
    for (int c0 = 0; c0 < nchunk; c0 += kUnroll) {
      float v[kUnroll][8];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const int k = (c0 + u) * 512 + 8 * lane;
        load8<F32>(x, rbase + k, real && k < K, v[u]);
      }
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const int k = (c0 + u) * 512 + 8 * lane;
        if (k < K) *(uint2*)(qrow + (int64_t)(k >> 6) * R * 64 + (k & 63)) = encode8(v[u], scale, rinv, fast, bad);
      }
    }
  }
}

template <bool F32, int NCH>
void launch_pc(const void* x, int64_t rows, int64_t K, int64_t ld, int64_t R, uint8_t* q, float* s,
               hipStream_t stream) {
  const unsigned blocks = (unsigned)((R + kRowsPerBlock - 1) / kRowsPerBlock);
  hipLaunchKernelGGL((pc_quantize_kernel<F32, NCH>), dim3(blocks), dim3(64 * kRowsPerBlock), 0, stream, x, rows,
                     (int)K, ld, R, q, s);
}

}  // namespace

hipError_t launch_pc_quantize_slab(int kind, const void* x, int64_t rows, int64_t K, int64_t ld, uint8_t* q, float* s,
                                   hipStream_t stream) {
  const int64_t R = slab_rows(rows);
  const int64_t nchunk = (K + 511) / 512;
  if (kind == 1)
    launch_pc<true, 0>(x, rows, K, ld, R, q, s, stream);
  else if (nchunk <= 4)
    launch_pc<false, 4>(x, rows, K, ld, R, q, s, stream);
  else if (nchunk <= 10)
    launch_pc<false, 10>(x, rows, K, ld, R, q, s, stream);
  else if (nchunk <= 16)
    launch_pc<false, 16>(x, rows, K, ld, R, q, s, stream);
  else if (nchunk <= 28)
    launch_pc<false, 28>(x, rows, K, ld, R, q, s, stream);
  else
    launch_pc<false, 0>(x, rows, K, ld, R, q, s, stream);
  return hipGetLastError();
}

}  // namespace mx
