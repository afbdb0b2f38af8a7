// Standalone MX quantizer: bf16 activations or f32/bf16 weights to E4M3
// codes + E8M0 scales (model card "Wan2.2-I2V-A14B-Lightning · MXFP8
// (AutoRound OptRTN)", section "Quantization Details": dynamic MXFP8
// activations, E4M3 weights with per-32 E8M0 scales).
//
// HBM-bound: each lane owns 8 consecutive elements (a quarter of a group of
// 32), so a wave streams 512 contiguous elements per item with 16- or 32-byte
// loads and 8-byte code stores; the group maximum is reduced across the four
// lanes of a DPP quad. Every thread keeps 4 items in flight.
#include "mx_device.h"
#include "mx_internal.h"

namespace mx {
namespace {

constexpr int kThreads = 256;
constexpr int kItems = 4;  // items (8-element quarters) in flight per thread

template <bool F32, typename Idx>
__global__ __launch_bounds__(kThreads) void quantize_kernel(const void* __restrict__ x, Idx rows, Idx K, Idx ld,
                                                            uint8_t* __restrict__ q, uint8_t* __restrict__ s) {
  const Idx qpr = K / 8;  // quarters per row; a multiple of 4
  const Idx total = rows * qpr;
  const Idx stride = (Idx)gridDim.x * kThreads;
  const Idx gpr = K / 32;
  for (Idx base = (Idx)blockIdx.x * kThreads + threadIdx.x; base < total; base += stride * kItems) {
    // All four lanes of a quad see the same validity: total and stride are
    // multiples of 4 and quads are 4-aligned.
    uint32_t raw[kItems][8];
    Idx row[kItems], cq[kItems];
    bool ok[kItems];
#pragma unroll
    for (int j = 0; j < kItems; ++j) {
      const Idx u = base + (Idx)j * stride;
      ok[j] = u < total;
      row[j] = ok[j] ? u / qpr : 0;
      cq[j] = ok[j] ? u - row[j] * qpr : 0;
      if (F32) {
        const float* p = (const float*)x + (size_t)row[j] * (size_t)ld + (size_t)cq[j] * 8;
        i32x4 a = ok[j] ? *(const i32x4*)p : i32x4{0, 0, 0, 0};
        i32x4 b = ok[j] ? *(const i32x4*)(p + 4) : i32x4{0, 0, 0, 0};
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          raw[j][t] = (uint32_t)a[t];
          raw[j][4 + t] = (uint32_t)b[t];
        }
      } else {
        const uint16_t* p = (const uint16_t*)x + (size_t)row[j] * (size_t)ld + (size_t)cq[j] * 8;
        i32x4 a = ok[j] ? *(const i32x4*)p : i32x4{0, 0, 0, 0};
#pragma unroll
        for (int t = 0; t < 4; ++t) raw[j][t] = (uint32_t)a[t];
      }
    }
#pragma unroll
    for (int j = 0; j < kItems; ++j) {
      if (!ok[j]) continue;  // uniform per quad
      uint32_t codes[2], sc;
      if (F32) {
        float f[8];
#pragma unroll
        for (int t = 0; t < 8; ++t) f[t] = __uint_as_float(raw[j][t]);
        quantize8_f32(f, codes, sc);
      } else {
        quantize8_bf16(raw[j], codes, sc);
      }
      *(i32x2*)(q + (size_t)row[j] * (size_t)K + (size_t)cq[j] * 8) = i32x2{(int)codes[0], (int)codes[1]};
      if ((cq[j] & 3) == 0) s[(size_t)row[j] * (size_t)gpr + (size_t)(cq[j] >> 2)] = (uint8_t)sc;
    }
  }
}

template <bool F32>
hipError_t launch_typed(const void* x, int64_t rows, int64_t K, int64_t ld, uint8_t* q, uint8_t* s, hipStream_t st) {
  const int64_t total = rows * (K / 8);
  int64_t blocks = (total + (int64_t)kThreads * kItems - 1) / ((int64_t)kThreads * kItems);
  if (blocks > 8192) blocks = 8192;
  if (blocks < 1) blocks = 1;
  if (total < (int64_t)1 << 31 && rows * ld < (int64_t)1 << 31) {
    hipLaunchKernelGGL((quantize_kernel<F32, uint32_t>), dim3((unsigned)blocks), dim3(kThreads), 0, st, x,
                       (uint32_t)rows, (uint32_t)K, (uint32_t)ld, q, s);
  } else {
    hipLaunchKernelGGL((quantize_kernel<F32, uint64_t>), dim3((unsigned)blocks), dim3(kThreads), 0, st, x,
                       (uint64_t)rows, (uint64_t)K, (uint64_t)ld, q, s);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_quantize(int kind, const void* x, int64_t rows, int64_t K, int64_t ld, uint8_t* q, uint8_t* s,
                           hipStream_t stream) {
  return kind == 1 ? launch_typed<true>(x, rows, K, ld, q, s, stream)
                   : launch_typed<false>(x, rows, K, ld, q, s, stream);
}

}  // namespace mx
