// Measurement probe: the scaled FP8 MFMA's throughput with operands held in
// registers, no memory traffic in the loop. One workgroup of 4 waves per CU
// (one wave per SIMD, 16 accumulator blocks of 32 x 32 each, the GEMM's own
// shape), each lane taking its 4 A and 4 B fragments (32 bytes each) from the
// caller's code buffers once, then issuing `iters` rounds of 16 independent
// v_mfma_scale_f32_32x32x64_f8f6f4 with unit block scales. The matrix cores'
// power, and so the clock the chip sustains, depends on the operand bits,
// which is why the codes are the caller's (e.g. the codes of the workload
// being measured) rather than constants.
#include "mx_device.h"
#include "mx_internal.h"

namespace mx {
namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));

__global__ __launch_bounds__(256, 1) void mfma_probe_kernel(const uint8_t* a, const uint8_t* b, uint32_t words,
                                                            int iters, float* sink) {
  const uint32_t t = blockIdx.x * 256 + threadIdx.x;
  const int* aw = (const int*)a;
  const int* bw = (const int*)b;
  i32x8 fa[4], fb[4];
#pragma unroll
  for (int f = 0; f < 4; ++f)
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      fa[f][i] = aw[(t * 32 + f * 8 + i) % words];
      fb[f][i] = bw[(t * 32 + f * 8 + i) % words];
    }
  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x16{};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fa[i], fb[j], acc[i][j], 0, 0, 0, 127, 0, 127);
  }
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) s += acc[i][j][e];
  sink[t] = s;  // keeps the MFMAs live
}

}  // namespace

hipError_t launch_mfma_probe(const uint8_t* a, const uint8_t* b, int64_t bytes, int iters, int blocks, float* sink,
                             hipStream_t stream) {
  hipLaunchKernelGGL(mfma_probe_kernel, dim3(blocks), dim3(256), 0, stream, a, b, (uint32_t)(bytes / 4), iters, sink);
  return hipGetLastError();
}

}  // namespace mx
