// Internal launchers shared by the C ABI layer (mx_api.cpp) and the kernels.
// Arguments are already validated when these are called.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mx {

// Elementwise MX quantization of `rows` rows of K elements (pitch ld
// elements). kind: 0 = bf16 input, 1 = f32 input.
hipError_t launch_quantize(int kind, const void* x, int64_t rows, int64_t K, int64_t ld,
                           uint8_t* q, uint8_t* s, hipStream_t stream);

// Rows of a slab-layout operand: `rows` rounded up to the 256-row tile.
inline int64_t slab_rows(int64_t rows) { return (rows + 255) / 256 * 256; }

// The same quantization written in the slab layout (codes [K/64][R][64],
// scales [K/64][R][2], R = slab_rows(rows); pad rows are zero). K % 64 == 0.
hipError_t launch_quantize_slab(int kind, const void* x, int64_t rows, int64_t K, int64_t ld,
                                uint8_t* q, uint8_t* s, hipStream_t stream);

// Row-major codes [rows][K] and scales [rows][K/32] to the slab layout.
hipError_t launch_slab_pack(const uint8_t* q, const uint8_t* s, int64_t rows, int64_t K,
                            uint8_t* qo, uint8_t* so, hipStream_t stream);

// The block-scaled GEMM. When xs == nullptr, x is bf16 [M][K] and is
// quantized in the prologue; otherwise x holds E4M3 codes [M][K] and xs the
// E8M0 scales [M][K/32]. epi: 0 none, 1 GELU-tanh.
hipError_t launch_linear(const void* x, const uint8_t* xs, int64_t M, int64_t K,
                         const uint8_t* wq, const uint8_t* ws, int64_t N,
                         const void* bias, int epi, void* y, hipStream_t stream);

// The block-scaled GEMM on operands in the slab layout (mx.h): codes
// [K/64][R][64], scales [K/64][R][2], R = rows rounded up to 256; K % 64 == 0.
hipError_t launch_linear_slab(const uint8_t* xq, const uint8_t* xs, int64_t M, int64_t K,
                              const uint8_t* wq, const uint8_t* ws, int64_t N,
                              const void* bias, int epi, void* y, hipStream_t stream);

// The same GEMM on 256 (weights) x 128 (tokens) tiles: twice the tiles of
// launch_linear_slab for the same shape, the same result bit for bit.
hipError_t launch_linear_slab_m128(const uint8_t* xq, const uint8_t* xs, int64_t M, int64_t K,
                                   const uint8_t* wq, const uint8_t* ws, int64_t N,
                                   const void* bias, int epi, void* y, hipStream_t stream);

// The slab GEMM writing, instead of y, the MX quantization of bf16 y in the
// slab layout with rows M and K' = N: hq [N/64][RM][64], hs [N/64][RM][2],
// RM = slab_rows(M). N % 64 == 0 and RM * N < 2^31.
hipError_t launch_linear_slab_requant(const uint8_t* xq, const uint8_t* xs, int64_t M, int64_t K,
                                      const uint8_t* wq, const uint8_t* ws, int64_t N, const void* bias,
                                      int epi, uint8_t* hq, uint8_t* hs, hipStream_t stream);

// Split-K slab GEMM: each tile's K/64 half-steps in `splits` ranges, one
// workgroup per (tile, range) writing fp32 partial sums into `part`
// (splits * tiles * 65536 floats), then a reduction kernel summing the
// ranges in order and applying bias, epilogue and bf16 into y [M][N].
// 1 <= splits <= K/64.
hipError_t launch_linear_slab_splitk(const uint8_t* xq, const uint8_t* xs, int64_t M, int64_t K, const uint8_t* wq,
                                     const uint8_t* ws, int64_t N, const void* bias, int epi, void* y, int splits,
                                     float* part, hipStream_t stream);

// Few-token slab GEMM (128-token x 64-weight-row tiles, see mx_small.hip):
// splits == 1 writes y directly; splits > 1 writes f32 partials [splits][M][N]
// into `part` and reduces them in range order. small_tiles gives the tile
// count. 1 <= splits <= K/64, N % 16 == 0.
int64_t small_tiles(int64_t M, int64_t N);

// Measurement probe (mx_probe.hip): `blocks` workgroups of 4 waves, each
// lane loading 128 bytes of A and B codes (word index modulo bytes / 4), then
// 16 * iters scaled 32x32x64 MFMAs; one float per thread to sink.
hipError_t launch_mfma_probe(const uint8_t* a, const uint8_t* b, int64_t bytes, int iters, int blocks, float* sink,
                             hipStream_t stream);

// A one-wave kernel that occupies `stream` for about `microseconds` (the
// tuner queues its timed runs behind it, so that they run back to back).
hipError_t launch_delay(int microseconds, hipStream_t stream);
hipError_t launch_linear_slab_small(const uint8_t* xq, const uint8_t* xs, int64_t M, int64_t K, const uint8_t* wq,
                                    const uint8_t* ws, int64_t N, const void* bias, int epi, void* y, int splits,
                                    float* part, hipStream_t stream);

// Balanced slab GEMM: the full rounds of ncu tiles data-parallel, the last,
// partial round split over K (at most 8 ranges, at least 2 slabs each) with
// fp32 partials in `part`. balanced_plan gives the number of data-parallel
// tiles, the split count (1: no split) and the partial bytes needed.
int64_t balanced_plan(int64_t M, int64_t K, int64_t N, int ncu, int64_t* full, int* splits);
hipError_t launch_linear_slab_balanced(const uint8_t* xq, const uint8_t* xs, int64_t M, int64_t K, const uint8_t* wq,
                                       const uint8_t* ws, int64_t N, const void* bias, int epi, void* y, int ncu,
                                       float* part, hipStream_t stream);

// Per-output-channel FP8: rows of x (bf16, kind 0, or f32, kind 1; pitch ld)
// to E4M3 codes in the slab layout q [K/64][R][64] and one f32 scale per row
// s [R] (R = slab_rows(rows); pad rows zero). K % 64 == 0.
hipError_t launch_pc_quantize_slab(int kind, const void* x, int64_t rows, int64_t K, int64_t ld, uint8_t* q, float* s,
                                   hipStream_t stream);

// The slab GEMM on per-channel operands: codes as for launch_linear_slab,
// scales f32 per token row (xs [RM]) and per weight row (ws [RN]);
// y = bf16(epi(xs[m] ws[n] acc + bias[n])).
hipError_t launch_pc_linear_slab(const uint8_t* xq, const float* xs, int64_t M, int64_t K, const uint8_t* wq,
                                 const float* ws, int64_t N, const void* bias, int epi, void* y, hipStream_t stream);

// Bytes of the library-owned scratch array of mx_linear_noalloc (per GPU).
constexpr int64_t kScratchBytes = int64_t(64) << 20;

// Device address of that array on the current device (looked up on the
// first call per device, then cached).
hipError_t scratch_buffer(void** ptr);

}  // namespace mx
