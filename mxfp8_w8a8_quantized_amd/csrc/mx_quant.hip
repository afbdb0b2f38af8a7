// Standalone MX quantizer: bf16 activations or f32/bf16 weights to E4M3
// codes + E8M0 scales (model card "Wan2.2-I2V-A14B-Lightning · MXFP8
// (AutoRound OptRTN)", section "Quantization Details": dynamic MXFP8
// activations, E4M3 weights with per-32 E8M0 scales).
//
// HBM-bound: each lane owns 8 consecutive elements (a quarter of a group of
// 32), loaded with 16- or 32-byte loads and stored as 8 code bytes; the group
// maximum is reduced across the four lanes of a DPP quad. Every thread keeps
// 2 items in flight.
//
// Row-major output: a wave streams 512 contiguous elements of one row.
// Slab output (codes [K/64][R][64], scales [K/64][R][2], R = rows rounded up
// to 256): from f32, 16 consecutive lanes cover two rows x 64 K, so each
// group of 16 lanes stores one whole 128-byte line of a slab; from bf16 (the
// activations), a block stages an 8-row x 512-K tile in LDS and stores each
// slab's part of it as one 512-byte run. Rows rows..R-1 are written as zero
// codes and zero scales.
#include "mx_device.h"
#include "mx_internal.h"

namespace mx {
namespace {

constexpr int kThreads = 256;
// Items (8-element quarters) in flight per thread, and the grid cap: two
// items with up to 65536 blocks measured best at 75348 x 5120 (0.230 ms,
// against 0.248 ms for four items with 8192 blocks).
constexpr int kItems = 2;
constexpr int64_t kMaxBlocks = 65536;

template <bool F32, bool SLAB, typename Idx>
__global__ __launch_bounds__(kThreads) void quantize_kernel(const void* __restrict__ x, Idx rows, Idx K, Idx ld,
                                                            Idx R, uint8_t* __restrict__ q, uint8_t* __restrict__ s) {
  const Idx qpr = K / 8;  // quarters per row; a multiple of 4
  const Idx total = (SLAB ? R : rows) * qpr;
  const Idx stride = (Idx)gridDim.x * kThreads;
  const Idx gpr = K / 32;
  const Idx nslab = K / 64;
  // Slab order: the 32 row pairs whose scales share one 128-byte line of a
  // scale slab are 5 blocks apart (at K = 5120). Blocks are dealt to the 8
  // XCDs in turn, so give each XCD a contiguous range of logical blocks:
  // the pieces of a scale line are then written by blocks on one XCD, at
  // about the same time, and its L2 merges them into whole lines (dealt
  // round-robin, the line's pieces reached several L2s, each of which wrote
  // back a partial line).
  Idx lb = blockIdx.x;
  if (SLAB) {
    const Idx nb = gridDim.x, q8 = nb >> 3, r8 = nb & 7, xcd = blockIdx.x & 7;
    lb = xcd * q8 + (xcd < r8 ? xcd : r8) + (blockIdx.x >> 3);
  }
  for (Idx base = lb * kThreads + threadIdx.x; base < total; base += stride * kItems) {
    // All four lanes of a quad see the same validity and row: total and
    // stride are multiples of 4 (of 16 in slab order) and quads are 4-aligned.
    uint32_t raw[kItems][8];
    Idx row[kItems], cq[kItems], qoff[kItems], soff[kItems];
    bool ok[kItems], in[kItems];
#pragma unroll
    for (int j = 0; j < kItems; ++j) {
      const Idx u = base + (Idx)j * stride;
      ok[j] = u < total;
      if (SLAB) {
        const Idx t = ok[j] ? (u & 15) : 0, rest = ok[j] ? (u >> 4) : 0;
        const Idx sl = rest % nslab, pair = rest / nslab;
        row[j] = 2 * pair + (t >> 3);
        cq[j] = sl * 8 + (t & 7);
        qoff[j] = sl * R * 64 + row[j] * 64 + (t & 7) * 8;
        soff[j] = sl * R * 2 + row[j] * 2 + ((t & 7) >> 2);
        in[j] = ok[j] && row[j] < rows;
      } else {
        row[j] = ok[j] ? u / qpr : 0;
        cq[j] = ok[j] ? u - row[j] * qpr : 0;
        qoff[j] = row[j] * K + cq[j] * 8;
        soff[j] = row[j] * gpr + (cq[j] >> 2);
        in[j] = ok[j];
      }
      if (F32) {
        const float* p = (const float*)x + (size_t)row[j] * (size_t)ld + (size_t)cq[j] * 8;
        i32x4 a = in[j] ? *(const i32x4*)p : i32x4{0, 0, 0, 0};
        i32x4 b = in[j] ? *(const i32x4*)(p + 4) : i32x4{0, 0, 0, 0};
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          raw[j][t] = (uint32_t)a[t];
          raw[j][4 + t] = (uint32_t)b[t];
        }
      } else {
        const uint16_t* p = (const uint16_t*)x + (size_t)row[j] * (size_t)ld + (size_t)cq[j] * 8;
        i32x4 a = in[j] ? *(const i32x4*)p : i32x4{0, 0, 0, 0};
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
      *(i32x2*)(q + (size_t)qoff[j]) = i32x2{(int)codes[0], (int)codes[1]};
      if ((cq[j] & 3) == 0) s[(size_t)soff[j]] = (uint8_t)sc;
    }
  }
}

// Slab output from bf16, staged through LDS: a block takes a tile of
// kTileRows rows x 512 K; each wave loads whole 1 KB row segments (64 lanes
// of 16 bytes, as in the row-major order), quantizes each lane's 8 elements
// (a DPP quad holds a group of 32), puts codes and scales into LDS in slab
// order, and then stores each of the tile's eight 64-K slabs as one
// contiguous run of kTileRows x 64 bytes, with its 2 x kTileRows scale bytes.
// Tiles run K fastest; blocks are numbered as in the slab order above, so the
// tiles that share a 128-byte scale line run on one XCD.
// 8 rows measured best at 75348 x 5120 (2.4% under the two-row order above;
// 16 or 32 rows the same as that order there, though faster at K = 13824).
constexpr int kTileRows = 8, kTileK = 512;
constexpr int64_t kMaxTiledBlocks = (int64_t)1 << 24;
constexpr int kTileItems = kTileRows / 4;  // 8-element items per thread and tile
// LDS bytes per slab of the tile: its rows plus 64 bytes of padding, so that
// the four slabs a half-wave writes at once start 16 banks apart and its 32
// eight-byte writes cover the 64 banks once.
constexpr int kSlabLds = kTileRows * 64 + 64;
static_assert(kTileRows % 8 == 0 && 256 % kTileRows == 0, "tile rows divide the slab row padding");
static_assert((kSlabLds / 4) % 64 == 16, "consecutive slabs of the tile start 16 LDS banks apart");

template <typename Idx>
__global__ __launch_bounds__(kThreads) void quantize_slab_tiled_kernel(const uint16_t* __restrict__ x, Idx rows, Idx K,
                                                                       Idx ld, Idx R, Idx tiles_per_block,
                                                                       uint8_t* __restrict__ q,
                                                                       uint8_t* __restrict__ s) {
  __shared__ __attribute__((aligned(16))) uint8_t lq[8 * kSlabLds];  // [slab][row][64], slabs kSlabLds apart
  __shared__ uint8_t ls[8 * kTileRows * 2];                           // [slab][row][2]
  const int t = threadIdx.x;
  const int lane = t & 63, wave = t >> 6;
  const int sl_l = lane >> 3;  // the lane's slab within the tile
  const Idx nkt = (K + kTileK - 1) / kTileK;
  const Idx tiles = (R / kTileRows) * nkt;
  const Idx nb = gridDim.x, q8 = nb >> 3, r8 = nb & 7, xcd = blockIdx.x & 7;
  const Idx lb = xcd * q8 + (xcd < r8 ? xcd : r8) + (blockIdx.x >> 3);
  const Idx first = lb * tiles_per_block;
  const Idx last = first + tiles_per_block < tiles ? first + tiles_per_block : tiles;
  for (Idx tile = first; tile < last; ++tile) {
    const Idx rg = tile / nkt, kt = tile - rg * nkt;
    const Idx r0 = rg * kTileRows, k0 = kt * kTileK;
    const bool kin = k0 + (Idx)(8 * lane) < K;
    uint32_t raw[kTileItems][4];
#pragma unroll
    for (int j = 0; j < kTileItems; ++j) {
      const Idx row = r0 + (Idx)(wave + 4 * j);
      const i32x4 a = (kin && row < rows) ? *(const i32x4*)(x + (size_t)row * (size_t)ld + (size_t)(k0 + 8 * lane))
                                          : i32x4{0, 0, 0, 0};
#pragma unroll
      for (int u = 0; u < 4; ++u) raw[j][u] = (uint32_t)a[u];
    }
#pragma unroll
    for (int j = 0; j < kTileItems; ++j) {
      uint32_t codes[2], sc;
      quantize8_bf16(raw[j], codes, sc);  // every lane: the quads stay whole
      const int row_l = wave + 4 * j;
      *(i32x2*)(lq + sl_l * kSlabLds + row_l * 64 + (lane & 7) * 8) = i32x2{(int)codes[0], (int)codes[1]};
      if ((lane & 3) == 0) ls[sl_l * (kTileRows * 2) + row_l * 2 + ((lane >> 2) & 1)] = (uint8_t)sc;
    }
    __syncthreads();
    {
      const int sl = t >> 5, piece = t & 31;  // 32 threads store slab sl of the tile
      if (k0 + (Idx)(64 * sl) < K) {
        const Idx gs = k0 / 64 + (Idx)sl;
        uint8_t* qrun = q + (size_t)(gs * R * 64 + r0 * 64);
        uint8_t* srun = s + (size_t)(gs * R * 2 + r0 * 2);
#pragma unroll
        for (int i = 0; i < kTileRows / 8; ++i)
          *(i32x4*)(qrun + (piece + 32 * i) * 16) = *(const i32x4*)(lq + sl * kSlabLds + (piece + 32 * i) * 16);
#pragma unroll
        for (int i = 0; i < (2 * kTileRows + 31) / 32; ++i)
          if (piece + 32 * i < 2 * kTileRows) srun[piece + 32 * i] = ls[sl * (kTileRows * 2) + piece + 32 * i];
      }
    }
    __syncthreads();
  }
}

// Row-major codes [rows][K] and scales [rows][K/32] to the slab layout: one
// 16-byte piece per thread, 8 consecutive threads per 128-byte slab line
// (two rows x 64 B); rows rows..R-1 become zeros.
template <typename Idx>
__global__ __launch_bounds__(kThreads) void slab_pack_kernel(const uint8_t* __restrict__ q, const uint8_t* __restrict__ s,
                                                             Idx rows, Idx K, Idx R, uint8_t* __restrict__ qo,
                                                             uint8_t* __restrict__ so) {
  const Idx total = R * (K / 16);
  const Idx nslab = K / 64;
  const Idx gpr = K / 32;
  for (Idx u = (Idx)blockIdx.x * kThreads + threadIdx.x; u < total; u += (Idx)gridDim.x * kThreads) {
    const Idx t = u & 7, rest = u >> 3;
    const Idx sl = rest % nslab, pair = rest / nslab;
    const Idx row = 2 * pair + (t >> 2), c = t & 3;
    const bool in = row < rows;
    const i32x4 v = in ? *(const i32x4*)(q + (size_t)row * K + sl * 64 + c * 16) : i32x4{0, 0, 0, 0};
    *(i32x4*)(qo + (size_t)sl * R * 64 + (size_t)pair * 128 + t * 16) = v;
    if (c == 0) {
      const uint16_t sc = in ? *(const uint16_t*)(s + (size_t)row * gpr + 2 * sl) : (uint16_t)0;
      *(uint16_t*)(so + (size_t)sl * R * 2 + (size_t)row * 2) = sc;
    }
  }
}

int64_t grid_for(int64_t units, int64_t per_block) {
  int64_t blocks = (units + per_block - 1) / per_block;
  if (blocks > kMaxBlocks) blocks = kMaxBlocks;
  if (blocks < 1) blocks = 1;
  return blocks;
}

template <bool F32, bool SLAB>
hipError_t launch_typed(const void* x, int64_t rows, int64_t K, int64_t ld, uint8_t* q, uint8_t* s, hipStream_t st) {
  const int64_t R = SLAB ? slab_rows(rows) : rows;
  const int64_t total = R * (K / 8);
  const unsigned blocks = (unsigned)grid_for(total, (int64_t)kThreads * kItems);
  if (total < (int64_t)1 << 31 && rows * ld < (int64_t)1 << 31 && R * K < (int64_t)1 << 31) {
    hipLaunchKernelGGL((quantize_kernel<F32, SLAB, uint32_t>), dim3(blocks), dim3(kThreads), 0, st, x,
                       (uint32_t)rows, (uint32_t)K, (uint32_t)ld, (uint32_t)R, q, s);
  } else {
    hipLaunchKernelGGL((quantize_kernel<F32, SLAB, uint64_t>), dim3(blocks), dim3(kThreads), 0, st, x,
                       (uint64_t)rows, (uint64_t)K, (uint64_t)ld, (uint64_t)R, q, s);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_quantize(int kind, const void* x, int64_t rows, int64_t K, int64_t ld, uint8_t* q, uint8_t* s,
                           hipStream_t stream) {
  return kind == 1 ? launch_typed<true, false>(x, rows, K, ld, q, s, stream)
                   : launch_typed<false, false>(x, rows, K, ld, q, s, stream);
}

hipError_t launch_quantize_slab(int kind, const void* x, int64_t rows, int64_t K, int64_t ld, uint8_t* q, uint8_t* s,
                                hipStream_t stream) {
  if (kind == 1) return launch_typed<true, true>(x, rows, K, ld, q, s, stream);
  const int64_t R = slab_rows(rows);
  const int64_t tiles = (R / kTileRows) * ((K + kTileK - 1) / kTileK);
  // One tile per block measured best (2% under two per block at 75348 x 5120,
  // 7% at 75348 x 13824); blocks loop over tiles only past 2^24 tiles.
  const int64_t per = (tiles + kMaxTiledBlocks - 1) / kMaxTiledBlocks;
  const unsigned blocks = (unsigned)((tiles + per - 1) / per);
  const uint16_t* xb = (const uint16_t*)x;
  if (R * K < (int64_t)1 << 31 && rows * ld < (int64_t)1 << 31) {
    hipLaunchKernelGGL((quantize_slab_tiled_kernel<uint32_t>), dim3(blocks), dim3(kThreads), 0, stream, xb,
                       (uint32_t)rows, (uint32_t)K, (uint32_t)ld, (uint32_t)R, (uint32_t)per, q, s);
  } else {
    hipLaunchKernelGGL((quantize_slab_tiled_kernel<uint64_t>), dim3(blocks), dim3(kThreads), 0, stream, xb,
                       (uint64_t)rows, (uint64_t)K, (uint64_t)ld, (uint64_t)R, (uint64_t)per, q, s);
  }
  return hipGetLastError();
}

hipError_t launch_slab_pack(const uint8_t* q, const uint8_t* s, int64_t rows, int64_t K, uint8_t* qo, uint8_t* so,
                            hipStream_t stream) {
  const int64_t R = slab_rows(rows);
  const int64_t total = R * (K / 16);
  const unsigned blocks = (unsigned)grid_for(total, (int64_t)kThreads * 4);
  if (R * K < (int64_t)1 << 31) {
    hipLaunchKernelGGL((slab_pack_kernel<uint32_t>), dim3(blocks), dim3(kThreads), 0, stream, q, s, (uint32_t)rows,
                       (uint32_t)K, (uint32_t)R, qo, so);
  } else {
    hipLaunchKernelGGL((slab_pack_kernel<uint64_t>), dim3(blocks), dim3(kThreads), 0, stream, q, s, (uint64_t)rows,
                       (uint64_t)K, (uint64_t)R, qo, so);
  }
  return hipGetLastError();
}

}  // namespace mx
