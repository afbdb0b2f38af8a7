// MXFP8 W8A8 linear on CDNA4 block-scaled FP8 matrix cores.
//
//   y[m][n] = bf16_rne( epi( sum_k xhat[m][k] * what[n][k] + f32(bias[n]) ) )
//
// (model card "Wan2.2-I2V-A14B-Lightning · MXFP8 (AutoRound OptRTN)", section
// "Quantization Details": W8A8 MXFP8 linears, E4M3 codes under one E8M0
// exponent per 32 elements, activations quantized on the fly, F16 biases;
// FP32 accumulation as in the FP32-accum FP8 mode of "Model Quantization
// Techniques", Conv3D mode table.)
//
// Three kernels, all with 256 (weight rows n) x 256 (tokens m) output tiles,
// the weights as the MFMA's A operand (a lane's accumulators are consecutive
// n of one token m) and the E8M0 scales handed straight to the MFMA:
//
// * linear_kernel (general): any K that is a multiple of 32, and the fused
//   prologue (FUSED) that quantizes the bf16 token tile inside the K loop.
//   4 waves, each a 128 x 128 sub-tile of v_mfma_scale_f32_16x16x128_f8f6f4,
//   operands staged global -> registers -> LDS, two 128-K stages.
// * pp::linear_prequant_pp: row-major pre-quantized operands with
//   K % 128 == 0; see its own comment.
// * slab::linear_slab_kernel: operands in the slab layout of mx.h (the
//   fastest path); see its own comment.
//
// 16x16x128 operand layout (32 bytes per lane in two 16-byte halves, found
// on the device): lane l holds row l%16, K bytes [16*(l/16), +16) in its
// first half and [64 + 16*(l/16), +16) in its second; the scale of lane l
// belongs to row l%16 and the 32-block l/16 (K [32b, 32b+32)). Reading the
// halves from memory K offsets 16*(l/16) and 64 + 16*(l/16) maps memory K
// to MFMA K one to one, so the scale of memory group b of the step is the
// one lane group b expects.
//
// General kernel LDS per stage: both operands 256 x 128 code bytes, rows of
// 128 B with the 16-byte chunks XOR-swizzled by (row & 7); scales stored as
// [32-block b][row permuted] so each lane reads the scales of its 8 MFMA
// tiles with one 8-byte load (op_sel picks the byte).
//
// Fused prologue: the token tile arrives as bf16 (256 B per row per step),
// each lane holds 8 elements, a DPP quad holds a 32-group, and the codes and
// scales go to LDS in the layout above.
//
// Ragged edges: buffer resources are rebased at the tile; rows past M (or N)
// load as zero and their stores are dropped.
#include <algorithm>

#include <type_traits>

#include "mx_device.h"
#include "mx_internal.h"

namespace mx {
namespace {

constexpr int BM = 256;  // tokens per tile
constexpr int BN = 256;  // weight rows per tile
constexpr int BK = 128;  // K per step
constexpr int NT = 256;  // threads
constexpr int TILE_BYTES = 256 * BK;        // one operand, one stage
constexpr int SCALE_BYTES = 4 * 256;        // one operand, one stage
constexpr int LDS_BYTES = 4 * TILE_BYTES + 4 * SCALE_BYTES;
constexpr int kDropOffset = 1 << 30;  // beyond every resource: the store is dropped
constexpr int kStoreAux = 2;
constexpr int64_t kMaxTailSplits = 8;  // as the split-K choice: partial traffic grows with it

struct Params {
  const uint8_t* x;   // bf16 tokens (fused) or E4M3 codes
  const uint8_t* xs;  // token scales (pre-quantized path)
  const uint8_t* wq;
  const uint8_t* ws;
  const uint16_t* bias;  // f16 bits, or null
  uint16_t* y;           // bf16 bits
  uint8_t* hq;           // requantized output: codes slab [N/64][RM][64] (or null)
  uint8_t* hs;           //                     scales slab [N/64][RM][2]
  float* part;           // split-K partial sums (or null), see slab::store_tile_part
  const float* sx;       // per-channel FP8: f32 scale per token row [RM] (or null)
  const float* sw;       //                  f32 scale per weight row [RN]
  int splits;            // K ranges per tile (split-K), else 1
  int tile_base;         // logical tile of this launch's first workgroup (tile_coords order)
  int part_tiles;        // split-K: tiles in this launch (partial tiles are numbered from 0)
  int M, N, K;
  int tiles_m, tiles_n;
};

template <int N>
struct Int {
  static constexpr int value = N;
};
template <int Begin, int End, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (Begin < End) {
    f(Int<Begin>{});
    static_for<Begin + 1, End>(f);
  }
}

// Bias of a lane's 32x32-MFMA accumulators: quad k = 4 i + q holds the f16
// bits of n = n0 + 128 wn + 32 i + 8 q + 4 (lane / 32) + 0..3. The 16 quads
// are loaded together (one memory round trip rather than one per quad, each
// behind a branch) through a buffer resource: zero past N, or everywhere
// without a bias.
struct BiasQuads {
  i32x2 v[16];
};

__device__ __forceinline__ void load_bias_quads(BiasQuads& B, const Params& p, int n0, int rows_n, int wn, int lane) {
  const bool has = p.bias != nullptr;
  const __amdgpu_buffer_rsrc_t rb = make_rsrc(has ? p.bias + n0 : nullptr, has ? (uint32_t)rows_n * 2u : 0u);
  const int base = (wn * 128 + 4 * (lane >> 5)) * 2;
#pragma unroll
  for (int k = 0; k < 16; ++k)
    B.v[k] = __builtin_bit_cast(i32x2, __builtin_amdgcn_raw_buffer_load_b64(rb, base + (32 * (k >> 2) + 8 * (k & 3)) * 2, 0, 0));
}

__device__ __forceinline__ float bias_at(const BiasQuads& B, int k, int r) {
  const uint32_t w = (uint32_t)B.v[k][r >> 1];
  return (float)__builtin_bit_cast(_Float16, (uint16_t)((r & 1) ? (w >> 16) : (w & 0xFFFFu)));
}

// Workgroup -> (token tile, weight tile). Workgroups are dealt round-robin to
// the 8 XCDs, so first give each XCD a contiguous range of logical tiles, then
// walk that range in groups of GM token tiles x all weight tiles (token tile
// fastest), so that concurrent tiles on one XCD share token and weight panels
// in its L2.
#ifndef MX_GM
#define MX_GM 4
#endif
__device__ inline void tile_coords(int pid, int tiles_m, int tiles_n, int& tm, int& tn) {
  constexpr int GM = MX_GM;
  const int nwg = tiles_m * tiles_n;
  const int q = nwg >> 3, r = nwg & 7;
  const int xcd = pid & 7, k = pid >> 3;
  const int lid = xcd * q + min(xcd, r) + k;
  const int group = lid / (GM * tiles_n);
  const int first_m = group * GM;
  const int gm = min(tiles_m - first_m, GM);
  const int in_group = lid - group * GM * tiles_n;
  tm = first_m + in_group % gm;
  tn = in_group / gm;
}

// LDS byte offset of 16-byte chunk c (0..7) of tile row `row`.
__device__ __forceinline__ int lds_chunk(int row, int c) { return row * BK + ((c ^ (row & 7)) << 4); }

// Scale slot of tile row `row` for 32-block b: [b][half][row%16][(row/16)%8].
__device__ __forceinline__ int lds_scale(int row, int b) {
  return b * 256 + (row >> 7) * 128 + (row & 15) * 8 + ((row >> 4) & 7);
}

// ---------------------------------------------------------------------------
// Global -> register loaders.
//
// E4M3 operand (weights, or pre-quantized tokens): thread t moves 8 chunks of
// 16 bytes, chunk c = t % 8 of rows t/8 + 32 i, plus the 4 scale bytes of row t.
struct Fp8Regs {
  i32x4 d[8];
  uint32_t sc;  // scales of row t for blocks 0..3 (byte b)
};

template <bool KTAIL>
__device__ __forceinline__ void load_fp8(Fp8Regs& r, __amdgpu_buffer_rsrc_t codes, __amdgpu_buffer_rsrc_t scales,
                                         int K, int ks) {
  const int t = threadIdx.x;
  const int c = t & 7;
  const int kk = ks * BK + c * 16;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int row = (t >> 3) + 32 * i;
    r.d[i] = __builtin_amdgcn_raw_buffer_load_b128(codes, row * K + kk, 0, 0);
    if (KTAIL && kk >= K) r.d[i] = i32x4{0, 0, 0, 0};
  }
  const int G = K >> 5;
  const int soff = t * G + ks * 4;
  uint32_t sc = 0;
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    uint32_t v = __builtin_amdgcn_raw_buffer_load_b8(scales, soff + b, 0, 0);
    if (KTAIL && ks * 4 + b >= G) v = 127;  // codes there are zero; keep the product finite
    sc |= v << (8 * b);
  }
  r.sc = sc;
}

__device__ __forceinline__ void store_fp8(const Fp8Regs& r, uint8_t* tile, uint8_t* sc) {
  const int t = threadIdx.x;
  const int c = t & 7;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int row = (t >> 3) + 32 * i;
    *(i32x4*)(tile + lds_chunk(row, c)) = r.d[i];
  }
#pragma unroll
  for (int b = 0; b < 4; ++b) sc[lds_scale(t, b)] = (uint8_t)(r.sc >> (8 * b));
}

// bf16 token tile for the fused prologue: thread t moves 16 chunks of 16
// bytes (8 elements), chunk c = t % 16 of rows t/16 + 16 j. Lanes 4g..4g+3 of
// a row's 16 hold 32-group g of the step, i.e. one DPP quad.
struct Bf16Regs {
  i32x4 d[16];
};

template <bool KTAIL>
__device__ __forceinline__ void load_bf16(Bf16Regs& r, __amdgpu_buffer_rsrc_t x, int K, int ks) {
  const int t = threadIdx.x;
  const int c = t & 15;
  const int kk = ks * BK + c * 8;  // element index
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const int row = (t >> 4) + 16 * j;
    r.d[j] = __builtin_amdgcn_raw_buffer_load_b128(x, (row * K + kk) * 2, 0, 0);
    if (KTAIL && kk >= K) r.d[j] = i32x4{0, 0, 0, 0};
  }
}

template <bool KTAIL>
__device__ __forceinline__ void quantize_store_bf16(const Bf16Regs& r, uint8_t* tile, uint8_t* sc, int K, int ks) {
  const int t = threadIdx.x;
  const int c = t & 15;
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const int row = (t >> 4) + 16 * j;
    uint32_t v[4] = {(uint32_t)r.d[j][0], (uint32_t)r.d[j][1], (uint32_t)r.d[j][2], (uint32_t)r.d[j][3]};
    uint32_t codes[2], s;
    quantize8_bf16(v, codes, s);
    *(i32x2*)(tile + lds_chunk(row, c >> 1) + (c & 1) * 8) = i32x2{(int)codes[0], (int)codes[1]};
    if ((c & 3) == 0) {
      if (KTAIL && ks * BK + c * 8 >= K) s = 127;
      sc[lds_scale(row, c >> 2)] = (uint8_t)s;
    }
  }
}

// ---------------------------------------------------------------------------
// One K step on the MFMAs: wave (wn, wm) multiplies its 128 weight rows by its
// 128 tokens.
__device__ __forceinline__ i32x8 read_frag(const uint8_t* tile, int row, int G) {
  const i32x4 lo = *(const i32x4*)(tile + lds_chunk(row, G));
  const i32x4 hi = *(const i32x4*)(tile + lds_chunk(row, 4 + G));
  return i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

__device__ __forceinline__ void mma_step(f32x4 (&acc)[8][8], const uint8_t* sW, const uint8_t* sX,
                                         const uint8_t* sWs, const uint8_t* sXs, int wn, int wm) {
  const int lane = threadIdx.x & 63;
  const int G = lane >> 4, r16 = lane & 15;
  i32x8 bx[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) bx[j] = read_frag(sX, wm * 128 + 16 * j + r16, G);
  const i32x2 sw = *(const i32x2*)(sWs + G * 256 + wn * 128 + r16 * 8);
  const i32x2 sx = *(const i32x2*)(sXs + G * 256 + wm * 128 + r16 * 8);
  static_for<0, 8>([&](auto I) {
    constexpr int i = decltype(I)::value;
    const i32x8 aw = read_frag(sW, wn * 128 + 16 * i + r16, G);
    static_for<0, 8>([&](auto J) {
      constexpr int j = decltype(J)::value;
      acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(aw, bx[j], acc[i][j], 0, 0, i & 3, sw[i >> 2],
                                                                  j & 3, sx[j >> 2]);
    });
  });
}

template <bool FUSED, bool KTAIL, int EPI>
__global__ __launch_bounds__(NT, 1) void linear_kernel(Params p) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  uint8_t* sW = smem;                       // [2][TILE_BYTES]
  uint8_t* sX = smem + 2 * TILE_BYTES;      // [2][TILE_BYTES]
  uint8_t* sWs = smem + 4 * TILE_BYTES;     // [2][SCALE_BYTES]
  uint8_t* sXs = sWs + 2 * SCALE_BYTES;     // [2][SCALE_BYTES]

  int tm, tn;
  tile_coords(blockIdx.x, p.tiles_m, p.tiles_n, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;
  const int K = p.K;
  const int G32 = K >> 5;
  const int nk = (K + BK - 1) / BK;
  // Rows of this tile that exist (> 0). Resources cover exactly those rows,
  // so everything past them reads as zero and is never written. K, N <= 2^20
  // keeps every byte offset below 2^30.
  const int rows_m = min(p.M - m0, BM);
  const int rows_n = min(p.N - n0, BN);
  const __amdgpu_buffer_rsrc_t rw = make_rsrc(p.wq + (size_t)n0 * K, (uint32_t)(rows_n * K));
  const __amdgpu_buffer_rsrc_t rws = make_rsrc(p.ws + (size_t)n0 * G32, (uint32_t)(rows_n * G32));
  __amdgpu_buffer_rsrc_t rx, rxs;
  if (FUSED) {
    rx = make_rsrc(p.x + (size_t)m0 * K * 2, (uint32_t)(rows_m * K * 2));
    rxs = rx;
  } else {
    rx = make_rsrc(p.x + (size_t)m0 * K, (uint32_t)(rows_m * K));
    rxs = make_rsrc(p.xs + (size_t)m0 * G32, (uint32_t)(rows_m * G32));
  }

  const int wave = threadIdx.x >> 6;
  const int wn = wave >> 1, wm = wave & 1;
  const int lane = threadIdx.x & 63;
  const int G = lane >> 4, r16 = lane & 15;

  // Accumulators start at the bias (bias + K sum in fp32, as every GEMM
  // kernel here computes it); lane holds n = 16 i + 4 G + r of its wave tile.
  f32x4 acc[8][8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int nl = wn * 128 + 16 * i + 4 * G;
    f32x4 b = {0.f, 0.f, 0.f, 0.f};
    if (p.bias != nullptr && nl < rows_n) {
      const uint16_t* bp = p.bias + n0 + nl;
#pragma unroll
      for (int r = 0; r < 4; ++r) b[r] = (float)__builtin_bit_cast(_Float16, bp[r]);
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[i][j] = b;
  }

  Fp8Regs wr;
  Fp8Regs xr8;
  Bf16Regs xr16;

  // Prologue: stage 0.
  load_fp8<KTAIL>(wr, rw, rws, K, 0);
  if (FUSED) load_bf16<KTAIL>(xr16, rx, K, 0);
  else load_fp8<KTAIL>(xr8, rx, rxs, K, 0);
  store_fp8(wr, sW, sWs);
  if (FUSED) quantize_store_bf16<KTAIL>(xr16, sX, sXs, K, 0);
  else store_fp8(xr8, sX, sXs);
  __syncthreads();

  for (int ks = 0; ks < nk; ++ks) {
    const int cur = ks & 1;
    const bool more = ks + 1 < nk;
    if (more) {
      load_fp8<KTAIL>(wr, rw, rws, K, ks + 1);
      if (FUSED) load_bf16<KTAIL>(xr16, rx, K, ks + 1);
      else load_fp8<KTAIL>(xr8, rx, rxs, K, ks + 1);
    }
    mma_step(acc, sW + cur * TILE_BYTES, sX + cur * TILE_BYTES, sWs + cur * SCALE_BYTES, sXs + cur * SCALE_BYTES,
             wn, wm);
    if (more) {
      const int nxt = cur ^ 1;
      store_fp8(wr, sW + nxt * TILE_BYTES, sWs + nxt * SCALE_BYTES);
      if (FUSED) quantize_store_bf16<KTAIL>(xr16, sX + nxt * TILE_BYTES, sXs + nxt * SCALE_BYTES, K, ks + 1);
      else store_fp8(xr8, sX + nxt * TILE_BYTES, sXs + nxt * SCALE_BYTES);
    }
    __syncthreads();
  }

  // Epilogue: lane holds D[n = 16 i + 4 G + r][m = 16 j + l%16] of its wave tile.
  const int N = p.N;
  const __amdgpu_buffer_rsrc_t ry = make_rsrc(p.y + (size_t)m0 * N, (uint32_t)(rows_m * N * 2));
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int nl = wn * 128 + 16 * i + 4 * G;  // local n of element r = 0
    const bool n_ok = nl < rows_n;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int ml = wm * 128 + 16 * j + r16;
      float v[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) v[r] = epilogue<EPI>(acc[i][j][r]);
      const bf16x2 p0 = {(__bf16)v[0], (__bf16)v[1]};
      const bf16x2 p1 = {(__bf16)v[2], (__bf16)v[3]};
      const i32x2 out = {__builtin_bit_cast(int, p0), __builtin_bit_cast(int, p1)};
      const int off = n_ok ? (ml * N + n0 + nl) * 2 : kDropOffset;
      __builtin_amdgcn_raw_buffer_store_b64(out, ry, off, 0, 0);
    }
  }
}

// ===========================================================================
// Fast path for K % 128 == 0 (every Wan2.2 shape) on pre-quantized tokens.
//
// v_mfma_scale_f32_32x32x64_f8f6f4 (the faster of the two scaled shapes on
// gfx950: 96% of peak in isolation against 81-88% for 16x16x128); operand
// layout, confirmed on the device: lane l holds row l%32, K bytes
// [16*(l/32), +16) and [32 + 16*(l/32), +16) of the 64; the scale of lane l
// belongs to row l%32 and 32-block l/32. Output: lane l holds
// D[8*(e/4) + 4*(l/32) + e%4][l%32], e = 0..15.
//
// LDS rows are 128 B; a ds_read_b128 is served 16 lanes (256 B, all 64
// banks) at a time, and 16 lanes read 16 consecutive rows at one logical
// chunk, so chunk c of row r is stored at physical chunk c ^ ((r >> 1) & 7):
// rows of equal parity then land on 8 distinct 16-byte slots.
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void* lds_ptr;

// ===========================================================================
// Eight-wave pipeline. On this shape the CU's load path, not the matrix
// core, is the constraint: strided 128-byte row segments sustain about
// 36 B/clk per CU (64-byte segments only about 24), a 256 x 256 tile needs
// 32 B/clk at MFMA peak, and a wave whose load instruction finds the
// address FIFO full stops issuing, MFMAs included. So:
//
//   * stages hold whole 128-byte row segments (two stages of 128 K, 132 KB);
//   * 8 waves, two per SIMD; each owns a 128 (n) x 64 (m) sub-tile
//     (128 accumulator registers);
//   * only waves 0..3 (one per SIMD) issue the stage refills, right after
//     the barrier that frees the stage; while one of them waits on the
//     address FIFO its SIMD sibling keeps the matrix core busy;
//   * one barrier per 128-K step; within a step the fragments of the second
//     64-K half are read while the first half's MFMAs run.
//
// LDS per stage: codes of both operands (256 rows x 128 B, chunk c of row r
// at c ^ ((r >> 1) & 7)), then scales as row-major dwords (4 groups per row),
// read back one byte per fragment.
namespace pp {

constexpr int NT8 = 512;
constexpr int OFF_W = 0, OFF_X = 32768, OFF_WS = 65536, OFF_XS = 66560;
constexpr int STAGE = 67584;
constexpr int LDS = 2 * STAGE;

struct Frags {
  i32x8 a[4];  // weights: rows wn*128 + 32 f + l%32
  i32x8 b[2];  // tokens:  rows wm*64 + 32 f + l%32
  int sa[4];
  int sb[2];
};

struct Src {
  __amdgpu_buffer_rsrc_t w, x, ws, xs;
  int K, G32;
  int voff, voff1;  // lane part of code DMA offsets for even / odd 8-row blocks
  int soff;         // lane part of a scale DMA offset (row L)
};

// Stage refill for K step kk (waves 0..3 only): wave w moves the 8-row
// blocks 8w..8w+7 of both operands (1 KB each) and 64 rows of scales each.
__device__ __forceinline__ void issue_stage(const Src& S, uint8_t* st, int kk, bool valid, int wave) {
  const int dbase = valid ? kk * 128 : kDropOffset;
  const int sbase = valid ? kk * 4 : kDropOffset;
  const int so = 64 * wave * S.G32 + sbase;
  __builtin_amdgcn_raw_ptr_buffer_load_lds(S.ws, (lds_ptr)(st + OFF_WS + wave * 256), 4, S.soff, so, 0, 0);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(S.xs, (lds_ptr)(st + OFF_XS + wave * 256), 4, S.soff, so, 0, 0);
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    const int q = wave * 8 + u;
    const int soff = 8 * q * S.K + dbase;
    const int vo = (u & 1) ? S.voff1 : S.voff;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(S.w, (lds_ptr)(st + OFF_W + q * 1024), 16, vo, soff, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(S.x, (lds_ptr)(st + OFF_X + q * 1024), 16, vo, soff, 0, 0);
  }
}

// Fragments of 64-K half h of a stage.
__device__ __forceinline__ void read_frags(Frags& F, const uint8_t* st, int wn, int wm, int h, int lane) {
  const int r32 = lane & 31, hi = lane >> 5;
  const int sw = (r32 >> 1) & 7;
  const int c0 = ((4 * h + hi) ^ sw) << 4, c1 = ((4 * h + 2 + hi) ^ sw) << 4;
  const int g = 2 * h + hi;
#pragma unroll
  for (int f = 0; f < 4; ++f) {
    const uint8_t* ra = st + OFF_W + (wn * 128 + 32 * f + r32) * 128;
    const i32x4 a0 = *(const i32x4*)(ra + c0), a1 = *(const i32x4*)(ra + c1);
    F.a[f] = i32x8{a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
    F.sa[f] = st[OFF_WS + (wn * 128 + 32 * f + r32) * 4 + g];
  }
#pragma unroll
  for (int f = 0; f < 2; ++f) {
    const uint8_t* rb = st + OFF_X + (wm * 64 + 32 * f + r32) * 128;
    const i32x4 b0 = *(const i32x4*)(rb + c0), b1 = *(const i32x4*)(rb + c1);
    F.b[f] = i32x8{b0[0], b0[1], b0[2], b0[3], b1[0], b1[1], b1[2], b1[3]};
    F.sb[f] = st[OFF_XS + (wm * 64 + 32 * f + r32) * 4 + g];
  }
}

__device__ __forceinline__ void mma8(f32x16 (&acc)[4][2], const Frags& F) {
  static_for<0, 4>([&](auto I) {
    constexpr int i = decltype(I)::value;
    static_for<0, 2>([&](auto J) {
      constexpr int j = decltype(J)::value;
      acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(F.a[i], F.b[j], acc[i][j], 0, 0, 0, F.sa[i], 0, F.sb[j]);
    });
  });
}

// Output of a wave's 128 (n) x 32 MF (m) tile: bias, epilogue and bf16
// rounding into LDS staging ([m][n] bf16, rows of 256 B, 8-byte block nb of
// row m at nb ^ (m & 31), so 32 lanes writing 32 consecutive rows hit 32
// distinct bank pairs), then 4 rows x 256 B per store instruction (16 bytes
// per lane) with non-temporal stores: whole 128-byte lines, no partial-line
// writebacks.
// PC (per-channel FP8): each accumulator is first multiplied by its token
// row's and weight row's f32 scales, read from the LDS table `tab`
// ([0, 256) weight rows of the tile, [256, 512) token rows).
template <int EPI, int MF = 2, bool PC = false, bool BIAS_IN_ACC = false>
__device__ __forceinline__ void store_tile8(const f32x16 (&acc)[4][MF], const BiasQuads& B, const Params& p,
                                            uint8_t* ep, int m0, int n0, int rows_m, int rows_n, int wn, int wm,
                                            int lane, const float* tab = nullptr) {
  const int r32 = lane & 31, hi = lane >> 5;
  // Per-channel output: the lane's token-row scales are read once, ahead of
  // the staging writes (read between them, each read waited out its own LDS
  // latency).
  float sx[MF];
  if constexpr (PC) {
#pragma unroll
    for (int j = 0; j < MF; ++j) sx[j] = tab[256 + wm * 32 * MF + 32 * j + r32];
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int nb = 8 * i + 2 * q + hi;
      float b[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) b[r] = BIAS_IN_ACC ? 0.f : bias_at(B, 4 * i + q, r);
      f32x4 swq = {1.f, 1.f, 1.f, 1.f};
      if constexpr (PC) swq = *(const f32x4*)(tab + wn * 128 + 4 * nb);
#pragma unroll
      for (int j = 0; j < MF; ++j) {
        const int m = 32 * j + r32;
        float v[4];
        if constexpr (PC) {
          const float sxm = sx[j];
#pragma unroll
          for (int r = 0; r < 4; ++r) v[r] = epilogue<EPI>(acc[i][j][4 * q + r] * (sxm * swq[r]) + b[r]);
        } else if constexpr (BIAS_IN_ACC) {
#pragma unroll
          for (int r = 0; r < 4; ++r) v[r] = epilogue<EPI>(acc[i][j][4 * q + r]);
        } else {
#pragma unroll
          for (int r = 0; r < 4; ++r) v[r] = epilogue<EPI>(acc[i][j][4 * q + r] + b[r]);
        }
        const bf16x2 p0 = {(__bf16)v[0], (__bf16)v[1]};
        const bf16x2 p1 = {(__bf16)v[2], (__bf16)v[3]};
        *(i32x2*)(ep + m * 256 + ((nb ^ (m & 31)) << 3)) =
            i32x2{__builtin_bit_cast(int, p0), __builtin_bit_cast(int, p1)};
      }
    }
  }
  // The staging rows pass data between lanes. Seen from one lane, the reads
  // below touch addresses it never wrote, so without this barrier the
  // compiler may move them above the other lanes' writes (it did, in an
  // eight-pass variant); the hardware keeps LDS order within a wave.
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  const int N = p.N;
  const __amdgpu_buffer_rsrc_t ry = make_rsrc(p.y + (size_t)m0 * N, (uint32_t)(rows_m * N * 2));
  // 16 bytes (8 values) per lane, 4 rows per store: blocks 2c and 2c + 1 of
  // row m sit at (2c) ^ s and (2c + 1) ^ s, s = m & 31: one aligned 16-byte
  // pair, its halves swapped when s is odd.
  const int c = lane & 15;
  const int nl = wn * 128 + 8 * c;
  const bool n_ok = nl < rows_n;
#pragma unroll 8
  for (int it = 0; it < 8 * MF; ++it) {
    const int m = 4 * it + (lane >> 4);
    const int sw = m & 31;
    const i32x4 v = *(const i32x4*)(ep + m * 256 + ((((2 * c) ^ sw) & ~1) << 3));
    const bool odd = sw & 1;
    const i32x4 w = odd ? i32x4{v[2], v[3], v[0], v[1]} : v;
    const int off = n_ok ? ((wm * 32 * MF + m) * N + n0 + nl) * 2 : kDropOffset;
    __builtin_amdgcn_raw_buffer_store_b128(w, ry, off, 0, kStoreAux);
  }
}

template <int EPI>
__global__ __launch_bounds__(NT8, 1) void linear_prequant_pp(Params p) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  int tm, tn;
  tile_coords(blockIdx.x, p.tiles_m, p.tiles_n, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;
  const int K = p.K, G32 = K >> 5, nk = K / 128;
  const int rows_m = min(p.M - m0, BM);
  const int rows_n = min(p.N - n0, BN);
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wn = wave & 1, wm = wave >> 1;
  const bool loader = wave < 4;

  Src S;
  S.w = make_rsrc(p.wq + (size_t)n0 * K, (uint32_t)(rows_n * K));
  S.ws = make_rsrc(p.ws + (size_t)n0 * G32, (uint32_t)(rows_n * G32));
  S.x = make_rsrc(p.x + (size_t)m0 * K, (uint32_t)(rows_m * K));
  S.xs = make_rsrc(p.xs + (size_t)m0 * G32, (uint32_t)(rows_m * G32));
  S.K = K;
  S.G32 = G32;
  S.voff = (lane >> 3) * K + (((lane & 7) ^ (lane >> 4)) << 4);
  S.voff1 = (lane >> 3) * K + (((lane & 7) ^ ((4 + (lane >> 4)) & 7)) << 4);
  S.soff = lane * G32;

  // Accumulators start at the bias (an output is bias + its K sum in fp32,
  // the order of the slab kernel, so the two layouts give identical bits).
  BiasQuads B;
  load_bias_quads(B, p, n0, rows_n, wn, lane);
  if (loader) issue_stage(S, smem, 0, true, wave);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  f32x16 acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float b = bias_at(B, 4 * i + q, r);
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j][4 * q + r] = b;
      }

  for (int k = 0; k < nk; ++k) {
    uint8_t* cur = smem + (k & 1) * STAGE;
    uint8_t* nxt = smem + ((k + 1) & 1) * STAGE;
    // This wave's refill of step k has landed and every wave is done with
    // the other stage (last read in step k-1): publish, then refill it.
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    if (loader) issue_stage(S, nxt, k + 1, k + 1 < nk, wave);
    __builtin_amdgcn_sched_barrier(0);
    Frags F0, F1;
    read_frags(F0, cur, wn, wm, 0, lane);
    read_frags(F1, cur, wn, wm, 1, lane);
    mma8(acc, F0);
    mma8(acc, F1);
  }
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_barrier();
  store_tile8<EPI, 2, false, true>(acc, B, p, smem + wave * 16384, m0, n0, rows_m, rows_n, wn, wm, lane);
}

template <int EPI>
hipError_t launch(const Params& p, int nwg, hipStream_t st) {
  static bool configured = false;  // per instantiation; benign race (idempotent)
  auto kern = linear_prequant_pp<EPI>;
  if (!configured) {
    hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, LDS);
    if (e != hipSuccess) return e;
    configured = true;
  }
  hipLaunchKernelGGL(kern, dim3(nwg), dim3(NT8), LDS, st, p);
  return hipGetLastError();
}

}  // namespace pp

// ---------------------------------------------------------------------------
// GEMM on the slab layout (see mx.h): operands as K-slabs of 64, codes
// [K/64][R][64] and scales [K/64][R][2] with R the row count rounded up to
// 256, so one tile's share of a slab is one contiguous run (16 KB of codes,
// 512 B of scales) instead of 256 row pieces 5 KB apart. This halves the
// cache-line requests per byte (the row-major scales alone cost as many line
// lookups as all the codes) and lets the loads stream from whole lines.
//
// Four waves of 128 (n) x 128 (m), one per SIMD, 256 accumulators each in
// AGPRs. Per 64-K half-step a wave reads 256 fragment rows (4 A + 4 B) for
// 16 MFMAs: 1 KB of LDS per MFMA, against 1.5 KB for eight 128 x 64 waves,
// so the CU's LDS traffic per half-step is 97 KB (64 KB of reads, 33 KB of
// DMA writes) instead of 129 KB, which also lowers power and so raises the
// clock a little. K advances through a ring of 4 LDS regions; each wave
// issues a quarter of the refill of half-step j+4 in half-step j, so a load
// has three half-steps to land and about 100 KB per CU are in flight:
//
//   half-step j:  wait for this wave's loads of j+1, barrier;
//                 16 MFMAs on the fragments of j (registers), with the LDS
//                 reads of the fragments of j+1 (region (j+1) % 4) and then
//                 the loads of j+4 into region j % 4 between them.
//
// Region layout: weight codes 256 rows x 64 B, 16-byte chunk c of row r at
// slot c ^ ((r >> 2) & 3) (conflict-free for 16-lane phases of b128 reads);
// token codes the same. The block scales of both operands sit in a ring of
// their own past the four regions (below). Loads past the last half-step use
// an empty resource and write zeros that nobody reads.
namespace slab {

constexpr int NT4 = 256;
constexpr int R_W = 0, R_X = 16384;
constexpr int REGION = 32768;  // codes of one half-step: 256 rows x 64 B, both operands
constexpr int LDS = 4 * REGION;
// Scale ring past the code regions: [weights, tokens][8 half-steps][256
// rows][2 groups], 512 bytes per operand and half-step. The scales of two
// consecutive half-steps (an even one and the next) sit side by side, so one
// 1 KB DMA fetches both: one scale DMA per wave every other half-step
// instead of one every half-step (each DMA instruction costs about the same
// whatever its size, and the scales are 3% of the bytes).
constexpr int SR = LDS;
constexpr int SR_OP = 8 * 512;

// Tile shapes. The tile is 256 weight rows x 64 JB tokens: four waves of 128
// (n) x 32 JB (m), each holding 4 x JB accumulator blocks of 32 x 32. JB = 4
// (256 x 256 tiles) is the GEMM of every large shape; JB = 2 (256 x 128)
// doubles the tile count for a few hundred tokens, where the 256 x 256 tiles
// would leave most CUs idle (the 512-token linear: 80 tiles on 256 CUs),
// without the partial sums of a K split. Both use the same LDS layout (the
// token half of each region only partly filled when JB = 2).
template <int JB>
struct Shape {
  static constexpr int MT = 64 * JB;           // tokens per tile
  static constexpr int CODE_LOADS = 4 + JB;    // code DMAs of 1 KB per wave and half-step
  static constexpr int NMFMA = 4 * JB;         // MFMAs per wave and half-step
  static constexpr int NCODE = 8 + 2 * JB;     // 16-byte code reads per wave and half-step
  static constexpr int NREAD = NCODE + 4 + JB;  // and the scale bytes
};

struct Src {
  const uint8_t* w;  // tile origin in slab 0: codes, then scales
  const uint8_t* x;
  const uint8_t* ws;
  const uint8_t* xs;
  uint64_t w_slab, x_slab;  // bytes between consecutive code slabs
  int nh;                   // half-steps (K / 64)
  int voff;                 // lane part of a code DMA offset
};

// Code loads of half-step j by wave `wave` (0..3): 16-row weight blocks
// 4 wave .. 4 wave + 3 and token blocks JB wave .. JB wave + JB - 1 (1 KB
// each; lane L takes row L/4, global chunk (L%4) ^ (L/16) into LDS slot L%4),
// in the order of the loop's load pieces.
template <int JB>
__device__ __forceinline__ void issue_codes(const Src& S, uint8_t* smem, int j, int wave) {
  uint8_t* reg = smem + (j & 3) * REGION;
  const uint32_t nc = j < S.nh ? 16384u : 0u;
  const __amdgpu_buffer_rsrc_t rw = make_rsrc(S.w + (uint64_t)j * S.w_slab, nc);
  const __amdgpu_buffer_rsrc_t rx = make_rsrc(S.x + (uint64_t)j * S.x_slab, JB == 4 ? nc : nc / 4 * JB);
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int q = wave * 4 + u;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rw, (lds_ptr)(reg + R_W + q * 1024), 16, S.voff, q * 1024, 0, 0);
    if (u < JB) {
      const int qx = wave * JB + u;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, (lds_ptr)(reg + R_X + qx * 1024), 16, S.voff, qx * 1024, 0, 0);
    }
  }
}

// Scales of half-steps s and s + 1 (s even) of one operand into ring slots
// s % 8 and s % 8 + 1: lanes 0..31 take half-step s's 512 bytes, lanes
// 32..63 half-step s + 1's (the next scale slab, `stride` bytes on). Waves 0
// and 1 both copy the weight scales, waves 2 and 3 the token scales (the
// same bytes to the same place, so every wave issues one DMA and all waves
// keep equal load counts). Half-steps past the range read zeros. With JB = 2
// a half-step's token scales are 256 bytes: lanes 0..15 and 32..47 fetch
// them, lanes 16..31 and 48..63 repeat those bytes into the slots' unused
// upper halves.
struct ScaleLoad {
  __amdgpu_buffer_rsrc_t r;
  uint8_t* dst;
  uint32_t voff;
};

template <int JB>
__device__ __forceinline__ ScaleLoad scale_res(const Src& S, uint8_t* smem, int s, int wave, int lane) {
  const bool wop = wave < 2;
  const uint32_t stride = (uint32_t)((wop ? S.w_slab : S.x_slab) >> 5);
  const uint32_t one = JB == 4 || wop ? 512u : 256u;  // bytes of one half-step
  const uint32_t n = s + 1 < S.nh ? stride + one : (s < S.nh ? one : 0u);
  ScaleLoad L;
  L.r = make_rsrc((wop ? S.ws : S.xs) + (uint64_t)s * stride, n);
  L.dst = smem + SR + (wop ? 0 : SR_OP) + (s & 7) * 512;
  L.voff = (JB == 4 || wop ? (lane & 31) : (lane & 15)) * 16 + (lane >> 5) * stride;
  return L;
}

__device__ __forceinline__ void issue_scale_load(const ScaleLoad& L) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(L.r, (lds_ptr)L.dst, 16, L.voff, 0, 0, 0);
}

template <int JB>
__device__ __forceinline__ void issue_scales(const Src& S, uint8_t* smem, int s, int wave, int lane) {
  issue_scale_load(scale_res<JB>(S, smem, s, wave, lane));
}

// The prologue's loads in the order the loop would have issued them (the
// scales of half-steps 0, 1 and 2, 3 each before the codes of the first of
// the pair): the loop's waits count on that order.
template <bool PC, int JB>
__device__ __forceinline__ void issue_prologue(const Src& S, uint8_t* smem, int wave, int lane) {
  if constexpr (!PC) issue_scales<JB>(S, smem, 0, wave, lane);
  issue_codes<JB>(S, smem, 0, wave);
  issue_codes<JB>(S, smem, 1, wave);
  if constexpr (!PC) issue_scales<JB>(S, smem, 2, wave, lane);
  issue_codes<JB>(S, smem, 2, wave);
  issue_codes<JB>(S, smem, 3, wave);
}

template <int JB>
struct Frags {
  i32x8 a[4];   // weights: rows wn*128 + 32 f + l%32
  i32x8 b[JB];  // tokens:  rows wm*32*JB + 32 f + l%32
  int sa[4];
  int sb[JB];
};

// Fragments of a region for the 32x32x64 MFMA: lane l, fragment f reads row
// base + 32 f + l%32, K bytes [16 (l/32), +16) and [32 + 16 (l/32), +16) of
// the 64, and the scale of group l/32 of the half-step.
template <bool PC, int JB>
__device__ __forceinline__ void read_frags(Frags<JB>& F, const uint8_t* reg, int wn, int wm, int lane) {
  // reg is region 0 (the LDS base): half-step 0, scale ring slot 0.
  const int r32 = lane & 31, hi = lane >> 5;
  const int sw = (r32 >> 2) & 3;
  const int c0 = (hi ^ sw) << 4, c1 = ((2 + hi) ^ sw) << 4;
#pragma unroll
  for (int f = 0; f < 4; ++f) {
    const int row = wn * 128 + 32 * f + r32;
    const uint8_t* ra = reg + R_W + row * 64;
    const i32x4 a0 = *(const i32x4*)(ra + c0), a1 = *(const i32x4*)(ra + c1);
    F.a[f] = i32x8{a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
    F.sa[f] = PC ? 127 : reg[SR + row * 2 + hi];
  }
#pragma unroll
  for (int f = 0; f < JB; ++f) {
    const int row = wm * 32 * JB + 32 * f + r32;
    const uint8_t* rb = reg + R_X + row * 64;
    const i32x4 b0 = *(const i32x4*)(rb + c0), b1 = *(const i32x4*)(rb + c1);
    F.b[f] = i32x8{b0[0], b0[1], b0[2], b0[3], b1[0], b1[1], b1[2], b1[3]};
    F.sb[f] = PC ? 127 : reg[SR + SR_OP + row * 2 + hi];
  }
}

// Per-channel FP8 (PC) runs the same MFMAs with unit block scales (E8M0
// 127 = 2^0); its row scales are applied in the epilogue.
// MFMAs t = B .. E - 1 of a half-step (t = JB i + j: weight fragment i,
// token fragment j).
template <bool PC, int JB, int B, int E>
__device__ __forceinline__ void mma16(f32x16 (&acc)[4][JB], const Frags<JB>& F) {
  static_for<B, E>([&](auto T) {
    constexpr int i = decltype(T)::value / JB, j = decltype(T)::value % JB;
    if constexpr (PC)
      acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(F.a[i], F.b[j], acc[i][j], 0, 0, 0, 127, 0, 127);
    else
      acc[i][j] =
          __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(F.a[i], F.b[j], acc[i][j], 0, 0, 0, F.sa[i], 0, F.sb[j]);
  });
}

// Pieces of a half-step, for interleaving in program order. Read piece r
// (0 .. NREAD - 1): r < 4 JB a 16-byte code half of fragment r / 4 (of A
// for r % 4 < 2, else of B; r % 2 picks the half); 4 JB <= r < NCODE a half
// of A fragment JB + (r - 4 JB) / 2 (JB = 2 only); then the scale bytes, 4 of
// A and JB of B. Load piece d (0 .. CODE_LOADS - 1) one 1 KB code DMA: for
// JB = 4 weights for d even, tokens for d odd (block 4 wave + d / 2, resp.
// JB wave + d / 2); for JB = 2 weights, tokens, weights, tokens, weights,
// weights. The scale DMA (even half-steps) is scheduled apart.
struct FragAddr {
  const uint8_t* a;  // row wn*128 + l%32 of the weight codes
  const uint8_t* b;  // row wm*128 + l%32 of the token codes
  int c0, c1;        // swizzled byte offsets of the two 16-byte halves
  const uint8_t* sa;
  const uint8_t* sb;
};

// Addresses of half-step h's fragments: codes in region h % 4, scales in
// ring slot h % 8.
template <int JB>
__device__ __forceinline__ FragAddr frag_addr(const uint8_t* smem, int h, int wn, int wm, int lane) {
  const int r32 = lane & 31, hi = lane >> 5;
  const int sw = (r32 >> 2) & 3;
  const uint8_t* reg = smem + (h & 3) * REGION;
  const uint8_t* sc = smem + SR + (h & 7) * 512;
  FragAddr A;
  A.a = reg + R_W + (wn * 128 + r32) * 64;
  A.b = reg + R_X + (wm * 32 * JB + r32) * 64;
  A.c0 = (hi ^ sw) << 4;
  A.c1 = ((2 + hi) ^ sw) << 4;
  A.sa = sc + (wn * 128 + r32) * 2 + hi;
  A.sb = sc + SR_OP + (wm * 32 * JB + r32) * 2 + hi;
  return A;
}

template <int R, int JB>
__device__ __forceinline__ void read_piece(Frags<JB>& F, const FragAddr& A) {
  constexpr int NC = Shape<JB>::NCODE;
  if constexpr (R < NC) {
    // Fragment f of A (part 0, 1) or of B (part 2, 3); part % 2: the half.
    constexpr int f = R < 4 * JB ? R / 4 : JB + (R - 4 * JB) / 2;
    constexpr int part = R < 4 * JB ? R % 4 : (R - 4 * JB) % 2;
    const uint8_t* base = (part < 2 ? A.a : A.b) + 32 * f * 64;
    const i32x4 v = *(const i32x4*)(base + ((part & 1) ? A.c1 : A.c0));
    i32x8& d = part < 2 ? F.a[f] : F.b[f < JB ? f : 0];
    if constexpr ((part & 1) == 0) {
      d[0] = v[0]; d[1] = v[1]; d[2] = v[2]; d[3] = v[3];
    } else {
      d[4] = v[0]; d[5] = v[1]; d[6] = v[2]; d[7] = v[3];
    }
  } else if constexpr (R < NC + 4) {
    F.sa[R - NC] = A.sa[32 * (R - NC) * 2];
  } else {
    F.sb[R - NC - 4] = A.sb[32 * (R - NC - 4) * 2];
  }
}

struct LoadRes {
  __amdgpu_buffer_rsrc_t w, x;
  uint8_t* reg;
};

template <int JB>
__device__ __forceinline__ LoadRes load_res(const Src& S, uint8_t* smem, int j) {
  LoadRes L;
  L.reg = smem + (j & 3) * REGION;
  const uint32_t nc = j < S.nh ? 16384u : 0u;
  L.w = make_rsrc(S.w + (uint64_t)j * S.w_slab, nc);
  L.x = make_rsrc(S.x + (uint64_t)j * S.x_slab, JB == 4 ? nc : nc / 4 * JB);
  return L;
}

// Code piece D (0 .. CODE_LOADS - 1) of the refill of half-step j + 4.
template <int D, int JB>
__device__ __forceinline__ void load_piece(const LoadRes& L, const Src& S, int wave) {
  constexpr bool W = (D & 1) == 0 || D >= 2 * JB;  // a weight block, else a token block
  constexpr int u = D < 2 * JB ? D / 2 : D - JB;    // its index among the wave's blocks
  if constexpr (W) {
    const int q = wave * 4 + u;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(L.w, (lds_ptr)(L.reg + R_W + q * 1024), 16, S.voff, q * 1024, 0, 0);
  } else {
    const int q = wave * JB + u;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(L.x, (lds_ptr)(L.reg + R_X + q * 1024), 16, S.voff, q * 1024, 0, 0);
  }
}

// MFMAs of a half-step issued ahead of its wait and barrier, and the most
// set-up instructions scheduled behind each of them. Against none (the
// set-up after the barrier): one 0.9% slower, two 1.8% faster, three and
// four 2.4-4.3% faster on the Wan shapes, five and six a little below
// three.
constexpr int PRE_MFMAS = 3;
constexpr int SETUP_PER_MFMA = 11;

// Reads and loads issued in slot i, the i-th MFMA after the barrier (0 ..
// 15 - PRE_MFMAS): reads 12i/5 .. 12(i+1)/5 - 1 in slots 0..9 (24 reads, the
// fragments the next half-step's first MFMAs need first), none after, and
// one DMA in each of slots 0..8 (the scale DMA first, on even half-steps),
// so the refill of j+4 leaves early and has the most time to land.
// Finishing the reads six MFMAs (about 380 cycles) before the next
// half-step's lgkmcnt(0) lets them complete before it, so the MFMA pipe
// does not drain there: 2% faster than spreading them over every slot
// (reads over 8, 12 or 14 of 16 slots: within 1% of 10; over 9, 11 or 13
// slots with three MFMAs ahead of the barrier: the same or slower). Placing
// the DMAs in every other slot, in the middle slots or one slot later
// measured the same within 1%. Slot i issues the DMAs [d0, d1) of the list
// (the scale DMA, then the code pieces 0, 1, ...): for JB = 4 one in each of
// slots 0..8; for JB = 2 (8 MFMAs, 5 slots after the barrier) the 18 reads
// in slots 0..3 and the 7 DMAs spread over slots 0..4.
template <int I, int JB>
struct Slot {
  static constexpr int NS = JB == 4 ? 10 : 4;  // slots holding reads
  static constexpr int NR = Shape<JB>::NREAD;
  static constexpr int r0 = I < NS ? NR * I / NS : NR, r1 = I < NS ? NR * (I + 1) / NS : NR;  // reads [r0, r1)
  static constexpr int ND = Shape<JB>::CODE_LOADS + 1;  // DMAs in the list
  static constexpr int DS = JB == 4 ? ND : 5;            // slots holding DMAs
  static constexpr int d0 = JB == 4 ? (I < ND ? I : ND) : (I < DS ? ND * I / DS : ND);
  static constexpr int d1 = JB == 4 ? (I < ND ? I + 1 : ND) : (I < DS ? ND * (I + 1) / DS : ND);
};

// Per-channel FP8 has no block scales: the scale read pieces and the scale
// DMA drop out; the other pieces keep their slots. Loads a wave has issued
// after half-step h + 1's codes, at the top of half-step h: those of
// half-steps h - 2 and h - 1, one of them even (2 x CODE_LOADS codes + 1
// scale DMA).
template <bool PC, int JB>
constexpr int loads_two_halves() { return PC ? 2 * Shape<JB>::CODE_LOADS : 2 * Shape<JB>::CODE_LOADS + 1; }
template <bool PC, int R, int JB>
constexpr bool has_read() { return !PC || R < Shape<JB>::NCODE; }
template <bool PC, int I, int JB>
constexpr int slot_reads() {
  int n = 0;
  for (int r = Slot<I, JB>::r0; r < Slot<I, JB>::r1; ++r) n += (!PC || r < Shape<JB>::NCODE) ? 1 : 0;
  return n;
}
// DMA k of the list is issued on this half-step (the scale DMA only on even
// half-steps of the MX GEMM).
template <bool PC, bool EVEN, int K>
constexpr bool dma_on() { return K > 0 || (EVEN && !PC); }
template <bool PC, bool EVEN, int I, int JB>
constexpr int slot_dmas() {
  int n = 0;
  for (int k = Slot<I, JB>::d0; k < Slot<I, JB>::d1; ++k) n += (k > 0 || (EVEN && !PC)) ? 1 : 0;
  return n;
}

// Half-step j. The lgkmcnt(0) in the wait keeps any wave's refill from
// overtaking another wave's last reads of the region being refilled. The LDS
// reads of the next fragments (region (j+1) % 4) and the refill DMAs of
// half-step j+4 (region j % 4) are interleaved in program order, since the
// compiler keeps them in that order (it cannot tell the regions apart), and
// the scheduling groups put each slot's reads and DMA behind one MFMA: with
// one wave per SIMD, this is what keeps the MFMA pipe fed and the address
// path free of bursts. EVEN: j is even, and the scales of half-steps j + 4
// and j + 5 are fetched too (slot 0).
template <bool PC, bool EVEN, int JB>
__device__ __forceinline__ void half_step(f32x16 (&acc)[4][JB], Frags<JB>& cur, Frags<JB>& nxt, const Src& S,
                                          uint8_t* smem, int j, int wave, int wn, int wm, int lane) {
  constexpr int NM = Shape<JB>::NMFMA;
  __builtin_amdgcn_sched_barrier(0);
  // The first MFMAs read registers only: issued ahead of the wait and the
  // barrier, with the half-step's address set-up in their shadow, they keep
  // the MFMA pipe busy through the wait, the barrier and the set-up.
  const FragAddr A = frag_addr<JB>(smem, j + 1, wn, wm, lane);
  const LoadRes L = load_res<JB>(S, smem, j + 4);
  ScaleLoad SLd;
  if constexpr (EVEN && !PC) SLd = scale_res<JB>(S, smem, j + 4, wave, lane);
  mma16<PC, JB, 0, PRE_MFMAS>(acc, cur);
  static_for<0, PRE_MFMAS>([&](auto I) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
    __builtin_amdgcn_sched_group_barrier(0x006, SETUP_PER_MFMA, 0);  // set-up VALU / SALU
  });
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)" ::"n"(loads_two_halves<PC, JB>()) : "memory");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
  static_for<0, NM - PRE_MFMAS>([&](auto I) {
    constexpr int i = decltype(I)::value;
    using SL = Slot<i, JB>;
    static_for<SL::r0, SL::r1>([&](auto Rr) {
      constexpr int r = decltype(Rr)::value;
      if constexpr (has_read<PC, r, JB>()) read_piece<r, JB>(nxt, A);
    });
    static_for<SL::d0, SL::d1>([&](auto Dk) {
      constexpr int k = decltype(Dk)::value;
      if constexpr (k == 0) {
        if constexpr (dma_on<PC, EVEN, 0>()) issue_scale_load(SLd);
      } else {
        load_piece<k - 1, JB>(L, S, wave);
      }
    });
  });
  mma16<PC, JB, PRE_MFMAS, NM>(acc, cur);
  static_for<0, NM - PRE_MFMAS>([&](auto I) {
    constexpr int i = decltype(I)::value;
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
    if constexpr (slot_reads<PC, i, JB>() > 0)
      __builtin_amdgcn_sched_group_barrier(0x100, slot_reads<PC, i, JB>(), 0);
    if constexpr (slot_dmas<PC, EVEN, i, JB>() > 0)
      __builtin_amdgcn_sched_group_barrier(0x020, slot_dmas<PC, EVEN, i, JB>(), 0);  // its DMAs
  });
  __builtin_amdgcn_sched_barrier(0);
}

// Requantizing epilogue: instead of y, the MX quantization of y (bf16) in
// the slab layout, as the next linear takes it (K' = N; the FFN
// down-projection after the GELU up-projection). The accumulators already
// hold the bias. The wave's 128 x 128 bf16 results are staged in LDS as in
// the plain epilogue (8-byte block nb of row m at nb ^ (m & 31): 32 lanes on
// 32 consecutive rows write 32 distinct bank pairs; the earlier swizzle
// nb ^ ((m & 15) << 1) kept block pairs adjacent but was 2-way bank
// conflicted, 16 M conflict cycles per launch at 75348 x 5120 x 13824); then
// each lane reads 8 consecutive values of a row (one aligned 16-byte pair,
// its halves swapped back when the row's swizzle is odd), the 4 lanes of a
// DPP quad hold one group of 32, and quantize8_bf16 encodes them exactly as
// the quantizer does. 16 lanes cover a row's 128 values, i.e. two 64-wide
// K'-slabs; 4 rows per read make whole 256-byte runs in each slab. Rows past
// M are written as zero codes and scales (the slab's pad rows); columns past
// N are dropped.
template <int EPI>
__device__ __forceinline__ void store_tile_q(const f32x16 (&acc)[4][4], const Params& p, uint8_t* ep, int m0, int n0,
                                             int wn, int wm, int lane) {
  const int r32 = lane & 31, hi = lane >> 5;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int nb = 8 * i + 2 * q + hi;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int m = 32 * j + r32;
        float v[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) v[r] = epilogue<EPI>(acc[i][j][4 * q + r]);
        const bf16x2 p0 = {(__bf16)v[0], (__bf16)v[1]};
        const bf16x2 p1 = {(__bf16)v[2], (__bf16)v[3]};
        *(i32x2*)(ep + m * 256 + ((nb ^ (m & 31)) << 3)) =
            i32x2{__builtin_bit_cast(int, p0), __builtin_bit_cast(int, p1)};
      }
    }
  }
  // The staging rows pass data between lanes (see store_tile8).
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  const int RM = p.tiles_m * BM;
  const __amdgpu_buffer_rsrc_t rq = make_rsrc(p.hq, (uint32_t)((size_t)RM * p.N));
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(p.hs, (uint32_t)((size_t)RM * (p.N / 32)));
  const int c = lane & 15;
  const int ng = n0 + wn * 128 + 8 * c;  // K' index of this lane's first value
  const bool n_ok = ng < p.N;
  const int slab = ng >> 6;
  // Eight rows' staging reads are issued together before their codes are
  // computed (one read at a time left each waiting out the LDS latency), and
  // the pad-row check is compiled in only for a tile that reaches past M:
  // 1.5% off the GELU up-projection at 75348 x 5120 x 13824, same bytes.
  auto rows8 = [&](auto tail_c) {
    constexpr bool TAIL = decltype(tail_c)::value;
    for (int g = 0; g < 32; g += 8) {
      i32x4 vv[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int row = 4 * (g + u) + (lane >> 4);
        vv[u] = *(const i32x4*)(ep + row * 256 + ((((2 * c) ^ (row & 31)) & ~1) << 3));
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int row = 4 * (g + u) + (lane >> 4);
        const int mg = m0 + wm * 128 + row;
        i32x4 v = vv[u];
        if (row & 1) v = i32x4{v[2], v[3], v[0], v[1]};
        if (TAIL && mg >= p.M) v = i32x4{0, 0, 0, 0};
        const uint32_t raw[4] = {(uint32_t)v[0], (uint32_t)v[1], (uint32_t)v[2], (uint32_t)v[3]};
        uint32_t codes[2], sc;
        quantize8_bf16(raw, codes, sc);
        const int qo = n_ok ? slab * RM * 64 + mg * 64 + (ng & 63) : kDropOffset;
        __builtin_amdgcn_raw_buffer_store_b64(i32x2{(int)codes[0], (int)codes[1]}, rq, qo, 0, 0);
        if ((c & 3) == 0) {
          const int so = n_ok ? slab * RM * 2 + mg * 2 + ((c >> 2) & 1) : kDropOffset;
          __builtin_amdgcn_raw_buffer_store_b8((uint8_t)sc, rs, so, 0, 0);
        }
      }
    }
  };
  if (m0 + wm * 128 + 128 > p.M)
    rows8(std::integral_constant<bool, true>{});
  else
    rows8(std::integral_constant<bool, false>{});
}

// Split-K output: the wave's fp32 accumulators as they sit in registers,
// for the split-K reduction. Partial tile (ks, tile) holds 65536
// floats; 16-byte chunk c = (((wave * 4 + i) * 4 + j) * 4 + q) * 64 + lane is
// acc[i][j][4q .. 4q+3] of that lane: token m = m0 + 128 wm + 32 j + lane%32,
// weight rows n = n0 + 128 wn + 32 i + 8 q + 4 (lane/32) + 0..3. One store
// instruction writes 1 KB of consecutive bytes. Chunks of tokens past M are
// not written (the reduction skips them).
__device__ __forceinline__ void store_tile_part(const f32x16 (&acc)[4][4], const Params& p, int tile, int ks, int m0,
                                                int wave, int wm, int lane) {
  float* base = p.part + ((size_t)ks * p.part_tiles + tile) * 65536;
  const __amdgpu_buffer_rsrc_t rp = make_rsrc(base, 65536u * 4u);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const bool ok = m0 + wm * 128 + 32 * j + (lane & 31) < p.M;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int chunk = (((wave * 4 + i) * 4 + j) * 4 + q) * 64 + lane;
        // Copy the elements out first: a bit_cast of a vector-element lvalue
        // reads from the start of the vector (element 0) in this compiler.
        const f32x4 f = {acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]};
        const i32x4 v = __builtin_bit_cast(i32x4, f);
        __builtin_amdgcn_raw_buffer_store_b128(v, rp, ok ? chunk * 16 : kDropOffset, 0, 0);
      }
    }
  }
}

// Outputs: bf16 y; the requantized MX slab of y; split-K partial sums; bf16 y
// of the per-channel FP8 linear (unit block scales, row scales in the
// epilogue from a 2 KB LDS table past the ring: [0, 256) weight rows n0..,
// [256, 512) token rows m0..).
enum { OUT_Y = 0, OUT_Q = 1, OUT_PART = 2, OUT_PCY = 3 };
constexpr int PC_TABLE = SR + 2 * SR_OP;  // byte offset of the per-channel scale table
constexpr int LDS_PC = PC_TABLE + 2048;
// Bias: each wave copies the 128 f16 bias values of its weight-row half (wn)
// into its own 256-byte LDS slot past the ring and the per-channel table,
// with one 4-byte DMA per lane issued before the ring's first stages; waiting
// for that one load (the oldest) leaves the ring's loads in flight. The bf16
// and requantizing outputs then start their accumulators at the bias (an
// output is bias + its K sum, in fp32), which takes the bias adds out of the
// epilogue and puts the accumulator initialization inside the first stage's
// load latency; the per-channel output, whose bias follows the row scales,
// reads its slot in the epilogue. Before: the epilogue waited a memory round
// trip for the bias after the last MFMA (0.85 us of a 61 us tile at
// 75348 x 5120 x 15360). Without a bias the slot is zeroed with ordinary LDS
// writes. Columns past N (a ragged last weight tile) read whatever the DMA
// leaves there; their outputs are not stored.
constexpr int BIAS_TABLE = LDS_PC;
constexpr int LDS_OUT = LDS_PC + 4 * 256;

template <int OUT>
constexpr int lds_bytes() { return LDS_OUT; }

__device__ __forceinline__ void issue_bias_slot(const Params& p, uint8_t* smem, int n0, int rows_n, int wave, int wn,
                                                int lane) {
  uint8_t* slot = smem + BIAS_TABLE + wave * 256;
  if (p.bias != nullptr) {
    const __amdgpu_buffer_rsrc_t rb = make_rsrc(p.bias + n0, (uint32_t)rows_n * 2u);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (lds_ptr)slot, 4, lane * 4, wn * 256, 0, 0);
  } else {
    *(int*)(slot + lane * 4) = 0;
  }
}

// The wave's bias quads from its slot, in the layout load_bias_quads gives.
__device__ __forceinline__ void read_bias_quads(BiasQuads& B, const uint8_t* smem, int wave, int lane) {
  const uint8_t* base = smem + BIAS_TABLE + wave * 256 + 4 * (lane >> 5) * 2;
#pragma unroll
  for (int k = 0; k < 16; ++k) B.v[k] = *(const i32x2*)(base + (32 * (k >> 2) + 8 * (k & 3)) * 2);
}

template <int EPI, int OUT, int JB = 4>
__global__ __launch_bounds__(NT4, 1) void linear_slab_kernel(Params p) {
  static_assert(JB == 4 || (JB == 2 && OUT == OUT_Y), "128-token tiles have the bf16 output only");
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  constexpr bool PC = OUT == OUT_PCY;
  constexpr int MT = Shape<JB>::MT;
  constexpr int CL = Shape<JB>::CODE_LOADS;
  int tm, tn;
  int bid = blockIdx.x, ks = 0;
  if constexpr (OUT == OUT_PART) {
    ks = bid % p.splits;
    bid /= p.splits;  // the partial tile, numbered within this launch
  }
  tile_coords(p.tile_base + bid, p.tiles_m, p.tiles_n, tm, tn);
  const int m0 = tm * MT, n0 = tn * BN;
  const int rows_m = min(p.M - m0, MT);
  const int rows_n = min(p.N - n0, BN);
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wn = wave & 1, wm = wave >> 1;

  // K range of this workgroup: all K/64 half-steps, or split-K range ks.
  int h0 = 0, nh_wg = p.K >> 6;
  if constexpr (OUT == OUT_PART) {
    const int tot = nh_wg;
    h0 = ks * tot / p.splits;
    nh_wg = (ks + 1) * tot / p.splits - h0;
  }
  Src S;
  S.w_slab = (uint64_t)p.tiles_n * BN * 64;
  // Token slab rows: the slab layout's row count (a multiple of 256).
  S.x_slab = JB == 4 ? (uint64_t)p.tiles_m * BM * 64 : (uint64_t)((p.tiles_m * MT + 255) & ~255) * 64;
  S.w = p.wq + (size_t)n0 * 64 + h0 * S.w_slab;
  S.x = p.x + (size_t)m0 * 64 + h0 * S.x_slab;
  S.ws = PC ? nullptr : p.ws + (size_t)n0 * 2 + h0 * (S.w_slab >> 5);
  S.xs = PC ? nullptr : p.xs + (size_t)m0 * 2 + h0 * (S.x_slab >> 5);
  S.nh = nh_wg;
  S.voff = (lane >> 2) * 64 + (((lane & 3) ^ (lane >> 4)) << 4);

  f32x16 acc[4][JB];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < JB; ++j) acc[i][j] = f32x16{};

  constexpr bool BIAS_IN_ACC = OUT == OUT_Y || OUT == OUT_Q;
  if constexpr (OUT != OUT_PART) issue_bias_slot(p, smem, n0, rows_n, wave, wn, lane);
  issue_prologue<PC, JB>(S, smem, wave, lane);
  __builtin_amdgcn_sched_barrier(0);
  // Loads issued after the bias: 4 x CL codes (+ 2 scale DMAs); after
  // half-step 0's codes: 3 x CL codes (+ 1 scale DMA).
  constexpr int AFTER_BIAS = 4 * CL + (PC ? 0 : 2);
  constexpr int AFTER_H0 = 3 * CL + (PC ? 0 : 1);
  if constexpr (BIAS_IN_ACC) {
    asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)" ::"n"(AFTER_BIAS) : "memory");
    BiasQuads B0;
    read_bias_quads(B0, smem, wave, lane);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float b = bias_at(B0, 4 * i + q, r);
#pragma unroll
          for (int jj = 0; jj < JB; ++jj) acc[i][jj][4 * q + r] = b;
        }
    // Materialize the accumulators here, inside the first stage's latency
    // (left alone, the compiler moves their writes past the barrier below).
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int jj = 0; jj < JB; ++jj) asm volatile("" : "+a"(acc[i][jj]));
    __builtin_amdgcn_sched_barrier(0);
  }
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)" ::"n"(AFTER_H0) : "memory");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
  Frags<JB> F0, F1;
  read_frags<PC, JB>(F0, smem, wn, wm, lane);
  const int nh = S.nh;
  int j = 0;
  for (; j + 1 < nh; j += 2) {
    half_step<PC, true, JB>(acc, F0, F1, S, smem, j, wave, wn, wm, lane);
    half_step<PC, false, JB>(acc, F1, F0, S, smem, j + 1, wave, wn, wm, lane);
  }
  if (j < nh) half_step<PC, true, JB>(acc, F0, F1, S, smem, j, wave, wn, wm, lane);
  __builtin_amdgcn_sched_barrier(0);
  BiasQuads B;
  if constexpr (OUT == OUT_PCY) read_bias_quads(B, smem, wave, lane);
  float scw = 0.f, scx = 0.f;
  if constexpr (PC) {
    // One weight-row and one token-row scale per thread; zero past N and M.
    const __amdgpu_buffer_rsrc_t rw = make_rsrc(p.sw + n0, (uint32_t)rows_n * 4u);
    const __amdgpu_buffer_rsrc_t rx = make_rsrc(p.sx + m0, (uint32_t)rows_m * 4u);
    scw = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rw, threadIdx.x * 4, 0, 0));
    scx = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rx, threadIdx.x * 4, 0, 0));
  }
  asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
  if constexpr (PC) {
    float* tab = (float*)(smem + PC_TABLE);
    tab[threadIdx.x] = scw;
    tab[256 + threadIdx.x] = scx;
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  }
  __builtin_amdgcn_s_barrier();
  if constexpr (OUT == OUT_Q)
    store_tile_q<EPI>(acc, p, smem + wave * 32768, m0, n0, wn, wm, lane);
  else if constexpr (OUT == OUT_PART)
    store_tile_part(acc, p, bid, ks, m0, wave, wm, lane);
  else
    pp::store_tile8<EPI, JB, PC, BIAS_IN_ACC>(acc, B, p, smem + wave * 32768, m0, n0, rows_m, rows_n, wn, wm, lane,
                                              (const float*)(smem + PC_TABLE));
}

// Split-K reduction: one thread per 16-byte chunk of the partial tiles (the
// layout of store_tile_part), summing the splits in order 0, 1, ... (so the
// result does not depend on timing), then bias, epilogue and bf16 as the
// other kernels' epilogues do; 8 bytes of y per thread.
template <int EPI>
__global__ __launch_bounds__(256) void splitk_reduce_kernel(Params p) {
  const int64_t u = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t tiles = p.part_tiles;
  if (u >= tiles * 16384) return;
  const int lane = (int)(u & 63), q = (int)(u >> 6) & 3, j = (int)(u >> 8) & 3, i = (int)(u >> 10) & 3;
  const int wave = (int)(u >> 12) & 3;
  const int tile = (int)(u >> 14);
  int tm, tn;
  tile_coords(p.tile_base + tile, p.tiles_m, p.tiles_n, tm, tn);
  const int m = tm * BM + (wave >> 1) * 128 + 32 * j + (lane & 31);
  const int n = tn * BN + (wave & 1) * 128 + 32 * i + 8 * q + 4 * (lane >> 5);
  if (m >= p.M || n >= p.N) return;
  const float* src = p.part + (size_t)tile * 65536 + (size_t)(u & 16383) * 4;
  f32x4 s = *(const f32x4*)src;
  for (int k = 1; k < p.splits; ++k) {
    const f32x4 v = *(const f32x4*)(src + (size_t)k * tiles * 65536);
    s[0] += v[0];
    s[1] += v[1];
    s[2] += v[2];
    s[3] += v[3];
  }
  float b[4] = {0.f, 0.f, 0.f, 0.f};
  if (p.bias != nullptr) {
#pragma unroll
    for (int r = 0; r < 4; ++r) b[r] = (float)__builtin_bit_cast(_Float16, p.bias[n + r]);
  }
  float v[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) v[r] = epilogue<EPI>(s[r] + b[r]);
  const bf16x2 p0 = {(__bf16)v[0], (__bf16)v[1]};
  const bf16x2 p1 = {(__bf16)v[2], (__bf16)v[3]};
  *(i32x2*)(p.y + (size_t)m * p.N + n) = i32x2{__builtin_bit_cast(int, p0), __builtin_bit_cast(int, p1)};
}

template <int EPI, int OUT = OUT_Y, int JB = 4>
hipError_t launch(const Params& p, int nwg, hipStream_t st) {
  static bool configured = false;  // per instantiation; benign race (idempotent)
  auto kern = linear_slab_kernel<EPI, OUT, JB>;
  constexpr int lds = lds_bytes<OUT>();
  if (!configured) {
    hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
    if (e != hipSuccess) return e;
    configured = true;
  }
  hipLaunchKernelGGL(kern, dim3(nwg), dim3(NT4), lds, st, p);
  return hipGetLastError();
}

// Split-K over the launch's p.part_tiles tiles (from logical tile
// p.tile_base): partial sums, then the ordered reduction.
hipError_t launch_split(const Params& p, int epi, hipStream_t stream) {
  hipError_t e = launch<0, OUT_PART>(p, p.part_tiles * p.splits, stream);
  if (e != hipSuccess) return e;
  const int nred = (int)(((int64_t)p.part_tiles * 16384 + 255) / 256);
  if (epi == 1)
    hipLaunchKernelGGL(splitk_reduce_kernel<1>, dim3(nred), dim3(256), 0, stream, p);
  else
    hipLaunchKernelGGL(splitk_reduce_kernel<0>, dim3(nred), dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace slab

template <bool FUSED, bool KTAIL, int EPI>
hipError_t launch_variant(const Params& p, int nwg, hipStream_t st) {
  static bool configured = false;  // per instantiation; benign race (idempotent)
  auto kern = linear_kernel<FUSED, KTAIL, EPI>;
  if (!configured) {
    hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, LDS_BYTES);
    if (e != hipSuccess) return e;
    configured = true;
  }
  hipLaunchKernelGGL(kern, dim3(nwg), dim3(NT), LDS_BYTES, st, p);
  return hipGetLastError();
}

template <bool FUSED>
hipError_t dispatch_epi(const Params& p, bool ktail, int epi, int nwg, hipStream_t st) {
  if (ktail) {
    return epi == 1 ? launch_variant<FUSED, true, 1>(p, nwg, st) : launch_variant<FUSED, true, 0>(p, nwg, st);
  }
  return epi == 1 ? launch_variant<FUSED, false, 1>(p, nwg, st) : launch_variant<FUSED, false, 0>(p, nwg, st);
}

}  // namespace

hipError_t launch_linear(const void* x, const uint8_t* xs, int64_t M, int64_t K, const uint8_t* wq,
                         const uint8_t* ws, int64_t N, const void* bias, int epi, void* y, hipStream_t stream) {
  Params p;
  p.x = (const uint8_t*)x;
  p.xs = xs;
  p.wq = wq;
  p.ws = ws;
  p.bias = (const uint16_t*)bias;
  p.y = (uint16_t*)y;
  p.hq = nullptr;
  p.hs = nullptr;
  p.part = nullptr;
  p.sx = nullptr;
  p.sw = nullptr;
  p.splits = 1;
  p.tile_base = 0;
  p.part_tiles = 0;
  p.M = (int)M;
  p.N = (int)N;
  p.K = (int)K;
  p.tiles_m = (int)((M + BM - 1) / BM);
  p.tiles_n = (int)((N + BN - 1) / BN);
  const int nwg = p.tiles_m * p.tiles_n;
  const bool ktail = (K % BK) != 0;
  if (xs != nullptr && !ktail)
    return epi == 1 ? pp::launch<1>(p, nwg, stream) : pp::launch<0>(p, nwg, stream);
  return xs == nullptr ? dispatch_epi<true>(p, ktail, epi, nwg, stream)
                       : dispatch_epi<false>(p, ktail, epi, nwg, stream);
}

hipError_t launch_linear_slab(const uint8_t* xq, const uint8_t* xs, int64_t M, int64_t K, const uint8_t* wq,
                              const uint8_t* ws, int64_t N, const void* bias, int epi, void* y, hipStream_t stream) {
  Params p;
  p.x = xq;
  p.xs = xs;
  p.wq = wq;
  p.ws = ws;
  p.bias = (const uint16_t*)bias;
  p.y = (uint16_t*)y;
  p.hq = nullptr;
  p.hs = nullptr;
  p.part = nullptr;
  p.sx = nullptr;
  p.sw = nullptr;
  p.splits = 1;
  p.tile_base = 0;
  p.part_tiles = 0;
  p.M = (int)M;
  p.N = (int)N;
  p.K = (int)K;
  p.tiles_m = (int)((M + BM - 1) / BM);
  p.tiles_n = (int)((N + BN - 1) / BN);
  const int nwg = p.tiles_m * p.tiles_n;
  return epi == 1 ? slab::launch<1>(p, nwg, stream) : slab::launch<0>(p, nwg, stream);
}

hipError_t launch_linear_slab_m128(const uint8_t* xq, const uint8_t* xs, int64_t M, int64_t K, const uint8_t* wq,
                                   const uint8_t* ws, int64_t N, const void* bias, int epi, void* y,
                                   hipStream_t stream) {
  Params p;
  p.x = xq;
  p.xs = xs;
  p.wq = wq;
  p.ws = ws;
  p.bias = (const uint16_t*)bias;
  p.y = (uint16_t*)y;
  p.hq = nullptr;
  p.hs = nullptr;
  p.part = nullptr;
  p.sx = nullptr;
  p.sw = nullptr;
  p.splits = 1;
  p.tile_base = 0;
  p.part_tiles = 0;
  p.M = (int)M;
  p.N = (int)N;
  p.K = (int)K;
  p.tiles_m = (int)((M + 127) / 128);
  p.tiles_n = (int)((N + BN - 1) / BN);
  const int nwg = p.tiles_m * p.tiles_n;
  return epi == 1 ? slab::launch<1, slab::OUT_Y, 2>(p, nwg, stream) : slab::launch<0, slab::OUT_Y, 2>(p, nwg, stream);
}

hipError_t launch_linear_slab_requant(const uint8_t* xq, const uint8_t* xs, int64_t M, int64_t K, const uint8_t* wq,
                                      const uint8_t* ws, int64_t N, const void* bias, int epi, uint8_t* hq,
                                      uint8_t* hs, hipStream_t stream) {
  Params p;
  p.x = xq;
  p.xs = xs;
  p.wq = wq;
  p.ws = ws;
  p.bias = (const uint16_t*)bias;
  p.y = nullptr;
  p.hq = hq;
  p.hs = hs;
  p.part = nullptr;
  p.sx = nullptr;
  p.sw = nullptr;
  p.splits = 1;
  p.tile_base = 0;
  p.part_tiles = 0;
  p.M = (int)M;
  p.N = (int)N;
  p.K = (int)K;
  p.tiles_m = (int)((M + BM - 1) / BM);
  p.tiles_n = (int)((N + BN - 1) / BN);
  const int nwg = p.tiles_m * p.tiles_n;
  return epi == 1 ? slab::launch<1, slab::OUT_Q>(p, nwg, stream) : slab::launch<0, slab::OUT_Q>(p, nwg, stream);
}

hipError_t launch_linear_slab_splitk(const uint8_t* xq, const uint8_t* xs, int64_t M, int64_t K, const uint8_t* wq,
                                     const uint8_t* ws, int64_t N, const void* bias, int epi, void* y, int splits,
                                     float* part, hipStream_t stream) {
  // One range is the plain kernel itself (its accumulators start at the
  // bias; the split form adds the bias after the ranges).
  if (splits == 1) return launch_linear_slab(xq, xs, M, K, wq, ws, N, bias, epi, y, stream);
  Params p;
  p.x = xq;
  p.xs = xs;
  p.wq = wq;
  p.ws = ws;
  p.bias = (const uint16_t*)bias;
  p.y = (uint16_t*)y;
  p.hq = nullptr;
  p.hs = nullptr;
  p.part = part;
  p.sx = nullptr;
  p.sw = nullptr;
  p.splits = splits;
  p.M = (int)M;
  p.N = (int)N;
  p.K = (int)K;
  p.tiles_m = (int)((M + BM - 1) / BM);
  p.tiles_n = (int)((N + BN - 1) / BN);
  p.tile_base = 0;
  p.part_tiles = p.tiles_m * p.tiles_n;
  return slab::launch_split(p, epi, stream);
}

int64_t balanced_plan(int64_t M, int64_t K, int64_t N, int ncu, int64_t* full, int* splits) {
  const int64_t tiles = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
  const int64_t tail = tiles % ncu;
  int64_t s = tail > 0 ? ncu / tail : 1;
  s = std::min<int64_t>(s, kMaxTailSplits);
  s = std::min<int64_t>(s, (K / 64) / 2);
  if (s < 2) {  // nothing to balance: every tile data-parallel
    *full = tiles;
    *splits = 1;
    return 0;
  }
  *full = tiles - tail;
  *splits = (int)s;
  return s * tail * 65536 * 4;
}

hipError_t launch_linear_slab_balanced(const uint8_t* xq, const uint8_t* xs, int64_t M, int64_t K, const uint8_t* wq,
                                       const uint8_t* ws, int64_t N, const void* bias, int epi, void* y, int ncu,
                                       float* part, hipStream_t stream) {
  int64_t full;
  int splits;
  balanced_plan(M, K, N, ncu, &full, &splits);
  Params p;
  p.x = xq;
  p.xs = xs;
  p.wq = wq;
  p.ws = ws;
  p.bias = (const uint16_t*)bias;
  p.y = (uint16_t*)y;
  p.hq = nullptr;
  p.hs = nullptr;
  p.part = part;
  p.sx = nullptr;
  p.sw = nullptr;
  p.splits = 1;
  p.tile_base = 0;
  p.part_tiles = 0;
  p.M = (int)M;
  p.N = (int)N;
  p.K = (int)K;
  p.tiles_m = (int)((M + BM - 1) / BM);
  p.tiles_n = (int)((N + BN - 1) / BN);
  const int64_t tiles = (int64_t)p.tiles_m * p.tiles_n;
  if (full > 0) {
    hipError_t e = epi == 1 ? slab::launch<1>(p, (int)full, stream) : slab::launch<0>(p, (int)full, stream);
    if (e != hipSuccess || full == tiles) return e;
  }
  p.splits = splits;
  p.tile_base = (int)full;
  p.part_tiles = (int)(tiles - full);
  return slab::launch_split(p, epi, stream);
}

hipError_t launch_pc_linear_slab(const uint8_t* xq, const float* xs, int64_t M, int64_t K, const uint8_t* wq,
                                 const float* ws, int64_t N, const void* bias, int epi, void* y, hipStream_t stream) {
  Params p;
  p.x = xq;
  p.xs = nullptr;
  p.wq = wq;
  p.ws = nullptr;
  p.bias = (const uint16_t*)bias;
  p.y = (uint16_t*)y;
  p.hq = nullptr;
  p.hs = nullptr;
  p.part = nullptr;
  p.sx = xs;
  p.sw = ws;
  p.splits = 1;
  p.tile_base = 0;
  p.part_tiles = 0;
  p.M = (int)M;
  p.N = (int)N;
  p.K = (int)K;
  p.tiles_m = (int)((M + BM - 1) / BM);
  p.tiles_n = (int)((N + BN - 1) / BN);
  const int nwg = p.tiles_m * p.tiles_n;
  return epi == 1 ? slab::launch<1, slab::OUT_PCY>(p, nwg, stream) : slab::launch<0, slab::OUT_PCY>(p, nwg, stream);
}

}  // namespace mx
