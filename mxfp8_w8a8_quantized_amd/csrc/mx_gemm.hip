// MXFP8 W8A8 linear on CDNA4 block-scaled FP8 matrix cores.
//
//   y[m][n] = bf16_rne( epi( sum_k xhat[m][k] * what[n][k] + f32(bias[n]) ) )
//
// (model card "Wan2.2-I2V-A14B-Lightning · MXFP8 (AutoRound OptRTN)", section
// "Quantization Details": W8A8 MXFP8 linears, E4M3 with per-32 E8M0 scales,
// dynamic activations, F16 biases; FP32 accumulation as in the FP32-accum
// FP8 mode of "Model Quantization Techniques", Conv3D mode table.)
//
// Tiling: one 256-thread workgroup per 256 (weight rows n) x 256 (tokens m)
// output tile, K in steps of 128. Each of the 4 waves owns a 128 x 128
// sub-tile as 8 x 8 tiles of v_mfma_scale_f32_16x16x128_f8f6f4, whose
// A operand is the weights (so a lane's four accumulators are four
// consecutive n of one token m, stored as 8 contiguous bytes of y) and whose
// B operand is the tokens. The scales go straight into the MFMA: per lane
// one E8M0 byte for (its row, its 32-block), selected by op_sel from a dword.
//
// MFMA operand layout (16x16x128, 32 bytes per lane in two 16-byte halves):
// lane l holds row l%16, K bytes [16*(l/16), +16) in its first half and
// [64 + 16*(l/16), +16) in its second; the scale of lane l belongs to row
// l%16 and the 32-block l/16 (K [32b, 32b+32)). Block b is thus held by the
// lanes of groups 2(b%2) and 2(b%2)+1, in their first halves for b < 2 and
// second halves otherwise; with these halves read from memory K offsets
// 16*(l/16) and 64 + 16*(l/16), memory K maps to MFMA K one to one, so the
// scale of memory group b of the step is exactly what lane group b expects.
//
// LDS per stage: weights and tokens 256 x 128 code bytes each, rows of 128 B
// with the eight 16-byte chunks XOR-swizzled by (row & 7) so that 8
// consecutive rows read the same logical chunk from 8 different bank groups
// (the fast path below swizzles by (row >> 1) & 7 instead, see there);
// scales stored as [32-block b][row permuted] so that each lane reads the
// scales of its 8 MFMA tiles with one 8-byte load. Two stages (132 KB):
// global loads of step k+1 are in flight while step k runs on the MFMAs.
//
// Fused prologue (FUSED): the token tile arrives as bf16 (256 B per row per
// step), each lane holds 8 elements, a DPP quad holds a 32-group, and the
// quantized codes and scales are written to LDS in the same layout as the
// pre-quantized path.
//
// Ragged edges: buffer resources are rebased at the tile; rows past M (or N)
// load as zero and their stores are dropped.
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
#ifndef MX_STORE_AUX
#define MX_STORE_AUX 2
#endif
constexpr int kStoreAux = MX_STORE_AUX;  // cache policy of output stores (2: non-temporal)
#ifndef MX_LOAD_AUX
#define MX_LOAD_AUX 0
#endif
constexpr int kLoadAux = MX_LOAD_AUX;  // cache policy of the direct operand loads

struct Params {
  const uint8_t* x;   // bf16 tokens (fused) or E4M3 codes
  const uint8_t* xs;  // token scales (pre-quantized path)
  const uint8_t* wq;
  const uint8_t* ws;
  const uint16_t* bias;  // f16 bits, or null
  uint16_t* y;           // bf16 bits
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

// Workgroup -> (token tile, weight tile). Workgroups are dealt round-robin to
// the 8 XCDs, so first give each XCD a contiguous range of logical tiles, then
// walk that range in groups of GM token tiles x all weight tiles (token tile
// fastest), so that concurrent tiles on one XCD share token and weight panels
// in its L2.
__device__ inline void tile_coords(int pid, int tiles_m, int tiles_n, int& tm, int& tn) {
  constexpr int GM = 4;
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

// ---------------------------------------------------------------------------
template <int EPI>
__device__ __forceinline__ float epilogue(float v) {
  if (EPI == 1) {
    // GELU, tanh form, as v * sigmoid(2u) = 0.5 v (1 + tanh(u)),
    // u = sqrt(2/pi) (v + 0.044715 v^3); this form has no cancellation.
    const float u = 0.7978845608028654f * (v + 0.044715f * v * v * v);
    return v / (1.0f + __expf(-2.0f * u));
  }
  return v;
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

  f32x4 acc[8][8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

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
  const int lane = threadIdx.x & 63;
  const int G = lane >> 4, r16 = lane & 15;
  const int N = p.N;
  const __amdgpu_buffer_rsrc_t ry = make_rsrc(p.y + (size_t)m0 * N, (uint32_t)(rows_m * N * 2));
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int nl = wn * 128 + 16 * i + 4 * G;  // local n of element r = 0
    const bool n_ok = nl < rows_n;
    float b[4] = {0.f, 0.f, 0.f, 0.f};
    if (p.bias != nullptr && n_ok) {
      const uint16_t* bp = p.bias + n0 + nl;
#pragma unroll
      for (int r = 0; r < 4; ++r) b[r] = (float)__builtin_bit_cast(_Float16, bp[r]);
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int ml = wm * 128 + 16 * j + r16;
      float v[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) v[r] = epilogue<EPI>(acc[i][j][r] + b[r]);
      const bf16x2 p0 = {(__bf16)v[0], (__bf16)v[1]};
      const bf16x2 p1 = {(__bf16)v[2], (__bf16)v[3]};
      const i32x2 out = {__builtin_bit_cast(int, p0), __builtin_bit_cast(int, p1)};
      const int off = n_ok ? (ml * N + n0 + nl) * 2 : kDropOffset;
      __builtin_amdgcn_raw_buffer_store_b64(out, ry, off, 0, 0);
    }
  }
}

// ===========================================================================
// Fast path for K % 128 == 0 (every Wan2.2 shape): v_mfma_scale_f32_32x32x64
// (the faster of the two scaled shapes on gfx950), operands moved global ->
// LDS by the buffer unit directly (no register staging), and a pipeline with
// one barrier per 128-K stage placed mid-iteration:
//
//   iteration k (stage s = k % 2 holds K step k):
//     1. 16 MFMAs on half-step (k, 0) from registers, while reading the
//        fragments of half-step (k, 1) from stage s; write the scales of
//        step k+1 (loaded one iteration earlier) into stage s^1
//     2. wait for this wave's loads of step k+1, barrier
//     3. issue the loads of step k+2 into stage s (free: no wave reads it
//        any more)
//     4. 16 MFMAs on half-step (k, 1), while reading the fragments of
//        half-step (k+1, 0) from stage s^1
//
// so every load has two half-steps (about 2000 MFMA cycles) to land, and no
// fragment read ever waits on the barrier.
//
// LDS rows are 128 B; a ds_read_b128 is served 16 lanes (256 B, all 64
// banks) at a time, and 16 lanes read 16 consecutive rows at one logical
// chunk, so chunk c of row r is stored at physical chunk c ^ ((r >> 1) & 7):
// rows of equal parity then land on 8 distinct 16-byte slots.
//
// 32x32x64 operand layout (confirmed on the device): lane l holds row l%32,
// K bytes [16*(l/32), +16) and [32 + 16*(l/32), +16) of the 64; the scale of
// lane l belongs to row l%32 and 32-block l/32. Output: lane l holds
// D[8*(e/4) + 4*(l/32) + e%4][l%32], e = 0..15.
namespace v2 {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void* lds_ptr;

constexpr int OFF_W = 0;        // weight codes, 256 rows x 128 B, chunks swizzled
constexpr int OFF_X = 32768;    // token codes, same layout
constexpr int OFF_WS = 65536;   // weight scales [g][row/128][row%32][(row/32)%4]
constexpr int OFF_XS = 66560;   // token scales, same layout
constexpr int STAGE = 67584;
constexpr int LDS = 2 * STAGE;  // 132 KB

__device__ __forceinline__ int scale_slot(int row, int g) {
  return g * 256 + (row >> 7) * 128 + (row & 31) * 4 + ((row >> 5) & 3);
}

struct Frags {
  i32x8 a[4];  // weights: rows wn*128 + 32 f + l%32
  i32x8 b[4];  // tokens:  rows wm*128 + 32 f + l%32
  int sa, sb;  // byte f = scale of frag f for this lane's 32-block
};

// Fragments of half-step h (K bytes 64h .. 64h+63 of the stage).
__device__ __forceinline__ void read_frags(Frags& F, const uint8_t* st, int wn, int wm, int h, int lane) {
  const int r32 = lane & 31, hi = lane >> 5;
  const int sw = (r32 >> 1) & 7;
  const int c0 = ((4 * h + hi) ^ sw) << 4, c1 = ((4 * h + 2 + hi) ^ sw) << 4;
#pragma unroll
  for (int f = 0; f < 4; ++f) {
    const uint8_t* ra = st + OFF_W + (wn * 128 + 32 * f + r32) * 128;
    const uint8_t* rb = st + OFF_X + (wm * 128 + 32 * f + r32) * 128;
    const i32x4 a0 = *(const i32x4*)(ra + c0), a1 = *(const i32x4*)(ra + c1);
    const i32x4 b0 = *(const i32x4*)(rb + c0), b1 = *(const i32x4*)(rb + c1);
    F.a[f] = i32x8{a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
    F.b[f] = i32x8{b0[0], b0[1], b0[2], b0[3], b1[0], b1[1], b1[2], b1[3]};
  }
  const int g = 2 * h + hi;
  F.sa = *(const int*)(st + OFF_WS + g * 256 + wn * 128 + r32 * 4);
  F.sb = *(const int*)(st + OFF_XS + g * 256 + wm * 128 + r32 * 4);
}

__device__ __forceinline__ void mma16(f32x16 (&acc)[4][4], const Frags& F) {
  static_for<0, 4>([&](auto I) {
    constexpr int i = decltype(I)::value;
    static_for<0, 4>([&](auto J) {
      constexpr int j = decltype(J)::value;
      acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(F.a[i], F.b[j], acc[i][j], 0, 0, i, F.sa, j, F.sb);
    });
  });
}

struct Src {
  __amdgpu_buffer_rsrc_t w, x, ws, xs;
  int K;       // bytes per code row
  int G32;     // bytes per scale row
  int voff;    // this lane's part of a direct-load offset
  int voff1;   // the same for odd 1 KB blocks
};

// Issue the loads of K step kk into stage st: 8 direct 1 KB loads per operand
// per wave (8 rows of 128 B each; lane L fills LDS bytes 16 L .. of its
// 1 KB, i.e. row r = 8q + L/8 at physical chunk L%8, which holds logical
// chunk (L%8) ^ ((r >> 1) & 7); voff / voff1 serve even / odd q), and
// this thread's row of 4 scale bytes per operand into registers. With
// valid == false every offset lies past the resources: the loads return
// zeros without touching memory, so the loop needs no branch.
__device__ __forceinline__ void issue_loads(const Src& S, uint8_t* st, int kk, bool valid, int wave, int& swv,
                                            int& sxv) {
  const int t = threadIdx.x;
  const int sbase = valid ? kk * 4 : kDropOffset;
  const int dbase = valid ? kk * 128 : kDropOffset;
  swv = __builtin_amdgcn_raw_buffer_load_b32(S.ws, t * S.G32, sbase, 0);
  sxv = __builtin_amdgcn_raw_buffer_load_b32(S.xs, t * S.G32, sbase, 0);
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    const int q = wave * 8 + u;
    const int soff = 8 * q * S.K + dbase;
    const int vo = (u & 1) ? S.voff1 : S.voff;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(S.w, (lds_ptr)(st + OFF_W + q * 1024), 16, vo, soff, 0, kLoadAux);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(S.x, (lds_ptr)(st + OFF_X + q * 1024), 16, vo, soff, 0, kLoadAux);
  }
}

__device__ __forceinline__ void write_scales(uint8_t* st, int swv, int sxv) {
  const int t = threadIdx.x;
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    st[OFF_WS + scale_slot(t, g)] = (uint8_t)(swv >> (8 * g));
    st[OFF_XS + scale_slot(t, g)] = (uint8_t)(sxv >> (8 * g));
  }
}

__device__ __forceinline__ void wait_all_and_barrier() {
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_waitcnt(0);  // vmcnt, lgkmcnt, expcnt all zero
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
}

// Interleave the 16 MFMAs of a half-step with the memory instructions issued
// beside them: one LDS read (and, when given, one LDS write or one global
// load) after each MFMA.
template <int DS_WRITES, int VMEM>
__device__ __forceinline__ void interleave_half_step() {
  static_for<0, 16>([&](auto I) {
    constexpr int i = decltype(I)::value;
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // LDS read
    if constexpr (i < DS_WRITES) __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);  // LDS write
    if constexpr (i < VMEM) __builtin_amdgcn_sched_group_barrier(0x010, 1, 0);  // global load
  });
}

// Slot-wise emission of half-step 4: slot i issues global loads
// kLoadsPerSlot*i .. of the stage after next, then MFMA i on the current
// fragments, then LDS read i of the next fragments, pinned in that order.
// Front-loading the global loads gives them the longest time to land.
#ifndef MX_LOADS_PER_SLOT
#define MX_LOADS_PER_SLOT 4
#endif
constexpr int kLoadsPerSlot = MX_LOADS_PER_SLOT;
struct FragAddr {
  const uint8_t* a;  // weight rows of this lane in the stage (chunk offsets applied below)
  const uint8_t* b;
  int c0, c1;        // swizzled byte offsets of the two 16-byte halves
  const uint8_t* sa;
  const uint8_t* sb;
};

__device__ __forceinline__ FragAddr frag_addr(const uint8_t* st, int wn, int wm, int h, int lane) {
  const int r32 = lane & 31, hi = lane >> 5;
  const int sw = (r32 >> 1) & 7;
  FragAddr A;
  A.a = st + OFF_W + (wn * 128 + r32) * 128;
  A.b = st + OFF_X + (wm * 128 + r32) * 128;
  A.c0 = ((4 * h + hi) ^ sw) << 4;
  A.c1 = ((4 * h + 2 + hi) ^ sw) << 4;
  const int g = 2 * h + hi;
  A.sa = st + OFF_WS + g * 256 + wn * 128 + r32 * 4;
  A.sb = st + OFF_XS + g * 256 + wm * 128 + r32 * 4;
  return A;
}

// LDS read number i (0..17) of a fragment set.
template <int I>
__device__ __forceinline__ void read_piece(Frags& F, const FragAddr& A) {
  if constexpr (I < 16) {
    constexpr int f = I / 4, part = I % 4;
    const uint8_t* base = (part < 2 ? A.a : A.b) + 32 * f * 128;
    const i32x4 v = *(const i32x4*)(base + ((part & 1) ? A.c1 : A.c0));
    i32x8& d = part < 2 ? F.a[f] : F.b[f];
    if constexpr ((part & 1) == 0) {
      d[0] = v[0]; d[1] = v[1]; d[2] = v[2]; d[3] = v[3];
    } else {
      d[4] = v[0]; d[5] = v[1]; d[6] = v[2]; d[7] = v[3];
    }
  } else if constexpr (I == 16) {
    F.sa = *(const int*)A.sa;
  } else {
    F.sb = *(const int*)A.sb;
  }
}

// Global load number i (0..17) of a stage: 0..15 direct code loads (W, X
// alternating, 8 each per wave), 16 and 17 the two scale rows.
template <int I>
__device__ __forceinline__ void load_piece(const Src& S, uint8_t* st, int kk, bool valid, int wave, int& swv,
                                           int& sxv) {
  const int dbase = valid ? kk * 128 : kDropOffset;
  if constexpr (I < 16) {
    constexpr int u = I / 2;
    const int q = wave * 8 + u;
    const int soff = 8 * q * S.K + dbase;
    const int vo = (u & 1) ? S.voff1 : S.voff;
    if constexpr ((I & 1) == 0)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(S.w, (lds_ptr)(st + OFF_W + q * 1024), 16, vo, soff, 0, kLoadAux);
    else
      __builtin_amdgcn_raw_ptr_buffer_load_lds(S.x, (lds_ptr)(st + OFF_X + q * 1024), 16, vo, soff, 0, kLoadAux);
  } else {
    const int sbase = valid ? kk * 4 : kDropOffset;
    if constexpr (I == 16)
      swv = __builtin_amdgcn_raw_buffer_load_b32(S.ws, threadIdx.x * S.G32, sbase, 0);
    else
      sxv = __builtin_amdgcn_raw_buffer_load_b32(S.xs, threadIdx.x * S.G32, sbase, 0);
  }
}

template <int I>
__device__ __forceinline__ void mfma_piece(f32x16 (&acc)[4][4], const Frags& F) {
  constexpr int i = I / 4, j = I % 4;
  acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(F.a[i], F.b[j], acc[i][j], 0, 0, i, F.sa, j, F.sb);
}

// Write a wave's 128 x 128 accumulator tile: bias, epilogue and bf16 rounding
// into LDS staging ([m][n] bf16, 256-byte rows, 8-byte block nb of row m at
// nb ^ (m & 31): 32 lanes writing 32 consecutive rows hit 32 distinct bank
// pairs), then 2 rows x 256 B per store instruction with streaming stores.
// Accumulator layout: lane l holds D[n = 32 i + 8 (e/4) + 4 (l/32) + e%4]
// [m = 32 j + l%32] of the wave tile.
template <int EPI>
__device__ __forceinline__ void store_tile(const f32x16 (&acc)[4][4], const Params& p, uint8_t* ep, int m0, int n0,
                                           int rows_m, int rows_n, int wn, int wm, int lane) {
  const int r32 = lane & 31, hi = lane >> 5;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int nb = 8 * i + 2 * q + hi;  // 4-column block within the wave tile
      const int nl = wn * 128 + 4 * nb;
      float b[4] = {0.f, 0.f, 0.f, 0.f};
      if (p.bias != nullptr && nl < rows_n) {
        const uint16_t* bp = p.bias + n0 + nl;
#pragma unroll
        for (int r = 0; r < 4; ++r) b[r] = (float)__builtin_bit_cast(_Float16, bp[r]);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int m = 32 * j + r32;
        float v[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) v[r] = epilogue<EPI>(acc[i][j][4 * q + r] + b[r]);
        const bf16x2 p0 = {(__bf16)v[0], (__bf16)v[1]};
        const bf16x2 p1 = {(__bf16)v[2], (__bf16)v[3]};
        *(i32x2*)(ep + m * 256 + ((nb ^ (m & 31)) << 3)) =
            i32x2{__builtin_bit_cast(int, p0), __builtin_bit_cast(int, p1)};
      }
    }
  }
  const int N = p.N;
  const __amdgpu_buffer_rsrc_t ry = make_rsrc(p.y + (size_t)m0 * N, (uint32_t)(rows_m * N * 2));
  const int nl = wn * 128 + 4 * r32;
  const bool n_ok = nl < rows_n;
#pragma unroll 8
  for (int it = 0; it < 64; ++it) {
    const int m = 2 * it + hi;
    const i32x2 v = *(const i32x2*)(ep + m * 256 + ((r32 ^ (m & 31)) << 3));
    const int off = n_ok ? ((wm * 128 + m) * N + n0 + nl) * 2 : kDropOffset;
    __builtin_amdgcn_raw_buffer_store_b64(v, ry, off, 0, kStoreAux);
  }
}

template <int EPI>
__global__ __launch_bounds__(NT, 1) void linear_prequant_kernel(Params p) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  int tm, tn;
  tile_coords(blockIdx.x, p.tiles_m, p.tiles_n, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;
  const int K = p.K, G32 = K >> 5, nk = K / 128;
  const int rows_m = min(p.M - m0, BM);
  const int rows_n = min(p.N - n0, BN);
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wn = wave >> 1, wm = wave & 1;

  Src S;
  S.w = make_rsrc(p.wq + (size_t)n0 * K, (uint32_t)(rows_n * K));
  S.ws = make_rsrc(p.ws + (size_t)n0 * G32, (uint32_t)(rows_n * G32));
  S.x = make_rsrc(p.x + (size_t)m0 * K, (uint32_t)(rows_m * K));
  S.xs = make_rsrc(p.xs + (size_t)m0 * G32, (uint32_t)(rows_m * G32));
  S.K = K;
  S.G32 = G32;
  S.voff = (lane >> 3) * K + (((lane & 7) ^ (lane >> 4)) << 4);
  S.voff1 = (lane >> 3) * K + (((lane & 7) ^ ((4 + (lane >> 4)) & 7)) << 4);

  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x16{};

  uint8_t* stage0 = smem;
  uint8_t* stage1 = smem + STAGE;
  int sw0, sx0, swn, sxn;  // (swn, sxn): scales of the step in flight to the other stage
  issue_loads(S, stage0, 0, true, wave, sw0, sx0);
  issue_loads(S, stage1, 1, nk > 1, wave, swn, sxn);
  __builtin_amdgcn_s_waitcnt(0);
  write_scales(stage0, sw0, sx0);
  wait_all_and_barrier();

  Frags F0, F1;
  read_frags(F0, stage0, wn, wm, 0, lane);

  for (int k = 0; k < nk; ++k) {
    uint8_t* st = (k & 1) ? stage1 : stage0;
    uint8_t* other = (k & 1) ? stage0 : stage1;
    // 1. MFMAs of (k, 0); read fragments of (k, 1).
    read_frags(F1, st, wn, wm, 1, lane);
    mma16(acc, F0);
    interleave_half_step<0, 0>();
    __builtin_amdgcn_sched_barrier(0);
    // 2. Scales of step k+1 (their loads finish with the data the barrier
    //    waits for anyway), then the barrier.
    write_scales(other, swn, sxn);
    wait_all_and_barrier();
    // 3. + 4. loads of step k+2 into stage s; MFMAs of (k, 1); fragments of (k+1, 0).
    {
      const FragAddr A = frag_addr(other, wn, wm, 0, lane);
      const bool valid = k + 2 < nk;
      static_for<0, 18>([&](auto I) {
        constexpr int i = decltype(I)::value;
        static_for<i * kLoadsPerSlot, (i + 1) * kLoadsPerSlot < 18 ? (i + 1) * kLoadsPerSlot : 18>([&](auto L) {
          load_piece<decltype(L)::value>(S, st, k + 2, valid, wave, swn, sxn);
        });
        if constexpr (i < 16) mfma_piece<i>(acc, F1);
        read_piece<i>(F0, A);
        __builtin_amdgcn_sched_barrier(0);
      });
    }
  }
  __builtin_amdgcn_s_waitcnt(0);

  // Epilogue. Every wave's loads have landed (including the out-of-range
  // ones of the last two iterations, which still write zeros into LDS), so
  // after one barrier the LDS is free: each wave stages its 128 x 128 bf16
  // result there and writes it back as whole 256-byte row segments.
  __builtin_amdgcn_s_barrier();
  store_tile<EPI>(acc, p, smem + wave * 32768, m0, n0, rows_m, rows_n, wn, wm, lane);
}

// ---------------------------------------------------------------------------
// Ring pipeline. The TA -> L1 -> L2 path of a CU sustains about 64 B/clk; a
// 256 x 256 tile needs 32 B/clk at MFMA peak. The two-stage loop above can
// only refill a stage after its mid-iteration barrier, so it pushes a whole
// stage (64 KB) through in half an iteration, fills the address FIFO and
// blocks the waves' instruction issue (MFMAs included). Here K advances in
// half-steps of 64 through a ring of 4 regions, each freed as soon as its
// fragments have been read, so the refill of half-step j+4 is issued at the
// start of half-step j and loads stream at the average rate with three
// half-steps (about 3000 cycles) to land:
//
//   half-step j:  wait for this wave's loads of j+1, barrier;
//                 issue the loads of j+4 into region j % 4;
//                 16 MFMAs on fragments of j (registers), interleaved with
//                 the LDS reads of the fragments of j+1 (region (j+1) % 4).
//
// Scales travel by LDS DMA too (one dword = 4 groups per row per 128-K step,
// a 4-slot ring), so no load result passes through registers and every wait
// is explicit. Each lane reads its 4 scale bytes per operand with byte loads
// and hands them to the MFMA with op_sel 0.
namespace ring {

constexpr int R_W = 0;          // weight codes: 256 rows x 64 B, chunk c of row r at c ^ ((r >> 2) & 3)
constexpr int R_X = 16384;      // token codes, same layout
constexpr int REGION = 32768;
constexpr int OFF_SC = 4 * REGION;       // scale slots: [slot 0..3][W 1 KB | X 1 KB], row-major dwords
constexpr int SLOT = 2048;
constexpr int LDS = OFF_SC + 4 * SLOT;   // 136 KB

struct Frags {
  i32x8 a[4];
  i32x8 b[4];
  int sa[4];  // scale byte (bits 0..7) of frag f
  int sb[4];
};

struct Src {
  __amdgpu_buffer_rsrc_t w, x, ws, xs;
  int K, G32;
  int voff;   // lane part of a code DMA offset: row L/4, logical chunk (L%4) ^ (L/16)
  int soff;   // lane part of a scale DMA offset: row L
};

// Load number I of half-step j into region j % 4: I = 0..7 code DMAs of
// 1 KB (16 rows x 64 B; W and X alternating, 4 each per wave), I = 8, 9 (even
// j only) the scale DMAs of its 128-K step into slot (j/2) % 4, 256 B each.
// Past the last half-step the offsets fall outside the resources: the DMAs
// then write zeros and touch no memory.
template <int I>
__device__ __forceinline__ void load_piece(const Src& S, uint8_t* smem, int j, int nh, int wave) {
  const bool valid = j < nh;
  if constexpr (I < 8) {
    uint8_t* reg = smem + (j & 3) * REGION;
    const int q = wave * 4 + I / 2;  // 16-row block
    const int so = 16 * q * S.K + (valid ? j * 64 : kDropOffset);
    if constexpr ((I & 1) == 0)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(S.w, (lds_ptr)(reg + R_W + q * 1024), 16, S.voff, so, 0, 0);
    else
      __builtin_amdgcn_raw_ptr_buffer_load_lds(S.x, (lds_ptr)(reg + R_X + q * 1024), 16, S.voff, so, 0, 0);
  } else {
    uint8_t* slot = smem + OFF_SC + ((j >> 1) & 3) * SLOT;
    const int so = 64 * wave * S.G32 + (valid ? (j >> 1) * 4 : kDropOffset);
    if constexpr (I == 8)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(S.ws, (lds_ptr)(slot + wave * 256), 4, S.soff, so, 0, 0);
    else
      __builtin_amdgcn_raw_ptr_buffer_load_lds(S.xs, (lds_ptr)(slot + 1024 + wave * 256), 4, S.soff, so, 0, 0);
  }
}

template <bool EVEN>
__device__ __forceinline__ void load_half(const Src& S, uint8_t* smem, int j, int nh, int wave) {
  static_for<0, EVEN ? 10 : 8>([&](auto I) { load_piece<decltype(I)::value>(S, smem, j, nh, wave); });
}

struct FragAddr {
  const uint8_t* a;
  const uint8_t* b;
  int c0, c1;
  const uint8_t* sa;
  const uint8_t* sb;
};

// Fragments of half-step j: lane l, frag f reads row base + 32 f + l%32,
// K bytes [16 (l/32), +16) and [32 + 16 (l/32), +16) of the 64, and the scale
// byte of group 2 (j % 2) + l/32 of its 128-K step.
__device__ __forceinline__ FragAddr frag_addr(const uint8_t* smem, int j, int wn, int wm, int lane) {
  const int r32 = lane & 31, hi = lane >> 5;
  const int sw = (r32 >> 2) & 3;
  const uint8_t* reg = smem + (j & 3) * REGION;
  FragAddr A;
  A.a = reg + R_W + (wn * 128 + r32) * 64;
  A.b = reg + R_X + (wm * 128 + r32) * 64;
  A.c0 = (hi ^ sw) << 4;
  A.c1 = ((2 + hi) ^ sw) << 4;
  const uint8_t* slot = smem + OFF_SC + ((j >> 1) & 3) * SLOT;
  const int g = 2 * (j & 1) + hi;
  A.sa = slot + (wn * 128 + r32) * 4 + g;
  A.sb = slot + 1024 + (wm * 128 + r32) * 4 + g;
  return A;
}

// LDS read number i (0..23) of a fragment set: 16 code halves, 8 scale bytes.
template <int I>
__device__ __forceinline__ void read_piece(Frags& F, const FragAddr& A) {
  if constexpr (I < 16) {
    constexpr int f = I / 4, part = I % 4;
    const uint8_t* base = (part < 2 ? A.a : A.b) + 32 * f * 64;
    const i32x4 v = *(const i32x4*)(base + ((part & 1) ? A.c1 : A.c0));
    i32x8& d = part < 2 ? F.a[f] : F.b[f];
    if constexpr ((part & 1) == 0) {
      d[0] = v[0]; d[1] = v[1]; d[2] = v[2]; d[3] = v[3];
    } else {
      d[4] = v[0]; d[5] = v[1]; d[6] = v[2]; d[7] = v[3];
    }
  } else if constexpr (I < 20) {
    F.sa[I - 16] = *(const uint8_t*)(A.sa + 32 * (I - 16) * 4);
  } else {
    F.sb[I - 20] = *(const uint8_t*)(A.sb + 32 * (I - 20) * 4);
  }
}

template <int I>
__device__ __forceinline__ void mfma_piece(f32x16 (&acc)[4][4], const Frags& F) {
  constexpr int i = I / 4, j = I % 4;
  acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(F.a[i], F.b[j], acc[i][j], 0, 0, 0, F.sa[i], 0, F.sb[j]);
}

// s_waitcnt vmcnt(N) lgkmcnt(0): written as asm because the compiler's own
// waitcnt pass relaxes the builtin form to the counts it tracks, and the
// lgkmcnt(0) here is what keeps another wave's DMA refill from overtaking
// this wave's last reads of the region being refilled.
template <int N>
__device__ __forceinline__ void wait_vm_lgkm0() {
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)" ::"n"(N));
}

// One half-step j (parity EVEN): barrier, loads of j+4, MFMAs of j on `cur`
// interleaved with the reads of j+1 into `nxt`.
template <bool EVEN>
__device__ __forceinline__ void half_step(f32x16 (&acc)[4][4], Frags& cur, Frags& nxt, const Src& S, uint8_t* smem,
                                          int j, int nh, int wave, int wn, int wm, int lane) {
  __builtin_amdgcn_sched_barrier(0);
  wait_vm_lgkm0<18>();  // loads of j+1 landed (those of j+2, j+3 may fly)
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
  const FragAddr A = frag_addr(smem, j + 1, wn, wm, lane);
  constexpr int NL = EVEN ? 10 : 8;  // loads of half-step j+4 (same parity as j)
  static_for<0, 16>([&](auto I) {
    constexpr int i = decltype(I)::value;
    if constexpr (i < NL) load_piece<i>(S, smem, j + 4, nh, wave);
    mfma_piece<i>(acc, cur);
    read_piece<i>(nxt, A);
    if constexpr (i < 8) read_piece<16 + i>(nxt, A);
    __builtin_amdgcn_sched_barrier(0);
  });
}

template <int EPI>
__global__ __launch_bounds__(NT, 1) void linear_prequant_ring(Params p) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  int tm, tn;
  tile_coords(blockIdx.x, p.tiles_m, p.tiles_n, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;
  const int K = p.K, G32 = K >> 5, nh = K / 64;  // nh is even (K % 128 == 0)
  const int rows_m = min(p.M - m0, BM);
  const int rows_n = min(p.N - n0, BN);
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wn = wave >> 1, wm = wave & 1;

  Src S;
  S.w = make_rsrc(p.wq + (size_t)n0 * K, (uint32_t)(rows_n * K));
  S.ws = make_rsrc(p.ws + (size_t)n0 * G32, (uint32_t)(rows_n * G32));
  S.x = make_rsrc(p.x + (size_t)m0 * K, (uint32_t)(rows_m * K));
  S.xs = make_rsrc(p.xs + (size_t)m0 * G32, (uint32_t)(rows_m * G32));
  S.K = K;
  S.G32 = G32;
  S.voff = (lane >> 2) * K + (((lane & 3) ^ (lane >> 4)) << 4);
  S.soff = lane * G32;

  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x16{};

  // Prologue: half-steps 0..3 in flight; wait for half-step 0.
  load_half<true>(S, smem, 0, nh, wave);
  load_half<false>(S, smem, 1, nh, wave);
  load_half<true>(S, smem, 2, nh, wave);
  load_half<false>(S, smem, 3, nh, wave);
  __builtin_amdgcn_sched_barrier(0);
  wait_vm_lgkm0<26>();  // half-step 0 (10 loads) landed; 8 + 10 + 8 may fly
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
  Frags F0, F1;
  {
    const FragAddr A = frag_addr(smem, 0, wn, wm, lane);
    static_for<0, 24>([&](auto I) { read_piece<decltype(I)::value>(F0, A); });
  }
  for (int j = 0; j < nh; j += 2) {
    half_step<true>(acc, F0, F1, S, smem, j, nh, wave, wn, wm, lane);
    half_step<false>(acc, F1, F0, S, smem, j + 1, nh, wave, wn, wm, lane);
  }
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_waitcnt(0);
  __builtin_amdgcn_s_barrier();
  store_tile<EPI>(acc, p, smem + wave * 32768, m0, n0, rows_m, rows_n, wn, wm, lane);
}

template <int EPI>
hipError_t launch(const Params& p, int nwg, hipStream_t st) {
  static bool configured = false;  // per instantiation; benign race (idempotent)
  auto kern = linear_prequant_ring<EPI>;
  if (!configured) {
    hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, LDS);
    if (e != hipSuccess) return e;
    configured = true;
  }
  hipLaunchKernelGGL(kern, dim3(nwg), dim3(NT), LDS, st, p);
  return hipGetLastError();
}

}  // namespace ring

template <int EPI>
hipError_t launch(const Params& p, int nwg, hipStream_t st) {
  static bool configured = false;  // per instantiation; benign race (idempotent)
  auto kern = linear_prequant_kernel<EPI>;
  if (!configured) {
    hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, LDS);
    if (e != hipSuccess) return e;
    configured = true;
  }
  hipLaunchKernelGGL(kern, dim3(nwg), dim3(NT), LDS, st, p);
  return hipGetLastError();
}

}  // namespace v2

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
  p.M = (int)M;
  p.N = (int)N;
  p.K = (int)K;
  p.tiles_m = (int)((M + BM - 1) / BM);
  p.tiles_n = (int)((N + BN - 1) / BN);
  const int nwg = p.tiles_m * p.tiles_n;
  const bool ktail = (K % BK) != 0;
  if (xs != nullptr && !ktail)
    return epi == 1 ? v2::ring::launch<1>(p, nwg, stream) : v2::ring::launch<0>(p, nwg, stream);
  return xs == nullptr ? dispatch_epi<true>(p, ktail, epi, nwg, stream)
                       : dispatch_epi<false>(p, ktail, epi, nwg, stream);
}

}  // namespace mx
