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
// consecutive rows read the same logical chunk from 8 different bank groups;
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
  return xs == nullptr ? dispatch_epi<true>(p, ktail, epi, nwg, stream)
                       : dispatch_epi<false>(p, ktail, epi, nwg, stream);
}

}  // namespace mx
