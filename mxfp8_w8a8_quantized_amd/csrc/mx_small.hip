// Block-scaled GEMM for few tokens (M up to a few hundred): the linears whose
// 256 x 256 tiles would leave most of the GPU idle (the 128-token linear, the
// 512 text tokens of attn2 k/v). Same operands and result as the slab GEMM
// (mx.h: y = bf16(epi(sum_k xhat what + bias)), slab layout, products exact
// on the scaled FP8 MFMA, FP32 sums).
//
// Tile: 128 tokens x 64 weight rows, 8 waves of one 32 x 32 block each (one
// 32x32x64 MFMA per 64-K slab, two waves per SIMD so that one issues while
// the other waits). Every workgroup streams its own 64 weight rows from HBM
// and the 128-token slab from the L2 (0.66 MB at 128 x 5120), and K is split
// into `splits` ranges so that there are about as many workgroups as CUs.
// Measured, a workgroup's loop is bound by its CU's load path (about 40 B
// per clock for these 1 KB LDS loads; 12.8 KB per slab), so the per-CU
// bytes, (128 + 64) per K element, set the loop time; launch, the first
// round trip to memory and the partial-sum reduction are of the same order
// at these sizes.
//
// The loop is written for few instructions: one buffer resource per operand
// for the whole K range (32-bit running offsets; slabs past the range read
// zeros), a ring of kSteps two-slab steps (12.8 KB per slab: 4 KB weight
// codes, 8 KB token codes, their scales) unrolled so that every LDS address
// is an immediate, and LDS fragment reads two steps ahead of their MFMAs.
//
// Output: splits == 1 writes y directly (bias, epilogue, bf16); otherwise
// each range writes f32 partial sums [splits][M][N] and small_reduce_kernel
// adds them in range order, so results do not depend on timing.
#include <type_traits>

#include "mx_device.h"
#include "mx_internal.h"

namespace mx {
namespace {

constexpr int TM = 128, TN = 64;
constexpr int R_W = 0, R_X = 4096, R_WS = 12288, R_XS = 12544;  // W scales use 128 of their 256 bytes
constexpr int SLAB = 12800;     // LDS bytes of one 64-K slab
constexpr int PAIR = 2 * SLAB;  // one pipeline step: two slabs
constexpr int kSteps = 6;       // LDS ring, in two-slab steps (153.6 KB)
constexpr int kDrop = 1 << 30;  // beyond every resource: the store is dropped

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void* lds_ptr;

template <int Begin, int End, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (Begin < End) {
    f(std::integral_constant<int, Begin>{});
    static_for<Begin + 1, End>(f);
  }
}

struct SmallParams {
  const uint8_t* x;   // token codes [K/64][RM][64]
  const uint8_t* xs;  // token scales [K/64][RM][2]
  const uint8_t* wq;  // weight codes [K/64][RN][64]
  const uint8_t* ws;  // weight scales [K/64][RN][2]
  const uint16_t* bias;
  uint16_t* y;
  float* part;  // [splits][M][N] f32 when splits > 1
  int M, N, K;
  int64_t RM, RN;
  int tiles_m, tiles_n, splits;
};

// Fragments of one 64-K slab for the 32x32x64 MFMA: lane l reads row l%32
// of each operand fragment, K bytes [16 (l/32), +16) and [32 + 16 (l/32),
// +16), and the scale of 32-group l/32.
struct Frag {
  i32x8 a;  // weight rows 32 wf + l%32
  i32x8 b;  // token rows 32 wt + l%32
  int sa, sb;
};
struct Pair {
  Frag s[2];
};

// 8 waves, two per SIMD: wave w computes the 32 x 32 block of token rows
// 32 (w%4) .. and weight rows 32 (w/4) ..; while one wave of a SIMD waits
// (for its MFMA to issue, at the barrier, for LDS data) the other issues.
template <int EPI, bool PART, int RP>
__global__ __launch_bounds__(512, 1) void small_kernel(SmallParams p) {
  static_assert(RP % 3 == 0 && RP >= 3, "the ring unrolls with three fragment sets");
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wt = wave & 3, wf = wave >> 2;
  // Work order: consecutive units on one XCD (workgroups are dealt to the 8
  // XCDs in turn), token tile fastest, then K range, then weight tile, so
  // that the units sharing a weight tile share an L2.
  const int units = p.tiles_m * p.tiles_n * p.splits;
  const int q8 = units >> 3, r8 = units & 7;
  const int xcd = blockIdx.x & 7;
  const int lid = xcd * q8 + min(xcd, r8) + (int)(blockIdx.x >> 3);
  const int tm = lid % p.tiles_m;
  const int rest = lid / p.tiles_m;
  const int ks = rest % p.splits, tn = rest / p.splits;
  const int m0 = tm * TM, n0 = tn * TN;
  const int nh_all = p.K >> 6;
  const int h0 = ks * nh_all / p.splits;
  const int nh = (ks + 1) * nh_all / p.splits - h0;
  const int np = (nh + 1) >> 1;  // pipeline steps of two slabs
  // Bytes between slabs (code and scale layouts [K/64][R][64], [K/64][R][2]);
  // the offsets below stay under 2^31 (checked by the host).
  const uint32_t xs_code = (uint32_t)p.RM * 64, ws_code = (uint32_t)p.RN * 64;
  const uint32_t xs_scale = (uint32_t)p.RM * 2, ws_scale = (uint32_t)p.RN * 2;
  // Loads per slab: token code block w (1 KB: 16 rows) by every wave,
  // weight code block w by waves 0..3, the weight scales by wave 4 (lanes
  // 32..63 repeat the 128 bytes of lanes 0..31 into the unused upper half),
  // the token scales (256 bytes) by wave 5. One resource per operand covers
  // the tile's K range; slabs past it read zeros. Lane L of a code load takes
  // row L/4 of the block and global 16-byte chunk (L%4) ^ (L/16) into LDS
  // slot L%4 (a 4-way swizzle); the block's offset goes in soffset, the
  // running slab offset in the lane offset.
  const __amdgpu_buffer_rsrc_t rx = make_rsrc(p.x + (uint64_t)m0 * 64 + (uint64_t)h0 * xs_code, (uint32_t)nh * xs_code);
  const __amdgpu_buffer_rsrc_t rw = make_rsrc(p.wq + (uint64_t)n0 * 64 + (uint64_t)h0 * ws_code, (uint32_t)nh * ws_code);
  const __amdgpu_buffer_rsrc_t rs =
      wave == 4 ? make_rsrc(p.ws + (uint64_t)n0 * 2 + (uint64_t)h0 * ws_scale, (uint32_t)nh * ws_scale)
                : make_rsrc(p.xs + (uint64_t)m0 * 2 + (uint64_t)h0 * xs_scale, (uint32_t)nh * xs_scale);
  const uint32_t s_stride = wave == 4 ? ws_scale : xs_scale;
  const uint32_t voff = (lane >> 2) * 64 + (((lane & 3) ^ (lane >> 4)) << 4);
  uint32_t ox = voff, ow = voff;
  uint32_t os = wave == 4 ? (uint32_t)(lane & 31) * 4 : (uint32_t)lane * 4;
  const int sblk = wave * 1024;
  const int nload = wave < 6 ? 2 : 1;  // loads per slab of this wave

  auto issue_slab = [&](uint8_t* reg) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, (lds_ptr)(reg + R_X + sblk), 16, ox, sblk, 0, 0);
    if (wave < 4) __builtin_amdgcn_raw_ptr_buffer_load_lds(rw, (lds_ptr)(reg + R_W + sblk), 16, ow, sblk, 0, 0);
    else if (wave < 6)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_ptr)(reg + (wave == 4 ? R_WS : R_XS)), 4, os, 0, 0, 0);
    ox += xs_code;
    ow += ws_code;
    os += s_stride;
  };
  auto issue = [&](auto k) {  // the step in ring slot k
    uint8_t* reg = smem + decltype(k)::value * PAIR;
    issue_slab(reg);
    issue_slab(reg + SLAB);
  };

  const int r32 = lane & 31, hi = lane >> 5;
  const int sw = (r32 >> 2) & 3;
  const int c0 = (hi ^ sw) << 4, c1 = ((2 + hi) ^ sw) << 4;
  const uint8_t* fa = smem + R_W + (32 * wf + r32) * 64;
  const uint8_t* fb = smem + R_X + (32 * wt + r32) * 64;
  const uint8_t* fsa = smem + R_WS + (32 * wf + r32) * 2 + hi;
  const uint8_t* fsb = smem + R_XS + (32 * wt + r32) * 2 + hi;
  auto read = [&](Pair& F, auto k) {  // fragments of the step in ring slot k
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int off = decltype(k)::value * PAIR + u * SLAB;
      const i32x4 a0 = *(const i32x4*)(fa + off + c0), a1 = *(const i32x4*)(fa + off + c1);
      const i32x4 b0 = *(const i32x4*)(fb + off + c0), b1 = *(const i32x4*)(fb + off + c1);
      F.s[u].a = i32x8{a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
      F.s[u].b = i32x8{b0[0], b0[1], b0[2], b0[3], b1[0], b1[1], b1[2], b1[3]};
      F.s[u].sa = fsa[off];
      F.s[u].sb = fsb[off];
    }
  };

  // One accumulator, slabs in K order, started at the bias for the direct
  // output (at zero for partial sums): with one range the result is the slab
  // GEMM's bit for bit (the same chain of MFMAs from the same start). The
  // slab past the range (the second of the last step when nh is odd, loaded
  // as zero codes) is not multiplied, so the chain has exactly nh MFMAs.
  f32x16 acc = f32x16{};
  auto mma = [&](const Pair& F, int t) {
    acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(F.s[0].a, F.s[0].b, acc, 0, 0, 0, F.s[0].sa, 0, F.s[0].sb);
    if (2 * t + 1 < nh)
      acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(F.s[1].a, F.s[1].b, acc, 0, 0, 0, F.s[1].sa, 0, F.s[1].sb);
  };
  // Step t (ring slot t % RP, fragment set t % 3): its MFMAs on fragments
  // read two steps earlier, then wait for step t + 2's slabs (this wave's
  // loads; every wave's by the barrier, which also means every wave has read
  // slot t), refill slot t with step t + RP and read step t + 2 into the set
  // step t + 2 will use. The barrier and the LDS latency thus overlap the
  // MFMAs of steps t and t + 1; RP - 3 later steps stay in flight.
  Pair F[3];
  auto step = [&](int t, auto k) {
    constexpr int K = decltype(k)::value;
    mma(F[K % 3], t);
    if (t + 2 < np) {
      if (nload == 2)
        asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)" ::"n"((RP - 3) * 4) : "memory");
      else
        asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)" ::"n"((RP - 3) * 2) : "memory");
      __builtin_amdgcn_s_barrier();
      issue(k);
      read(F[(K + 2) % 3], std::integral_constant<int, (K + 2) % RP>{});
    }
  };

  // The bias quads of this lane's outputs (direct output only), loaded
  // before the first slabs; they are older than every slab load, so the
  // first slabs' wait below (loads complete in order) covers them too.
  i32x2 bq[4];
  if constexpr (!PART) {
    const bool has_b = p.bias != nullptr;
    const __amdgpu_buffer_rsrc_t rb = make_rsrc(has_b ? p.bias + n0 : nullptr, has_b ? (uint32_t)(p.N - n0) * 2u : 0u);
#pragma unroll
    for (int q = 0; q < 4; ++q)
      bq[q] = __builtin_bit_cast(
          i32x2, __builtin_amdgcn_raw_buffer_load_b64(rb, (32 * wf + 8 * q + 4 * (lane >> 5)) * 2, 0, 0));
  }
  static_for<0, RP>([&](auto k) { issue(k); });
  if (nload == 2)  // steps 0 and 1 landed
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"((RP - 2) * 4) : "memory");
  else
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"((RP - 2) * 2) : "memory");
  __builtin_amdgcn_s_barrier();
  if constexpr (!PART) {
    // The bias (landed with the first slabs): lane holds n = n0 + 32 wf +
    // 8 q + 4 (lane/32) + r in element 4 q + r.
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint32_t w0 = (uint32_t)bq[q][0], w1 = (uint32_t)bq[q][1];
      acc[4 * q] = (float)__builtin_bit_cast(_Float16, (uint16_t)(w0 & 0xFFFFu));
      acc[4 * q + 1] = (float)__builtin_bit_cast(_Float16, (uint16_t)(w0 >> 16));
      acc[4 * q + 2] = (float)__builtin_bit_cast(_Float16, (uint16_t)(w1 & 0xFFFFu));
      acc[4 * q + 3] = (float)__builtin_bit_cast(_Float16, (uint16_t)(w1 >> 16));
    }
  }
  read(F[0], std::integral_constant<int, 0>{});
  read(F[1], std::integral_constant<int, 1>{});
  for (int t = 0; t < np; t += RP) {
    static_for<0, RP>([&](auto k) {
      if (t + decltype(k)::value < np) step(t + decltype(k)::value, k);
    });
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  // A lane holds n = n0 + 32 wf + 8 q + 4 (lane/32) + 0..3 (q = 0..3) of
  // token m = m0 + 32 wt + lane%32.
  const int m = m0 + 32 * wt + r32;
  const bool m_ok = m < p.M;
  if constexpr (PART) {
    float* prow = p.part + ((size_t)ks * p.M + (m_ok ? m : 0)) * p.N;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int n = n0 + 32 * wf + 8 * q + 4 * hi;
      if (m_ok && n < p.N) {
        const f32x4 v = {acc[4 * q], acc[4 * q + 1], acc[4 * q + 2], acc[4 * q + 3]};
        *(f32x4*)(prow + n) = v;
      }
    }
  } else {
    const int rows = min(p.M - m0, TM);
    const __amdgpu_buffer_rsrc_t ry = make_rsrc(p.y + (size_t)m0 * p.N, (uint32_t)rows * (uint32_t)p.N * 2u);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int n = n0 + 32 * wf + 8 * q + 4 * hi;
      float v[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) v[r] = epilogue<EPI>(acc[4 * q + r]);
      const bf16x2 p0 = {(__bf16)v[0], (__bf16)v[1]};
      const bf16x2 p1 = {(__bf16)v[2], (__bf16)v[3]};
      const int off = (m_ok && n < p.N) ? ((m - m0) * p.N + n) * 2 : kDrop;
      __builtin_amdgcn_raw_buffer_store_b64(i32x2{__builtin_bit_cast(int, p0), __builtin_bit_cast(int, p1)}, ry, off,
                                            0, 0);
    }
  }
}

// Sum of the ranges' partials in range order, then bias, epilogue, bf16:
// one thread per 4 consecutive outputs of a row.
template <int EPI>
__global__ __launch_bounds__(256) void small_reduce_kernel(SmallParams p) {
  const int64_t u = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t n4 = p.N / 4;
  if (u >= (int64_t)p.M * n4) return;
  const int64_t m = u / n4;
  const int n = (int)(u - m * n4) * 4;
  const size_t plane = (size_t)p.M * p.N;
  const float* src = p.part + (size_t)m * p.N + n;
  f32x4 s = *(const f32x4*)src;
  for (int k = 1; k < p.splits; ++k) {
    const f32x4 v = *(const f32x4*)(src + k * plane);
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

template <int EPI, bool PART>
hipError_t launch_small_kernel(const SmallParams& p, int nwg, hipStream_t st) {
  static bool configured = false;  // per instantiation; benign race (idempotent)
  auto kern = small_kernel<EPI, PART, kSteps>;
  constexpr int lds = kSteps * PAIR;
  if (!configured) {
    hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
    if (e != hipSuccess) return e;
    configured = true;
  }
  hipLaunchKernelGGL(kern, dim3(nwg), dim3(512), lds, st, p);
  return hipGetLastError();
}

// One wave that waits until `ticks` of the constant-rate wall clock have
// passed (bounded: it always exits).
__global__ __launch_bounds__(64) void delay_kernel(uint64_t ticks) {
  const uint64_t t0 = wall_clock64();
  while (wall_clock64() - t0 < ticks) __builtin_amdgcn_s_sleep(8);
}

}  // namespace

hipError_t launch_delay(int microseconds, hipStream_t stream) {
  int dev = 0, khz = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if ((e = hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev)) != hipSuccess) return e;
  const uint64_t ticks = (uint64_t)(khz > 0 ? khz : 100000) * (uint64_t)microseconds / 1000u;
  hipLaunchKernelGGL(delay_kernel, dim3(1), dim3(64), 0, stream, ticks);
  return hipGetLastError();
}

int64_t small_tiles(int64_t M, int64_t N) { return ((M + TM - 1) / TM) * ((N + TN - 1) / TN); }

hipError_t launch_linear_slab_small(const uint8_t* xq, const uint8_t* xs, int64_t M, int64_t K, const uint8_t* wq,
                                    const uint8_t* ws, int64_t N, const void* bias, int epi, void* y, int splits,
                                    float* part, hipStream_t stream) {
  SmallParams p;
  p.x = xq;
  p.xs = xs;
  p.wq = wq;
  p.ws = ws;
  p.bias = (const uint16_t*)bias;
  p.y = (uint16_t*)y;
  p.part = part;
  p.M = (int)M;
  p.N = (int)N;
  p.K = (int)K;
  p.RM = slab_rows(M);
  p.RN = slab_rows(N);
  p.tiles_m = (int)((M + TM - 1) / TM);
  p.tiles_n = (int)((N + TN - 1) / TN);
  p.splits = splits;
  const int nwg = p.tiles_m * p.tiles_n * p.splits;
  if (p.splits == 1)
    return epi == 1 ? launch_small_kernel<1, false>(p, nwg, stream) : launch_small_kernel<0, false>(p, nwg, stream);
  hipError_t e = launch_small_kernel<0, true>(p, nwg, stream);
  if (e != hipSuccess) return e;
  const unsigned nred = (unsigned)((M * (N / 4) + 255) / 256);
  if (epi == 1)
    hipLaunchKernelGGL(small_reduce_kernel<1>, dim3(nred), dim3(256), 0, stream, p);
  else
    hipLaunchKernelGGL(small_reduce_kernel<0>, dim3(nred), dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace mx
