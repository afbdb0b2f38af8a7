// C ABI of the MXFP8 W8A8 linear (include/mx.h): argument checks on the
// host, the gfx950 check, and the launches. Every argument check runs before
// any HIP call, so the error paths need no GPU.
#include <hip/hip_runtime_api.h>

#include <algorithm>
#include <atomic>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <map>
#include <mutex>
#include <tuple>

#include "mx.h"
#include "mx_internal.h"

namespace {

thread_local int t_last_hip = 0;
thread_local char t_msg[512] = "";

int fail(int status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(t_msg, sizeof(t_msg), fmt, ap);
  va_end(ap);
  return status;
}

int hip_fail(hipError_t e, const char* what) {
  t_last_hip = (int)e;
  return fail(MX_ERR_HIP, "%s failed: %s (%d)", what, hipGetErrorString(e), (int)e);
}

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p % a) == 0; }

// Byte ranges [a, a+na) and [b, b+nb) intersect.
bool overlap(const void* a, uint64_t na, const void* b, uint64_t nb) {
  if (a == nullptr || b == nullptr || na == 0 || nb == 0) return false;
  const uintptr_t pa = (uintptr_t)a, pb = (uintptr_t)b;
  return pa < pb + nb && pb < pa + na;
}

constexpr int64_t kMaxKN = int64_t(1) << 20;   // keeps in-tile byte offsets below 2^30
constexpr int64_t kMaxRows = int64_t(1) << 30;
constexpr int64_t kSplitTargetWorkgroups = 256;  // one workgroup per CU of an MI355X
constexpr int64_t kMaxSplitWorkgroups = int64_t(1) << 24;
constexpr int64_t kMaxAutoSplits = 8;  // 128 x 5120 x 5120: 8 splits 19.5 us, 12 splits 20.7 us
// Default plan: the few-token kernel up to 256 tokens (MI355X, K = 5120: 16.0
// vs 20.4 us at 128 tokens, 19.1 vs 25.7 at 256; split-K wins from 512).
constexpr int64_t kSmallMaxTokens = 256;
constexpr int64_t kTuneSmallMaxTokens = 1024;  // the tuner tries the few-token kernel up to here
constexpr int kMaxTuneCandidates = 24;

int check_k(int64_t K) {
  if (K <= 0 || K % 32 != 0) return fail(MX_ERR_INVALID_ARGUMENT, "K = %lld must be a positive multiple of 32", (long long)K);
  if (K > kMaxKN) return fail(MX_ERR_UNSUPPORTED, "K = %lld exceeds the supported 2^20", (long long)K);
  return MX_OK;
}

int check_rows(const char* name, int64_t R) {
  if (R < 0) return fail(MX_ERR_INVALID_ARGUMENT, "%s = %lld is negative", name, (long long)R);
  if (R > kMaxRows) return fail(MX_ERR_UNSUPPORTED, "%s = %lld exceeds the supported 2^30", name, (long long)R);
  return MX_OK;
}

// Current device is gfx950 (cached per device), unless forced off.
int check_device() {
  const char* force = getenv("MX_FORCE_UNSUPPORTED");
  if (force != nullptr && force[0] == '1') return fail(MX_ERR_UNSUPPORTED, "MX_FORCE_UNSUPPORTED=1");
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  static std::atomic<int> cache[64];  // 0 unknown, 1 gfx950, 2 other
  if (dev < 0 || dev >= 64) return fail(MX_ERR_UNSUPPORTED, "device index %d out of range", dev);
  int c = cache[dev].load(std::memory_order_acquire);
  if (c == 0) {
    hipDeviceProp_t prop;
    e = hipGetDeviceProperties(&prop, dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDeviceProperties");
    c = strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
    cache[dev].store(c, std::memory_order_release);
    if (c == 2) return fail(MX_ERR_UNSUPPORTED, "device %d is %s, not gfx950", dev, prop.gcnArchName);
  }
  if (c != 1) return fail(MX_ERR_UNSUPPORTED, "device %d is not gfx950", dev);
  return MX_OK;
}

int finish(hipError_t e, const char* what) {
  if (e != hipSuccess) return hip_fail(e, what);
  t_msg[0] = '\0';
  return MX_OK;
}

int check_linear_common(int64_t M, int64_t K, const uint8_t* wq, const uint8_t* ws, int64_t N, const void* bias,
                        int epilogue, const void* y) {
  int st;
  if ((st = check_rows("M", M)) != MX_OK) return st;
  if ((st = check_k(K)) != MX_OK) return st;
  if (N < 0) return fail(MX_ERR_INVALID_ARGUMENT, "N = %lld is negative", (long long)N);
  if (N > kMaxKN) return fail(MX_ERR_UNSUPPORTED, "N = %lld exceeds the supported 2^20", (long long)N);
  if (epilogue != MX_EPI_NONE && epilogue != MX_EPI_GELU_TANH)
    return fail(MX_ERR_INVALID_ARGUMENT, "unknown epilogue %d", epilogue);
  if (M == 0 || N == 0) return MX_OK;
  if (N % 16 != 0) return fail(MX_ERR_UNSUPPORTED, "N = %lld must be a multiple of 16", (long long)N);
  if (wq == nullptr || ws == nullptr || y == nullptr) return fail(MX_ERR_INVALID_ARGUMENT, "NULL weight or output pointer");
  if (!aligned(wq, 16) || !aligned(y, 16)) return fail(MX_ERR_INVALID_ARGUMENT, "wq and y must be 16-byte aligned");
  if (bias != nullptr && !aligned(bias, 2)) return fail(MX_ERR_INVALID_ARGUMENT, "bias must be 2-byte aligned");
  const uint64_t ybytes = (uint64_t)M * N * 2;
  if (overlap(y, ybytes, wq, (uint64_t)N * K) || overlap(y, ybytes, ws, (uint64_t)N * (K / 32)) ||
      overlap(y, ybytes, bias, (uint64_t)N * 2))
    return fail(MX_ERR_INVALID_ARGUMENT, "y overlaps an input");
  return MX_OK;
}

// Quantizer arguments: x [rows][ld] of dtype dt; outputs row-major or slab.
int check_quantize(const void* x, int dt, int64_t rows, int64_t K, int64_t ld, const uint8_t* q, const uint8_t* s,
                   bool slab) {
  int st;
  if (dt != MX_DT_BF16 && dt != MX_DT_F32) return fail(MX_ERR_INVALID_ARGUMENT, "unknown weight dtype %d", dt);
  if ((st = check_rows("rows", rows)) != MX_OK) return st;
  if ((st = check_k(K)) != MX_OK) return st;
  if (slab && K % 64 != 0)
    return fail(MX_ERR_INVALID_ARGUMENT, "K = %lld must be a multiple of 64 for the slab layout", (long long)K);
  const int64_t es = dt == MX_DT_F32 ? 4 : 2;
  if (ld < K || (ld * es) % 16 != 0)
    return fail(MX_ERR_INVALID_ARGUMENT, "pitch %lld must be >= K with 16-byte aligned rows", (long long)ld);
  if (rows == 0) return MX_OK;
  if (x == nullptr || q == nullptr || s == nullptr) return fail(MX_ERR_INVALID_ARGUMENT, "NULL pointer");
  if (!aligned(x, 16) || !aligned(q, 16)) return fail(MX_ERR_INVALID_ARGUMENT, "input and codes must be 16-byte aligned");
  const uint64_t R = slab ? (uint64_t)mx::slab_rows(rows) : (uint64_t)rows;
  const uint64_t xbytes = ((uint64_t)(rows - 1) * ld + K) * es;
  const uint64_t nq = R * K, ns = R * (K / 32);
  if (overlap(q, nq, x, xbytes) || overlap(s, ns, x, xbytes) || overlap(q, nq, s, ns))
    return fail(MX_ERR_INVALID_ARGUMENT, "outputs overlap an input or each other");
  return check_device();
}

// Slab-linear operand arguments (shared by the bf16 and requantizing outputs).
int check_linear_slab(const uint8_t* xq, const uint8_t* xs, int64_t M, int64_t K, const uint8_t* wq,
                      const uint8_t* ws, int64_t N, const void* bias, int epilogue) {
  int st;
  if ((st = check_rows("M", M)) != MX_OK) return st;
  if ((st = check_k(K)) != MX_OK) return st;
  if (K % 64 != 0) return fail(MX_ERR_INVALID_ARGUMENT, "K = %lld must be a multiple of 64 for the slab layout", (long long)K);
  if (N < 0) return fail(MX_ERR_INVALID_ARGUMENT, "N = %lld is negative", (long long)N);
  if (N > kMaxKN) return fail(MX_ERR_UNSUPPORTED, "N = %lld exceeds the supported 2^20", (long long)N);
  if (epilogue != MX_EPI_NONE && epilogue != MX_EPI_GELU_TANH)
    return fail(MX_ERR_INVALID_ARGUMENT, "unknown epilogue %d", epilogue);
  if (M == 0 || N == 0) return MX_OK;
  if (N % 16 != 0) return fail(MX_ERR_UNSUPPORTED, "N = %lld must be a multiple of 16", (long long)N);
  if (xq == nullptr || xs == nullptr || wq == nullptr || ws == nullptr)
    return fail(MX_ERR_INVALID_ARGUMENT, "NULL operand pointer");
  if (!aligned(xq, 16) || !aligned(wq, 16) || !aligned(xs, 4) || !aligned(ws, 4))
    return fail(MX_ERR_INVALID_ARGUMENT, "codes must be 16-byte aligned, scales 4-byte aligned");
  if (bias != nullptr && !aligned(bias, 2)) return fail(MX_ERR_INVALID_ARGUMENT, "bias must be 2-byte aligned");
  return MX_OK;
}

// An output range [out, out + bytes) must not overlap any slab-linear input.
int check_slab_output(const uint8_t* xq, const uint8_t* xs, int64_t M, int64_t K, const uint8_t* wq,
                      const uint8_t* ws, int64_t N, const void* bias, const void* out, uint64_t bytes,
                      const char* name) {
  const uint64_t RM = (uint64_t)mx::slab_rows(M), RN = (uint64_t)mx::slab_rows(N);
  if (overlap(out, bytes, xq, RM * K) || overlap(out, bytes, xs, RM * (K / 32)) || overlap(out, bytes, wq, RN * K) ||
      overlap(out, bytes, ws, RN * (K / 32)) || overlap(out, bytes, bias, (uint64_t)N * 2))
    return fail(MX_ERR_INVALID_ARGUMENT, "%s overlaps an input", name);
  return MX_OK;
}

// Per-channel quantizer arguments: x [rows][ld] of dtype dt; slab codes, f32 row scales.
int check_pc_quantize(const void* x, int dt, int64_t rows, int64_t K, int64_t ld, const uint8_t* q,
                      const float* sc) {
  int st;
  if (dt != MX_DT_BF16 && dt != MX_DT_F32) return fail(MX_ERR_INVALID_ARGUMENT, "unknown weight dtype %d", dt);
  if ((st = check_rows("rows", rows)) != MX_OK) return st;
  if ((st = check_k(K)) != MX_OK) return st;
  if (K % 64 != 0) return fail(MX_ERR_INVALID_ARGUMENT, "K = %lld must be a multiple of 64 for the slab layout", (long long)K);
  const int64_t es = dt == MX_DT_F32 ? 4 : 2;
  if (ld < K || (ld * es) % 16 != 0)
    return fail(MX_ERR_INVALID_ARGUMENT, "pitch %lld must be >= K with 16-byte aligned rows", (long long)ld);
  if (rows == 0) return MX_OK;
  if (x == nullptr || q == nullptr || sc == nullptr) return fail(MX_ERR_INVALID_ARGUMENT, "NULL pointer");
  if (!aligned(x, 16) || !aligned(q, 16) || !aligned(sc, 4))
    return fail(MX_ERR_INVALID_ARGUMENT, "input and codes must be 16-byte aligned, scales 4-byte aligned");
  const uint64_t R = (uint64_t)mx::slab_rows(rows);
  const uint64_t xbytes = ((uint64_t)(rows - 1) * ld + K) * es;
  const uint64_t nq = R * K, ns = R * 4;
  if (overlap(q, nq, x, xbytes) || overlap(sc, ns, x, xbytes) || overlap(q, nq, sc, ns))
    return fail(MX_ERR_INVALID_ARGUMENT, "outputs overlap an input or each other");
  return check_device();
}

// Shape limits of the few-token kernel: it addresses a tile's K range with
// 32-bit offsets that run a few slabs past it, and launches tiles x splits
// workgroups.
int check_small_shape(int64_t M, int64_t K, int64_t N, int splits) {
  const int64_t span = K / 64 + 16;
  if (span * mx::slab_rows(M) * 64 >= (int64_t(1) << 31) || span * mx::slab_rows(N) * 64 >= (int64_t(1) << 31))
    return fail(MX_ERR_UNSUPPORTED, "(K/64 + 16) * 64 * rows must be below 2^31 for M and N (M = %lld, N = %lld)",
                (long long)M, (long long)N);
  const int64_t tiles = mx::small_tiles(M, N);
  if (tiles * splits > kMaxSplitWorkgroups)
    return fail(MX_ERR_UNSUPPORTED, "%lld tiles x %d splits exceed 2^24 workgroups", (long long)tiles, splits);
  return MX_OK;
}

// Split-K on 256 x 256 tiles launches tiles x splits workgroups.
int check_splitk_shape(int64_t M, int64_t N, int splits) {
  const int64_t tiles = ((M + 255) / 256) * ((N + 255) / 256);
  if (tiles * splits > kMaxSplitWorkgroups)
    return fail(MX_ERR_UNSUPPORTED, "%lld tiles x %d splits exceed 2^24 workgroups", (long long)tiles, splits);
  return MX_OK;
}

// Compute units of the current device (the balanced GEMM's round size).
int cu_count() {
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      n <= 0)
    return 256;
  return n;
}

}  // namespace

extern "C" {

int mx_abi_version(void) { return MX_ABI_VERSION; }

const char* mx_status_string(int status) {
  switch (status) {
    case MX_OK: return "MX_OK";
    case MX_ERR_INVALID_ARGUMENT: return "MX_ERR_INVALID_ARGUMENT";
    case MX_ERR_UNSUPPORTED: return "MX_ERR_UNSUPPORTED";
    case MX_ERR_HIP: return "MX_ERR_HIP";
    default: return "MX_UNKNOWN_STATUS";
  }
}

int mx_last_hip_error(void) { return t_last_hip; }

const char* mx_last_error_message(void) { return t_msg; }

int mx_quantize_act(const void* x, int64_t M, int64_t K, int64_t ldx, uint8_t* q, uint8_t* s, void* stream) {
  const int st = check_quantize(x, MX_DT_BF16, M, K, ldx, q, s, false);
  if (st != MX_OK || M == 0) return st;
  (void)hipGetLastError();
  return finish(mx::launch_quantize(0, x, M, K, ldx, q, s, (hipStream_t)stream), "quantize launch");
}

int mx_quantize_weight(const void* w, int wdtype, int64_t N, int64_t K, int64_t ldw, uint8_t* q, uint8_t* s,
                       void* stream) {
  const int st = check_quantize(w, wdtype, N, K, ldw, q, s, false);
  if (st != MX_OK || N == 0) return st;
  (void)hipGetLastError();
  return finish(mx::launch_quantize(wdtype == MX_DT_F32 ? 1 : 0, w, N, K, ldw, q, s, (hipStream_t)stream),
                "quantize launch");
}

int64_t mx_slab_rows(int64_t rows) { return rows < 0 ? -1 : mx::slab_rows(rows); }

int mx_quantize_act_slab(const void* x, int64_t M, int64_t K, int64_t ldx, uint8_t* q, uint8_t* s, void* stream) {
  const int st = check_quantize(x, MX_DT_BF16, M, K, ldx, q, s, true);
  if (st != MX_OK || M == 0) return st;
  (void)hipGetLastError();
  return finish(mx::launch_quantize_slab(0, x, M, K, ldx, q, s, (hipStream_t)stream), "quantize launch");
}

int mx_quantize_weight_slab(const void* w, int wdtype, int64_t N, int64_t K, int64_t ldw, uint8_t* q, uint8_t* s,
                            void* stream) {
  const int st = check_quantize(w, wdtype, N, K, ldw, q, s, true);
  if (st != MX_OK || N == 0) return st;
  (void)hipGetLastError();
  return finish(mx::launch_quantize_slab(wdtype == MX_DT_F32 ? 1 : 0, w, N, K, ldw, q, s, (hipStream_t)stream),
                "quantize launch");
}

int mx_slab_pack(const uint8_t* q, const uint8_t* s, int64_t rows, int64_t K, uint8_t* qslab, uint8_t* sslab,
                 void* stream) {
  int st;
  if ((st = check_rows("rows", rows)) != MX_OK) return st;
  if ((st = check_k(K)) != MX_OK) return st;
  if (K % 64 != 0) return fail(MX_ERR_INVALID_ARGUMENT, "K = %lld must be a multiple of 64 for the slab layout", (long long)K);
  if (rows == 0) return MX_OK;
  if (q == nullptr || s == nullptr || qslab == nullptr || sslab == nullptr)
    return fail(MX_ERR_INVALID_ARGUMENT, "NULL pointer");
  if (!aligned(q, 16) || !aligned(qslab, 16) || !aligned(s, 2) || !aligned(sslab, 2))
    return fail(MX_ERR_INVALID_ARGUMENT, "codes must be 16-byte and scales 2-byte aligned");
  const uint64_t R = (uint64_t)mx::slab_rows(rows);
  const uint64_t nq = (uint64_t)rows * K, ns = (uint64_t)rows * (K / 32);
  const uint64_t oq = R * K, os = R * (K / 32);
  if (overlap(qslab, oq, q, nq) || overlap(qslab, oq, s, ns) || overlap(sslab, os, q, nq) ||
      overlap(sslab, os, s, ns) || overlap(qslab, oq, sslab, os))
    return fail(MX_ERR_INVALID_ARGUMENT, "outputs overlap an input or each other");
  if ((st = check_device()) != MX_OK) return st;
  (void)hipGetLastError();
  return finish(mx::launch_slab_pack(q, s, rows, K, qslab, sslab, (hipStream_t)stream), "slab pack launch");
}

int mx_linear_fused(const void* x, int64_t M, int64_t K, const uint8_t* wq, const uint8_t* ws, int64_t N,
                    const void* bias, int epilogue, void* y, void* stream) {
  int st = check_linear_common(M, K, wq, ws, N, bias, epilogue, y);
  if (st != MX_OK || M == 0 || N == 0) return st;
  if (x == nullptr) return fail(MX_ERR_INVALID_ARGUMENT, "NULL x");
  if (!aligned(x, 16)) return fail(MX_ERR_INVALID_ARGUMENT, "x must be 16-byte aligned");
  if (overlap(y, (uint64_t)M * N * 2, x, (uint64_t)M * K * 2)) return fail(MX_ERR_INVALID_ARGUMENT, "y overlaps x");
  if ((st = check_device()) != MX_OK) return st;
  (void)hipGetLastError();
  return finish(mx::launch_linear(x, nullptr, M, K, wq, ws, N, bias, epilogue, y, (hipStream_t)stream), "linear launch");
}

int mx_linear_q(const uint8_t* xq, const uint8_t* xs, int64_t M, int64_t K, const uint8_t* wq, const uint8_t* ws,
                int64_t N, const void* bias, int epilogue, void* y, void* stream) {
  int st = check_linear_common(M, K, wq, ws, N, bias, epilogue, y);
  if (st != MX_OK || M == 0 || N == 0) return st;
  if (xq == nullptr || xs == nullptr) return fail(MX_ERR_INVALID_ARGUMENT, "NULL xq or xs");
  if (!aligned(xq, 16)) return fail(MX_ERR_INVALID_ARGUMENT, "xq must be 16-byte aligned");
  const uint64_t yb = (uint64_t)M * N * 2;
  if (overlap(y, yb, xq, (uint64_t)M * K) || overlap(y, yb, xs, (uint64_t)M * (K / 32)))
    return fail(MX_ERR_INVALID_ARGUMENT, "y overlaps xq or xs");
  if ((st = check_device()) != MX_OK) return st;
  (void)hipGetLastError();
  return finish(mx::launch_linear(xq, xs, M, K, wq, ws, N, bias, epilogue, y, (hipStream_t)stream), "linear launch");
}

int mx_linear_slab(const uint8_t* xq, const uint8_t* xs, int64_t M, int64_t K, const uint8_t* wq, const uint8_t* ws,
                   int64_t N, const void* bias, int epilogue, void* y, void* stream) {
  int st = check_linear_slab(xq, xs, M, K, wq, ws, N, bias, epilogue);
  if (st != MX_OK || M == 0 || N == 0) return st;
  if (y == nullptr) return fail(MX_ERR_INVALID_ARGUMENT, "NULL y");
  if (!aligned(y, 16)) return fail(MX_ERR_INVALID_ARGUMENT, "y must be 16-byte aligned");
  if ((st = check_slab_output(xq, xs, M, K, wq, ws, N, bias, y, (uint64_t)M * N * 2, "y")) != MX_OK) return st;
  if ((st = check_device()) != MX_OK) return st;
  (void)hipGetLastError();
  return finish(mx::launch_linear_slab(xq, xs, M, K, wq, ws, N, bias, epilogue, y, (hipStream_t)stream),
                "linear launch");
}

int mx_linear_slab_m128(const uint8_t* xq, const uint8_t* xs, int64_t M, int64_t K, const uint8_t* wq,
                        const uint8_t* ws, int64_t N, const void* bias, int epilogue, void* y, void* stream) {
  int st = check_linear_slab(xq, xs, M, K, wq, ws, N, bias, epilogue);
  if (st != MX_OK || M == 0 || N == 0) return st;
  if (y == nullptr) return fail(MX_ERR_INVALID_ARGUMENT, "NULL y");
  if (!aligned(y, 16)) return fail(MX_ERR_INVALID_ARGUMENT, "y must be 16-byte aligned");
  if ((st = check_slab_output(xq, xs, M, K, wq, ws, N, bias, y, (uint64_t)M * N * 2, "y")) != MX_OK) return st;
  if ((st = check_device()) != MX_OK) return st;
  (void)hipGetLastError();
  return finish(mx::launch_linear_slab_m128(xq, xs, M, K, wq, ws, N, bias, epilogue, y, (hipStream_t)stream),
                "linear launch");
}

int mx_linear_slab_requant(const uint8_t* xq, const uint8_t* xs, int64_t M, int64_t K, const uint8_t* wq,
                           const uint8_t* ws, int64_t N, const void* bias, int epilogue, uint8_t* hq, uint8_t* hs,
                           void* stream) {
  int st = check_linear_slab(xq, xs, M, K, wq, ws, N, bias, epilogue);
  if (st != MX_OK || M == 0 || N == 0) return st;
  if (N % 64 != 0)
    return fail(MX_ERR_INVALID_ARGUMENT, "N = %lld must be a multiple of 64 (it is the next linear's K)", (long long)N);
  if (hq == nullptr || hs == nullptr) return fail(MX_ERR_INVALID_ARGUMENT, "NULL hq or hs");
  if (!aligned(hq, 16)) return fail(MX_ERR_INVALID_ARGUMENT, "hq must be 16-byte aligned");
  const uint64_t RM = (uint64_t)mx::slab_rows(M);
  if (RM * (uint64_t)N >= (uint64_t(1) << 31))
    return fail(MX_ERR_UNSUPPORTED, "output slab of %llu bytes exceeds 2^31", (unsigned long long)(RM * N));
  if ((st = check_slab_output(xq, xs, M, K, wq, ws, N, bias, hq, RM * N, "hq")) != MX_OK) return st;
  if ((st = check_slab_output(xq, xs, M, K, wq, ws, N, bias, hs, RM * (N / 32), "hs")) != MX_OK) return st;
  if (overlap(hq, RM * N, hs, RM * (N / 32))) return fail(MX_ERR_INVALID_ARGUMENT, "hq overlaps hs");
  if ((st = check_device()) != MX_OK) return st;
  (void)hipGetLastError();
  return finish(mx::launch_linear_slab_requant(xq, xs, M, K, wq, ws, N, bias, epilogue, hq, hs, (hipStream_t)stream),
                "linear launch");
}

int64_t mx_linear_splitk_ws_bytes(int64_t M, int64_t N, int splits) {
  if (M < 0 || N < 0 || M > kMaxRows || N > kMaxKN || splits < 1 || splits > kMaxKN / 64) return -1;
  const int64_t tiles = ((M + 255) / 256) * ((N + 255) / 256);
  return (int64_t)splits * tiles * 65536 * 4;
}

int mx_linear_splitk_choose(int64_t M, int64_t K, int64_t N) {
  if (M <= 0 || N <= 0 || K < 64 || K % 64 != 0 || M > kMaxRows || N > kMaxKN || K > kMaxKN) return 1;
  const int64_t tiles = ((M + 255) / 256) * ((N + 255) / 256);
  const int64_t nh = K / 64;
  int64_t s = kSplitTargetWorkgroups / tiles;  // fill the CUs once, without a second partial round
  s = std::min<int64_t>(s, kMaxAutoSplits);    // partial-sum traffic grows with the split count
  s = std::min<int64_t>(s, nh / 2);            // at least two half-steps per range
  return (int)std::max<int64_t>(s, 1);
}

int mx_linear_slab_splitk(const uint8_t* xq, const uint8_t* xs, int64_t M, int64_t K, const uint8_t* wq,
                          const uint8_t* ws, int64_t N, const void* bias, int epilogue, void* y, int splits,
                          void* workspace, int64_t workspace_bytes, void* stream) {
  int st = check_linear_slab(xq, xs, M, K, wq, ws, N, bias, epilogue);
  if (st != MX_OK) return st;
  if (splits < 1 || splits > K / 64)
    return fail(MX_ERR_INVALID_ARGUMENT, "splits = %d must be in [1, K/64 = %lld]", splits, (long long)(K / 64));
  if (M == 0 || N == 0) return MX_OK;
  if (y == nullptr || workspace == nullptr) return fail(MX_ERR_INVALID_ARGUMENT, "NULL y or workspace");
  if (!aligned(y, 16) || !aligned(workspace, 256))
    return fail(MX_ERR_INVALID_ARGUMENT, "y must be 16-byte aligned, workspace 256-byte aligned");
  if ((st = check_splitk_shape(M, N, splits)) != MX_OK) return st;
  const int64_t need = mx_linear_splitk_ws_bytes(M, N, splits);
  if (workspace_bytes < need)
    return fail(MX_ERR_INVALID_ARGUMENT, "workspace of %lld bytes, %lld needed", (long long)workspace_bytes, (long long)need);
  const uint64_t ybytes = (uint64_t)M * N * 2;
  if ((st = check_slab_output(xq, xs, M, K, wq, ws, N, bias, y, ybytes, "y")) != MX_OK) return st;
  if ((st = check_slab_output(xq, xs, M, K, wq, ws, N, bias, workspace, (uint64_t)need, "workspace")) != MX_OK)
    return st;
  if (overlap(workspace, (uint64_t)need, y, ybytes)) return fail(MX_ERR_INVALID_ARGUMENT, "workspace overlaps y");
  if ((st = check_device()) != MX_OK) return st;
  (void)hipGetLastError();
  return finish(mx::launch_linear_slab_splitk(xq, xs, M, K, wq, ws, N, bias, epilogue, y, splits, (float*)workspace,
                                              (hipStream_t)stream),
                "linear launch");
}

int64_t mx_linear_small_ws_bytes(int64_t M, int64_t N, int splits) {
  if (M < 0 || N < 0 || M > kMaxRows || N > kMaxKN || splits < 1 || splits > kMaxKN / 64) return -1;
  return splits > 1 ? (int64_t)splits * M * N * 4 : 0;
}

int mx_linear_small_choose(int64_t M, int64_t K, int64_t N) {
  if (M <= 0 || N <= 0 || K < 64 || K % 64 != 0 || M > kMaxRows || N > kMaxKN || K > kMaxKN) return 1;
  int64_t s = cu_count() / mx::small_tiles(M, N);  // about one workgroup per CU
  s = std::min<int64_t>(s, kMaxAutoSplits);         // partial-sum traffic grows with the split count
  s = std::min<int64_t>(s, K / 128);                // at least two 64-K slabs per range
  return (int)std::max<int64_t>(s, 1);
}

int mx_linear_slab_small(const uint8_t* xq, const uint8_t* xs, int64_t M, int64_t K, const uint8_t* wq,
                         const uint8_t* ws, int64_t N, const void* bias, int epilogue, void* y, int splits,
                         void* workspace, int64_t workspace_bytes, void* stream) {
  int st = check_linear_slab(xq, xs, M, K, wq, ws, N, bias, epilogue);
  if (st != MX_OK) return st;
  if (splits < 1 || splits > K / 64)
    return fail(MX_ERR_INVALID_ARGUMENT, "splits = %d must be in [1, K/64 = %lld]", splits, (long long)(K / 64));
  if (M == 0 || N == 0) return MX_OK;
  if (y == nullptr) return fail(MX_ERR_INVALID_ARGUMENT, "NULL y");
  if (!aligned(y, 16)) return fail(MX_ERR_INVALID_ARGUMENT, "y must be 16-byte aligned");
  if ((st = check_small_shape(M, K, N, splits)) != MX_OK) return st;
  const int64_t need = mx_linear_small_ws_bytes(M, N, splits);
  const uint64_t ybytes = (uint64_t)M * N * 2;
  if ((st = check_slab_output(xq, xs, M, K, wq, ws, N, bias, y, ybytes, "y")) != MX_OK) return st;
  if (need > 0) {
    if (workspace == nullptr) return fail(MX_ERR_INVALID_ARGUMENT, "NULL workspace (%lld bytes needed)", (long long)need);
    if (!aligned(workspace, 256)) return fail(MX_ERR_INVALID_ARGUMENT, "workspace must be 256-byte aligned");
    if (workspace_bytes < need)
      return fail(MX_ERR_INVALID_ARGUMENT, "workspace of %lld bytes, %lld needed", (long long)workspace_bytes,
                  (long long)need);
    if ((st = check_slab_output(xq, xs, M, K, wq, ws, N, bias, workspace, (uint64_t)need, "workspace")) != MX_OK)
      return st;
    if (overlap(workspace, (uint64_t)need, y, ybytes)) return fail(MX_ERR_INVALID_ARGUMENT, "workspace overlaps y");
  }
  if ((st = check_device()) != MX_OK) return st;
  (void)hipGetLastError();
  return finish(mx::launch_linear_slab_small(xq, xs, M, K, wq, ws, N, bias, epilogue, y, splits, (float*)workspace,
                                             (hipStream_t)stream),
                "linear launch");
}

int mx_pc_quantize_act_slab(const void* x, int64_t M, int64_t K, int64_t ldx, uint8_t* q, float* s, void* stream) {
  const int st = check_pc_quantize(x, MX_DT_BF16, M, K, ldx, q, s);
  if (st != MX_OK || M == 0) return st;
  (void)hipGetLastError();
  return finish(mx::launch_pc_quantize_slab(0, x, M, K, ldx, q, s, (hipStream_t)stream), "quantize launch");
}

int mx_pc_quantize_weight_slab(const void* w, int wdtype, int64_t N, int64_t K, int64_t ldw, uint8_t* q, float* s,
                               void* stream) {
  const int st = check_pc_quantize(w, wdtype, N, K, ldw, q, s);
  if (st != MX_OK || N == 0) return st;
  (void)hipGetLastError();
  return finish(mx::launch_pc_quantize_slab(wdtype == MX_DT_F32 ? 1 : 0, w, N, K, ldw, q, s, (hipStream_t)stream),
                "quantize launch");
}

int mx_pc_linear_slab(const uint8_t* xq, const float* xs, int64_t M, int64_t K, const uint8_t* wq, const float* ws,
                      int64_t N, const void* bias, int epilogue, void* y, void* stream) {
  int st;
  if ((st = check_rows("M", M)) != MX_OK) return st;
  if ((st = check_k(K)) != MX_OK) return st;
  if (K % 64 != 0) return fail(MX_ERR_INVALID_ARGUMENT, "K = %lld must be a multiple of 64 for the slab layout", (long long)K);
  if (N < 0) return fail(MX_ERR_INVALID_ARGUMENT, "N = %lld is negative", (long long)N);
  if (N > kMaxKN) return fail(MX_ERR_UNSUPPORTED, "N = %lld exceeds the supported 2^20", (long long)N);
  if (epilogue != MX_EPI_NONE && epilogue != MX_EPI_GELU_TANH)
    return fail(MX_ERR_INVALID_ARGUMENT, "unknown epilogue %d", epilogue);
  if (M == 0 || N == 0) return MX_OK;
  if (N % 16 != 0) return fail(MX_ERR_UNSUPPORTED, "N = %lld must be a multiple of 16", (long long)N);
  if (xq == nullptr || xs == nullptr || wq == nullptr || ws == nullptr || y == nullptr)
    return fail(MX_ERR_INVALID_ARGUMENT, "NULL operand or output pointer");
  if (!aligned(xq, 16) || !aligned(wq, 16) || !aligned(xs, 4) || !aligned(ws, 4) || !aligned(y, 16))
    return fail(MX_ERR_INVALID_ARGUMENT, "codes and y must be 16-byte aligned, scales 4-byte aligned");
  if (bias != nullptr && !aligned(bias, 2)) return fail(MX_ERR_INVALID_ARGUMENT, "bias must be 2-byte aligned");
  const uint64_t RM = (uint64_t)mx::slab_rows(M), RN = (uint64_t)mx::slab_rows(N);
  const uint64_t yb = (uint64_t)M * N * 2;
  if (overlap(y, yb, xq, RM * K) || overlap(y, yb, xs, RM * 4) || overlap(y, yb, wq, RN * K) ||
      overlap(y, yb, ws, RN * 4) || overlap(y, yb, bias, (uint64_t)N * 2))
    return fail(MX_ERR_INVALID_ARGUMENT, "y overlaps an input");
  if ((st = check_device()) != MX_OK) return st;
  (void)hipGetLastError();
  return finish(mx::launch_pc_linear_slab(xq, xs, M, K, wq, ws, N, bias, epilogue, y, (hipStream_t)stream),
                "linear launch");
}

int64_t mx_linear_balanced_ws_bytes(int64_t M, int64_t K, int64_t N) {
  if (M < 0 || N < 0 || K <= 0 || K % 64 != 0 || M > kMaxRows || N > kMaxKN || K > kMaxKN) return -1;
  if (M == 0 || N == 0) return 0;
  int64_t full;
  int splits;
  return mx::balanced_plan(M, K, N, cu_count(), &full, &splits);
}

int mx_linear_slab_balanced(const uint8_t* xq, const uint8_t* xs, int64_t M, int64_t K, const uint8_t* wq,
                            const uint8_t* ws, int64_t N, const void* bias, int epilogue, void* y, void* workspace,
                            int64_t workspace_bytes, void* stream) {
  int st = check_linear_slab(xq, xs, M, K, wq, ws, N, bias, epilogue);
  if (st != MX_OK || M == 0 || N == 0) return st;
  if (y == nullptr) return fail(MX_ERR_INVALID_ARGUMENT, "NULL y");
  if (!aligned(y, 16)) return fail(MX_ERR_INVALID_ARGUMENT, "y must be 16-byte aligned");
  const uint64_t ybytes = (uint64_t)M * N * 2;
  if ((st = check_slab_output(xq, xs, M, K, wq, ws, N, bias, y, ybytes, "y")) != MX_OK) return st;
  const int ncu = cu_count();
  int64_t full;
  int splits;
  const int64_t need = mx::balanced_plan(M, K, N, ncu, &full, &splits);
  if (need > 0) {
    if (workspace == nullptr || !aligned(workspace, 256))
      return fail(MX_ERR_INVALID_ARGUMENT, "workspace must be non-NULL and 256-byte aligned");
    if (workspace_bytes < need)
      return fail(MX_ERR_INVALID_ARGUMENT, "workspace of %lld bytes, %lld needed", (long long)workspace_bytes,
                  (long long)need);
    if ((st = check_slab_output(xq, xs, M, K, wq, ws, N, bias, workspace, (uint64_t)need, "workspace")) != MX_OK)
      return st;
    if (overlap(workspace, (uint64_t)need, y, ybytes)) return fail(MX_ERR_INVALID_ARGUMENT, "workspace overlaps y");
  }
  if ((st = check_device()) != MX_OK) return st;
  (void)hipGetLastError();
  return finish(mx::launch_linear_slab_balanced(xq, xs, M, K, wq, ws, N, bias, epilogue, y, ncu, (float*)workspace,
                                                (hipStream_t)stream),
                "linear launch");
}

/* ---- Per-shape plans: default rule, tuner, process-local cache ---------- */

int mx_linear_plan_default(int64_t M, int64_t K, int64_t N, int* kind, int* splits) {
  if (kind == nullptr || splits == nullptr) return fail(MX_ERR_INVALID_ARGUMENT, "NULL kind or splits");
  if (M < 0 || N < 0 || K < 64 || K % 64 != 0 || M > kMaxRows || N > kMaxKN || K > kMaxKN)
    return fail(MX_ERR_INVALID_ARGUMENT, "bad shape %lld x %lld x %lld", (long long)M, (long long)K, (long long)N);
  const int64_t tiles = ((M + 255) / 256) * ((N + 255) / 256);
  if (M > 0 && M <= kSmallMaxTokens) {
    *kind = MX_PLAN_SMALL;
    *splits = mx_linear_small_choose(M, K, N);
  } else if (2 * tiles <= kSplitTargetWorkgroups && 8 * tiles >= kSplitTargetWorkgroups) {
    // One round of 128-token tiles keeps at least a quarter of the CUs busy:
    // measured faster than split-K there (512 x 5120 x 10240: 31.5 against
    // 45.9 us; 512 x 5120 x 5120: 26.0 against 30.8), with no partial sums.
    *kind = MX_PLAN_SLAB_M128;
    *splits = 1;
  } else {
    const int s = mx_linear_splitk_choose(M, K, N);
    *kind = s > 1 ? MX_PLAN_SPLITK : MX_PLAN_SLAB;
    *splits = s > 1 ? s : 1;
  }
  t_msg[0] = '\0';
  return MX_OK;
}

int64_t mx_linear_plan_ws_bytes(int kind, int splits, int64_t M, int64_t K, int64_t N) {
  if (M < 0 || N < 0 || K < 64 || K % 64 != 0 || M > kMaxRows || N > kMaxKN || K > kMaxKN) return -1;
  switch (kind) {
    case MX_PLAN_SLAB:
      return splits == 1 ? 0 : -1;
    case MX_PLAN_SPLITK:
      return mx_linear_splitk_ws_bytes(M, N, splits);
    case MX_PLAN_SMALL:
      return mx_linear_small_ws_bytes(M, N, splits);
    case MX_PLAN_BALANCED:
      return splits == 1 ? mx_linear_balanced_ws_bytes(M, K, N) : -1;
    case MX_PLAN_SLAB_M128:
      return splits == 1 ? 0 : -1;
    default:
      return -1;
  }
}

int mx_linear_slab_plan(int kind, int splits, const uint8_t* xq, const uint8_t* xs, int64_t M, int64_t K,
                        const uint8_t* wq, const uint8_t* ws, int64_t N, const void* bias, int epilogue, void* y,
                        void* workspace, int64_t workspace_bytes, void* stream) {
  switch (kind) {
    case MX_PLAN_SLAB:
      if (splits != 1) return fail(MX_ERR_INVALID_ARGUMENT, "the slab plan takes splits = 1, not %d", splits);
      return mx_linear_slab(xq, xs, M, K, wq, ws, N, bias, epilogue, y, stream);
    case MX_PLAN_SPLITK:
      return mx_linear_slab_splitk(xq, xs, M, K, wq, ws, N, bias, epilogue, y, splits, workspace, workspace_bytes,
                                   stream);
    case MX_PLAN_SMALL:
      return mx_linear_slab_small(xq, xs, M, K, wq, ws, N, bias, epilogue, y, splits, workspace, workspace_bytes,
                                  stream);
    case MX_PLAN_BALANCED:
      if (splits != 1) return fail(MX_ERR_INVALID_ARGUMENT, "the balanced plan takes splits = 1, not %d", splits);
      return mx_linear_slab_balanced(xq, xs, M, K, wq, ws, N, bias, epilogue, y, workspace, workspace_bytes, stream);
    case MX_PLAN_SLAB_M128:
      if (splits != 1) return fail(MX_ERR_INVALID_ARGUMENT, "the 128-token-tile plan takes splits = 1, not %d", splits);
      return mx_linear_slab_m128(xq, xs, M, K, wq, ws, N, bias, epilogue, y, stream);
    default:
      return fail(MX_ERR_INVALID_ARGUMENT, "unknown plan kind %d", kind);
  }
}

}  // extern "C"

namespace {

struct Plan {
  int kind, splits;
};

// Candidate plans of the tuner for one shape (the default plan first).
int tune_candidates(int64_t M, int64_t K, int64_t N, Plan* out, int cap) {
  int n = 0;
  auto add = [&](int kind, int splits) {
    for (int i = 0; i < n; ++i)
      if (out[i].kind == kind && out[i].splits == splits) return;
    if (n < cap) out[n++] = Plan{kind, splits};
  };
  int k0, s0;
  if (mx_linear_plan_default(M, K, N, &k0, &s0) != MX_OK) return 0;
  add(k0, s0);
  add(MX_PLAN_SLAB, 1);
  const int64_t nh = K / 64;
  const int64_t tiles = ((M + 255) / 256) * ((N + 255) / 256);
  static const int kSplits[] = {2, 3, 4, 6, 8};
  if (tiles < cu_count()) {
    for (int s : kSplits)
      if (s <= nh) add(MX_PLAN_SPLITK, s);
  }
  if (M > 128 && tiles < 2 * cu_count()) add(MX_PLAN_SLAB_M128, 1);
  if (M <= kTuneSmallMaxTokens) {
    add(MX_PLAN_SMALL, 1);
    for (int s : kSplits)
      if (s <= nh) add(MX_PLAN_SMALL, s);
  }
  if (tiles > cu_count() && tiles % cu_count() != 0 && mx_linear_balanced_ws_bytes(M, K, N) > 0)
    add(MX_PLAN_BALANCED, 1);
  return n;
}

using PlanKey = std::tuple<int, int64_t, int64_t, int64_t, int>;  // device, M, K, N, epilogue
std::mutex g_plan_mutex;
std::map<PlanKey, Plan> g_plans;

bool cached_plan(const PlanKey& key, Plan* p) {
  std::lock_guard<std::mutex> lock(g_plan_mutex);
  auto it = g_plans.find(key);
  if (it == g_plans.end()) return false;
  *p = it->second;
  return true;
}

}  // namespace

extern "C" {

int64_t mx_linear_tune_ws_bytes(int64_t M, int64_t K, int64_t N) {
  if (M < 0 || N < 0 || K < 64 || K % 64 != 0 || M > kMaxRows || N > kMaxKN || K > kMaxKN) return -1;
  Plan c[kMaxTuneCandidates];
  const int n = tune_candidates(M, K, N, c, kMaxTuneCandidates);
  int64_t need = 0;
  for (int i = 0; i < n; ++i) need = std::max(need, mx_linear_plan_ws_bytes(c[i].kind, c[i].splits, M, K, N));
  return need;
}

int mx_linear_tune(const uint8_t* xq, const uint8_t* xs, int64_t M, int64_t K, const uint8_t* wq, const uint8_t* ws,
                   int64_t N, const void* bias, int epilogue, void* y, void* workspace, int64_t workspace_bytes,
                   int reps, void* stream, int* kind, int* splits) {
  if (kind == nullptr || splits == nullptr) return fail(MX_ERR_INVALID_ARGUMENT, "NULL kind or splits");
  if (reps < 1 || reps > 1000) return fail(MX_ERR_INVALID_ARGUMENT, "reps = %d must be in [1, 1000]", reps);
  int st = check_linear_slab(xq, xs, M, K, wq, ws, N, bias, epilogue);
  if (st != MX_OK) return st;
  if (M == 0 || N == 0) return fail(MX_ERR_INVALID_ARGUMENT, "nothing to tune for an empty shape");
  if ((st = check_device()) != MX_OK) return st;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  Plan c[kMaxTuneCandidates];
  const int n = tune_candidates(M, K, N, c, kMaxTuneCandidates);
  hipEvent_t ev[2];
  if ((e = hipEventCreate(&ev[0])) != hipSuccess) return hip_fail(e, "hipEventCreate");
  if ((e = hipEventCreate(&ev[1])) != hipSuccess) {
    (void)hipEventDestroy(ev[0]);
    return hip_fail(e, "hipEventCreate");
  }
  hipStream_t hs = (hipStream_t)stream;
  Plan best{-1, 0};
  float best_ms = 0.f;
  int result = MX_OK;
  for (int i = 0; i < n && result == MX_OK; ++i) {
    const int64_t need = mx_linear_plan_ws_bytes(c[i].kind, c[i].splits, M, K, N);
    if (need < 0 || need > workspace_bytes) continue;  // the caller's workspace does not fit this candidate
    // Warm-up run: a candidate the entry point rejects (a size limit) is
    // skipped; a HIP failure ends the tuning.
    const int wst = mx_linear_slab_plan(c[i].kind, c[i].splits, xq, xs, M, K, wq, ws, N, bias, epilogue, y, workspace,
                                        workspace_bytes, stream);
    if (wst == MX_ERR_HIP) {
      result = wst;
      break;
    }
    if (wst != MX_OK) continue;
    // The timed runs queue behind a delay long enough for the host to submit
    // them all (about 10 us per launch, at most two launches per run), so the
    // events measure the GPU's back-to-back time, not the host's launch rate.
    float ms = 0.f;
    if ((e = mx::launch_delay(std::min(20 * reps + 50, 20000), hs)) != hipSuccess) { result = hip_fail(e, "delay launch"); break; }
    if ((e = hipEventRecord(ev[0], hs)) != hipSuccess) { result = hip_fail(e, "hipEventRecord"); break; }
    for (int r = 0; r < reps && result == MX_OK; ++r)
      result = mx_linear_slab_plan(c[i].kind, c[i].splits, xq, xs, M, K, wq, ws, N, bias, epilogue, y, workspace,
                                   workspace_bytes, stream);
    if (result != MX_OK) break;
    if ((e = hipEventRecord(ev[1], hs)) != hipSuccess) { result = hip_fail(e, "hipEventRecord"); break; }
    if ((e = hipEventSynchronize(ev[1])) != hipSuccess) { result = hip_fail(e, "hipEventSynchronize"); break; }
    if ((e = hipEventElapsedTime(&ms, ev[0], ev[1])) != hipSuccess) { result = hip_fail(e, "hipEventElapsedTime"); break; }
    if (best.kind < 0 || ms < best_ms) {
      best = c[i];
      best_ms = ms;
    }
  }
  (void)hipEventDestroy(ev[0]);
  (void)hipEventDestroy(ev[1]);
  if (result != MX_OK) return result;
  if (best.kind < 0) return fail(MX_ERR_INVALID_ARGUMENT, "no candidate plan fits a workspace of %lld bytes",
                                 (long long)workspace_bytes);
  {
    std::lock_guard<std::mutex> lock(g_plan_mutex);
    g_plans[PlanKey{dev, M, K, N, epilogue}] = best;
  }
  *kind = best.kind;
  *splits = best.splits;
  t_msg[0] = '\0';
  return MX_OK;
}

int mx_linear_plan_lookup(int64_t M, int64_t K, int64_t N, int epilogue, int* kind, int* splits) {
  if (kind == nullptr || splits == nullptr) return fail(MX_ERR_INVALID_ARGUMENT, "NULL kind or splits");
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  Plan p;
  if (cached_plan(PlanKey{dev, M, K, N, epilogue}, &p)) {
    *kind = p.kind;
    *splits = p.splits;
    t_msg[0] = '\0';
    return MX_OK;
  }
  return mx_linear_plan_default(M, K, N, kind, splits);
}

int mx_linear_slab_auto(const uint8_t* xq, const uint8_t* xs, int64_t M, int64_t K, const uint8_t* wq,
                        const uint8_t* ws, int64_t N, const void* bias, int epilogue, void* y, void* workspace,
                        int64_t workspace_bytes, void* stream) {
  int kind, splits;
  int st = check_linear_slab(xq, xs, M, K, wq, ws, N, bias, epilogue);
  if (st != MX_OK || M == 0 || N == 0) return st;
  if ((st = mx_linear_plan_lookup(M, K, N, epilogue, &kind, &splits)) != MX_OK) return st;
  return mx_linear_slab_plan(kind, splits, xq, xs, M, K, wq, ws, N, bias, epilogue, y, workspace, workspace_bytes,
                             stream);
}

int mx_probe_mfma(const uint8_t* a, const uint8_t* b, int64_t bytes, int iters, int blocks, float* sink,
                  void* stream) {
  if (a == nullptr || b == nullptr || sink == nullptr) return fail(MX_ERR_INVALID_ARGUMENT, "NULL pointer");
  if (!aligned(a, 4) || !aligned(b, 4) || !aligned(sink, 4))
    return fail(MX_ERR_INVALID_ARGUMENT, "a, b and sink must be 4-byte aligned");
  if (bytes < 4 || bytes % 4 != 0 || bytes > (int64_t(1) << 31))
    return fail(MX_ERR_INVALID_ARGUMENT, "bytes = %lld must be a positive multiple of 4, at most 2^31", (long long)bytes);
  if (iters < 1 || iters > (1 << 20)) return fail(MX_ERR_INVALID_ARGUMENT, "iters = %d must be in [1, 2^20]", iters);
  if (blocks < 1 || blocks > 65536) return fail(MX_ERR_INVALID_ARGUMENT, "blocks = %d must be in [1, 65536]", blocks);
  int st;
  if ((st = check_device()) != MX_OK) return st;
  (void)hipGetLastError();
  return finish(mx::launch_mfma_probe(a, b, bytes, iters, blocks, sink, (hipStream_t)stream), "probe launch");
}

void mx_linear_plan_clear(void) {
  std::lock_guard<std::mutex> lock(g_plan_mutex);
  g_plans.clear();
}

}  // extern "C"

/* ---- The one-call linear: quantize into the workspace, then the plan ---- */

namespace {

int64_t round256(int64_t v) { return (v + 255) / 256 * 256; }

// Workspace layout of mx_linear: the activation slab (codes, then scales),
// then the plan's partial sums.
struct LinearWs {
  int64_t act, part;  // byte offsets
};

LinearWs linear_ws_layout(int64_t M, int64_t K) {
  const int64_t RM = mx::slab_rows(M);
  LinearWs L;
  L.act = 0;
  L.part = round256(RM * K + RM * (K / 32));
  return L;
}

// One linear on the slab operands in the workspace, by plan. The shape
// checks of the plan's own entry point run first.
int run_linear_plan(int kind, int splits, const void* x, int64_t M, int64_t K, int64_t ldx, const uint8_t* wq,
                    const uint8_t* ws, int64_t N, const void* bias, int epilogue, void* y, uint8_t* work,
                    hipStream_t stream) {
  const LinearWs L = linear_ws_layout(M, K);
  const int64_t RM = mx::slab_rows(M);
  uint8_t* xq = work + L.act;
  uint8_t* xs = xq + RM * K;
  float* part = (float*)(work + L.part);
  int st = MX_OK;
  if (kind == MX_PLAN_SMALL) st = check_small_shape(M, K, N, splits);
  if (kind == MX_PLAN_SPLITK) st = check_splitk_shape(M, N, splits);
  if (st != MX_OK) return st;
  hipError_t e = mx::launch_quantize_slab(0, x, M, K, ldx, xq, xs, stream);
  if (e != hipSuccess) return hip_fail(e, "quantize launch");
  switch (kind) {
    case MX_PLAN_SLAB:
      e = mx::launch_linear_slab(xq, xs, M, K, wq, ws, N, bias, epilogue, y, stream);
      break;
    case MX_PLAN_SMALL:
      e = mx::launch_linear_slab_small(xq, xs, M, K, wq, ws, N, bias, epilogue, y, splits, part, stream);
      break;
    case MX_PLAN_SPLITK:
      e = mx::launch_linear_slab_splitk(xq, xs, M, K, wq, ws, N, bias, epilogue, y, splits, part, stream);
      break;
    case MX_PLAN_BALANCED:
      e = mx::launch_linear_slab_balanced(xq, xs, M, K, wq, ws, N, bias, epilogue, y, cu_count(), part, stream);
      break;
    case MX_PLAN_SLAB_M128:
      e = mx::launch_linear_slab_m128(xq, xs, M, K, wq, ws, N, bias, epilogue, y, stream);
      break;
    default:
      return fail(MX_ERR_INVALID_ARGUMENT, "unknown plan kind %d", kind);
  }
  return finish(e, "linear launch");
}

// mx_linear's checks and run. library_scratch: the workspace is the
// library's own scratch array (mx_linear_noalloc; `workspace` is ignored and
// the array's device address looked up after the host-side checks), so a
// shape that needs more than it holds is MX_ERR_UNSUPPORTED rather than a
// short workspace, and it cannot overlap the caller's buffers.
int linear_one_call(const void* x, int64_t M, int64_t K, int64_t ldx, const uint8_t* wq, const uint8_t* ws, int64_t N,
                    const void* bias, int epilogue, void* y, void* workspace, int64_t workspace_bytes, void* stream,
                    bool library_scratch) {
  // The token slab lives in the workspace: check it as the operand it
  // becomes (any 256-aligned stand-in for the library's array).
  if (library_scratch) workspace = (void*)(uintptr_t)256;
  const uint64_t RM0 = M > 0 && M <= kMaxRows ? (uint64_t)mx::slab_rows(M) : 0;
  const uint8_t* wxq = (const uint8_t*)workspace;
  const uint8_t* wxs = workspace != nullptr && K > 0 ? wxq + RM0 * (uint64_t)K : nullptr;
  int st = check_linear_slab(wxq, wxs, M, K, wq, ws, N, bias, epilogue);
  if (st != MX_OK || M == 0 || N == 0) return st;
  if (x == nullptr || y == nullptr || workspace == nullptr) return fail(MX_ERR_INVALID_ARGUMENT, "NULL x, y or workspace");
  if (ldx < K || ldx % 8 != 0) return fail(MX_ERR_INVALID_ARGUMENT, "ldx = %lld must be >= K and a multiple of 8", (long long)ldx);
  if (!aligned(x, 16) || !aligned(y, 16) || !aligned(workspace, 256))
    return fail(MX_ERR_INVALID_ARGUMENT, "x and y must be 16-byte aligned, workspace 256-byte aligned");
  // The activation slab comes first in the workspace; the plan's partial
  // sums follow.
  const int64_t base = linear_ws_layout(M, K).part;
  if (workspace_bytes < base)
    return fail(library_scratch ? MX_ERR_UNSUPPORTED : MX_ERR_INVALID_ARGUMENT,
                "workspace of %lld bytes, at least %lld needed (mx_linear_ws_bytes gives %lld)",
                (long long)workspace_bytes, (long long)base, (long long)mx_linear_ws_bytes(M, K, N));
  const uint64_t RN = (uint64_t)mx::slab_rows(N);
  const uint64_t xbytes = ((uint64_t)(M - 1) * ldx + K) * 2, ybytes = (uint64_t)M * N * 2;
  auto overlaps_args = [&](uint64_t nbytes) {
    return !library_scratch &&
           (overlap(workspace, nbytes, x, xbytes) || overlap(workspace, nbytes, y, ybytes) ||
            overlap(workspace, nbytes, wq, RN * K) || overlap(workspace, nbytes, ws, RN * (K / 32)) ||
            overlap(workspace, nbytes, bias, (uint64_t)N * 2));
  };
  if (overlaps_args((uint64_t)base)) return fail(MX_ERR_INVALID_ARGUMENT, "workspace overlaps an argument");
  if (overlap(y, ybytes, x, xbytes) || overlap(y, ybytes, wq, RN * K) || overlap(y, ybytes, ws, RN * (K / 32)) ||
      overlap(y, ybytes, bias, (uint64_t)N * 2))
    return fail(MX_ERR_INVALID_ARGUMENT, "y overlaps an input");
  if ((st = check_device()) != MX_OK) return st;
  if (library_scratch) {
    const hipError_t e = mx::scratch_buffer(&workspace);
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress of the scratch array");
  }
  // The plan: the tuned one cached for this shape, else the default rule; a
  // tuned plan whose partial sums do not fit the workspace gives way to the
  // default plan.
  int kind, splits;
  if ((st = mx_linear_plan_lookup(M, K, N, epilogue, &kind, &splits)) != MX_OK) return st;
  int64_t need = base + round256(mx_linear_plan_ws_bytes(kind, splits, M, K, N));
  if (need > workspace_bytes) {
    if ((st = mx_linear_plan_default(M, K, N, &kind, &splits)) != MX_OK) return st;
    need = base + round256(mx_linear_plan_ws_bytes(kind, splits, M, K, N));
  }
  if (workspace_bytes < need)
    return fail(library_scratch ? MX_ERR_UNSUPPORTED : MX_ERR_INVALID_ARGUMENT,
                "workspace of %lld bytes, %lld needed (mx_linear_ws_bytes gives %lld)", (long long)workspace_bytes,
                (long long)need, (long long)mx_linear_ws_bytes(M, K, N));
  if (overlaps_args((uint64_t)need)) return fail(MX_ERR_INVALID_ARGUMENT, "workspace overlaps an argument");
  (void)hipGetLastError();
  return run_linear_plan(kind, splits, x, M, K, ldx, wq, ws, N, bias, epilogue, y, (uint8_t*)workspace,
                         (hipStream_t)stream);
}

}  // namespace

extern "C" {

int64_t mx_linear_ws_bytes(int64_t M, int64_t K, int64_t N) {
  if (M < 0 || N < 0 || K < 64 || K % 64 != 0 || M > kMaxRows || N > kMaxKN || K > kMaxKN) return -1;
  if (M == 0 || N == 0) return 0;
  const int64_t part = mx_linear_tune_ws_bytes(M, K, N);  // the largest any candidate plan needs
  if (part < 0) return -1;
  return linear_ws_layout(M, K).part + round256(part);
}

int mx_linear(const void* x, int64_t M, int64_t K, int64_t ldx, const uint8_t* wq, const uint8_t* ws, int64_t N,
              const void* bias, int epilogue, void* y, void* workspace, int64_t workspace_bytes, void* stream) {
  return linear_one_call(x, M, K, ldx, wq, ws, N, bias, epilogue, y, workspace, workspace_bytes, stream, false);
}

int mx_linear_noalloc(const void* x, int64_t M, int64_t K, int64_t ldx, const uint8_t* wq, const uint8_t* ws,
                      int64_t N, const void* bias, int epilogue, void* y, void* stream) {
  return linear_one_call(x, M, K, ldx, wq, ws, N, bias, epilogue, y, nullptr, mx::kScratchBytes, stream, true);
}

}  // extern "C"
