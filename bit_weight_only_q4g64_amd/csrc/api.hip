// Host side of the q4g64 C ABI: argument validation, launch configuration and
// error reporting. Every entry point validates on the host first and enqueues
// nothing when an argument is rejected.
#include "../../include/q4g64.h"

#include <math.h>
#include <stdarg.h>
#include <stdio.h>

#include <atomic>
#include <mutex>

#include "common.h"
#include "ffn.h"
#include "ffn_flow.h"
#include "pack.h"
#include "pgemm.h"
#include "pgemm_flow.h"
#include "pgemm_narrow.h"
#include "qmv.h"
#include "rope.h"

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return code;
}

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p % a) == 0; }

constexpr int64_t kMaxDim = int64_t(1) << 30;
constexpr int64_t kMaxElems = int64_t(1) << 40;
// Row strides (elements) and the elements a strided array spans: small enough
// that no offset a call forms, on the host or in a kernel, overflows int64.
constexpr int64_t kMaxStride = int64_t(1) << 40;
constexpr int64_t kMaxSpan = int64_t(1) << 48;
constexpr size_t kMaxLds = 64 * 1024;
// Window GEMM: one column tile's codes (K / 128 pairs of 1 KiB) are addressed
// with 32-bit offsets.
constexpr int64_t kPgemmMaxK = int64_t(1) << 20;
constexpr int64_t kPgemmMaxM = int64_t(1) << 24;
// One-launch FFN step: at most two segments per wave in each phase.
constexpr int64_t kFfnMaxK1 = 4096;
constexpr int64_t kFfnMaxN1 = 8192;

int check_nk(const char* fn, int64_t N, int64_t K) {
  if (N <= 0 || K <= 0 || N % 64 != 0 || K % 64 != 0)
    return fail(Q4_EINVAL, "%s: N=%lld and K=%lld must be positive multiples of 64", fn, (long long)N, (long long)K);
  if (N > kMaxDim || K > kMaxDim || N * K > kMaxElems)
    return fail(Q4_EINVAL, "%s: N=%lld x K=%lld is too large", fn, (long long)N, (long long)K);
  return Q4_OK;
}

int check_ld(const char* fn, const char* name, int64_t ld) {
  if (ld > kMaxStride) return fail(Q4_EINVAL, "%s: %s=%lld exceeds 2^40 elements", fn, name, (long long)ld);
  return Q4_OK;
}

int check_ptr(const char* fn, const char* name, const void* p, uintptr_t align) {
  if (p == nullptr) return fail(Q4_EALIGN, "%s: %s is NULL", fn, name);
  if (!aligned(p, align)) return fail(Q4_EALIGN, "%s: %s is not %u-byte aligned", fn, name, (unsigned)align);
  return Q4_OK;
}

int launched(const char* fn) {
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(Q4_EDEVICE, "%s: launch failed: %s", fn, hipGetErrorString(e));
  return Q4_OK;
}

unsigned grid_for(int64_t total, int block) {
  int64_t g = (total + block - 1) / block;
  if (g > 65536) g = 65536;
  if (g < 1) g = 1;
  return (unsigned)g;
}

int check_x(const char* fn, const void* x, int x_dtype, int64_t ldx, int64_t K) {
  if (x_dtype != Q4_BF16 && x_dtype != Q4_F32 && x_dtype != Q4_BF16X3 && x_dtype != Q4_BF16X3T)
    return fail(Q4_EINVAL, "%s: x_dtype %d is not Q4_BF16, Q4_F32, Q4_BF16X3 or Q4_BF16X3T", fn, x_dtype);
  if (int rc = check_ptr(fn, "x", x, 16)) return rc;
  if (x_dtype == Q4_BF16X3T && ldx != K)
    return fail(Q4_EINVAL, "%s: fragment-ordered planes have no row stride (ldx=%lld must equal K=%lld)", fn, (long long)ldx,
                (long long)K);
  if (ldx < K) return fail(Q4_EINVAL, "%s: ldx=%lld < K=%lld", fn, (long long)ldx, (long long)K);
  if (int rc = check_ld(fn, "ldx", ldx)) return rc;
  const int64_t es = x_dtype == Q4_F32 ? 4 : 2;
  if ((ldx * es) % 16 != 0) return fail(Q4_EALIGN, "%s: ldx=%lld elements does not keep rows 16-byte aligned", fn, (long long)ldx);
  return Q4_OK;
}

int check_bits(const char* fn, int bits) {
  if (bits != 4 && bits != 6 && bits != 8) return fail(Q4_EINVAL, "%s: bits=%d is not 4, 6 or 8", fn, bits);
  return Q4_OK;
}

// Internal: the MLX widths or block FP8.
int check_fmt(const char* fn, int fmt) {
  if (fmt == q4::kFmtFp8) return Q4_OK;
  return check_bits(fn, fmt);
}

size_t packed_bytes_impl(int bits, int64_t N, int64_t K) {
  if (bits != 4 && bits != 6 && bits != 8) return 0;
  if (N <= 0 || K <= 0 || N % 64 != 0 || K % 64 != 0 || N > kMaxDim || K > kMaxDim || N * K > kMaxElems) return 0;
  return (size_t)q4::packed_bytes(N, K, bits);
}

int pack_impl(const char* fn, int bits, const uint32_t* wq, const uint16_t* scales, const uint16_t* biases, int64_t N, int64_t K,
              void* packed, hipStream_t s) {
  if (int rc = check_bits(fn, bits)) return rc;
  if (int rc = check_nk(fn, N, K)) return rc;
  if (int rc = check_ptr(fn, "wq", wq, 16)) return rc;
  if (int rc = check_ptr(fn, "scales", scales, 2)) return rc;
  if (int rc = check_ptr(fn, "biases", biases, 2)) return rc;
  if (int rc = check_ptr(fn, "packed", packed, 16)) return rc;
  const int64_t words = q4::codes_bytes(N, K, bits) / 4;
  const int64_t sb_entries = (N / q4::kTileN) * q4::n_pairs(K) * q4::kTileN;
  uint8_t* out = (uint8_t*)packed;
  if (bits == 4)
    hipLaunchKernelGGL(q4::pack_codes_kernel, dim3(grid_for(words, 256)), dim3(256), 0, s, wq, N, K, (uint32_t*)out);
  else if (bits == 6)
    hipLaunchKernelGGL(q4::pack_codes_wide_kernel<6>, dim3(grid_for(words, 256)), dim3(256), 0, s, wq, N, K, (uint32_t*)out);
  else
    hipLaunchKernelGGL(q4::pack_codes_wide_kernel<8>, dim3(grid_for(words, 256)), dim3(256), 0, s, wq, N, K, (uint32_t*)out);
  if (int rc = launched(fn)) return rc;
  hipLaunchKernelGGL(q4::pack_sb_kernel, dim3(grid_for(sb_entries, 256)), dim3(256), 0, s, scales, biases, N, K,
                     (q4::u32x2*)(out + q4::codes_bytes(N, K, bits)));
  return launched(fn);
}

int unpack_impl(const char* fn, int bits, const void* packed, int64_t N, int64_t K, uint32_t* wq, uint16_t* scales,
                uint16_t* biases, hipStream_t s) {
  if (int rc = check_bits(fn, bits)) return rc;
  if (int rc = check_nk(fn, N, K)) return rc;
  if (int rc = check_ptr(fn, "packed", packed, 16)) return rc;
  if (int rc = check_ptr(fn, "wq", wq, 16)) return rc;
  if (int rc = check_ptr(fn, "scales", scales, 2)) return rc;
  if (int rc = check_ptr(fn, "biases", biases, 2)) return rc;
  const uint8_t* in = (const uint8_t*)packed;
  const int64_t cwords = N * (K * bits / 32);
  if (bits == 4)
    hipLaunchKernelGGL(q4::unpack_codes_kernel, dim3(grid_for(cwords, 256)), dim3(256), 0, s, (const uint32_t*)in, N, K, wq);
  else if (bits == 6)
    hipLaunchKernelGGL(q4::unpack_codes_wide_kernel<6>, dim3(grid_for(cwords, 256)), dim3(256), 0, s, (const uint32_t*)in, N, K, wq);
  else
    hipLaunchKernelGGL(q4::unpack_codes_wide_kernel<8>, dim3(grid_for(cwords, 256)), dim3(256), 0, s, (const uint32_t*)in, N, K, wq);
  if (int rc = launched(fn)) return rc;
  hipLaunchKernelGGL(q4::unpack_sb_kernel, dim3(grid_for(N * (K / 64), 256)), dim3(256), 0, s,
                     (const q4::u32x2*)(in + q4::codes_bytes(N, K, bits)), N, K, scales, biases);
  return launched(fn);
}

// Decode activation forms: 0 bf16 rows, 1 float32 rows, 2 float32 rows as three
// bf16 planes, 3 the planes in fragment order.
int xmode_of(int x_dtype) { return x_dtype == Q4_F32 ? 1 : (x_dtype == Q4_BF16X3 ? 2 : (x_dtype == Q4_BF16X3T ? 3 : 0)); }

int qmv_rows_impl(const char* fn, int bits, const void* packed, int64_t N, int64_t K, const void* x, int x_dtype, int64_t ldx,
                  int R, float* y, int64_t ldy, hipStream_t s) {
  if (int rc = check_fmt(fn, bits)) return rc;
  if (int rc = check_nk(fn, N, K)) return rc;
  if (R < 1 || R > 16) return fail(Q4_EINVAL, "%s: R=%d is outside 1..16", fn, R);
  if (int rc = check_ptr(fn, "packed", packed, 16)) return rc;
  if (int rc = check_x(fn, x, x_dtype, ldx, K)) return rc;
  if (int rc = check_ptr(fn, "y", y, 4)) return rc;
  if (ldy < N) return fail(Q4_EINVAL, "%s: ldy=%lld < N=%lld", fn, (long long)ldy, (long long)N);
  if (int rc = check_ld(fn, "ldy", ldy)) return rc;
  const int64_t xrows = x_dtype == Q4_BF16X3 ? 3 * (int64_t)R : R;  // planes: three rows per activation row
  if (xrows * ldx * (x_dtype == Q4_F32 ? 4 : 2) >= (int64_t(1) << 31))
    return fail(Q4_EUNSUPPORTED, "%s: R * ldx spans more than 2 GiB of activations", fn);
  // up to 4 segments per wave, 16 waves: K <= 16384
  if (K > q4::kQmvMaxK) return fail(Q4_EUNSUPPORTED, "%s: K=%lld exceeds the decode limit of 16384", fn, (long long)K);
  const size_t lds = q4::qmv_lds_bytes(K, x_dtype != Q4_BF16, 1, R);
  if (lds > kMaxLds) return fail(Q4_EUNSUPPORTED, "%s: K=%lld exceeds the decode limit of 16384", fn, (long long)K);
  q4::qmv_launch((const uint8_t*)packed, (const uint8_t*)packed, 1, (int)N, (int)K, x, xmode_of(x_dtype), ldx, R, y, ldy, s, bits);
  return launched(fn);
}

// K split of a one-matrix matvec: workgroups per column tile. 0 picks the
// smallest power of two that gives at least one workgroup per CU, with at
// least one segment each; the result never depends on the choice.
constexpr int kSplitMax = 16;
constexpr int kSplitTargetWgs = 256;
int split_shares(int splits, int xmode, int64_t N, int64_t K, int R) {
  const int nseg = q4::qmv_segments(K);
  if (splits > 0) return splits < nseg ? splits : nseg;
  int s = 1;
  while (2 * s <= nseg && 2 * s <= kSplitMax) {
    const q4::QmvSplitShape sh = q4::qmv_split_shape(1, xmode, (int)N, (int)K, R, s);
    if (sh.tile_ids * s >= kSplitTargetWgs) break;
    s *= 2;
  }
  return s;
}

int qmv_split_check(const char* fn, int bits, const void* packed, int64_t N, int64_t K, const void* x, int x_dtype, int64_t ldx,
                    int R, float* y, int64_t ldy, int splits) {
  if (int rc = check_fmt(fn, bits)) return rc;
  if (int rc = check_nk(fn, N, K)) return rc;
  if (R < 1 || R > 16) return fail(Q4_EINVAL, "%s: R=%d is outside 1..16", fn, R);
  if (splits < 0 || splits > kSplitMax) return fail(Q4_EINVAL, "%s: splits=%d is outside 0..%d", fn, splits, kSplitMax);
  if (int rc = check_ptr(fn, "packed", packed, 16)) return rc;
  if (int rc = check_x(fn, x, x_dtype, ldx, K)) return rc;
  if (int rc = check_ptr(fn, "y", y, 4)) return rc;
  if (ldy < N) return fail(Q4_EINVAL, "%s: ldy=%lld < N=%lld", fn, (long long)ldy, (long long)N);
  if (int rc = check_ld(fn, "ldy", ldy)) return rc;
  const int64_t xrows = x_dtype == Q4_BF16X3 ? 3 * (int64_t)R : R;
  if (xrows * ldx * (x_dtype == Q4_F32 ? 4 : 2) >= (int64_t(1) << 31))
    return fail(Q4_EUNSUPPORTED, "%s: R * ldx spans more than 2 GiB of activations", fn);
  if (K > q4::kQmvMaxK) return fail(Q4_EUNSUPPORTED, "%s: K=%lld exceeds the decode limit of 16384", fn, (long long)K);
  const size_t lds = q4::qmv_lds_bytes(K, x_dtype != Q4_BF16, 1, R);
  if (lds > kMaxLds) return fail(Q4_EUNSUPPORTED, "%s: K=%lld exceeds the decode limit of 16384", fn, (long long)K);
  return Q4_OK;
}

// The split matvec on a workspace of at least work_bytes (checked by the caller).
int qmv_split_launch(const char* fn, int bits, const void* packed, int64_t N, int64_t K, const void* x, int x_dtype, int64_t ldx,
                     int R, float* y, int64_t ldy, int nshare, uint8_t* work, hipStream_t s) {
  const int xmode = xmode_of(x_dtype);
  q4::QmvSplit sp{nshare, nullptr, nullptr};
  if (nshare > 1) {
    const q4::QmvSplitShape sh = q4::qmv_split_shape(1, xmode, (int)N, (int)K, R, nshare);
    sp.cnt = (uint32_t*)work;
    sp.part = (float*)(work + q4::qmv_split_counter_bytes(sh));
  }
  q4::qmv_launch((const uint8_t*)packed, (const uint8_t*)packed, 1, (int)N, (int)K, x, xmode, ldx, R, y, ldy, s, bits, 0, sp);
  return launched(fn);
}

// y3: 0 float32 y [R][ldy]; 1 Q4_BF16X3 planes [3][R][ldy]; 2 Q4_BF16X3T
// (ldy is then N, the activations per row).
int qmv_w13_impl(const char* fn, int bits, const void* packed_w1, const void* packed_w3, int64_t N, int64_t K, const uint16_t* x,
                 int64_t ldx, int R, void* y, int64_t ldy, hipStream_t s, int y3 = 0) {
  if (int rc = check_fmt(fn, bits)) return rc;
  if (int rc = check_nk(fn, N, K)) return rc;
  if (R < 1 || R > 16) return fail(Q4_EINVAL, "%s: R=%d is outside 1..16", fn, R);
  if (int rc = check_ptr(fn, "packed_w1", packed_w1, 16)) return rc;
  if (int rc = check_ptr(fn, "packed_w3", packed_w3, 16)) return rc;
  if (int rc = check_x(fn, x, Q4_BF16, ldx, K)) return rc;
  if (int rc = check_ptr(fn, y3 ? "z3" : "y", y, y3 ? 16 : 4)) return rc;
  if (ldy < N) return fail(Q4_EINVAL, "%s: %s=%lld < N=%lld", fn, y3 ? "ldz" : "ldy", (long long)ldy, (long long)N);
  if (int rc = check_ld(fn, y3 ? "ldz" : "ldy", ldy)) return rc;
  if (y3 == 1 && (ldy * 2) % 16 != 0)
    return fail(Q4_EALIGN, "%s: ldz=%lld elements does not keep rows 16-byte aligned", fn, (long long)ldy);
  if (y3 == 2 && N > q4::kQmvMaxK)
    return fail(Q4_EUNSUPPORTED, "%s: N=%lld exceeds the decode limit of 16384 for the next matvec's K", fn, (long long)N);
  if ((int64_t)R * ldx * 2 >= (int64_t(1) << 31))
    return fail(Q4_EUNSUPPORTED, "%s: R * ldx spans more than 2 GiB of activations", fn);
  // up to 2 segments per wave, 16 waves: K <= 8192
  if (K > q4::kQmvMaxK / 2) return fail(Q4_EUNSUPPORTED, "%s: K=%lld exceeds the fused decode limit of 8192", fn, (long long)K);
  const size_t lds = q4::qmv_lds_bytes(K, 0, 2, R);
  if (lds > kMaxLds) return fail(Q4_EUNSUPPORTED, "%s: K=%lld exceeds the fused decode limit of 8192", fn, (long long)K);
  q4::qmv_launch((const uint8_t*)packed_w1, (const uint8_t*)packed_w3, 2, (int)N, (int)K, x, 0, ldx, R, (float*)y, ldy, s, bits, y3);
  return launched(fn);
}

// Workgroup grid of a window: column blocks x row blocks, as one dimension.
int64_t pgemm_blocks(int64_t N, int64_t M, bool swiglu, int* nblk, int* mblk) {
  const int cols = q4::pgemm_cols(swiglu);
  const int64_t nb = (N + cols - 1) / cols, mb = (M + q4::kPgemmRows - 1) / q4::kPgemmRows;
  *nblk = (int)nb;
  *mblk = (int)mb;
  return nb * mb;
}

template <int BITS>
void pgemm_launch_bits(bool swiglu, bool obf16, dim3 grid, dim3 block, hipStream_t s, const uint8_t* a, const uint8_t* b, int n,
                       int k, const uint16_t* x, int64_t ldx, int m, void* y, int64_t ldy, int nblk, int mblk) {
  using namespace q4;
  if (swiglu) {
    if (obf16)
      hipLaunchKernelGGL((pgemm_kernel<true, true, BITS>), grid, block, 0, s, a, b, n, k, x, ldx, m, y, ldy, nblk, mblk);
    else
      hipLaunchKernelGGL((pgemm_kernel<true, false, BITS>), grid, block, 0, s, a, b, n, k, x, ldx, m, y, ldy, nblk, mblk);
  } else {
    if (obf16)
      hipLaunchKernelGGL((pgemm_kernel<false, true, BITS>), grid, block, 0, s, a, b, n, k, x, ldx, m, y, ldy, nblk, mblk);
    else
      hipLaunchKernelGGL((pgemm_kernel<false, false, BITS>), grid, block, 0, s, a, b, n, k, x, ldx, m, y, ldy, nblk, mblk);
  }
}

// Below this many 256-column workgroups a window runs on the 64-column
// workgroups of pgemm_narrow_kernel (every code format; the same bits per
// row).
constexpr int64_t kNarrowBelow = 256;

template <int BITS>
void narrow_launch_bits(bool swiglu, bool obf16, dim3 grid, dim3 block, hipStream_t s, const uint8_t* a, const uint8_t* b, int n, int k,
                        const uint16_t* x, int64_t ldx, int m, void* y, int64_t ldy, int nb, int mblk) {
  using namespace q4;
  if (swiglu) {
    if (obf16) hipLaunchKernelGGL((pgemm_narrow_kernel<true, true, BITS>), grid, block, 0, s, a, b, n, k, x, ldx, m, y, ldy, nb, mblk);
    else hipLaunchKernelGGL((pgemm_narrow_kernel<true, false, BITS>), grid, block, 0, s, a, b, n, k, x, ldx, m, y, ldy, nb, mblk);
  } else {
    if (obf16) hipLaunchKernelGGL((pgemm_narrow_kernel<false, true, BITS>), grid, block, 0, s, a, b, n, k, x, ldx, m, y, ldy, nb, mblk);
    else hipLaunchKernelGGL((pgemm_narrow_kernel<false, false, BITS>), grid, block, 0, s, a, b, n, k, x, ldx, m, y, ldy, nb, mblk);
  }
}
// Among those, a window whose 32 x 32 tiles fit twice on the compute units
// runs on pgemm_flow_kernel: plain with 3 producer waves and a ring of 8
// (74.5 KiB of LDS, two workgroups per compute unit); SwiGLU with 3 producers
// and a ring of 8 when its tiles fit once (120 KiB), else with 2 producers and
// a ring of 4 (72.7 KiB, two per compute unit). Measured on MI355X (us per
// window, flow / narrow): 128-row w2 25.6 / 79.5, o 9.7 / 22.8, qkv 12.2 /
// 23.1; SwiGLU 8192 x 2048 at 16 rows 13.1 / 23.5, at 64 rows 20.9 / 24.4.
template <bool SW, int NP, int R, int BITS>
void flow_launch_cfg(bool obf16, const uint8_t* a, const uint8_t* b, int n, int k, const uint16_t* x, int64_t ldx, int m, void* y,
                     int64_t ldy, int nb, int mb, hipStream_t s) {
  using namespace q4;
  const dim3 grid((unsigned)((int64_t)nb * mb)), block(64 * (NP + 1));
  if (obf16) hipLaunchKernelGGL((pgemm_flow_kernel<SW, true, NP, R, BITS>), grid, block, 0, s, a, b, n, k, x, ldx, m, y, ldy, nb, mb);
  else hipLaunchKernelGGL((pgemm_flow_kernel<SW, false, NP, R, BITS>), grid, block, 0, s, a, b, n, k, x, ldx, m, y, ldy, nb, mb);
}

template <int BITS>
bool flow_launch_bits(bool swiglu, bool obf16, const uint8_t* a, const uint8_t* b, int64_t N, int k, const uint16_t* x, int64_t ldx,
                      int64_t M, void* y, int64_t ldy, hipStream_t s) {
  using namespace q4;
  const int64_t nb = (N + kFlowRows - 1) / kFlowRows, mb = (M + kFlowRows - 1) / kFlowRows, cus = device_cus();
  const int n = (int)N, m = (int)M;
  // Past two rounds of tiles (SwiGLU) the narrow kernel wins for every code
  // format; past two (4-bit) or four (wider codes) rounds of plain tiles as
  // well. Measured, us per window, this kernel / narrow: 6-bit w1/w3 at 128
  // rows 49.6 / 32.7, FP8 37.1 / 20.0; 6-bit w2 at 384 rows (3 rounds)
  // 69.1 / 108.6, at 768 rows (6 rounds) 125.6 / 112.9; 6-bit o at 512 rows
  // (4 rounds) 26.9 / 30.9, q/k/v at 512 rows (6 rounds) 38.4 / 32.0.
  const int64_t plain_max = (BITS == 4 ? 2 : 4) * cus, sw_max = 2 * cus;
  if (!swiglu && nb * mb <= plain_max) flow_launch_cfg<false, 3, 8, BITS>(obf16, a, b, n, k, x, ldx, m, y, ldy, (int)nb, (int)mb, s);
  else if (swiglu && nb * mb <= cus) flow_launch_cfg<true, 3, 8, BITS>(obf16, a, b, n, k, x, ldx, m, y, ldy, (int)nb, (int)mb, s);
  else if (swiglu && nb * mb <= sw_max) flow_launch_cfg<true, 2, 4, BITS>(obf16, a, b, n, k, x, ldx, m, y, ldy, (int)nb, (int)mb, s);
  else return false;
  return true;
}

// true when the window ran on pgemm_flow_kernel
bool flow_launch(int bits, bool swiglu, bool obf16, const uint8_t* a, const uint8_t* b, int64_t N, int k, const uint16_t* x, int64_t ldx,
                 int64_t M, void* y, int64_t ldy, hipStream_t s) {
  switch (bits) {
    case 4: return flow_launch_bits<4>(swiglu, obf16, a, b, N, k, x, ldx, M, y, ldy, s);
    case 6: return flow_launch_bits<6>(swiglu, obf16, a, b, N, k, x, ldx, M, y, ldy, s);
    case 8: return flow_launch_bits<8>(swiglu, obf16, a, b, N, k, x, ldx, M, y, ldy, s);
    case q4::kFmtFp8: return flow_launch_bits<q4::kFmtFp8>(swiglu, obf16, a, b, N, k, x, ldx, M, y, ldy, s);
  }
  return false;
}

int qmm_window_impl(const char* fn, int bits, const void* packed_a, const void* packed_b, int64_t N, int64_t K, const uint16_t* x,
                    int64_t ldx, int64_t M, void* y, int y_dtype, int64_t ldy, hipStream_t s) {
  using namespace q4;
  const bool swiglu = packed_b != nullptr;
  const bool obf16 = y_dtype == Q4_BF16;
  int nblk, mblk;
  const int64_t blocks = pgemm_blocks(N, M, swiglu, &nblk, &mblk);
  if (blocks > INT32_MAX) return fail(Q4_EUNSUPPORTED, "%s: N=%lld x M=%lld needs too many workgroups", fn, (long long)N, (long long)M);
  dim3 grid((unsigned)blocks), block(kPgemmThreads);
  const uint8_t* a = (const uint8_t*)packed_a;
  const uint8_t* b = swiglu ? (const uint8_t*)packed_b : a;
  const int n = (int)N, k = (int)K, m = (int)M;
  // short windows: the dataflow kernel where its tiles fit twice on the CUs
  // (plain windows of the wider codes: four times), else the narrow kernel
  if (blocks < kNarrowBelow && flow_launch(bits, swiglu, obf16, a, b, N, k, x, ldx, M, y, ldy, s)) return launched(fn);
  if (blocks < kNarrowBelow) {
    const int cols = pgemm_narrow_cols(swiglu);
    const int nb = (n + cols - 1) / cols;
    const dim3 ngrid((unsigned)((int64_t)nb * mblk));
    if (bits == 6)
      narrow_launch_bits<6>(swiglu, obf16, ngrid, block, s, a, b, n, k, x, ldx, m, y, ldy, nb, mblk);
    else if (bits == 8)
      narrow_launch_bits<8>(swiglu, obf16, ngrid, block, s, a, b, n, k, x, ldx, m, y, ldy, nb, mblk);
    else if (bits == kFmtFp8)
      narrow_launch_bits<kFmtFp8>(swiglu, obf16, ngrid, block, s, a, b, n, k, x, ldx, m, y, ldy, nb, mblk);
    else
      narrow_launch_bits<4>(swiglu, obf16, ngrid, block, s, a, b, n, k, x, ldx, m, y, ldy, nb, mblk);
    return launched(fn);
  }
  if (bits == 6)
    pgemm_launch_bits<6>(swiglu, obf16, grid, block, s, a, b, n, k, x, ldx, m, y, ldy, nblk, mblk);
  else if (bits == 8)
    pgemm_launch_bits<8>(swiglu, obf16, grid, block, s, a, b, n, k, x, ldx, m, y, ldy, nblk, mblk);
  else if (bits == kFmtFp8)
    pgemm_launch_bits<kFmtFp8>(swiglu, obf16, grid, block, s, a, b, n, k, x, ldx, m, y, ldy, nblk, mblk);
  else
    pgemm_launch_bits<4>(swiglu, obf16, grid, block, s, a, b, n, k, x, ldx, m, y, ldy, nblk, mblk);
  return launched(fn);
}

int check_window_args(const char* fn, const void* packed_a, const void* packed_b, int64_t N, int64_t K,
                      const uint16_t* x, int64_t ldx, const void* y, int y_dtype, int64_t ldy) {
  if (int rc = check_nk(fn, N, K)) return rc;
  if (int rc = check_ptr(fn, "packed_a", packed_a, 16)) return rc;
  if (packed_b != nullptr && !aligned(packed_b, 16)) return fail(Q4_EALIGN, "%s: packed_b is not 16-byte aligned", fn);
  if (int rc = check_x(fn, x, Q4_BF16, ldx, K)) return rc;
  if (y_dtype != Q4_BF16 && y_dtype != Q4_F32) return fail(Q4_EINVAL, "%s: y_dtype %d is not Q4_BF16 or Q4_F32", fn, y_dtype);
  if (int rc = check_ptr(fn, "y", y, y_dtype == Q4_F32 ? 4 : 2)) return rc;
  if (ldy < N) return fail(Q4_EINVAL, "%s: ldy=%lld < N=%lld", fn, (long long)ldy, (long long)N);
  if (int rc = check_ld(fn, "ldy", ldy)) return rc;
  if ((int64_t)q4::kPgemmRows * ldx * 2 >= (int64_t(1) << 31))
    return fail(Q4_EUNSUPPORTED, "%s: ldx=%lld is too large for a %d-row window tile", fn, (long long)ldx, q4::kPgemmRows);
  if (K > kPgemmMaxK) return fail(Q4_EUNSUPPORTED, "%s: K=%lld exceeds the window GEMM limit of %lld", fn, (long long)K, (long long)kPgemmMaxK);
  return Q4_OK;
}

// The one-launch dataflow step (up to 2 rows, whole 256-wide segments in K1
// and N1): one workgroup per CU, every one resident at once. From 3 rows the
// two decode calls are faster (w1/w3 + SwiGLU 8192 x 2048 then w2 2048 x
// 8192, us: 4 rows 20.1 / 15.3, 8 rows 33.1 / 16.0 for the grid-barrier
// launch this replaced, 16 rows 53.7 / 20.0); at 1 and 2 rows the one launch
// is (11.8 / 13.3, 13.0 / 14.1).
constexpr int kFfnFlowRows = 2;
bool ffn_flow_applies(int64_t N1, int64_t K1, int R) { return R <= kFfnFlowRows && K1 % 256 == 0 && N1 % 256 == 0; }
// Workspace: the error word and the dataflow step's state (call counter,
// tagged z, hand-overs) for up to kFfnFlowRows rows, then, 256-byte aligned,
// the fragment-ordered planes of z for up to 16 rows, which the two-call
// schedule hands from the first call to the second. The size does not depend
// on R, so one workspace serves every row count.
size_t ffn_planes_off(int64_t N1, int64_t N2) { return (q4::flow_work_bytes(N1, N2, kFfnFlowRows) + 255) / 256 * 256; }

template <int NV, int SPW1>
int flow_launch_t(const uint8_t* p1, const uint8_t* p3, const uint8_t* p2, int N1, int K1, int N2, const uint16_t* x, int64_t ldx,
                  int R, float* z, int64_t ldz, float* y, int64_t ldy, uint8_t* work, hipStream_t s) {
  const size_t lds = q4::flow_lds_bytes(K1, R);
  auto kern = q4::ffn_flow_kernel<NV, SPW1>;
  static const bool lds_ok = q4::allow_max_dynamic_lds((const void*)kern);
  (void)lds_ok;
  int dev = 0, cus = 0, per_cu = 0;
  if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, q4::kFfnThreads, lds) != hipSuccess)
    return fail(Q4_EDEVICE, "qmv_ffn: device query failed");
  if (per_cu < 1) return fail(Q4_EUNSUPPORTED, "qmv_ffn: a %zu-byte workgroup does not fit on a CU", lds);
  // every workgroup produces z (at most one per w1/w3 tile pair), so each
  // has read the call counter before any upper-half item advances it
  const int pairs1 = N1 / q4::kTileN / 2;
  const int nwg = cus < pairs1 ? cus : pairs1;
  hipLaunchKernelGGL(kern, dim3((unsigned)nwg), dim3(q4::kFfnThreads), lds, s, p1, p3, p2, N1, K1, N2, x, ldx, R, z, ldz, y, ldy, work);
  return launched("qmv_ffn");
}

template <int NV>
int flow_launch_s1(int spw1, const uint8_t* p1, const uint8_t* p3, const uint8_t* p2, int N1, int K1, int N2, const uint16_t* x,
                   int64_t ldx, int R, float* z, int64_t ldz, float* y, int64_t ldy, uint8_t* work, hipStream_t s) {
  if (spw1 <= 1) return flow_launch_t<NV, 1>(p1, p3, p2, N1, K1, N2, x, ldx, R, z, ldz, y, ldy, work, s);
  return flow_launch_t<NV, 2>(p1, p3, p2, N1, K1, N2, x, ldx, R, z, ldz, y, ldy, work, s);
}

// The rows of a window (a cut) must lie within 2^48 elements of x and of y.
int check_rows_span(const char* fn, int64_t rows, int64_t ldx, int64_t ldy) {
  if (rows > kMaxSpan / ldx || rows > kMaxSpan / ldy)
    return fail(Q4_EINVAL, "%s: %lld rows of strides ldx=%lld, ldy=%lld span more than 2^48 elements", fn, (long long)rows,
                (long long)ldx, (long long)ldy);
  return Q4_OK;
}

int qmm_window_checked(const char* fn, int bits, const void* packed_a, const void* packed_b, int64_t N, int64_t K,
                       const uint16_t* x, int64_t ldx, int64_t M, void* y, int y_dtype, int64_t ldy, hipStream_t s) {
  if (int rc = check_fmt(fn, bits)) return rc;
  if (int rc = check_window_args(fn, packed_a, packed_b, N, K, x, ldx, y, y_dtype, ldy)) return rc;
  if (M < 1 || M > kPgemmMaxM) return fail(Q4_EINVAL, "%s: M=%lld is outside 1..%lld", fn, (long long)M, (long long)kPgemmMaxM);
  if (int rc = check_rows_span(fn, M, ldx, ldy)) return rc;
  return qmm_window_impl(fn, bits, packed_a, packed_b, N, K, x, ldx, M, y, y_dtype, ldy, s);
}

int qmm_cut_impl(const char* fn, int bits, const void* packed_a, const void* packed_b, int64_t N, int64_t K, const uint16_t* x,
                 int64_t ldx, const int64_t* window_rows, int n_windows, void* y, int y_dtype, int64_t ldy, hipStream_t s) {
  if (int rc = check_fmt(fn, bits)) return rc;
  if (int rc = check_window_args(fn, packed_a, packed_b, N, K, x, ldx, y, y_dtype, ldy)) return rc;
  if (window_rows == nullptr || n_windows < 1) return fail(Q4_EINVAL, "%s: need at least one window", fn);
  for (int w = 0; w < n_windows; ++w)
    if (window_rows[w] < 1 || window_rows[w] > kPgemmMaxM)
      return fail(Q4_EINVAL, "%s: window %d has %lld rows", fn, w, (long long)window_rows[w]);
  int64_t rows = 0;  // at most 2^31 windows of at most 2^24 rows: no overflow
  for (int w = 0; w < n_windows; ++w) rows += window_rows[w];
  if (int rc = check_rows_span(fn, rows, ldx, ldy)) return rc;
  const int64_t es = y_dtype == Q4_F32 ? 4 : 2;
  int64_t row0 = 0;
  for (int w = 0; w < n_windows; ++w) {
    const uint16_t* xw = x + row0 * ldx;
    void* yw = (uint8_t*)y + row0 * ldy * es;
    if (int rc = qmm_window_impl(fn, bits, packed_a, packed_b, N, K, xw, ldx, window_rows[w], yw, y_dtype, ldy, s)) return rc;
    row0 += window_rows[w];
  }
  return Q4_OK;
}

int check_rope_args(const char* fn, const q4_rope_kv* a, int R, q4::RopeKvArgs* out) {
  if (a == nullptr) return fail(Q4_EINVAL, "%s: args is NULL", fn);
  if (a->n_q_heads < 1 || a->n_kv_heads < 1 || a->n_q_heads > 4096 || a->n_kv_heads > 4096)
    return fail(Q4_EINVAL, "%s: n_q_heads=%d and n_kv_heads=%d must be 1..4096", fn, a->n_q_heads, a->n_kv_heads);
  if (a->rot_dims < 0 || a->rot_dims > 64 || (a->rot_dims & 1))
    return fail(Q4_EINVAL, "%s: rot_dims=%d is not an even number in 0..64", fn, a->rot_dims);
  if (!(a->theta > 0.f) || !isfinite(a->theta)) return fail(Q4_EINVAL, "%s: theta must be positive and finite", fn);
  if (!(a->eps >= 0.f) || !isfinite(a->eps)) return fail(Q4_EINVAL, "%s: eps must be >= 0 and finite", fn);
  if (a->cache_dtype != Q4_F32 && a->cache_dtype != Q4_BF16) return fail(Q4_EINVAL, "%s: cache_dtype %d is not Q4_F32 or Q4_BF16", fn, a->cache_dtype);
  // positions are int32, so a longer ring would never be filled
  if (a->ring_len < 1 || a->ring_len > (int64_t(1) << 31))
    return fail(Q4_EINVAL, "%s: ring_len=%lld is outside 1..2^31", fn, (long long)a->ring_len);
  if (a->ldq < (int64_t)a->n_q_heads * 64) return fail(Q4_EINVAL, "%s: ldq=%lld < n_q_heads * 64", fn, (long long)a->ldq);
  if (int rc = check_ld(fn, "ldq", a->ldq)) return rc;
  if (int rc = check_ptr(fn, "pos", a->pos, 4)) return rc;
  if (int rc = check_ptr(fn, "q_out", a->q_out, 4)) return rc;
  const uintptr_t ce = a->cache_dtype == Q4_F32 ? 4 : 2;
  if (int rc = check_ptr(fn, "k_cache", a->k_cache, ce)) return rc;
  if (int rc = check_ptr(fn, "v_cache", a->v_cache, ce)) return rc;
  if (a->gamma_q != nullptr && !aligned(a->gamma_q, 4)) return fail(Q4_EALIGN, "%s: gamma_q is not 4-byte aligned", fn);
  if (a->gamma_k != nullptr && !aligned(a->gamma_k, 4)) return fail(Q4_EALIGN, "%s: gamma_k is not 4-byte aligned", fn);
  if (a->n_gate_heads < 0 || a->n_gate_heads > 4096) return fail(Q4_EINVAL, "%s: n_gate_heads=%d must be 0..4096", fn, a->n_gate_heads);
  if (a->n_gate_heads > 0) {
    if (a->ldg < (int64_t)a->n_gate_heads * 64) return fail(Q4_EINVAL, "%s: ldg=%lld < n_gate_heads * 64", fn, (long long)a->ldg);
    if (int rc = check_ld(fn, "ldg", a->ldg)) return rc;
    if (int rc = check_ptr(fn, "gate_out", a->gate_out, 4)) return rc;
  }
  if (a->cache_row_stride < 0) return fail(Q4_EINVAL, "%s: cache_row_stride=%lld < 0", fn, (long long)a->cache_row_stride);
  if (int rc = check_ld(fn, "cache_row_stride", a->cache_row_stride)) return rc;
  if (a->cache_row_stride > 0 && a->cache_row_stride < a->ring_len * a->n_kv_heads * 64)
    return fail(Q4_EINVAL, "%s: cache_row_stride=%lld is below ring_len * n_kv_heads * 64: the rows' rings would overlap", fn,
                (long long)a->cache_row_stride);
  (void)R;
  q4::RopeKvArgs r{};
  for (int i = 0; i < a->rot_dims / 2; ++i) r.inv[i] = pow((double)a->theta, -2.0 * (double)i / (double)a->rot_dims);
  r.pos = a->pos;
  r.n_q = a->n_q_heads;
  r.n_kv = a->n_kv_heads;
  r.rot = a->rot_dims;
  r.theta = a->theta;
  r.eps = a->eps;
  r.gamma_q = a->gamma_q;
  r.gamma_k = a->gamma_k;
  r.q_out = a->q_out;
  r.ldq = a->ldq;
  r.k_cache = a->k_cache;
  r.v_cache = a->v_cache;
  r.cache_bf16 = a->cache_dtype == Q4_BF16;
  r.ring = a->ring_len;
  r.row_stride = a->cache_row_stride;
  r.n_gate = a->n_gate_heads;
  r.gate_out = a->n_gate_heads > 0 ? a->gate_out : nullptr;
  r.ldg = a->n_gate_heads > 0 ? a->ldg : 0;
  *out = r;
  return Q4_OK;
}

template <int SPW, int NV, int BITS>
int qkv_rope_launch_t(const uint8_t* pk, int N, int K, const uint16_t* x, int64_t ldx, int R, const q4::RopeKvArgs& a, size_t lds,
                      int heads, hipStream_t s) {
  auto kern = q4::qkv_rope_kernel<SPW, NV, BITS>;
  static const bool lds_ok = q4::allow_max_dynamic_lds((const void*)kern);
  (void)lds_ok;
  hipLaunchKernelGGL(kern, dim3((unsigned)heads), dim3(q4::kQkvWaves * 64), lds, s, pk, N, K, x, ldx, R, a);
  return launched("qmv_qkv_rope");
}

template <int SPW, int BITS>
int qkv_rope_launch_nv(int nv, const uint8_t* pk, int N, int K, const uint16_t* x, int64_t ldx, int R, const q4::RopeKvArgs& a,
                       size_t lds, int heads, hipStream_t s) {
  if (nv == 1) return qkv_rope_launch_t<SPW, 1, BITS>(pk, N, K, x, ldx, R, a, lds, heads, s);
  if (nv == 2) return qkv_rope_launch_t<SPW, 2, BITS>(pk, N, K, x, ldx, R, a, lds, heads, s);
  return qkv_rope_launch_t<SPW, 4, BITS>(pk, N, K, x, ldx, R, a, lds, heads, s);
}

template <int BITS>
int qkv_rope_launch_bits(int spw, int nv, const uint8_t* pk, int N, int K, const uint16_t* x, int64_t ldx, int R,
                         const q4::RopeKvArgs& a, size_t lds, int heads, hipStream_t s) {
  if (spw <= 1) return qkv_rope_launch_nv<1, BITS>(nv, pk, N, K, x, ldx, R, a, lds, heads, s);
  if (spw <= 2) return qkv_rope_launch_nv<2, BITS>(nv, pk, N, K, x, ldx, R, a, lds, heads, s);
  return qkv_rope_launch_nv<4, BITS>(nv, pk, N, K, x, ldx, R, a, lds, heads, s);
}

}  // namespace

// ---- the split matvec without a caller workspace ---------------------------
// Its workspace is this file-scope device array: one copy per GPU, held from
// the library's load until the process ends. In host code `scratch` names a
// host-side stand-in, never the device memory: the device address comes from
// hipGetSymbolAddress, taken once per device with that device current.
constexpr size_t kScratchBytes = size_t(8) << 20;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];
namespace {

constexpr int kScratchDevices = 64;
std::atomic<uint8_t*> g_scratch[kScratchDevices];
std::mutex g_scratch_mu;

__global__ void zero_words_kernel(uint32_t* p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) p[i] = 0u;
}

// This device's copy of the scratch array; at the first call on a device its
// address is looked up and the counter area cleared by a kernel on `s` (a
// kernel rather than a memset, so that a graph that captures the first call
// replays correctly). Returns nullptr with the error recorded on failure.
uint8_t* scratch_on_device(const char* fn, hipStream_t s) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kScratchDevices) {
    fail(Q4_EDEVICE, "%s: no usable current device", fn);
    return nullptr;
  }
  uint8_t* p = g_scratch[dev].load(std::memory_order_acquire);
  if (p != nullptr) return p;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  p = g_scratch[dev].load(std::memory_order_relaxed);
  if (p != nullptr) return p;
  void* addr = nullptr;
  const hipError_t e = hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch));
  if (e != hipSuccess || addr == nullptr) {
    fail(Q4_EDEVICE, "%s: hipGetSymbolAddress(scratch) failed on device %d: %s", fn, dev, hipGetErrorString(e));
    return nullptr;
  }
  // every counter block a split matvec can use lies in the first 1 MiB
  hipLaunchKernelGGL(zero_words_kernel, dim3(256), dim3(256), 0, s, (uint32_t*)addr, (int64_t)(size_t(1) << 20) / 4);
  if (hipGetLastError() != hipSuccess) {
    fail(Q4_EDEVICE, "%s: clearing the scratch counters failed on device %d", fn, dev);
    return nullptr;
  }
  p = (uint8_t*)addr;
  g_scratch[dev].store(p, std::memory_order_release);
  return p;
}

}  // namespace

extern "C" {

int q4g64_abi_version(void) { return 4; }

const char* q4_last_error(void) { return g_err; }

size_t q4g64_packed_bytes(int64_t N, int64_t K) { return packed_bytes_impl(4, N, K); }

size_t qg64_packed_bytes(int bits, int64_t N, int64_t K) { return packed_bytes_impl(bits, N, K); }

size_t q4g64_x3t_bytes(int64_t K, int R) {
  if (K <= 0 || K % 64 != 0 || K > q4::kQmvMaxK || R < 1 || R > 16) return 0;
  return (size_t)q4::qmv_x3t_bytes(K, R);
}

int pack_q4g64(const uint32_t* wq, const uint16_t* scales, const uint16_t* biases, int64_t N, int64_t K, void* packed,
               void* stream) {
  return pack_impl("pack_q4g64", 4, wq, scales, biases, N, K, packed, (hipStream_t)stream);
}

int pack_qg64(int bits, const uint32_t* wq, const uint16_t* scales, const uint16_t* biases, int64_t N, int64_t K, void* packed,
              void* stream) {
  return pack_impl("pack_qg64", bits, wq, scales, biases, N, K, packed, (hipStream_t)stream);
}

int unpack_q4g64(const void* packed, int64_t N, int64_t K, uint32_t* wq, uint16_t* scales, uint16_t* biases,
                 void* stream) {
  return unpack_impl("unpack_q4g64", 4, packed, N, K, wq, scales, biases, (hipStream_t)stream);
}

int unpack_qg64(int bits, const void* packed, int64_t N, int64_t K, uint32_t* wq, uint16_t* scales, uint16_t* biases,
                void* stream) {
  return unpack_impl("unpack_qg64", bits, packed, N, K, wq, scales, biases, (hipStream_t)stream);
}

int qmv_rows(const void* packed, int64_t N, int64_t K, const void* x, int x_dtype, int64_t ldx, int R, float* y,
             int64_t ldy, void* stream) {
  return qmv_rows_impl("qmv_rows", 4, packed, N, K, x, x_dtype, ldx, R, y, ldy, (hipStream_t)stream);
}

int qmv_rows_qg64(int bits, const void* packed, int64_t N, int64_t K, const void* x, int x_dtype, int64_t ldx, int R, float* y,
                  int64_t ldy, void* stream) {
  if (int rc = check_bits("qmv_rows_qg64", bits)) return rc;
  return qmv_rows_impl("qmv_rows_qg64", bits, packed, N, K, x, x_dtype, ldx, R, y, ldy, (hipStream_t)stream);
}

int qmv_w13_swiglu(const void* packed_w1, const void* packed_w3, int64_t N, int64_t K, const uint16_t* x, int64_t ldx,
                   int R, float* y, int64_t ldy, void* stream) {
  return qmv_w13_impl("qmv_w13_swiglu", 4, packed_w1, packed_w3, N, K, x, ldx, R, y, ldy, (hipStream_t)stream);
}

int qmv_w13_swiglu_qg64(int bits, const void* packed_w1, const void* packed_w3, int64_t N, int64_t K, const uint16_t* x,
                        int64_t ldx, int R, float* y, int64_t ldy, void* stream) {
  if (int rc = check_bits("qmv_w13_swiglu_qg64", bits)) return rc;
  return qmv_w13_impl("qmv_w13_swiglu_qg64", bits, packed_w1, packed_w3, N, K, x, ldx, R, y, ldy, (hipStream_t)stream);
}

int qmv_w13_swiglu_x3(int bits, const void* packed_w1, const void* packed_w3, int64_t N, int64_t K, const uint16_t* x,
                      int64_t ldx, int R, uint16_t* z3, int64_t ldz, void* stream) {
  if (int rc = check_bits("qmv_w13_swiglu_x3", bits)) return rc;
  return qmv_w13_impl("qmv_w13_swiglu_x3", bits, packed_w1, packed_w3, N, K, x, ldx, R, z3, ldz, (hipStream_t)stream, 1);
}

int qmv_w13_swiglu_x3t(int bits, const void* packed_w1, const void* packed_w3, int64_t N, int64_t K, const uint16_t* x,
                       int64_t ldx, int R, uint16_t* z3t, void* stream) {
  if (int rc = check_bits("qmv_w13_swiglu_x3t", bits)) return rc;
  return qmv_w13_impl("qmv_w13_swiglu_x3t", bits, packed_w1, packed_w3, N, K, x, ldx, R, z3t, N, (hipStream_t)stream, 2);
}

int qmm_window(const void* packed_a, const void* packed_b, int64_t N, int64_t K, const uint16_t* x, int64_t ldx, int64_t M,
               void* y, int y_dtype, int64_t ldy, void* stream) {
  return qmm_window_checked("qmm_window", 4, packed_a, packed_b, N, K, x, ldx, M, y, y_dtype, ldy, (hipStream_t)stream);
}

int qmm_window_qg64(int bits, const void* packed_a, const void* packed_b, int64_t N, int64_t K, const uint16_t* x, int64_t ldx,
                    int64_t M, void* y, int y_dtype, int64_t ldy, void* stream) {
  if (int rc = check_bits("qmm_window_qg64", bits)) return rc;
  return qmm_window_checked("qmm_window_qg64", bits, packed_a, packed_b, N, K, x, ldx, M, y, y_dtype, ldy, (hipStream_t)stream);
}

int qmm_cut(const void* packed_a, const void* packed_b, int64_t N, int64_t K, const uint16_t* x, int64_t ldx,
            const int64_t* window_rows, int n_windows, void* y, int y_dtype, int64_t ldy, void* stream) {
  return qmm_cut_impl("qmm_cut", 4, packed_a, packed_b, N, K, x, ldx, window_rows, n_windows, y, y_dtype, ldy, (hipStream_t)stream);
}

int qmm_cut_qg64(int bits, const void* packed_a, const void* packed_b, int64_t N, int64_t K, const uint16_t* x, int64_t ldx,
                 const int64_t* window_rows, int n_windows, void* y, int y_dtype, int64_t ldy, void* stream) {
  if (int rc = check_bits("qmm_cut_qg64", bits)) return rc;
  return qmm_cut_impl("qmm_cut_qg64", bits, packed_a, packed_b, N, K, x, ldx, window_rows, n_windows, y, y_dtype, ldy,
                      (hipStream_t)stream);
}

size_t q4g64_ffn_work_bytes(int64_t N1, int64_t N2, int R) {
  if (N1 <= 0 || N1 % 64 != 0 || N1 > kFfnMaxN1 || N2 <= 0 || N2 % 64 != 0 || N2 > kMaxDim || R < 1 || R > 16) return 0;
  return ffn_planes_off(N1, N2) + (size_t)q4::qmv_x3t_bytes(N1, 16);
}

int qmv_ffn(const void* packed_w1, const void* packed_w3, const void* packed_w2, int64_t N1, int64_t K1, int64_t N2,
            const uint16_t* x, int64_t ldx, int R, float* z, int64_t ldz, float* y, int64_t ldy, void* work, void* stream) {
  const char* fn = "qmv_ffn";
  if (int rc = check_nk(fn, N1, K1)) return rc;
  if (int rc = check_nk(fn, N2, N1)) return rc;
  if (R < 1 || R > 16) return fail(Q4_EINVAL, "%s: R=%d is outside 1..16", fn, R);
  if (int rc = check_ptr(fn, "packed_w1", packed_w1, 16)) return rc;
  if (int rc = check_ptr(fn, "packed_w3", packed_w3, 16)) return rc;
  if (int rc = check_ptr(fn, "packed_w2", packed_w2, 16)) return rc;
  if (int rc = check_x(fn, x, Q4_BF16, ldx, K1)) return rc;
  if (int rc = check_ptr(fn, "z", z, 4)) return rc;
  if (int rc = check_ptr(fn, "y", y, 4)) return rc;
  if (int rc = check_ptr(fn, "work", work, 256)) return rc;
  if (ldz < N1) return fail(Q4_EINVAL, "%s: ldz=%lld < N1=%lld", fn, (long long)ldz, (long long)N1);
  if (ldy < N2) return fail(Q4_EINVAL, "%s: ldy=%lld < N2=%lld", fn, (long long)ldy, (long long)N2);
  if (int rc = check_ld(fn, "ldz", ldz)) return rc;
  if (int rc = check_ld(fn, "ldy", ldy)) return rc;
  if ((int64_t)R * ldx * 2 >= (int64_t(1) << 31))
    return fail(Q4_EUNSUPPORTED, "%s: R * ldx spans more than 2 GiB of activations", fn);
  // the dataflow step's shape limits (8 waves per w1/w3 tile and 16 per w2
  // half-tile, up to 2 segments each; a 1024-thread workgroup leaves 128
  // registers per lane), kept for every row count
  if (K1 > kFfnMaxK1) return fail(Q4_EUNSUPPORTED, "%s: K1=%lld exceeds the decode FFN step limit of 4096", fn, (long long)K1);
  if (N1 > kFfnMaxN1) return fail(Q4_EUNSUPPORTED, "%s: N1=%lld exceeds the decode FFN step limit of 8192", fn, (long long)N1);
  const uint8_t *a = (const uint8_t*)packed_w1, *c = (const uint8_t*)packed_w3, *d = (const uint8_t*)packed_w2;
  uint8_t* w = (uint8_t*)work;
  hipStream_t s = (hipStream_t)stream;
  const int n1 = (int)N1, k1 = (int)K1, n2 = (int)N2;
  if (ffn_flow_applies(N1, K1, R) && q4::flow_lds_bytes(K1, R) <= q4::qmv_max_lds()) {
    const int spw1 = (q4::qmv_segments(K1) + q4::kFfnP1Waves - 1) / q4::kFfnP1Waves;
    if (R == 1) return flow_launch_s1<1>(spw1, a, c, d, n1, k1, n2, x, ldx, R, z, ldz, y, ldy, w, s);
    return flow_launch_s1<2>(spw1, a, c, d, n1, k1, n2, x, ldx, R, z, ldz, y, ldy, w, s);
  }
  // two calls: w1/w3 + SwiGLU writing z as float32 rows and as its
  // fragment-ordered planes in the workspace, then w2 reading the planes
  // (the same bits as from the float32 rows)
  if (q4::qmv_lds_bytes(K1, 0, 2, R) > kMaxLds || q4::qmv_lds_bytes(N1, 1, 1, R) > kMaxLds)
    return fail(Q4_EUNSUPPORTED, "%s: K1=%lld, N1=%lld with R=%d exceed the decode partials' LDS", fn, (long long)K1, (long long)N1, R);
  uint16_t* planes = (uint16_t*)(w + ffn_planes_off(N1, N2));
  q4::QmvSplit sp{1, nullptr, nullptr};
  sp.z32 = z;
  sp.ldz32 = ldz;
  q4::qmv_launch(a, c, 2, n1, k1, x, 0, ldx, R, (float*)planes, N1, s, 4, 2, sp);
  q4::qmv_launch(d, d, 1, n2, n1, planes, 3, N1, R, y, ldy, s, 4);
  return launched(fn);
}

size_t fp8b_packed_bytes(int64_t N, int64_t K) { return packed_bytes_impl(8, N, K); }

int pack_fp8b(const uint8_t* w8, const float* scales, int64_t N, int64_t K, void* packed, void* stream) {
  const char* fn = "pack_fp8b";
  if (int rc = check_nk(fn, N, K)) return rc;
  if (int rc = check_ptr(fn, "w8", w8, 16)) return rc;
  if (int rc = check_ptr(fn, "scales", scales, 4)) return rc;
  if (int rc = check_ptr(fn, "packed", packed, 16)) return rc;
  hipStream_t s = (hipStream_t)stream;
  const int64_t words = q4::codes_bytes(N, K, 8) / 4;
  const int64_t sb_entries = (N / q4::kTileN) * q4::n_pairs(K) * q4::kTileN;
  uint8_t* out = (uint8_t*)packed;
  hipLaunchKernelGGL(q4::pack_codes_wide_kernel<8>, dim3(grid_for(words, 256)), dim3(256), 0, s, (const uint32_t*)w8, N, K,
                     (uint32_t*)out);
  if (int rc = launched(fn)) return rc;
  hipLaunchKernelGGL(q4::pack_scale_fp8_kernel, dim3(grid_for(sb_entries, 256)), dim3(256), 0, s, scales, N, K,
                     (q4::u32x2*)(out + q4::codes_bytes(N, K, 8)));
  return launched(fn);
}

int unpack_fp8b(const void* packed, int64_t N, int64_t K, uint8_t* w8, float* scales, void* stream) {
  const char* fn = "unpack_fp8b";
  if (int rc = check_nk(fn, N, K)) return rc;
  if (int rc = check_ptr(fn, "packed", packed, 16)) return rc;
  if (int rc = check_ptr(fn, "w8", w8, 16)) return rc;
  if (int rc = check_ptr(fn, "scales", scales, 4)) return rc;
  hipStream_t s = (hipStream_t)stream;
  const uint8_t* in = (const uint8_t*)packed;
  hipLaunchKernelGGL(q4::unpack_codes_wide_kernel<8>, dim3(grid_for(N * (K / 4), 256)), dim3(256), 0, s, (const uint32_t*)in, N, K,
                     (uint32_t*)w8);
  if (int rc = launched(fn)) return rc;
  const int64_t blocks = ((N + 127) / 128) * q4::n_pairs(K);
  hipLaunchKernelGGL(q4::unpack_scale_fp8_kernel, dim3(grid_for(blocks, 256)), dim3(256), 0, s,
                     (const q4::u32x2*)(in + q4::codes_bytes(N, K, 8)), N, K, scales);
  return launched(fn);
}

int qmv_rows_fp8b(const void* packed, int64_t N, int64_t K, const void* x, int x_dtype, int64_t ldx, int R, float* y, int64_t ldy,
                  void* stream) {
  return qmv_rows_impl("qmv_rows_fp8b", q4::kFmtFp8, packed, N, K, x, x_dtype, ldx, R, y, ldy, (hipStream_t)stream);
}

int qmv_w13_swiglu_fp8b(const void* packed_w1, const void* packed_w3, int64_t N, int64_t K, const uint16_t* x, int64_t ldx, int R,
                        float* y, int64_t ldy, void* stream) {
  return qmv_w13_impl("qmv_w13_swiglu_fp8b", q4::kFmtFp8, packed_w1, packed_w3, N, K, x, ldx, R, y, ldy, (hipStream_t)stream);
}

int qmv_w13_swiglu_x3_fp8b(const void* packed_w1, const void* packed_w3, int64_t N, int64_t K, const uint16_t* x, int64_t ldx,
                           int R, uint16_t* z3, int64_t ldz, void* stream) {
  return qmv_w13_impl("qmv_w13_swiglu_x3_fp8b", q4::kFmtFp8, packed_w1, packed_w3, N, K, x, ldx, R, z3, ldz, (hipStream_t)stream, 1);
}

int qmv_w13_swiglu_x3t_fp8b(const void* packed_w1, const void* packed_w3, int64_t N, int64_t K, const uint16_t* x, int64_t ldx,
                            int R, uint16_t* z3t, void* stream) {
  return qmv_w13_impl("qmv_w13_swiglu_x3t_fp8b", q4::kFmtFp8, packed_w1, packed_w3, N, K, x, ldx, R, z3t, N, (hipStream_t)stream, 2);
}

int qmm_window_fp8b(const void* packed_a, const void* packed_b, int64_t N, int64_t K, const uint16_t* x, int64_t ldx, int64_t M,
                    void* y, int y_dtype, int64_t ldy, void* stream) {
  return qmm_window_checked("qmm_window_fp8b", q4::kFmtFp8, packed_a, packed_b, N, K, x, ldx, M, y, y_dtype, ldy,
                            (hipStream_t)stream);
}

int qmm_cut_fp8b(const void* packed_a, const void* packed_b, int64_t N, int64_t K, const uint16_t* x, int64_t ldx,
                 const int64_t* window_rows, int n_windows, void* y, int y_dtype, int64_t ldy, void* stream) {
  return qmm_cut_impl("qmm_cut_fp8b", q4::kFmtFp8, packed_a, packed_b, N, K, x, ldx, window_rows, n_windows, y, y_dtype, ldy,
                      (hipStream_t)stream);
}

int rope_kv_store(const float* qkv, int64_t ldqkv, int R, const q4_rope_kv* args, void* stream) {
  const char* fn = "rope_kv_store";
  q4::RopeKvArgs a;
  if (int rc = check_rope_args(fn, args, R, &a)) return rc;
  if (R < 1 || R > 65535) return fail(Q4_EINVAL, "%s: R=%d is outside 1..65535", fn, R);
  if (int rc = check_ptr(fn, "qkv", qkv, 4)) return rc;
  const int heads = a.n_q + 2 * a.n_kv + a.n_gate;
  if (ldqkv < (int64_t)heads * 64)
    return fail(Q4_EINVAL, "%s: ldqkv=%lld < (n_q_heads + 2 n_kv_heads + n_gate_heads) * 64", fn, (long long)ldqkv);
  if (int rc = check_ld(fn, "ldqkv", ldqkv)) return rc;
  hipLaunchKernelGGL(q4::rope_kv_kernel, dim3((unsigned)heads, (unsigned)R), dim3(64), 0, (hipStream_t)stream, qkv, ldqkv, a);
  return launched(fn);
}

int qmv_qkv_rope(int bits, const void* packed_qkv, int64_t K, const uint16_t* x, int64_t ldx, int R, const q4_rope_kv* args,
                 void* stream) {
  const char* fn = "qmv_qkv_rope";
  if (int rc = check_bits(fn, bits)) return rc;
  q4::RopeKvArgs a;
  if (int rc = check_rope_args(fn, args, R, &a)) return rc;
  const int heads = a.n_q + 2 * a.n_kv + a.n_gate;
  const int64_t N = (int64_t)heads * 64;
  if (int rc = check_nk(fn, N, K)) return rc;
  if (R < 1 || R > 16) return fail(Q4_EINVAL, "%s: R=%d is outside 1..16", fn, R);
  if (int rc = check_ptr(fn, "packed_qkv", packed_qkv, 16)) return rc;
  if (int rc = check_x(fn, x, Q4_BF16, ldx, K)) return rc;
  if ((int64_t)R * ldx * 2 >= (int64_t(1) << 31)) return fail(Q4_EUNSUPPORTED, "%s: R * ldx spans more than 2 GiB of activations", fn);
  // four waves per 16-column tile, up to 4 segments each
  if (K > 4096) return fail(Q4_EUNSUPPORTED, "%s: K=%lld exceeds the fused limit of 4096", fn, (long long)K);
  const int nv = q4::qmv_nv(R);
  const size_t lds = q4::qkv_rope_lds_bytes(K, nv, R);
  if (lds > q4::qmv_max_lds()) return fail(Q4_EUNSUPPORTED, "%s: K=%lld with R=%d needs %zu bytes of LDS", fn, (long long)K, R, lds);
  const int nseg = q4::qmv_segments(K), spw = (nseg + 3) / 4;
  const uint8_t* pk = (const uint8_t*)packed_qkv;
  hipStream_t s = (hipStream_t)stream;
  if (bits == 6) return qkv_rope_launch_bits<6>(spw, nv, pk, (int)N, (int)K, x, ldx, R, a, lds, heads, s);
  if (bits == 8) return qkv_rope_launch_bits<8>(spw, nv, pk, (int)N, (int)K, x, ldx, R, a, lds, heads, s);
  return qkv_rope_launch_bits<4>(spw, nv, pk, (int)N, (int)K, x, ldx, R, a, lds, heads, s);
}

size_t qmv_split_work_bytes(int bits, int64_t N, int64_t K, int x_dtype, int R, int splits) {
  if ((bits != 4 && bits != 6 && bits != 8) || N <= 0 || K <= 0 || N % 64 || K % 64 || N > kMaxDim || K > q4::kQmvMaxK || R < 1 ||
      R > 16 || splits < 0 || splits > kSplitMax)
    return 0;
  if (x_dtype != Q4_BF16 && x_dtype != Q4_F32 && x_dtype != Q4_BF16X3 && x_dtype != Q4_BF16X3T) return 0;
  const int xmode = xmode_of(x_dtype);
  const int nshare = split_shares(splits, xmode, N, K, R);
  return q4::qmv_split_work_bytes(1, xmode, (int)N, (int)K, R, nshare);
}

size_t qmv_split_noalloc_max_bytes(void) { return kScratchBytes; }

int qmv_rows_split_noalloc(int bits, const void* packed, int64_t N, int64_t K, const void* x, int x_dtype, int64_t ldx, int R,
                           float* y, int64_t ldy, int splits, void* stream) {
  const char* fn = "qmv_rows_split_noalloc";
  if (int rc = qmv_split_check(fn, bits, packed, N, K, x, x_dtype, ldx, R, y, ldy, splits)) return rc;
  const int xmode = xmode_of(x_dtype);
  const int nshare = split_shares(splits, xmode, N, K, R);
  uint8_t* work = nullptr;
  if (nshare > 1) {
    const size_t need = q4::qmv_split_work_bytes(1, xmode, (int)N, (int)K, R, nshare);
    const q4::QmvSplitShape sh = q4::qmv_split_shape(1, xmode, (int)N, (int)K, R, nshare);
    if (need > kScratchBytes || q4::qmv_split_counter_bytes(sh) > (size_t(1) << 20))
      return fail(Q4_EUNSUPPORTED, "%s: this shape needs %zu bytes of scratch, more than the %zu the library holds per GPU", fn, need,
                  kScratchBytes);
    work = scratch_on_device(fn, (hipStream_t)stream);
    if (work == nullptr) return Q4_EDEVICE;
  }
  return qmv_split_launch(fn, bits, packed, N, K, x, x_dtype, ldx, R, y, ldy, nshare, work, (hipStream_t)stream);
}

int qmv_rows_split(int bits, const void* packed, int64_t N, int64_t K, const void* x, int x_dtype, int64_t ldx, int R, float* y,
                   int64_t ldy, int splits, void* work, size_t work_bytes, void* stream) {
  const char* fn = "qmv_rows_split";
  if (int rc = qmv_split_check(fn, bits, packed, N, K, x, x_dtype, ldx, R, y, ldy, splits)) return rc;
  const int xmode = xmode_of(x_dtype);
  const int nshare = split_shares(splits, xmode, N, K, R);
  if (nshare > 1) {
    const size_t need = q4::qmv_split_work_bytes(1, xmode, (int)N, (int)K, R, nshare);
    if (int rc = check_ptr(fn, "work", work, 256)) return rc;
    if (work_bytes < need) return fail(Q4_EINVAL, "%s: work_bytes=%zu < %zu needed for this shape", fn, work_bytes, need);
  }
  return qmv_split_launch(fn, bits, packed, N, K, x, x_dtype, ldx, R, y, ldy, nshare, (uint8_t*)work, (hipStream_t)stream);
}

static const int kCostRows[5] = {1, 2, 4, 8, 16};

int qmv_window_costs(int bits, const void* packed, int64_t N, int64_t K, const void* x, int x_dtype, int64_t ldx, float* y,
                     int64_t ldy, int reps, float* us_out, void* stream) {
  const char* fn = "qmv_window_costs";
  if (int rc = check_bits(fn, bits)) return rc;
  if (us_out == nullptr) return fail(Q4_EINVAL, "%s: us_out is NULL", fn);
  if (reps < 1 || reps > 10000) return fail(Q4_EINVAL, "%s: reps=%d is outside 1..10000", fn, reps);
  hipStream_t s = (hipStream_t)stream;
  // validates every argument at the largest row count, and warms every kernel up twice
  for (int rep = 0; rep < 2; ++rep)
    for (int i = 4; i >= 0; --i)
      if (int rc = qmv_rows_impl(fn, bits, packed, N, K, x, x_dtype, ldx, kCostRows[i], y, ldy, s)) return rc;
  hipEvent_t e0 = nullptr, e1 = nullptr;
  if (hipEventCreate(&e0) != hipSuccess || hipEventCreate(&e1) != hipSuccess) {
    if (e0) (void)hipEventDestroy(e0);
    return fail(Q4_EDEVICE, "%s: could not create timing events", fn);
  }
  int rc = Q4_OK;
  for (int i = 0; i < 5 && rc == Q4_OK; ++i) {
    if (hipEventRecord(e0, s) != hipSuccess) { rc = fail(Q4_EDEVICE, "%s: event record failed", fn); break; }
    for (int r = 0; r < reps && rc == Q4_OK; ++r) rc = qmv_rows_impl(fn, bits, packed, N, K, x, x_dtype, ldx, kCostRows[i], y, ldy, s);
    if (rc != Q4_OK) break;
    float ms = 0.f;
    if (hipEventRecord(e1, s) != hipSuccess || hipEventSynchronize(e1) != hipSuccess || hipEventElapsedTime(&ms, e0, e1) != hipSuccess)
      rc = fail(Q4_EDEVICE, "%s: event timing failed", fn);
    else
      us_out[i] = ms * 1000.f / (float)reps;
  }
  (void)hipEventDestroy(e0);
  (void)hipEventDestroy(e1);
  return rc;
}

float qmv_window_cost(const float* us, int R) {
  if (us == nullptr || R < 1 || R > 16) return NAN;
  for (int i = 0; i < 5; ++i)
    if (R == kCostRows[i]) return us[i];  // a timed row count reads back its own entry
  for (int i = 0; i < 4; ++i) {
    if (R < kCostRows[i + 1]) {
      const float t = (float)(R - kCostRows[i]) / (float)(kCostRows[i + 1] - kCostRows[i]);
      return us[i] + t * (us[i + 1] - us[i]);
    }
  }
  return us[4];
}

}  // extern "C"
