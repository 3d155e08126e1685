// Host-side argument validation of every q4g64.h entry point, for a build of
// the library's host code under AddressSanitizer and UndefinedBehaviorSanitizer.
//
// Every call below carries at least one invalid argument, so validation must
// reject it before anything is enqueued: the device pointers are fake,
// suitably aligned addresses that nothing may dereference (a host read of one
// would fault), and host arrays (window rows, the rope struct, the cost table)
// are heap copies of exactly the documented length, so a read past them is a
// sanitizer report. The host-only queries (sizes, the cost interpolation) are
// checked against their documented values. The program prints one line per
// failed expectation and exits with the number of failures.
#include "q4g64.h"

#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include <vector>

namespace {

int g_cases = 0, g_bad = 0;

void expect_rc(int line, const char* what, int rc, int want, const char* fn) {
  ++g_cases;
  const char* msg = q4_last_error();
  if (rc != want) {
    ++g_bad;
    printf("FAIL line %d: %s returned %d, expected %d (%s)\n", line, what, rc, want, msg);
    return;
  }
  // every rejection names its entry point in the message
  if (want != Q4_OK && (msg == nullptr || strncmp(msg, fn, strlen(fn)) != 0)) {
    ++g_bad;
    printf("FAIL line %d: %s: message \"%s\" does not start with %s\n", line, what, msg ? msg : "(null)", fn);
  }
}

void expect_size(int line, const char* what, size_t got, size_t want) {
  ++g_cases;
  if (got != want) {
    ++g_bad;
    printf("FAIL line %d: %s = %zu, expected %zu\n", line, what, got, want);
  }
}

void expect_true(int line, const char* what, bool ok) {
  ++g_cases;
  if (!ok) {
    ++g_bad;
    printf("FAIL line %d: %s\n", line, what);
  }
}

#define RC(fn, call, want) expect_rc(__LINE__, #call, (call), (want), #fn)
#define SIZE(call, want) expect_size(__LINE__, #call, (size_t)(call), (size_t)(want))
#define TRUE(cond) expect_true(__LINE__, #cond, (cond))

// Fake device addresses: 4 KiB aligned, never mapped on the host.
char* const D = reinterpret_cast<char*>(uintptr_t(0x7e0000000000ull));
void* const P = D;                                       // a packed matrix
void* const P2 = D + (1 << 20);
void* const P3 = D + (2 << 20);
uint16_t* const X = reinterpret_cast<uint16_t*>(D + (3 << 20));
float* const Y = reinterpret_cast<float*>(D + (4 << 20));
float* const Z = reinterpret_cast<float*>(D + (5 << 20));
void* const W = D + (6 << 20);                           // a workspace

const int64_t I64MAX = INT64_MAX, I64MIN = INT64_MIN;
const int IMAX = 2147483647, IMIN = -2147483647 - 1;

template <class T>
T* off(T* p, int bytes) { return reinterpret_cast<T*>(reinterpret_cast<uintptr_t>(p) + (uintptr_t)bytes); }

void sizes() {
  TRUE(q4g64_abi_version() == 4);
  SIZE(q4g64_packed_bytes(64, 64), 16 * 1152 / 4);  // 4 column tiles, one pair of 1 KiB + 128 B
  SIZE(q4g64_packed_bytes(128, 256), 8 * 2 * 1152);
  SIZE(q4g64_packed_bytes(0, 64), 0);
  SIZE(q4g64_packed_bytes(64, 100), 0);
  SIZE(q4g64_packed_bytes(-64, 64), 0);
  SIZE(q4g64_packed_bytes(I64MAX, 64), 0);
  SIZE(q4g64_packed_bytes(64, I64MIN), 0);
  SIZE(q4g64_packed_bytes(int64_t(1) << 31, 64), 0);            // a dimension above 2^30
  SIZE(q4g64_packed_bytes(int64_t(1) << 25, int64_t(1) << 25), 0);  // N*K above 2^40
  SIZE(qg64_packed_bytes(5, 64, 64), 0);
  SIZE(qg64_packed_bytes(IMIN, 64, 64), 0);
  TRUE(qg64_packed_bytes(6, 128, 256) > q4g64_packed_bytes(128, 256));
  TRUE(qg64_packed_bytes(8, 128, 256) > qg64_packed_bytes(6, 128, 256));
  SIZE(fp8b_packed_bytes(128, 256), qg64_packed_bytes(8, 128, 256));
  SIZE(fp8b_packed_bytes(128, 32), 0);
  // fragment-ordered pieces: 32 bytes per k per row tile of 4 (1, 2 or 4 tiles)
  SIZE(q4g64_x3t_bytes(256, 1), 32 * 256);
  SIZE(q4g64_x3t_bytes(256, 5), 2 * 32 * 256);
  SIZE(q4g64_x3t_bytes(256, 16), 4 * 32 * 256);
  SIZE(q4g64_x3t_bytes(0, 1), 0);
  SIZE(q4g64_x3t_bytes(100, 1), 0);
  SIZE(q4g64_x3t_bytes(16384 + 64, 1), 0);
  SIZE(q4g64_x3t_bytes(I64MAX, 1), 0);
  SIZE(q4g64_x3t_bytes(256, 0), 0);
  SIZE(q4g64_x3t_bytes(256, 17), 0);
  SIZE(q4g64_x3t_bytes(256, IMIN), 0);
  // split workspace: 0 for anything invalid
  TRUE(qmv_split_work_bytes(4, 128, 512, Q4_BF16, 1, 2) > 0);
  SIZE(qmv_split_work_bytes(5, 128, 512, Q4_BF16, 1, 2), 0);
  SIZE(qmv_split_work_bytes(4, 100, 512, Q4_BF16, 1, 2), 0);
  SIZE(qmv_split_work_bytes(4, 128, 16384 + 64, Q4_BF16, 1, 2), 0);
  SIZE(qmv_split_work_bytes(4, I64MAX, 512, Q4_BF16, 1, 2), 0);
  SIZE(qmv_split_work_bytes(4, 128, I64MIN, Q4_BF16, 1, 2), 0);
  SIZE(qmv_split_work_bytes(4, 128, 512, 7, 1, 2), 0);
  SIZE(qmv_split_work_bytes(4, 128, 512, -1, 1, 2), 0);
  SIZE(qmv_split_work_bytes(4, 128, 512, Q4_BF16, 0, 2), 0);
  SIZE(qmv_split_work_bytes(4, 128, 512, Q4_BF16, 17, 2), 0);
  SIZE(qmv_split_work_bytes(4, 128, 512, Q4_BF16, 1, -1), 0);
  SIZE(qmv_split_work_bytes(4, 128, 512, Q4_BF16, 1, 17), 0);
  SIZE(qmv_split_work_bytes(4, 128, 512, Q4_BF16, 1, IMAX), 0);
  TRUE(qmv_split_noalloc_max_bytes() >= (size_t(1) << 20));
  // decode FFN workspace: the one-launch step's state for up to 2 rows, then
  // the two-call step's fragment-ordered planes for up to 16 rows; any R
  SIZE(q4g64_ffn_work_bytes(256, 128, 1), 4352 + 8 * 2 * 256 + 32 * 128 + 128 * 256);
  SIZE(q4g64_ffn_work_bytes(8192, 4096, 4), 4352 + 8 * 2 * 8192 + 32 * 4096 + 128 * 8192);
  SIZE(q4g64_ffn_work_bytes(192, 128, 1), 4352 + 8 * 2 * 192 + 32 * 128 + 128 * 192);
  SIZE(q4g64_ffn_work_bytes(256, 128, 5), 4352 + 8 * 2 * 256 + 32 * 128 + 128 * 256);
  SIZE(q4g64_ffn_work_bytes(256, 128, 16), 4352 + 8 * 2 * 256 + 32 * 128 + 128 * 256);
  SIZE(q4g64_ffn_work_bytes(0, 128, 1), 0);
  SIZE(q4g64_ffn_work_bytes(256, 100, 1), 0);
  SIZE(q4g64_ffn_work_bytes(8192 + 256, 128, 1), 0);
  SIZE(q4g64_ffn_work_bytes(256, I64MAX, 1), 0);
  SIZE(q4g64_ffn_work_bytes(I64MIN, 128, 1), 0);
  SIZE(q4g64_ffn_work_bytes(256, 128, 0), 0);
  SIZE(q4g64_ffn_work_bytes(256, 128, 17), 0);
}

void cost_table() {
  std::vector<float> us = {1.f, 2.f, 4.f, 8.f, 16.f};
  for (int r = 1; r <= 16; ++r) TRUE(qmv_window_cost(us.data(), r) == (float)r);  // linear table reads back R
  std::vector<float> c = {3.f, 5.f, 6.f, 10.f, 12.f};
  TRUE(qmv_window_cost(c.data(), 3) == 5.5f);
  TRUE(qmv_window_cost(c.data(), 12) == 11.f);
  TRUE(isnan(qmv_window_cost(c.data(), 0)));
  TRUE(isnan(qmv_window_cost(c.data(), 17)));
  TRUE(isnan(qmv_window_cost(c.data(), IMIN)));
  TRUE(isnan(qmv_window_cost(nullptr, 4)));
}

void pack_calls() {
  const uint32_t* wq = reinterpret_cast<const uint32_t*>(X);
  const uint16_t* sc = X;
  RC(pack_q4g64, pack_q4g64(wq, sc, sc, 100, 64, P, nullptr), Q4_EINVAL);
  RC(pack_q4g64, pack_q4g64(wq, sc, sc, 64, I64MIN, P, nullptr), Q4_EINVAL);
  RC(pack_q4g64, pack_q4g64(wq, sc, sc, int64_t(1) << 25, int64_t(1) << 25, P, nullptr), Q4_EINVAL);
  RC(pack_q4g64, pack_q4g64(nullptr, sc, sc, 64, 64, P, nullptr), Q4_EALIGN);
  RC(pack_q4g64, pack_q4g64(off(wq, 4), sc, sc, 64, 64, P, nullptr), Q4_EALIGN);
  RC(pack_q4g64, pack_q4g64(wq, nullptr, sc, 64, 64, P, nullptr), Q4_EALIGN);
  RC(pack_q4g64, pack_q4g64(wq, off(sc, 1), sc, 64, 64, P, nullptr), Q4_EALIGN);
  RC(pack_q4g64, pack_q4g64(wq, sc, off(sc, 1), 64, 64, P, nullptr), Q4_EALIGN);
  RC(pack_q4g64, pack_q4g64(wq, sc, sc, 64, 64, nullptr, nullptr), Q4_EALIGN);
  RC(pack_q4g64, pack_q4g64(wq, sc, sc, 64, 64, off(P, 8), nullptr), Q4_EALIGN);
  RC(pack_qg64, pack_qg64(5, wq, sc, sc, 64, 64, P, nullptr), Q4_EINVAL);
  RC(pack_qg64, pack_qg64(IMAX, wq, sc, sc, 64, 64, P, nullptr), Q4_EINVAL);
  RC(pack_qg64, pack_qg64(6, wq, sc, sc, 64, -64, P, nullptr), Q4_EINVAL);
  RC(pack_qg64, pack_qg64(8, wq, sc, nullptr, 64, 64, P, nullptr), Q4_EALIGN);
  uint32_t* owq = reinterpret_cast<uint32_t*>(Y);
  uint16_t* osc = reinterpret_cast<uint16_t*>(Z);
  RC(unpack_q4g64, unpack_q4g64(P, 64, 32, owq, osc, osc, nullptr), Q4_EINVAL);
  RC(unpack_q4g64, unpack_q4g64(nullptr, 64, 64, owq, osc, osc, nullptr), Q4_EALIGN);
  RC(unpack_q4g64, unpack_q4g64(off(P, 8), 64, 64, owq, osc, osc, nullptr), Q4_EALIGN);
  RC(unpack_q4g64, unpack_q4g64(P, 64, 64, nullptr, osc, osc, nullptr), Q4_EALIGN);
  RC(unpack_q4g64, unpack_q4g64(P, 64, 64, owq, off(osc, 1), osc, nullptr), Q4_EALIGN);
  RC(unpack_qg64, unpack_qg64(7, P, 64, 64, owq, osc, osc, nullptr), Q4_EINVAL);
  RC(unpack_qg64, unpack_qg64(6, P, I64MAX, 64, owq, osc, osc, nullptr), Q4_EINVAL);
  RC(unpack_qg64, unpack_qg64(8, P, 64, 64, owq, osc, nullptr, nullptr), Q4_EALIGN);
  const uint8_t* w8 = reinterpret_cast<const uint8_t*>(X);
  const float* fsc = Y;
  RC(pack_fp8b, pack_fp8b(w8, fsc, 64, 100, P, nullptr), Q4_EINVAL);
  RC(pack_fp8b, pack_fp8b(nullptr, fsc, 64, 64, P, nullptr), Q4_EALIGN);
  RC(pack_fp8b, pack_fp8b(off(w8, 8), fsc, 64, 64, P, nullptr), Q4_EALIGN);
  RC(pack_fp8b, pack_fp8b(w8, off(fsc, 2), 64, 64, P, nullptr), Q4_EALIGN);
  RC(pack_fp8b, pack_fp8b(w8, fsc, 64, 64, off(P, 4), nullptr), Q4_EALIGN);
  RC(unpack_fp8b, unpack_fp8b(P, -64, 64, reinterpret_cast<uint8_t*>(Z), Y, nullptr), Q4_EINVAL);
  RC(unpack_fp8b, unpack_fp8b(P, 64, 64, nullptr, Y, nullptr), Q4_EALIGN);
  RC(unpack_fp8b, unpack_fp8b(P, 64, 64, reinterpret_cast<uint8_t*>(Z), off(Y, 1), nullptr), Q4_EALIGN);
}

// Decode matvecs: base shape N = 128, K = 256, one bf16 row.
void decode_calls() {
  RC(qmv_rows, qmv_rows(P, 100, 256, X, Q4_BF16, 256, 1, Y, 128, nullptr), Q4_EINVAL);
  RC(qmv_rows, qmv_rows(P, 128, 0, X, Q4_BF16, 256, 1, Y, 128, nullptr), Q4_EINVAL);
  RC(qmv_rows, qmv_rows(P, I64MAX, 256, X, Q4_BF16, 256, 1, Y, 128, nullptr), Q4_EINVAL);
  RC(qmv_rows, qmv_rows(P, 128, I64MIN, X, Q4_BF16, 256, 1, Y, 128, nullptr), Q4_EINVAL);
  RC(qmv_rows, qmv_rows(P, 128, 256, X, Q4_BF16, 256, 0, Y, 128, nullptr), Q4_EINVAL);
  RC(qmv_rows, qmv_rows(P, 128, 256, X, Q4_BF16, 256, 17, Y, 128, nullptr), Q4_EINVAL);
  RC(qmv_rows, qmv_rows(P, 128, 256, X, Q4_BF16, 256, IMIN, Y, 128, nullptr), Q4_EINVAL);
  RC(qmv_rows, qmv_rows(P, 128, 256, X, Q4_BF16, 256, IMAX, Y, 128, nullptr), Q4_EINVAL);
  RC(qmv_rows, qmv_rows(nullptr, 128, 256, X, Q4_BF16, 256, 1, Y, 128, nullptr), Q4_EALIGN);
  RC(qmv_rows, qmv_rows(off(P, 8), 128, 256, X, Q4_BF16, 256, 1, Y, 128, nullptr), Q4_EALIGN);
  RC(qmv_rows, qmv_rows(P, 128, 256, X, 4, 256, 1, Y, 128, nullptr), Q4_EINVAL);
  RC(qmv_rows, qmv_rows(P, 128, 256, X, -1, 256, 1, Y, 128, nullptr), Q4_EINVAL);
  RC(qmv_rows, qmv_rows(P, 128, 256, X, IMAX, 256, 1, Y, 128, nullptr), Q4_EINVAL);
  RC(qmv_rows, qmv_rows(P, 128, 256, nullptr, Q4_BF16, 256, 1, Y, 128, nullptr), Q4_EALIGN);
  RC(qmv_rows, qmv_rows(P, 128, 256, off(X, 2), Q4_BF16, 256, 1, Y, 128, nullptr), Q4_EALIGN);
  RC(qmv_rows, qmv_rows(P, 128, 256, X, Q4_BF16, 255, 1, Y, 128, nullptr), Q4_EINVAL);
  RC(qmv_rows, qmv_rows(P, 128, 256, X, Q4_BF16, I64MIN, 1, Y, 128, nullptr), Q4_EINVAL);
  RC(qmv_rows, qmv_rows(P, 128, 256, X, Q4_BF16, 260, 1, Y, 128, nullptr), Q4_EALIGN);  // 520-byte rows
  RC(qmv_rows, qmv_rows(P, 128, 256, X, Q4_F32, 258, 1, Y, 128, nullptr), Q4_EALIGN);   // 1032-byte rows
  RC(qmv_rows, qmv_rows(P, 128, 256, X, Q4_BF16, I64MAX, 1, Y, 128, nullptr), Q4_EINVAL);
  RC(qmv_rows, qmv_rows(P, 128, 256, X, Q4_F32, I64MAX - 7, 1, Y, 128, nullptr), Q4_EINVAL);
  RC(qmv_rows, qmv_rows(P, 128, 256, X, Q4_BF16, int64_t(1) << 30, 1, Y, 128, nullptr), Q4_EUNSUPPORTED);  // 2 GiB of x
  RC(qmv_rows, qmv_rows(P, 128, 256, X, Q4_BF16X3, int64_t(1) << 28, 2, Y, 128, nullptr), Q4_EUNSUPPORTED);
  RC(qmv_rows, qmv_rows(P, 128, 256, X, Q4_BF16X3T, 512, 1, Y, 128, nullptr), Q4_EINVAL);  // no row stride
  RC(qmv_rows, qmv_rows(P, 128, 256, X, Q4_BF16, 256, 1, nullptr, 128, nullptr), Q4_EALIGN);
  RC(qmv_rows, qmv_rows(P, 128, 256, X, Q4_BF16, 256, 1, off(Y, 2), 128, nullptr), Q4_EALIGN);
  RC(qmv_rows, qmv_rows(P, 128, 256, X, Q4_BF16, 256, 1, Y, 127, nullptr), Q4_EINVAL);
  RC(qmv_rows, qmv_rows(P, 128, 256, X, Q4_BF16, 256, 1, Y, I64MIN, nullptr), Q4_EINVAL);
  RC(qmv_rows, qmv_rows(P, 128, 256, X, Q4_BF16, 256, 16, Y, I64MAX, nullptr), Q4_EINVAL);
  RC(qmv_rows, qmv_rows(P, 128, 16384 + 64, X, Q4_BF16, 16384 + 64, 1, Y, 128, nullptr), Q4_EUNSUPPORTED);
  RC(qmv_rows_qg64, qmv_rows_qg64(5, P, 128, 256, X, Q4_BF16, 256, 1, Y, 128, nullptr), Q4_EINVAL);
  RC(qmv_rows_qg64, qmv_rows_qg64(0, P, 128, 256, X, Q4_BF16, 256, 1, Y, 128, nullptr), Q4_EINVAL);
  RC(qmv_rows_qg64, qmv_rows_qg64(IMIN, P, 128, 256, X, Q4_BF16, 256, 1, Y, 128, nullptr), Q4_EINVAL);
  RC(qmv_rows_qg64, qmv_rows_qg64(6, P, 128, 256, X, Q4_BF16, 256, 1, Y, 64, nullptr), Q4_EINVAL);
  RC(qmv_rows_qg64, qmv_rows_qg64(8, P, 128, 256, X, Q4_BF16, 256, 0, Y, 128, nullptr), Q4_EINVAL);
  RC(qmv_rows_fp8b, qmv_rows_fp8b(P, 128, 200, X, Q4_BF16, 256, 1, Y, 128, nullptr), Q4_EINVAL);
  RC(qmv_rows_fp8b, qmv_rows_fp8b(P, 128, 256, X, Q4_BF16, 256, 1, off(Y, 1), 128, nullptr), Q4_EALIGN);

  // K split: K = 512 has two segments, so splits = 2 needs a workspace
  const size_t need = qmv_split_work_bytes(4, 128, 512, Q4_BF16, 1, 2);
  RC(qmv_rows_split, qmv_rows_split(4, P, 128, 512, X, Q4_BF16, 512, 1, Y, 128, -1, W, need, nullptr), Q4_EINVAL);
  RC(qmv_rows_split, qmv_rows_split(4, P, 128, 512, X, Q4_BF16, 512, 1, Y, 128, 17, W, need, nullptr), Q4_EINVAL);
  RC(qmv_rows_split, qmv_rows_split(4, P, 128, 512, X, Q4_BF16, 512, 1, Y, 128, IMIN, W, need, nullptr), Q4_EINVAL);
  RC(qmv_rows_split, qmv_rows_split(3, P, 128, 512, X, Q4_BF16, 512, 1, Y, 128, 2, W, need, nullptr), Q4_EINVAL);
  RC(qmv_rows_split, qmv_rows_split(4, P, 128, 512, X, Q4_BF16, 512, 1, Y, 128, 2, nullptr, need, nullptr), Q4_EALIGN);
  RC(qmv_rows_split, qmv_rows_split(4, P, 128, 512, X, Q4_BF16, 512, 1, Y, 128, 2, off(W, 16), need, nullptr), Q4_EALIGN);
  RC(qmv_rows_split, qmv_rows_split(4, P, 128, 512, X, Q4_BF16, 512, 1, Y, 128, 2, W, need - 1, nullptr), Q4_EINVAL);
  RC(qmv_rows_split, qmv_rows_split(4, P, 128, 512, X, Q4_BF16, 512, 1, Y, 128, 2, W, 0, nullptr), Q4_EINVAL);
  RC(qmv_rows_split, qmv_rows_split(4, P, 128, 512, X, Q4_BF16, I64MAX, 1, Y, 128, 2, W, need, nullptr), Q4_EINVAL);
  RC(qmv_rows_split, qmv_rows_split(4, P, 128, 512, X, Q4_BF16, 512, 1, Y, I64MAX, 2, W, need, nullptr), Q4_EINVAL);
  RC(qmv_rows_split_noalloc, qmv_rows_split_noalloc(4, P, 128, 512, X, Q4_BF16, 512, 1, Y, 128, -1, nullptr), Q4_EINVAL);
  RC(qmv_rows_split_noalloc, qmv_rows_split_noalloc(4, P, 100, 512, X, Q4_BF16, 512, 1, Y, 128, 2, nullptr), Q4_EINVAL);
  RC(qmv_rows_split_noalloc, qmv_rows_split_noalloc(4, P, 128, 512, X, Q4_BF16, 512, 1, off(Y, 2), 128, 2, nullptr), Q4_EALIGN);
  // partial sums beyond the fixed scratch array
  RC(qmv_rows_split_noalloc,
     qmv_rows_split_noalloc(4, P, int64_t(1) << 20, 16384, X, Q4_BF16, 16384, 16, Y, int64_t(1) << 20, 16, nullptr), Q4_EUNSUPPORTED);
}

void fused_decode_calls() {
  RC(qmv_w13_swiglu, qmv_w13_swiglu(P, P2, 100, 256, X, 256, 1, Y, 128, nullptr), Q4_EINVAL);
  RC(qmv_w13_swiglu, qmv_w13_swiglu(P, P2, 128, 256, X, 256, 0, Y, 128, nullptr), Q4_EINVAL);
  RC(qmv_w13_swiglu, qmv_w13_swiglu(nullptr, P2, 128, 256, X, 256, 1, Y, 128, nullptr), Q4_EALIGN);
  RC(qmv_w13_swiglu, qmv_w13_swiglu(P, nullptr, 128, 256, X, 256, 1, Y, 128, nullptr), Q4_EALIGN);
  RC(qmv_w13_swiglu, qmv_w13_swiglu(P, off(P2, 8), 128, 256, X, 256, 1, Y, 128, nullptr), Q4_EALIGN);
  RC(qmv_w13_swiglu, qmv_w13_swiglu(P, P2, 128, 256, off(X, 8), 256, 1, Y, 128, nullptr), Q4_EALIGN);
  RC(qmv_w13_swiglu, qmv_w13_swiglu(P, P2, 128, 256, X, 255, 1, Y, 128, nullptr), Q4_EINVAL);
  RC(qmv_w13_swiglu, qmv_w13_swiglu(P, P2, 128, 256, X, I64MAX, 1, Y, 128, nullptr), Q4_EINVAL);
  RC(qmv_w13_swiglu, qmv_w13_swiglu(P, P2, 128, 256, X, 256, 1, Y, 120, nullptr), Q4_EINVAL);
  RC(qmv_w13_swiglu, qmv_w13_swiglu(P, P2, 128, 256, X, 256, 1, Y, I64MAX, nullptr), Q4_EINVAL);
  RC(qmv_w13_swiglu, qmv_w13_swiglu(P, P2, 128, 8192 + 64, X, 8192 + 64, 1, Y, 128, nullptr), Q4_EUNSUPPORTED);
  RC(qmv_w13_swiglu, qmv_w13_swiglu(P, P2, 128, 256, X, int64_t(1) << 30, 1, Y, 128, nullptr), Q4_EUNSUPPORTED);
  RC(qmv_w13_swiglu_qg64, qmv_w13_swiglu_qg64(2, P, P2, 128, 256, X, 256, 1, Y, 128, nullptr), Q4_EINVAL);
  RC(qmv_w13_swiglu_qg64, qmv_w13_swiglu_qg64(6, P, P2, 128, 256, X, 256, 1, nullptr, 128, nullptr), Q4_EALIGN);
  uint16_t* z3 = reinterpret_cast<uint16_t*>(Z);
  RC(qmv_w13_swiglu_x3, qmv_w13_swiglu_x3(4, P, P2, 128, 256, X, 256, 1, z3, 132, nullptr), Q4_EALIGN);  // 264-byte planes rows
  RC(qmv_w13_swiglu_x3, qmv_w13_swiglu_x3(4, P, P2, 128, 256, X, 256, 1, off(z3, 8), 128, nullptr), Q4_EALIGN);
  RC(qmv_w13_swiglu_x3, qmv_w13_swiglu_x3(4, P, P2, 128, 256, X, 256, 1, z3, 64, nullptr), Q4_EINVAL);
  RC(qmv_w13_swiglu_x3, qmv_w13_swiglu_x3(4, P, P2, 128, 256, X, 256, 1, z3, I64MAX, nullptr), Q4_EINVAL);
  RC(qmv_w13_swiglu_x3, qmv_w13_swiglu_x3(9, P, P2, 128, 256, X, 256, 1, z3, 128, nullptr), Q4_EINVAL);
  RC(qmv_w13_swiglu_x3t, qmv_w13_swiglu_x3t(4, P, P2, 16384 + 64, 256, X, 256, 1, z3, nullptr), Q4_EUNSUPPORTED);
  RC(qmv_w13_swiglu_x3t, qmv_w13_swiglu_x3t(4, P, P2, 128, 256, X, 256, 17, z3, nullptr), Q4_EINVAL);
  RC(qmv_w13_swiglu_x3t, qmv_w13_swiglu_x3t(4, P, P2, 128, 256, X, 256, 1, nullptr, nullptr), Q4_EALIGN);
  RC(qmv_w13_swiglu_fp8b, qmv_w13_swiglu_fp8b(P, P2, 128, 256, X, 256, 1, Y, 127, nullptr), Q4_EINVAL);
  RC(qmv_w13_swiglu_x3_fp8b, qmv_w13_swiglu_x3_fp8b(P, P2, 128, 256, X, 256, 1, z3, 132, nullptr), Q4_EALIGN);
  RC(qmv_w13_swiglu_x3t_fp8b, qmv_w13_swiglu_x3t_fp8b(P, P2, 128, 256, X, 256, 1, off(z3, 2), nullptr), Q4_EALIGN);
}

// Prompt windows: base shape N = 256, K = 256, M = 128 bf16 rows.
void window_calls() {
  RC(qmm_window, qmm_window(P, nullptr, 256, 100, X, 256, 128, Y, Q4_F32, 256, nullptr), Q4_EINVAL);
  RC(qmm_window, qmm_window(P, nullptr, 256, 256, X, 256, 0, Y, Q4_F32, 256, nullptr), Q4_EINVAL);
  RC(qmm_window, qmm_window(P, nullptr, 256, 256, X, 256, -5, Y, Q4_F32, 256, nullptr), Q4_EINVAL);
  RC(qmm_window, qmm_window(P, nullptr, 256, 256, X, 256, (int64_t(1) << 24) + 1, Y, Q4_F32, 256, nullptr), Q4_EINVAL);
  RC(qmm_window, qmm_window(P, nullptr, 256, 256, X, 256, I64MAX, Y, Q4_F32, 256, nullptr), Q4_EINVAL);
  RC(qmm_window, qmm_window(nullptr, nullptr, 256, 256, X, 256, 128, Y, Q4_F32, 256, nullptr), Q4_EALIGN);
  RC(qmm_window, qmm_window(P, off(P2, 8), 256, 256, X, 256, 128, Y, Q4_F32, 256, nullptr), Q4_EALIGN);
  RC(qmm_window, qmm_window(P, nullptr, 256, 256, X, 250, 128, Y, Q4_F32, 256, nullptr), Q4_EINVAL);
  RC(qmm_window, qmm_window(P, nullptr, 256, 256, X, 260, 128, Y, Q4_F32, 256, nullptr), Q4_EALIGN);
  RC(qmm_window, qmm_window(P, nullptr, 256, 256, X, I64MAX, 128, Y, Q4_F32, 256, nullptr), Q4_EINVAL);
  RC(qmm_window, qmm_window(P, nullptr, 256, 256, X, int64_t(1) << 30, 128, Y, Q4_F32, 256, nullptr), Q4_EUNSUPPORTED);
  RC(qmm_window, qmm_window(P, nullptr, 256, 256, X, 256, 128, Y, 2, 256, nullptr), Q4_EINVAL);
  RC(qmm_window, qmm_window(P, nullptr, 256, 256, X, 256, 128, Y, Q4_BF16X3, 256, nullptr), Q4_EINVAL);
  RC(qmm_window, qmm_window(P, nullptr, 256, 256, X, 256, 128, off(Y, 2), Q4_F32, 256, nullptr), Q4_EALIGN);
  RC(qmm_window, qmm_window(P, nullptr, 256, 256, X, 256, 128, off(Y, 1), Q4_BF16, 256, nullptr), Q4_EALIGN);
  RC(qmm_window, qmm_window(P, nullptr, 256, 256, X, 256, 128, Y, Q4_F32, 255, nullptr), Q4_EINVAL);
  RC(qmm_window, qmm_window(P, nullptr, 256, 256, X, 256, 128, Y, Q4_F32, I64MAX, nullptr), Q4_EINVAL);
  RC(qmm_window, qmm_window(P, nullptr, 64, (int64_t(1) << 20) + 64, X, (int64_t(1) << 20) + 64, 128, Y, Q4_F32, 64, nullptr),
     Q4_EUNSUPPORTED);
  // more workgroups than a launch holds
  RC(qmm_window, qmm_window(P, nullptr, int64_t(1) << 28, 64, X, 64, int64_t(1) << 20, Y, Q4_F32, int64_t(1) << 28, nullptr),
     Q4_EUNSUPPORTED);
  // a window's rows must lie within 2^48 elements of x and of y
  RC(qmm_window, qmm_window(P, nullptr, 256, 256, X, 256, int64_t(1) << 24, Y, Q4_F32, int64_t(1) << 25, nullptr), Q4_EINVAL);
  RC(qmm_window_qg64, qmm_window_qg64(4 + 1, P, nullptr, 256, 256, X, 256, 128, Y, Q4_F32, 256, nullptr), Q4_EINVAL);
  RC(qmm_window_qg64, qmm_window_qg64(6, P, P2, 256, 256, X, 256, 128, Y, Q4_F32, 100, nullptr), Q4_EINVAL);
  RC(qmm_window_fp8b, qmm_window_fp8b(P, nullptr, 256, 256, X, 256, 0, Y, Q4_F32, 256, nullptr), Q4_EINVAL);
  RC(qmm_window_fp8b, qmm_window_fp8b(off(P, 4), nullptr, 256, 256, X, 256, 128, Y, Q4_F32, 256, nullptr), Q4_EALIGN);

  // window drivers: the rows array is read only within n_windows
  std::vector<int64_t>* rows = new std::vector<int64_t>{64, 128, 0};
  RC(qmm_cut, qmm_cut(P, nullptr, 256, 256, X, 256, rows->data(), 3, Y, Q4_F32, 256, nullptr), Q4_EINVAL);
  (*rows)[2] = -64;
  RC(qmm_cut, qmm_cut(P, nullptr, 256, 256, X, 256, rows->data(), 3, Y, Q4_F32, 256, nullptr), Q4_EINVAL);
  (*rows)[2] = (int64_t(1) << 24) + 1;
  RC(qmm_cut, qmm_cut(P, nullptr, 256, 256, X, 256, rows->data(), 3, Y, Q4_F32, 256, nullptr), Q4_EINVAL);
  (*rows)[2] = I64MAX;
  RC(qmm_cut, qmm_cut(P, nullptr, 256, 256, X, 256, rows->data(), 3, Y, Q4_F32, 256, nullptr), Q4_EINVAL);
  (*rows)[2] = 64;
  RC(qmm_cut, qmm_cut(P, nullptr, 256, 256, X, 256, rows->data(), 0, Y, Q4_F32, 256, nullptr), Q4_EINVAL);
  RC(qmm_cut, qmm_cut(P, nullptr, 256, 256, X, 256, rows->data(), -1, Y, Q4_F32, 256, nullptr), Q4_EINVAL);
  RC(qmm_cut, qmm_cut(P, nullptr, 256, 256, X, 256, rows->data(), IMIN, Y, Q4_F32, 256, nullptr), Q4_EINVAL);
  RC(qmm_cut, qmm_cut(P, nullptr, 256, 256, X, 256, nullptr, 3, Y, Q4_F32, 256, nullptr), Q4_EINVAL);
  RC(qmm_cut, qmm_cut(P, nullptr, 256, 256, X, 256, rows->data(), 3, Y, 5, 256, nullptr), Q4_EINVAL);
  RC(qmm_cut, qmm_cut(P, nullptr, 256, 256, X, 250, rows->data(), 3, Y, Q4_F32, 256, nullptr), Q4_EINVAL);
  // windows that each fit, while the later ones would start beyond 2^48 elements of y
  std::vector<int64_t>* big = new std::vector<int64_t>(1024, int64_t(1) << 18);
  RC(qmm_cut, qmm_cut(P, nullptr, 256, 256, X, 256, big->data(), 1024, Y, Q4_F32, int64_t(1) << 30, nullptr), Q4_EINVAL);
  RC(qmm_cut, qmm_cut(P, nullptr, 256, 256, X, int64_t(1) << 22, big->data(), 1024, Y, Q4_F32, 256, nullptr), Q4_EINVAL);
  RC(qmm_cut_qg64, qmm_cut_qg64(7, P, nullptr, 256, 256, X, 256, rows->data(), 3, Y, Q4_F32, 256, nullptr), Q4_EINVAL);
  RC(qmm_cut_qg64, qmm_cut_qg64(8, P, nullptr, 256, 256, X, 256, rows->data(), 3, nullptr, Q4_F32, 256, nullptr), Q4_EALIGN);
  RC(qmm_cut_fp8b, qmm_cut_fp8b(P, nullptr, 256, 256, X, 256, rows->data(), 0, Y, Q4_F32, 256, nullptr), Q4_EINVAL);
  delete big;
  delete rows;
}

void ffn_calls() {
  // base: N1 = 512, K1 = 256, N2 = 128, one row
  RC(qmv_ffn, qmv_ffn(P, P2, P3, 500, 256, 128, X, 256, 1, Z, 512, Y, 128, W, nullptr), Q4_EINVAL);
  RC(qmv_ffn, qmv_ffn(P, P2, P3, 512, 0, 128, X, 256, 1, Z, 512, Y, 128, W, nullptr), Q4_EINVAL);
  RC(qmv_ffn, qmv_ffn(P, P2, P3, 512, 256, -128, X, 256, 1, Z, 512, Y, 128, W, nullptr), Q4_EINVAL);
  RC(qmv_ffn, qmv_ffn(P, P2, P3, 512, 256, I64MAX, X, 256, 1, Z, 512, Y, 128, W, nullptr), Q4_EINVAL);
  RC(qmv_ffn, qmv_ffn(P, P2, P3, 512, 256, 128, X, 256, 0, Z, 512, Y, 128, W, nullptr), Q4_EINVAL);
  RC(qmv_ffn, qmv_ffn(P, P2, P3, 512, 256, 128, X, 256, 17, Z, 512, Y, 128, W, nullptr), Q4_EINVAL);
  RC(qmv_ffn, qmv_ffn(nullptr, P2, P3, 512, 256, 128, X, 256, 1, Z, 512, Y, 128, W, nullptr), Q4_EALIGN);
  RC(qmv_ffn, qmv_ffn(P, nullptr, P3, 512, 256, 128, X, 256, 1, Z, 512, Y, 128, W, nullptr), Q4_EALIGN);
  RC(qmv_ffn, qmv_ffn(P, P2, off(P3, 8), 512, 256, 128, X, 256, 1, Z, 512, Y, 128, W, nullptr), Q4_EALIGN);
  RC(qmv_ffn, qmv_ffn(P, P2, P3, 512, 256, 128, off(X, 4), 256, 1, Z, 512, Y, 128, W, nullptr), Q4_EALIGN);
  RC(qmv_ffn, qmv_ffn(P, P2, P3, 512, 256, 128, X, 200, 1, Z, 512, Y, 128, W, nullptr), Q4_EINVAL);
  RC(qmv_ffn, qmv_ffn(P, P2, P3, 512, 256, 128, X, I64MAX, 1, Z, 512, Y, 128, W, nullptr), Q4_EINVAL);
  RC(qmv_ffn, qmv_ffn(P, P2, P3, 512, 256, 128, X, 256, 1, nullptr, 512, Y, 128, W, nullptr), Q4_EALIGN);
  RC(qmv_ffn, qmv_ffn(P, P2, P3, 512, 256, 128, X, 256, 1, Z, 512, off(Y, 2), 128, W, nullptr), Q4_EALIGN);
  RC(qmv_ffn, qmv_ffn(P, P2, P3, 512, 256, 128, X, 256, 1, Z, 512, Y, 128, nullptr, nullptr), Q4_EALIGN);
  RC(qmv_ffn, qmv_ffn(P, P2, P3, 512, 256, 128, X, 256, 1, Z, 512, Y, 128, off(W, 128), nullptr), Q4_EALIGN);
  RC(qmv_ffn, qmv_ffn(P, P2, P3, 512, 256, 128, X, 256, 1, Z, 511, Y, 128, W, nullptr), Q4_EINVAL);
  RC(qmv_ffn, qmv_ffn(P, P2, P3, 512, 256, 128, X, 256, 1, Z, I64MAX, Y, 128, W, nullptr), Q4_EINVAL);
  RC(qmv_ffn, qmv_ffn(P, P2, P3, 512, 256, 128, X, 256, 1, Z, 512, Y, 64, W, nullptr), Q4_EINVAL);
  RC(qmv_ffn, qmv_ffn(P, P2, P3, 512, 256, 128, X, 256, 1, Z, 512, Y, I64MAX, W, nullptr), Q4_EINVAL);
  RC(qmv_ffn, qmv_ffn(P, P2, P3, 512, 4096 + 64, 128, X, 4096 + 64, 1, Z, 512, Y, 128, W, nullptr), Q4_EUNSUPPORTED);
  RC(qmv_ffn, qmv_ffn(P, P2, P3, 8192 + 64, 256, 128, X, 256, 1, Z, 8192 + 64, Y, 128, W, nullptr), Q4_EUNSUPPORTED);
  RC(qmv_ffn, qmv_ffn(P, P2, P3, 512, 256, 128, X, int64_t(1) << 30, 1, Z, 512, Y, 128, W, nullptr), Q4_EUNSUPPORTED);
}

q4_rope_kv rope_base() {
  q4_rope_kv a;
  memset(&a, 0, sizeof a);
  a.pos = reinterpret_cast<const int32_t*>(D + (7 << 20));
  a.n_q_heads = 4;
  a.n_kv_heads = 2;
  a.rot_dims = 32;
  a.theta = 10000.f;
  a.eps = 1e-6f;
  a.q_out = Y;
  a.ldq = 256;
  a.k_cache = D + (8 << 20);
  a.v_cache = D + (9 << 20);
  a.cache_dtype = Q4_F32;
  a.ring_len = 64;
  a.ldg = 0;
  a.cache_row_stride = 0;
  return a;
}

// One invalid field at a time, through both rope entry points. The struct
// lives on the heap so a read past it is reported.
void rope_case(int line, void (*edit)(q4_rope_kv*), int want) {
  q4_rope_kv* a = new q4_rope_kv(rope_base());
  edit(a);
  const float* qkv = Z;
  expect_rc(line, "rope_kv_store(edited args)", rope_kv_store(qkv, 1024, 1, a, nullptr), want, "rope_kv_store");
  expect_rc(line, "qmv_qkv_rope(edited args)", qmv_qkv_rope(4, P, 256, X, 256, 1, a, nullptr), want, "qmv_qkv_rope");
  delete a;
}

#define ROPE(body, want) rope_case(__LINE__, [](q4_rope_kv* a) { body; }, want)

void rope_calls() {
  ROPE(a->n_q_heads = 0, Q4_EINVAL);
  ROPE(a->n_q_heads = 4097, Q4_EINVAL);
  ROPE(a->n_kv_heads = -1, Q4_EINVAL);
  ROPE(a->n_kv_heads = IMAX, Q4_EINVAL);
  ROPE(a->rot_dims = 3, Q4_EINVAL);
  ROPE(a->rot_dims = -2, Q4_EINVAL);
  ROPE(a->rot_dims = 66, Q4_EINVAL);
  ROPE(a->rot_dims = IMIN, Q4_EINVAL);
  ROPE(a->theta = 0.f, Q4_EINVAL);
  ROPE(a->theta = -1.f, Q4_EINVAL);
  ROPE(a->theta = NAN, Q4_EINVAL);
  ROPE(a->theta = INFINITY, Q4_EINVAL);
  ROPE(a->eps = -1e-6f, Q4_EINVAL);
  ROPE(a->eps = NAN, Q4_EINVAL);
  ROPE(a->eps = INFINITY, Q4_EINVAL);
  ROPE(a->cache_dtype = Q4_BF16X3, Q4_EINVAL);
  ROPE(a->cache_dtype = -1, Q4_EINVAL);
  ROPE(a->ring_len = 0, Q4_EINVAL);
  ROPE(a->ring_len = I64MIN, Q4_EINVAL);
  ROPE(a->ring_len = (int64_t(1) << 31) + 1, Q4_EINVAL);  // positions are int32
  ROPE(a->ring_len = I64MAX; a->cache_row_stride = 1, Q4_EINVAL);
  ROPE(a->ldq = 255, Q4_EINVAL);
  ROPE(a->ldq = I64MIN, Q4_EINVAL);
  ROPE(a->ldq = I64MAX, Q4_EINVAL);
  ROPE(a->pos = nullptr, Q4_EALIGN);
  ROPE(a->pos = off(a->pos, 2), Q4_EALIGN);
  ROPE(a->q_out = nullptr, Q4_EALIGN);
  ROPE(a->q_out = off(a->q_out, 1), Q4_EALIGN);
  ROPE(a->k_cache = off(a->k_cache, 2), Q4_EALIGN);
  ROPE(a->v_cache = nullptr, Q4_EALIGN);
  ROPE(a->cache_dtype = Q4_BF16; a->v_cache = off(a->v_cache, 1), Q4_EALIGN);
  ROPE(a->gamma_q = off(Y, 2), Q4_EALIGN);
  ROPE(a->gamma_k = off(Y, 1), Q4_EALIGN);
  ROPE(a->n_gate_heads = -1, Q4_EINVAL);
  ROPE(a->n_gate_heads = 4097, Q4_EINVAL);
  ROPE(a->n_gate_heads = 2; a->ldg = 127; a->gate_out = Z, Q4_EINVAL);
  ROPE(a->n_gate_heads = 2; a->ldg = I64MAX; a->gate_out = Z, Q4_EINVAL);
  ROPE(a->n_gate_heads = 2; a->ldg = 128; a->gate_out = nullptr, Q4_EALIGN);
  ROPE(a->cache_row_stride = -1, Q4_EINVAL);
  ROPE(a->cache_row_stride = I64MIN, Q4_EINVAL);
  ROPE(a->cache_row_stride = 64 * 2 * 64 - 1, Q4_EINVAL);  // rings would overlap
  ROPE(a->cache_row_stride = I64MAX, Q4_EINVAL);

  q4_rope_kv* a = new q4_rope_kv(rope_base());
  RC(rope_kv_store, rope_kv_store(Z, 1024, 1, nullptr, nullptr), Q4_EINVAL);
  RC(rope_kv_store, rope_kv_store(Z, 1024, 0, a, nullptr), Q4_EINVAL);
  RC(rope_kv_store, rope_kv_store(Z, 1024, 65536, a, nullptr), Q4_EINVAL);
  RC(rope_kv_store, rope_kv_store(Z, 1024, IMIN, a, nullptr), Q4_EINVAL);
  RC(rope_kv_store, rope_kv_store(nullptr, 1024, 1, a, nullptr), Q4_EALIGN);
  RC(rope_kv_store, rope_kv_store(off(Z, 2), 1024, 1, a, nullptr), Q4_EALIGN);
  RC(rope_kv_store, rope_kv_store(Z, 511, 1, a, nullptr), Q4_EINVAL);  // (4 + 2*2) heads of 64
  RC(rope_kv_store, rope_kv_store(Z, I64MIN, 1, a, nullptr), Q4_EINVAL);
  RC(rope_kv_store, rope_kv_store(Z, I64MAX, 1, a, nullptr), Q4_EINVAL);
  RC(qmv_qkv_rope, qmv_qkv_rope(5, P, 256, X, 256, 1, a, nullptr), Q4_EINVAL);
  RC(qmv_qkv_rope, qmv_qkv_rope(4, P, 256, X, 256, 1, nullptr, nullptr), Q4_EINVAL);
  RC(qmv_qkv_rope, qmv_qkv_rope(4, P, 100, X, 256, 1, a, nullptr), Q4_EINVAL);
  RC(qmv_qkv_rope, qmv_qkv_rope(4, P, 256, X, 256, 0, a, nullptr), Q4_EINVAL);
  RC(qmv_qkv_rope, qmv_qkv_rope(4, P, 256, X, 256, 17, a, nullptr), Q4_EINVAL);
  RC(qmv_qkv_rope, qmv_qkv_rope(4, nullptr, 256, X, 256, 1, a, nullptr), Q4_EALIGN);
  RC(qmv_qkv_rope, qmv_qkv_rope(6, P, 256, off(X, 2), 256, 1, a, nullptr), Q4_EALIGN);
  RC(qmv_qkv_rope, qmv_qkv_rope(8, P, 256, X, 128, 1, a, nullptr), Q4_EINVAL);
  RC(qmv_qkv_rope, qmv_qkv_rope(4, P, 256, X, I64MAX, 1, a, nullptr), Q4_EINVAL);
  RC(qmv_qkv_rope, qmv_qkv_rope(4, P, 4096 + 64, X, 4096 + 64, 1, a, nullptr), Q4_EUNSUPPORTED);
  RC(qmv_qkv_rope, qmv_qkv_rope(4, P, 256, X, int64_t(1) << 30, 1, a, nullptr), Q4_EUNSUPPORTED);
  delete a;
}

void cost_calls() {
  float* us = new float[5];
  RC(qmv_window_costs, qmv_window_costs(5, P, 128, 256, X, Q4_BF16, 256, Y, 128, 10, us, nullptr), Q4_EINVAL);
  RC(qmv_window_costs, qmv_window_costs(4, P, 128, 256, X, Q4_BF16, 256, Y, 128, 10, nullptr, nullptr), Q4_EINVAL);
  RC(qmv_window_costs, qmv_window_costs(4, P, 128, 256, X, Q4_BF16, 256, Y, 128, 0, us, nullptr), Q4_EINVAL);
  RC(qmv_window_costs, qmv_window_costs(4, P, 128, 256, X, Q4_BF16, 256, Y, 128, 10001, us, nullptr), Q4_EINVAL);
  RC(qmv_window_costs, qmv_window_costs(4, P, 128, 256, X, Q4_BF16, 256, Y, 128, IMIN, us, nullptr), Q4_EINVAL);
  RC(qmv_window_costs, qmv_window_costs(4, P, 100, 256, X, Q4_BF16, 256, Y, 128, 10, us, nullptr), Q4_EINVAL);
  RC(qmv_window_costs, qmv_window_costs(6, P, 128, 256, X, Q4_BF16, 256, off(Y, 2), 128, 10, us, nullptr), Q4_EALIGN);
  RC(qmv_window_costs, qmv_window_costs(8, P, 128, 256, X, Q4_BF16, I64MAX, Y, 128, 10, us, nullptr), Q4_EINVAL);
  delete[] us;
}

}  // namespace

int main() {
  sizes();
  cost_table();
  pack_calls();
  decode_calls();
  fused_decode_calls();
  window_calls();
  ffn_calls();
  rope_calls();
  cost_calls();
  printf("%d cases, %d failed\n", g_cases, g_bad);
  return g_bad == 0 ? 0 : 1;
}
