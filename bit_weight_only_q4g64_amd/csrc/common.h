// Shared device helpers for the q4g64 kernels (gfx950 / CDNA4).
//
// Numerics. Every kernel forms only exact products: a 4-bit code q (0..15) is
// turned into an exact bf16 integer, multiplied by a bf16 activation on the
// matrix cores (8 x 4 significant bits fit in float32), and each 64-wide group
// is reduced on the matrix cores into a float32 partial P_g = sum q*x together
// with the activation sum S_g = sum x. The group's scale and bias enter once
// per group in float32: acc <- fma(s_g, P_g, fma(b_g, S_g, acc)). This is the
// affine MLX dequantization w = s*q + b applied after the in-group sum
// (TensorFold PR #1696, later revision, "What it adds", prompt GEMM item: a
// chain per 64-wide k block, blocks added in order).
//
// Determinism. The result of v_mfma_f32_16x16x32_bf16 in one output slot
// depends only on that slot's A row, B column and C input, so a row's bits do
// not depend on which slot it occupies or on the other rows sharing the
// instruction. The order of operations per output is a function of K only.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace q4 {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kGroup = 64;        // k per quantization group
constexpr int kTileN = 16;        // output columns per column tile
constexpr int kPairCodeBytes = 1024;  // codes of one column tile x 128 k (two groups)
constexpr int kPairSbBytes = 128;     // scale+bias of one column tile x two groups

// Device layout sizes (see include/q4g64.h for the full description). Codes
// of b bits take 256 * b bytes per column tile and group pair; the scale/bias
// block is the same for every width.
// Code formats: 4, 6 and 8 are MLX affine codes of that width; kFmtFp8 is
// block FP8 (OCP E4M3 bytes in the 8-bit layout, a float32 block scale in
// place of each group's scale/bias word, no bias term).
constexpr int kFmtFp8 = 9;
__host__ __device__ constexpr int code_bits(int fmt) { return fmt == kFmtFp8 ? 8 : fmt; }
__host__ __device__ constexpr int pair_code_bytes(int fmt) { return 256 * code_bits(fmt); }
__host__ __device__ inline int64_t n_pairs(int64_t K) { return (K / kGroup + 1) / 2; }
__host__ __device__ inline int64_t codes_bytes(int64_t N, int64_t K, int bits = 4) {
  return (N / kTileN) * n_pairs(K) * pair_code_bytes(bits);
}
__host__ __device__ inline int64_t packed_bytes(int64_t N, int64_t K, int bits = 4) {
  return (N / kTileN) * n_pairs(K) * (pair_code_bytes(bits) + kPairSbBytes);
}

// Position of code e (k offset e within an 8-code word) in a device word.
// Codes 0..3 sit at even nibbles, 4..7 at odd nibbles, so masking the word
// with 0x0F0F0F0F yields codes 0..3 one per byte and (w >> 4) yields 4..7.
__host__ __device__ constexpr int dev_nibble(int e) { return e < 4 ? 2 * e : 2 * (e - 4) + 1; }

// 8 codes of a device word -> 8 exact bf16 integers in k order.
// A byte holding a code q (0..15) read as an OCP e4m3 value is q * 2^-9
// (exponent field 0 or 1), so the scaled conversion by 2^9 gives q exactly.
__device__ __forceinline__ bf16x8 codes_to_bf16(uint32_t w) {
  const uint32_t lo = w & 0x0F0F0F0Fu;
  const uint32_t hi = (w >> 4) & 0x0F0F0F0Fu;
  const bf16x2 c01 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 512.0f, false);
  const bf16x2 c23 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 512.0f, true);
  const bf16x2 c45 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 512.0f, false);
  const bf16x2 c67 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 512.0f, true);
  const auto c0123 = __builtin_shufflevector(c01, c23, 0, 1, 2, 3);
  const auto c4567 = __builtin_shufflevector(c45, c67, 0, 1, 2, 3);
  return __builtin_shufflevector(c0123, c4567, 0, 1, 2, 3, 4, 5, 6, 7);
}

// 8 codes given as bytes (codes 0..3 in w0, 4..7 in w1, byte e = code e) ->
// 8 exact bf16 integers in k order. A byte converts exactly to float32 and
// an integer below 256 has at most 8 significant bits, so its float32 bits
// end in 16 zeros and the top half is the exact bf16.
__device__ __forceinline__ bf16x8 bytes_to_bf16(uint32_t w0, uint32_t w1) {
  auto pair = [](uint32_t w, int sh) -> uint32_t {
    const float f0 = (float)((w >> sh) & 0xFFu), f1 = (float)((w >> (sh + 8)) & 0xFFu);
    return __builtin_amdgcn_perm(__float_as_uint(f1), __float_as_uint(f0), 0x07060302u);
  };
  const u32x4 v = {pair(w0, 0), pair(w0, 16), pair(w1, 0), pair(w1, 16)};
  return __builtin_bit_cast(bf16x8, v);
}

// 8 six-bit codes: the low nibbles in a 4-bit device word (nib) and the high
// bit pairs in byte lanes of H (half 0 of a group: bits 0-1 codes 0..3, bits
// 2-3 codes 4..7; half 1: bits 4-5 and 6-7) -> codes as bytes -> exact bf16.
template <int HALF>
__device__ __forceinline__ bf16x8 six_to_bf16(uint32_t nib, uint32_t H) {
  uint32_t lo = nib & 0x0F0F0F0Fu, hi = (nib >> 4) & 0x0F0F0F0Fu;
  if constexpr (HALF == 0) {
    lo |= (H & 0x03030303u) << 4;
    hi |= (H & 0x0C0C0C0Cu) << 2;
  } else {
    lo |= H & 0x30303030u;
    hi |= (H >> 2) & 0x30303030u;
  }
  return bytes_to_bf16(lo, hi);
}

// One lane's codes of one group pair (halves h = 0..3: group h >> 1, half
// h & 1). 4-bit: a[h]. 6-bit: low nibbles a[h], high pairs b[h >> 1].
// 8-bit: a = group 0 (half hh in a[2hh], a[2hh + 1]), b = group 1.
template <int BITS>
struct CodeWords;
template <>
struct CodeWords<4> {
  u32x4 a;
};
template <>
struct CodeWords<6> {
  u32x4 a;
  u32x2 b;
};
template <>
struct CodeWords<8> {
  u32x4 a;
  u32x4 b;
};
template <>
struct CodeWords<kFmtFp8> {
  u32x4 a;
  u32x4 b;
};

// 8 OCP E4M3 bytes (codes 0..3 in w0, 4..7 in w1) -> 8 bf16 in k order.
// Every finite E4M3 value (4 significant bits, exponents 2^-9 .. 2^8) is a
// bf16 value, so the conversion with scale 1 is exact.
__device__ __forceinline__ bf16x8 fp8_to_bf16(uint32_t w0, uint32_t w1) {
  const bf16x2 c01 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, false);
  const bf16x2 c23 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, true);
  const bf16x2 c45 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, false);
  const bf16x2 c67 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, true);
  const auto c0123 = __builtin_shufflevector(c01, c23, 0, 1, 2, 3);
  const auto c4567 = __builtin_shufflevector(c45, c67, 0, 1, 2, 3);
  return __builtin_shufflevector(c0123, c4567, 0, 1, 2, 3, 4, 5, 6, 7);
}

// The bf16 B-operand fragment of group gh (0/1 within the pair), half hh.
template <int BITS, int GH, int HH>
__device__ __forceinline__ bf16x8 code_frag(const CodeWords<BITS>& c) {
  if constexpr (BITS == 4) {
    return codes_to_bf16(c.a[2 * GH + HH]);
  } else if constexpr (BITS == 6) {
    return six_to_bf16<HH>(c.a[2 * GH + HH], c.b[GH]);
  } else if constexpr (BITS == kFmtFp8) {
    if constexpr (GH == 0) return fp8_to_bf16(c.a[2 * HH], c.a[2 * HH + 1]);
    else return fp8_to_bf16(c.b[2 * HH], c.b[2 * HH + 1]);
  } else {
    if constexpr (GH == 0) return bytes_to_bf16(c.a[2 * HH], c.a[2 * HH + 1]);
    else return bytes_to_bf16(c.b[2 * HH], c.b[2 * HH + 1]);
  }
}

__device__ __forceinline__ bf16x8 ones_bf16x8() {
  const u32x4 one = {0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};
  return __builtin_bit_cast(bf16x8, one);
}

__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// bf16 bit pattern in the low / high half of a word -> float32 (exact).
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// float32 -> bf16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  const uint32_t u = __float_as_uint(f);
  return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

// float32 x = h + m + l exactly, each a bf16 (truncation keeps the top 8
// significant bits; each remainder is exact in float32).
__device__ __forceinline__ void split3(float x, uint32_t& h, uint32_t& m, uint32_t& l) {
  const uint32_t hu = __float_as_uint(x) & 0xFFFF0000u;
  const float r1 = x - __uint_as_float(hu);
  const uint32_t mu = __float_as_uint(r1) & 0xFFFF0000u;
  const float r2 = r1 - __uint_as_float(mu);
  h = hu >> 16;
  m = mu >> 16;
  l = __float_as_uint(r2) >> 16;
}

// Raw buffer access: a scalar resource (base, size in bytes) and a 32-bit
// per-lane byte offset plus a scalar byte offset. Reads past `bytes` return 0.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr int kRsrcWord3 = 0x00020000;  // raw buffer, gfx9 family
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, kRsrcWord3);
}
// A per-lane offset past every buffer this library builds (all are < 2 GiB):
// a load there returns zeros without touching memory.
constexpr uint32_t kOffBuffer = 0x80000000u;
__device__ __forceinline__ u32x4 buf_load16(rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
}
// The same with the non-temporal (streaming) cache policy, for data a launch
// reads exactly once (the decode kernels' weights): measured 6% off the
// fused w1/w3 decode kernel and 3% off w2, against the default policy.
constexpr int kCachePolicyNT = 2;
__device__ __forceinline__ u32x4 buf_load16_nt(rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, kCachePolicyNT));
}
__device__ __forceinline__ u32x2 buf_load8_nt(rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, kCachePolicyNT));
}

// SwiGLU gate in float32: silu(a) = a / (1 + exp(-a)), within 7 * 2^-24
// relative of the exact value wherever |silu(a)| > 2^-100:
//   exp(-a) = 2^(t + t_lo) with t + t_lo = -a * log2(e) carried in two
//   floats (the product's rounding error recovered by an fma, plus the
//   constant's tail), 2^t on the hardware exp2 (1 ulp), and the tail applied
//   as e * (1 + t_lo * ln 2) in one fma (|t_lo| <= 2^-17, so the dropped
//   second-order term is below 2^-35): 3 units;
//   1 + e: 1 unit; the hardware reciprocal (1 ulp): 2 units; a * r: 1 unit.
// The exponent argument is clamped to [-80, 88] so nothing overflows: above
// 88, exp(-a) < 2^-126 and the result is a; below -80 the result is -0,
// within |a| exp(a) <= 80 exp(-80) < 2^-100 of the exact value.
__device__ __forceinline__ float silu_f32(float a) {
  constexpr float kLog2e = 0x1.715476p+0f;      // log2(e) rounded to float
  constexpr float kLog2eTail = 0x1.4ae0c0p-26f; // log2(e) - kLog2e
  constexpr float kLn2 = 0x1.62e430p-1f;        // ln(2) rounded to float
  const float ac = __builtin_amdgcn_fmed3f(a, -80.0f, 88.0f);
  const float t = -ac * kLog2e;
  const float t_lo = __builtin_fmaf(-ac, kLog2e, -t) + (-ac) * kLog2eTail;
  const float e = __builtin_amdgcn_exp2f(t);
  const float e2 = __builtin_fmaf(e, t_lo * kLn2, e);
  const float r = a * __builtin_amdgcn_rcpf(1.0f + e2);
  return a < -80.0f ? -0.0f : r;
}

}  // namespace q4
