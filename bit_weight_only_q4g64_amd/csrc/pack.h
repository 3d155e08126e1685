// pack / unpack between the canonical MLX q4g64 tensors and the device layout.
// Integer permutations only: every output bit is one input bit (or a zero pad).
#pragma once

#include "common.h"

namespace q4 {

__device__ __forceinline__ uint32_t canon_to_dev_word(uint32_t cw) {
  uint32_t d = 0;
#pragma unroll
  for (int e = 0; e < 8; ++e) d |= ((cw >> (4 * e)) & 0xFu) << (4 * dev_nibble(e));
  return d;
}

__device__ __forceinline__ uint32_t dev_to_canon_word(uint32_t dw) {
  uint32_t c = 0;
#pragma unroll
  for (int e = 0; e < 8; ++e) c |= ((dw >> (4 * dev_nibble(e))) & 0xFu) << (4 * e);
  return c;
}

// One thread per 32-bit device code word (grid-stride).
__global__ void pack_codes_kernel(const uint32_t* __restrict__ wq, int64_t N, int64_t K, uint32_t* __restrict__ out) {
  const int64_t P = n_pairs(K);
  const int64_t total = (N / kTileN) * P * (kPairCodeBytes / 4);
  const int64_t kw = K / 8;
  for (int64_t w = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; w < total; w += (int64_t)gridDim.x * blockDim.x) {
    const int64_t blk = w >> 8;
    const int j = (int)(w & 255);
    const int lane = j >> 2, h = j & 3;
    const int64_t t = blk / P, p = blk - t * P;
    const int64_t n = t * kTileN + (lane & 15);
    const int64_t kb = p * 128 + h * 32 + (lane >> 4) * 8;
    out[w] = kb < K ? canon_to_dev_word(wq[n * kw + kb / 8]) : 0u;
  }
}

// One thread per (column tile, pair, column): 8 bytes [s_2p, b_2p, s_2p+1, b_2p+1].
__global__ void pack_sb_kernel(const uint16_t* __restrict__ sc, const uint16_t* __restrict__ bi, int64_t N, int64_t K,
                               u32x2* __restrict__ out) {
  const int64_t P = n_pairs(K), G = K / kGroup;
  const int64_t total = (N / kTileN) * P * kTileN;
  for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < total; e += (int64_t)gridDim.x * blockDim.x) {
    const int c = (int)(e & 15);
    const int64_t blk = e >> 4;
    const int64_t t = blk / P, p = blk - t * P;
    const int64_t n = t * kTileN + c;
    const int64_t g0 = 2 * p, g1 = 2 * p + 1;
    u32x2 v;
    v.x = (uint32_t)sc[n * G + g0] | ((uint32_t)bi[n * G + g0] << 16);
    v.y = g1 < G ? ((uint32_t)sc[n * G + g1] | ((uint32_t)bi[n * G + g1] << 16)) : 0u;
    out[e] = v;
  }
}

// Inverse of pack: one thread per canonical word (n, k/8).
__global__ void unpack_codes_kernel(const uint32_t* __restrict__ dev, int64_t N, int64_t K, uint32_t* __restrict__ wq) {
  const int64_t P = n_pairs(K);
  const int64_t kw = K / 8;
  const int64_t total = N * kw;
  for (int64_t w = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; w < total; w += (int64_t)gridDim.x * blockDim.x) {
    const int64_t n = w / kw, kb = (w - n * kw) * 8;
    const int64_t t = n / kTileN, c = n - t * kTileN;
    const int64_t p = kb / 128;
    const int h = (int)((kb % 128) / 32), kc = (int)((kb % 32) / 8);
    const int lane = (int)c + 16 * kc;
    wq[w] = dev_to_canon_word(dev[(t * P + p) * 256 + lane * 4 + h]);
  }
}

__global__ void unpack_sb_kernel(const u32x2* __restrict__ sb, int64_t N, int64_t K, uint16_t* __restrict__ sc,
                                 uint16_t* __restrict__ bi) {
  const int64_t P = n_pairs(K), G = K / kGroup;
  const int64_t total = N * G;
  for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < total; e += (int64_t)gridDim.x * blockDim.x) {
    const int64_t n = e / G, g = e - n * G;
    const int64_t t = n / kTileN, c = n - t * kTileN;
    const u32x2 v = sb[(t * P + g / 2) * kTileN + c];
    const uint32_t word = (g & 1) ? v.y : v.x;
    sc[e] = (uint16_t)(word & 0xFFFFu);
    bi[e] = (uint16_t)(word >> 16);
  }
}

// ---- 6- and 8-bit codes -------------------------------------------------
// Canonical rows are little-endian bit streams: code k at bits bits*k .. of
// the row's words (8-bit: the bytes in order; 6-bit: straddling words).
__device__ __forceinline__ uint32_t canon_code(const uint32_t* __restrict__ row, int64_t k, int bits) {
  const int64_t pos = k * bits;
  const int64_t w = pos >> 5;
  const int sh = (int)(pos & 31);
  uint64_t v = row[w];
  if (sh + bits > 32) v |= (uint64_t)row[w + 1] << 32;
  return (uint32_t)(v >> sh) & ((1u << bits) - 1u);
}

// Device layout of one column tile x group pair (64 * BITS words):
//  8-bit: sub-block j (groups 2p + j) of 256 words; word lane*4 + hh*2 + ws
//         holds codes 4*ws .. 4*ws + 3 of half hh of that group, one per
//         byte in k order;
//  6-bit: 256 words of low nibbles laid out exactly as the 4-bit codes, then
//         128 words of high bit pairs; word lane*2 + j covers halves 2j and
//         2j + 1, byte b holding (from bit 0) the high pairs of codes b and
//         4 + b of the even half, then of the odd half.
// Column n = 16 t + (lane & 15); half h = 0..3 spans k = 128 p + 32 h +
// 8 (lane >> 4) .. + 7. Codes past K are zero.
template <int BITS>
__global__ void pack_codes_wide_kernel(const uint32_t* __restrict__ wq, int64_t N, int64_t K, uint32_t* __restrict__ out) {
  constexpr int kWords = 64 * BITS;
  const int64_t P = n_pairs(K);
  const int64_t total = (N / kTileN) * P * kWords;
  const int64_t rw = K * BITS / 32;
  for (int64_t w = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; w < total; w += (int64_t)gridDim.x * blockDim.x) {
    const int64_t blk = w / kWords;
    const int r = (int)(w - blk * kWords);
    const int64_t t = blk / P, p = blk - t * P;
    uint32_t d = 0;
    if constexpr (BITS == 8) {
      const int j = r >> 8, q = r & 255, lane = q >> 2, hh = (q >> 1) & 1, ws = q & 1;
      const uint32_t* row = wq + (t * kTileN + (lane & 15)) * rw;
      const int64_t k0 = p * 128 + j * 64 + hh * 32 + (lane >> 4) * 8 + ws * 4;
      if (k0 < K)
        for (int e = 0; e < 4; ++e) d |= canon_code(row, k0 + e, 8) << (8 * e);
    } else {
      static_assert(BITS == 6, "wide codes are 6 or 8 bits");
      if (r < 256) {
        const int lane = r >> 2, h = r & 3;
        const uint32_t* row = wq + (t * kTileN + (lane & 15)) * rw;
        const int64_t k0 = p * 128 + h * 32 + (lane >> 4) * 8;
        if (k0 < K)
          for (int e = 0; e < 8; ++e) d |= (canon_code(row, k0 + e, 6) & 15u) << (4 * dev_nibble(e));
      } else {
        const int q = r - 256, lane = q >> 1, j = q & 1;
        const uint32_t* row = wq + (t * kTileN + (lane & 15)) * rw;
        for (int hh = 0; hh < 2; ++hh) {
          const int64_t k0 = p * 128 + (2 * j + hh) * 32 + (lane >> 4) * 8;
          if (k0 >= K) continue;
          for (int e = 0; e < 8; ++e) {
            const int field = (e >> 2) + 2 * hh;
            d |= (canon_code(row, k0 + e, 6) >> 4) << (8 * (e & 3) + 2 * field);
          }
        }
      }
    }
    out[w] = d;
  }
}

// Code k of column n read back from the wide device layout.
template <int BITS>
__device__ __forceinline__ uint32_t dev_wide_code(const uint32_t* __restrict__ dev, int64_t P, int64_t n, int64_t k) {
  const int64_t t = n / kTileN, p = k / 128;
  const int c = (int)(n - t * kTileN), h = (int)((k % 128) / 32), kc = (int)((k % 32) / 8), e = (int)(k % 8);
  const int lane = c + 16 * kc;
  const uint32_t* base = dev + (t * P + p) * (64 * BITS);
  if constexpr (BITS == 8) {
    const uint32_t word = base[(h >> 1) * 256 + lane * 4 + (h & 1) * 2 + (e >> 2)];
    return (word >> (8 * (e & 3))) & 255u;
  } else {
    const uint32_t lo = (base[lane * 4 + h] >> (4 * dev_nibble(e))) & 15u;
    const uint32_t hw = base[256 + lane * 2 + (h >> 1)];
    const int field = (e >> 2) + 2 * (h & 1);
    return lo | (((hw >> (8 * (e & 3) + 2 * field)) & 3u) << 4);
  }
}

// Inverse: one thread per canonical word (n, cw), rebuilt from the codes that
// overlap its 32 bits.
template <int BITS>
__global__ void unpack_codes_wide_kernel(const uint32_t* __restrict__ dev, int64_t N, int64_t K, uint32_t* __restrict__ wq) {
  const int64_t P = n_pairs(K);
  const int64_t rw = K * BITS / 32;
  const int64_t total = N * rw;
  for (int64_t w = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; w < total; w += (int64_t)gridDim.x * blockDim.x) {
    const int64_t n = w / rw, cw = w - n * rw;
    const int64_t b0 = cw * 32;
    uint64_t v = 0;
    for (int64_t k = b0 / BITS; k * BITS < b0 + 32; ++k) {
      const int64_t pos = k * BITS - b0;
      const uint64_t code = dev_wide_code<BITS>(dev, P, n, k);
      v |= pos >= 0 ? code << pos : code >> (-pos);
    }
    wq[w] = (uint32_t)v;
  }
}

// ---- block FP8 -----------------------------------------------------------
// Codes are E4M3 bytes [N][K], packed by pack_codes_wide_kernel<8> (the
// canonical 8-bit stream is the bytes in k order). The float32 scale of
// block (n / 128, p) (128 rows x the 128 k of group pair p) goes into both
// group words of pair p for column n (zero past G).
__global__ void pack_scale_fp8_kernel(const float* __restrict__ sc, int64_t N, int64_t K, u32x2* __restrict__ out) {
  const int64_t P = n_pairs(K), G = K / kGroup;
  const int64_t total = (N / kTileN) * P * kTileN;
  for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < total; e += (int64_t)gridDim.x * blockDim.x) {
    const int c = (int)(e & 15);
    const int64_t blk = e >> 4;
    const int64_t t = blk / P, p = blk - t * P;
    const int64_t n = t * kTileN + c;
    const uint32_t v = __float_as_uint(sc[(n / 128) * P + p]);
    out[e] = u32x2{v, 2 * p + 1 < G ? v : 0u};
  }
}

// Inverse: block (i, p) read back from column 128 i of pair p.
__global__ void unpack_scale_fp8_kernel(const u32x2* __restrict__ sb, int64_t N, int64_t K, float* __restrict__ sc) {
  const int64_t P = n_pairs(K), NB = (N + 127) / 128;
  const int64_t total = NB * P;
  for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < total; e += (int64_t)gridDim.x * blockDim.x) {
    const int64_t i = e / P, p = e - i * P;
    const int64_t t = (i * 128) / kTileN;
    sc[e] = __uint_as_float(sb[(t * P + p) * kTileN].x);
  }
}

}  // namespace q4
