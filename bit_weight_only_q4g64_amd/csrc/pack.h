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

}  // namespace q4
