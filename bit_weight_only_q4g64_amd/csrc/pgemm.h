// Prefill window GEMM (pgemm) on the matrix cores.
//
// A workgroup of 8 waves owns 256 window rows and 16 weight column tiles of
// 16 columns (256 output columns; SwiGLU: 128 output columns, 8 tiles of w1
// and the same 8 tiles of w3). Wave w covers rows 128 * (w / 4) .. + 127 and
// four of the tiles (w % 4 picks which), so each wave holds 8 x 4 output
// tiles of 16 x 16 in registers.
//
// Operands move from HBM to LDS by buffer-to-LDS DMA, which costs no
// registers while in flight: the 256 x 64 activation tile of a group in
// three stages (two groups of lookahead), the codes and scale/bias words of
// a pair of groups in two stages. One barrier per group. Each wave turns the
// codes of its four tiles into exact bf16 integers once per group and reuses
// them for its eight row tiles. The activation sum S_g of a row is formed
// once per workgroup (each of the four waves sharing a row half forms it for
// two of the eight row tiles) and shared through LDS.
//
// Per output (r, n) the order is, with chunks of 8 consecutive groups:
//
//   acc = 0
//   for each chunk (ascending):
//     for each group g of the chunk (ascending):
//       P_g = mfma(x[g, 32..63], q, mfma(x[g, 0..31], q, 0))     exact products
//       acc = fma(s_g, P_g, acc)                                  one VALU op per output
//       S_g = sum of x[g, :] on the matrix cores (A = ones)
//     acc = mfma(A = exact bf16 pieces h, m, l of S_g for the chunk's groups,
//                B = b_g repeated over the pieces, C = acc)        the bias term
//   y = acc
//
// Nothing in it depends on M, on the row's offset in the window or on the
// other rows, so a row's bits are the same for every cut of the prompt
// (TensorFold PR #1696, later revision, "What it adds", prompt GEMM item: a
// chain per 64-wide k block, blocks added in order; "Checks": every row alone
// equals the row inside a window).
#pragma once

#include <type_traits>

#include "common.h"

namespace q4 {

constexpr int kPgemmWaves = 8;                  // 2 row halves x 4 column quarters
constexpr int kPgemmThreads = kPgemmWaves * 64;
constexpr int kPgemmRT = 8;                     // 16-row tiles per wave
constexpr int kPgemmNT = 4;                     // 16-column weight tiles per wave
constexpr int kPgemmRows = 256;                 // window rows per workgroup
constexpr int kPgemmSlots = 16;                 // 16-column weight tiles per workgroup
constexpr int kPgemmChunk = 8;                  // groups per bias chunk
constexpr int kXStages = 3;
constexpr int kXRowBytes = kGroup * 2;          // one staged activation row of a group
constexpr int kXStageBytes = kPgemmRows * kXRowBytes;       // 32 KiB
constexpr int kCStageBytes = kPgemmSlots * kPairCodeBytes;  // 16 KiB
constexpr int kSbStageBytes = kPgemmSlots * kPairSbBytes;   // 2 KiB
constexpr int kSumFloats = 2 * kPgemmRows * kPgemmChunk;    // activation sums, 2 chunks
static_assert(kPgemmRows == 2 * kPgemmRT * 16, "two row halves of kPgemmRT tiles");
static_assert(kPgemmSlots == 4 * kPgemmNT, "four column quarters");
static_assert(kPgemmRows * kXRowBytes == kPgemmWaves * 4 * 1024, "each wave stages 4 KiB of a group");

// Output columns covered by one workgroup.
__host__ __device__ constexpr int pgemm_cols(bool swiglu) { return swiglu ? 8 * kTileN : kPgemmSlots * kTileN; }

// LDS slot of 16-byte chunk c (0..7) of staged row r. Rows are 128 bytes;
// XOR-ing the chunk with the row's low 3 bits spreads the rows of a fragment
// read over the banks (measured: a quarter of the conflict cycles of the
// unswizzled layout, and of an XOR that also folds in row bit 3).
__device__ __forceinline__ int xs_slot(int r, int c) { return c ^ (r & 7); }
__device__ __forceinline__ int xs_off(int r, int c) { return r * kXRowBytes + (xs_slot(r, c) << 4); }

// Buffer-to-LDS DMA. Lane L's bytes land at LDS address lds + L * size;
// lds (m0) and the resource are wave-uniform. Written as inline assembly so
// that the compiler neither reorders nor waits on them: every wait on these
// loads is an explicit s_waitcnt vmcnt before a barrier.
typedef int i32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ i32x4 make_srsrc(const void* base, uint32_t bytes) {
  const uint64_t b = (uint64_t)base;
  return i32x4{(int)(uint32_t)b, (int)((uint32_t)(b >> 32) & 0xFFFFu), (int)bytes, kRsrcWord3};
}
__device__ __forceinline__ void dma_b128(i32x4 r, uint32_t voff, uint32_t soff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %3\n\tbuffer_load_dwordx4 %0, %1, %2 offen lds" ::"v"(voff), "s"(r), "s"(soff), "s"(lds) : "m0");
}
__device__ __forceinline__ void dma_b32(i32x4 r, uint32_t voff, uint32_t soff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %3\n\tbuffer_load_dword %0, %1, %2 offen lds" ::"v"(voff), "s"(r), "s"(soff), "s"(lds) : "m0");
}
template <typename T>
__device__ __forceinline__ uint32_t lds_addr(T* p) {
  return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) void*)p;
}
// Wait until at most n of this wave's DMA loads are in flight, wait for its
// LDS accesses, then meet the workgroup barrier.
template <int n>
__device__ __forceinline__ void dma_wait_barrier() {
  static_assert(n == 0 || n == 4 || n == 7, "wait depths used by the pipeline");
  if constexpr (n == 7) asm volatile("s_waitcnt vmcnt(7)\n\ts_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  else if constexpr (n == 4) asm volatile("s_waitcnt vmcnt(4)\n\ts_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  else asm volatile("s_waitcnt vmcnt(0)\n\ts_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Workgroup b -> (row block, column block). Workgroups are dealt to the 8
// XCDs round robin, so b is first renumbered so that those on one XCD are
// consecutive; consecutive numbers then walk 4 row blocks before the next
// column block, so the workgroups an XCD runs together share their
// activation rows and weight columns in its L2.
__host__ __device__ inline void pgemm_tile(int b, int nblk, int mblk, int& mb, int& nb) {
  const int T = nblk * mblk;
  const int q = T / 8, r = T % 8;
  const int xcd = b % 8, j = b / 8;
  const int t = xcd * q + (xcd < r ? xcd : r) + j;
  const int gsz = 4 * nblk;
  const int grp = t / gsz, first = grp * 4;
  const int h = mblk - first < 4 ? mblk - first : 4;
  const int in = t - grp * gsz;
  mb = first + in % h;
  nb = in / h;
}

template <bool SWIGLU, bool OUT_BF16>
__global__ __launch_bounds__(kPgemmThreads, 1) void pgemm_kernel(const uint8_t* __restrict__ pa, const uint8_t* __restrict__ pb,
                                                                  int N, int K, const uint16_t* __restrict__ x, int64_t ldx, int M,
                                                                  void* __restrict__ yv, int64_t ldy, int nblk, int mblk) {
  __shared__ __align__(16) uint8_t xs[kXStages * kXStageBytes];
  __shared__ __align__(16) uint8_t cs[2 * kCStageBytes];
  __shared__ __align__(16) uint8_t sbs[2 * kSbStageBytes];
  __shared__ __align__(16) float ssum[kSumFloats];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int cw = wave & 3, hh = wave >> 2;
  const int i = lane & 15, kc = lane >> 4;
  int mb, nb;
  pgemm_tile(blockIdx.x, nblk, mblk, mb, nb);
  const int m0 = mb * kPgemmRows;
  const int mt = M - m0 < kPgemmRows ? M - m0 : kPgemmRows;  // rows of this tile inside the window
  const int G = K / kGroup;
  const int P = (G + 1) / 2;
  const int ntiles = N / kTileN;
  const int64_t cb = codes_bytes(N, K);
  const bf16x8 ones = ones_bf16x8();

  // slot (0..15) -> weight tile (unclamped)
  auto slot_tile = [&](int slot) { return SWIGLU ? nb * 8 + (slot & 7) : nb * kPgemmSlots + slot; };
  auto clamp_tile = [&](int t) { return t < ntiles ? t : ntiles - 1; };

  // ---- DMA set-up --------------------------------------------------------
  // activations: wave w stages rows 32w + 8u + lane / 8 (u < 4) into LDS slot
  // lane % 8 of each row; rows past the window re-read its last row (their
  // results are never stored)
  const i32x4 xr = make_srsrc(x + (int64_t)m0 * ldx, (uint32_t)((int64_t)mt * ldx * 2));
  uint32_t xvo[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int r = 32 * wave + 8 * u + (lane >> 3);
    const int rc = r < mt ? r : mt - 1;
    xvo[u] = (uint32_t)(rc * ldx * 2) + (uint32_t)(xs_slot(r, lane & 7) << 4);
  }
  const uint32_t xs_lds = lds_addr(xs) + wave * 4096;
  // codes and scale/bias words: wave w stages slots 2w and 2w + 1 (one matrix)
  const uint8_t* mat = (SWIGLU && wave >= 4) ? pb : pa;
  const int t0 = clamp_tile(slot_tile(2 * wave)), t1 = clamp_tile(slot_tile(2 * wave + 1));
  const i32x4 cr0 = make_srsrc(mat + (int64_t)t0 * P * kPairCodeBytes, (uint32_t)P * kPairCodeBytes);
  const i32x4 cr1 = make_srsrc(mat + (int64_t)t1 * P * kPairCodeBytes, (uint32_t)P * kPairCodeBytes);
  const i32x4 sr = make_srsrc(mat + cb + (int64_t)t0 * P * kPairSbBytes, (uint32_t)((t1 - t0 + 1) * P * kPairSbBytes));
  const uint32_t cvo = (uint32_t)lane * 16u;
  const uint32_t svo = (uint32_t)((lane >> 5) * (t1 - t0) * P * kPairSbBytes) + (uint32_t)(lane & 31) * 4u;
  const uint32_t cs_lds = lds_addr(cs) + 2 * wave * kPairCodeBytes;
  const uint32_t sb_lds = lds_addr(sbs) + 2 * wave * kPairSbBytes;

  auto issue_x = [&](int g) {
    const uint32_t dst = xs_lds + (uint32_t)(g % kXStages) * kXStageBytes;
#pragma unroll
    for (int u = 0; u < 4; ++u) dma_b128(xr, xvo[u], (uint32_t)g * kXRowBytes, dst + u * 1024);
  };
  auto issue_c = [&](int p) {
    const uint32_t st = (uint32_t)(p & 1);
    dma_b128(cr0, cvo, (uint32_t)p * kPairCodeBytes, cs_lds + st * kCStageBytes);
    dma_b128(cr1, cvo, (uint32_t)p * kPairCodeBytes, cs_lds + st * kCStageBytes + kPairCodeBytes);
    dma_b32(sr, svo, (uint32_t)p * kPairSbBytes, sb_lds + st * kSbStageBytes);
  };

  // ---- consumer set-up ---------------------------------------------------
  int cslot[kPgemmNT];
#pragma unroll
  for (int s = 0; s < kPgemmNT; ++s) cslot[s] = SWIGLU ? (s < 2 ? 2 * cw + s : 8 + 2 * cw + (s - 2)) : kPgemmNT * cw + s;
  const int rbase = hh * (kPgemmRows / 2);
  // a wave computes only where its row half meets the window; every wave of
  // a live half forms its share of the activation sums
  const bool live = rbase < mt;

  f32x4 acc[kPgemmRT][kPgemmNT];
#pragma unroll
  for (int rt = 0; rt < kPgemmRT; ++rt)
#pragma unroll
    for (int s = 0; s < kPgemmNT; ++s) acc[rt][s] = f32x4{0.f, 0.f, 0.f, 0.f};
  // raw scale/bias words of groups 2*kc, 2*kc+1 of the current chunk
  uint32_t bsel[kPgemmNT][2];
#pragma unroll
  for (int s = 0; s < kPgemmNT; ++s) bsel[s][0] = bsel[s][1] = 0u;

  // the bias term of chunk c on the matrix cores, added into acc
  auto bias_chunk = [&](int c) {
    const float* sp = ssum + (c & 1) * kPgemmRows * kPgemmChunk;
    const bool v0 = kPgemmChunk * c + 2 * kc < G, v1 = kPgemmChunk * c + 2 * kc + 1 < G;
    bf16x8 bfr[kPgemmNT];
#pragma unroll
    for (int s = 0; s < kPgemmNT; ++s) {
      const uint32_t b0 = bsel[s][0] >> 16, b1 = bsel[s][1] >> 16;
      bfr[s] = __builtin_bit_cast(bf16x8, u32x4{b0 | (b0 << 16), b0, b1 | (b1 << 16), b1});
      bsel[s][0] = bsel[s][1] = 0u;
    }
#pragma unroll
    for (int rt = 0; rt < kPgemmRT; ++rt) {
      const int row = rbase + rt * 16 + i;
      const float2 S2 = *(const float2*)(sp + row * kPgemmChunk + 2 * kc);
      // groups past K hold no sum in this chunk; their slots must be zero
      const float s0 = v0 ? S2.x : 0.f, s1 = v1 ? S2.y : 0.f;
      uint32_t h0, mm0, l0, h1, mm1, l1;
      split3(s0, h0, mm0, l0);
      split3(s1, h1, mm1, l1);
      const bf16x8 afr = __builtin_bit_cast(bf16x8, u32x4{h0 | (mm0 << 16), l0, h1 | (mm1 << 16), l1});
#pragma unroll
      for (int s = 0; s < kPgemmNT; ++s) acc[rt][s] = mfma16(afr, bfr[s], acc[rt][s]);
    }
  };

  // one group; gh (compile time) is the group's half of its pair
  auto group = [&](int g, auto ghc) {
    constexpr int gh = decltype(ghc)::value;
    const int p = g >> 1, gg = g & (kPgemmChunk - 1);
    const uint8_t* xb = xs + (g % kXStages) * kXStageBytes;
    const uint8_t* cb0 = cs + (p & 1) * kCStageBytes;
    const uint8_t* sb0 = sbs + (p & 1) * kSbStageBytes;

    if constexpr (gh == 0) {
      if (gg == 0 && g > 0) bias_chunk(g / kPgemmChunk - 1);
    }

    bf16x8 q[kPgemmNT][2];
    float sc[kPgemmNT];
#pragma unroll
    for (int s = 0; s < kPgemmNT; ++s) {
      const uint32_t w = *(const uint32_t*)(sb0 + cslot[s] * kPairSbBytes + i * 8 + gh * 4);
      sc[s] = bf16_lo(w);
      if (kc == (gg >> 1)) bsel[s][gh] = w;
      const u32x2 cwd = *(const u32x2*)(cb0 + cslot[s] * kPairCodeBytes + lane * 16 + gh * 8);
      q[s][0] = codes_to_bf16(cwd[0]);
      q[s][1] = codes_to_bf16(cwd[1]);
    }

    // activation sums of this wave's share of the row tiles
    float* sw = ssum + ((g / kPgemmChunk) & 1) * kPgemmRows * kPgemmChunk + gg;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int row = rbase + (2 * cw + u) * 16 + i;
      const bf16x8 xa0 = __builtin_bit_cast(bf16x8, *(const u32x4*)(xb + xs_off(row, kc)));
      const bf16x8 xa1 = __builtin_bit_cast(bf16x8, *(const u32x4*)(xb + xs_off(row, kc + 4)));
      f32x4 S = mfma16(ones, xa0, f32x4{0.f, 0.f, 0.f, 0.f});
      S = mfma16(ones, xa1, S);
      if (kc == 0) sw[row * kPgemmChunk] = S[0];
    }

#pragma unroll
    for (int rt = 0; rt < kPgemmRT; ++rt) {
      const int row = rbase + rt * 16 + i;
      const bf16x8 xa0 = __builtin_bit_cast(bf16x8, *(const u32x4*)(xb + xs_off(row, kc)));
      const bf16x8 xa1 = __builtin_bit_cast(bf16x8, *(const u32x4*)(xb + xs_off(row, kc + 4)));
#pragma unroll
      for (int s = 0; s < kPgemmNT; ++s) {
        f32x4 Pm = mfma16(xa0, q[s][0], f32x4{0.f, 0.f, 0.f, 0.f});
        Pm = mfma16(xa1, q[s][1], Pm);
#pragma unroll
        for (int v = 0; v < 4; ++v) acc[rt][s][v] = __builtin_fmaf(sc[s], Pm[v], acc[rt][s][v]);
      }
    }
  };

  // ---- pipeline ------------------------------------------------------------
  // In flight at the top of group g is what was issued during group g - 1:
  // the activations of group g + 1 (4 loads) and, when g is odd, the weights
  // of the next pair (3 loads). Everything older has landed once the wave's
  // vmcnt is that low; the barrier then makes every wave's stage visible and
  // frees the stage the next DMA overwrites (read during group g - 1).
  issue_x(0);
  issue_c(0);
  if (G > 1) issue_x(1);
  for (int p = 0; p < P; ++p) {
    const int g = 2 * p;
    if (g + 1 < G) dma_wait_barrier<4>();
    else dma_wait_barrier<0>();
    if (g + 2 < G) issue_x(g + 2);
    if (p + 1 < P) issue_c(p + 1);
    if (live) group(g, std::integral_constant<int, 0>{});
    if (g + 1 < G) {
      // p + 1 < P implies g + 2 < G
      if (p + 1 < P) dma_wait_barrier<7>();
      else if (g + 2 < G) dma_wait_barrier<4>();
      else dma_wait_barrier<0>();
      if (g + 3 < G) issue_x(g + 3);
      if (live) group(g + 1, std::integral_constant<int, 1>{});
    }
  }
  dma_wait_barrier<0>();  // the last group's sums from every wave
  if (!live) return;
  bias_chunk((G - 1) / kPgemmChunk);

  // ---- epilogue: lane holds rows m0 + rbase + rt*16 + 4*kc + v of column i of each tile
#pragma unroll
  for (int rt = 0; rt < kPgemmRT; ++rt) {
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int row = rbase + rt * 16 + 4 * kc + v;
      if (row >= mt) continue;
      const int64_t yrow = (int64_t)(m0 + row) * ldy;
      if constexpr (SWIGLU) {
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          const int t = slot_tile(cslot[s]);
          if (t >= ntiles) continue;
          const float z = silu_f32(acc[rt][s][v]) * acc[rt][s + 2][v];
          const int64_t at = yrow + (int64_t)t * kTileN + i;
          if constexpr (OUT_BF16) ((uint16_t*)yv)[at] = f32_to_bf16_rne(z);
          else ((float*)yv)[at] = z;
        }
      } else {
#pragma unroll
        for (int s = 0; s < kPgemmNT; ++s) {
          const int t = slot_tile(cslot[s]);
          if (t >= ntiles) continue;
          const int64_t at = yrow + (int64_t)t * kTileN + i;
          if constexpr (OUT_BF16) ((uint16_t*)yv)[at] = f32_to_bf16_rne(acc[rt][s][v]);
          else ((float*)yv)[at] = acc[rt][s][v];
        }
      }
    }
  }
}

}  // namespace q4
