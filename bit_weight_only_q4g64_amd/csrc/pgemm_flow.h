// Prompt GEMM for short windows: producer waves and one folder wave per
// 32 x 32 output tile. Codes of 4, 6 or 8 bits (MLX affine) or block FP8.
//
// A window of up to a few hundred rows has few output tiles: a 128-row window
// of w2 (2048 x 8192) is 256 tiles of 32 x 32, each a chain over 128 groups
// of k. Run as one wave per tile, each group costs about 1000 cycles of
// exposed latency (operand loads, four dependent matrix steps, the fold) on
// a quarter of the SIMDs. But in the window order only the fold
// acc = fma(s_g, P_g, acc) is a chain: the products P_g of different groups
// are independent. So a workgroup here owns one tile (SwiGLU: the w1 tile and
// the same w3 tile) with NP producer waves and one folder wave:
//
//   - producer p takes group pairs p, p + NP, p + 2 NP, ...: the pair's 32
//     activation rows, code blocks and scale/bias blocks arrive in its LDS
//     stage by buffer-to-LDS DMA; it reads them into registers and at once
//     issues the DMA of its next pair into the same stage, so that the next
//     pair's loads run while this one is computed. It forms P_g on the
//     matrix cores exactly as the other window kernels do, and the row sums
//     S_g with the same matrix steps against ones, on operands moved between
//     lanes of the fragments it already holds (two lane swaps, no second LDS
//     read). It hands each group to the folder: P_g and the column scales
//     through a ring of R entries in LDS, and the exact bf16 pieces of S_g
//     and the biases b_g into its chunk's bias operands, at the lanes the bias
//     term's matrix steps read them from;
//   - the folder takes the entries in ascending g and applies the order step
//     for step: acc = fma(s_g, P_g, acc), and after the fold of the first
//     group of each chunk of 8 the previous chunk's bias term on the matrix
//     cores; then the epilogue. It reads a pair's entries one pair ahead, so
//     the reads run under the folds of the pair before.
//
// Ring protocol (LDS): entry g % R holds group g once ready[g % R] = g + 1
// (stored after the entry's writes have completed), and is free again once
// the folder stores done[g % R] = g + 1 (after the folds that used its values).
// Every wait is bounded (at most 2^22 polls), so no wave can hang.
//
// LDS is 74.5 KiB with NP = 3, R = 8 (plain) and 72.7 KiB with NP = 2, R = 4
// (SwiGLU) for 4-bit codes, 80.7 and 80.9 KiB for the wider ones, so two
// workgroups share a compute unit and a window of up to two rounds of tiles
// is resident at once; SwiGLU with NP = 3, R = 8 takes 120 to 130 KiB.
//
// Measured on MI355X and dropped: more producers (4 to 7, two per SIMD), two
// folders each folding half the accumulators, a ring of 16 and deeper
// staging were all within 5% or slower. LDS writes are what waits: with
// buffer-to-LDS DMA streaming, one wave's 128-bit LDS write took 140 to 520
// cycles to complete against 70 idle (reads stayed near 64), so the ring's
// hand-off writes, not the folds or the matrix work, pace a workgroup.
//
// Per output the arithmetic is pgemm_kernel's: the same four chained
// 32 x 32 x 16 matrix steps per group on the same exact bf16 codes and
// activation fragments, the same fold, the same activation sums (16 x 16 x 32
// against ones, two per 16 rows, on the same operand values) and the same
// bias term per chunk of 8 groups. A row's bits are the same whichever kernel
// computes them, and the window cut stays free (TensorFold PR #1696, later
// revision, "What it adds", prompt GEMM item: a chain per 64-wide k block;
// "Checks": every row alone equals the row inside a window).
#pragma once

#include "pgemm.h"

namespace q4 {

constexpr int kFlowRows = 32;  // window rows per workgroup

// Per-producer DMA stage: a pair's activations (2 groups x 32 rows x 128
// bytes), its code blocks (per weight slot 1 KiB for 4-bit codes; 2 KiB for
// the wider ones: 8-bit and FP8 the pair's block as it is, 6-bit its 1 KiB of
// nibble words and then its 512 bytes of high-pair words) and scale/bias blocks.
__host__ __device__ constexpr int flow_slots(bool swiglu) { return swiglu ? 4 : 2; }
__host__ __device__ constexpr int flow_slot_code_bytes(int bits) { return bits == 4 ? kPairCodeBytes : 2048; }
__host__ __device__ constexpr int flow_stage_bytes(bool swiglu, int bits = 4) {
  return 2 * kFlowRows * kXRowBytes + flow_slots(swiglu) * (flow_slot_code_bytes(bits) + kPairSbBytes);
}
// A buffer resource from workgroup-uniform values, pinned to scalar registers.
__device__ __forceinline__ i32x4 flow_rsrc(const void* base, uint32_t bytes) {
  const i32x4 r = make_srsrc(base, bytes);
  return i32x4{__builtin_amdgcn_readfirstlane(r[0]), __builtin_amdgcn_readfirstlane(r[1]), __builtin_amdgcn_readfirstlane(r[2]),
               __builtin_amdgcn_readfirstlane(r[3])};
}

template <bool SWIGLU, bool OUT_BF16, int NP, int R, int BITS = 4>
__global__ __launch_bounds__(64 * (NP + 1)) void pgemm_flow_kernel(const uint8_t* __restrict__ pa, const uint8_t* __restrict__ pb, int N,
                                                                   int K, const uint16_t* __restrict__ x, int64_t ldx, int M,
                                                                   void* __restrict__ yv, int64_t ldy, int nblk, int mblk) {
  constexpr int kTiles = SWIGLU ? 2 : 1;
  __shared__ __align__(16) f32x4 ringP[R][kTiles][4][64];  // P_g, element quad i of lane L at [i][L]
  __shared__ float ringC[R][kTiles][64];                   // the lane's column scale s_g
  // the bias term's matrix operands of chunk c (at c & 1), in the lanes of
  // its 32 x 32 x 16 steps m = 0, 1: A = the exact bf16 pieces of S_g of row j
  // for groups 4 m + 2 hl + e in lane j + 32 hl, B = b_g of column j likewise
  __shared__ __align__(16) u32x4 biasA[2][2][64];
  __shared__ __align__(16) u32x4 biasB[2][kTiles][2][64];
  __shared__ uint32_t ready[R], done[R];
  constexpr int kSlots = flow_slots(SWIGLU);
  constexpr int kXBytes = 2 * kFlowRows * kXRowBytes;
  constexpr int kStageBytes = flow_stage_bytes(SWIGLU, BITS);
  constexpr int kPcb = pair_code_bytes(BITS);           // a pair's code block in memory
  constexpr int kSlotCode = flow_slot_code_bytes(BITS);  // and in the stage
  constexpr bool kBias = BITS != kFmtFp8;                // block FP8 has no bias term
  static_assert(BITS == 4 || BITS == 6 || BITS == 8 || BITS == kFmtFp8, "4-, 6- or 8-bit codes or block FP8");
  // chunk c + 2 reuses chunk c's bias operands: a producer writes group g
  // only after the release of group g - R, and the release of group
  // 8 (c + 1) follows chunk c's bias term, so R may not exceed a chunk
  static_assert(R >= 2 && R <= kPgemmChunk && (R & (R - 1)) == 0, "ring of 2, 4 or 8 entries");
  __shared__ __align__(16) uint8_t smem_stages[NP * kStageBytes];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  int mb, nb;
  pgemm_tile(blockIdx.x, nblk, mblk, mb, nb);
  const int m0 = mb * kFlowRows;
  const int mt = M - m0 < kFlowRows ? M - m0 : kFlowRows;  // rows of this block inside the window
  const int G = K / kGroup;
  const int P = (G + 1) / 2;
  const int ntiles = N / kTileN;
  const int j = lane & 31, hl = lane >> 5, jj = j & 15;
  // this lane's weight tile in output tile t: tiles 2 nb and 2 nb + 1 (of w1,
  // and of w3 for t = 1 with SwiGLU), column jj
  const int wtile = 2 * nb + (j >> 4);

  if (threadIdx.x < R) ready[threadIdx.x] = done[threadIdx.x] = 0u;
  __syncthreads();

  // Ring flags. Only LDS is ordered (a C++ release would also wait for the
  // producer's loads in flight): a producer completes its entry writes
  // (lgkmcnt(0)) before it stores the flag; the folder stores a release
  // after the folds that consumed the entry's values. Waits are bounded.
  if (wave < NP) {
    // ---------------- producer --------------------------------------------
    // the workgroup's two weight tiles 2 nb, 2 nb + 1 (SwiGLU: of w1, then of
    // w3), clamped at N (columns past N are never stored)
    const int t0 = 2 * nb < ntiles ? 2 * nb : ntiles - 1;
    const int t1 = 2 * nb + 1 < ntiles ? 2 * nb + 1 : ntiles - 1;
    const int64_t cb = codes_bytes(N, K, BITS);
    const i32x4 xr = flow_rsrc(x + (int64_t)m0 * ldx, (uint32_t)((int64_t)mt * ldx * 2));
    const i32x4 cra = flow_rsrc(pa + (int64_t)t0 * P * kPcb, (uint32_t)((t1 - t0 + 1) * P * kPcb));
    const i32x4 sra = flow_rsrc(pa + cb + (int64_t)t0 * P * kPairSbBytes, (uint32_t)((t1 - t0 + 1) * P * kPairSbBytes));
    const uint8_t* pbm = SWIGLU ? pb : pa;
    const i32x4 crb = flow_rsrc(pbm + (int64_t)t0 * P * kPcb, (uint32_t)((t1 - t0 + 1) * P * kPcb));
    const i32x4 srb = flow_rsrc(pbm + cb + (int64_t)t0 * P * kPairSbBytes, (uint32_t)((t1 - t0 + 1) * P * kPairSbBytes));
    // activation DMA: load i (0..7) of a pair is group half i / 4, rows
    // 8 (i % 4) + lane / 8, 16-byte chunk lane % 8 at its swizzled slot; rows
    // past the window re-read its last row (their results are never stored)
    uint32_t xvo[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int r = 8 * u + (lane >> 3);
      const int rc = r < mt ? r : mt - 1;
      xvo[u] = (uint32_t)(rc * ldx * 2) + (uint32_t)(xs_slot(r, lane & 7) << 4);
    }
    // scale/bias DMA: lanes 0..31 the block of tile t0, lanes 32..63 of t1
    const uint32_t svo = (uint32_t)((lane >> 5) * (t1 - t0) * P * kPairSbBytes) + (uint32_t)(lane & 31) * 4u;
    uint8_t* const st = smem_stages + wave * kStageBytes;
    const uint32_t st_lds = lds_addr(st);
    const bf16x8 ones = ones_bf16x8();

    // 6-bit high-pair words: 512 bytes, lanes 0..31 (lanes 32..63 read out of
    // range: zeros into the rest of the slot)
    const uint32_t hvo = lane < 32 ? 1024u + (uint32_t)lane * 16u : kOffBuffer;
    // pair q into the stage: 8 activation loads, one or two code loads per
    // slot, one scale/bias load per two slots
    auto issue = [&](int q) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        int g = 2 * q + i / 4;
        g = g < G ? g : G - 1;
        dma_b128(xr, xvo[i % 4], (uint32_t)g * kXRowBytes, st_lds + (uint32_t)((i / 4) * kFlowRows * kXRowBytes + (i % 4) * 1024));
      }
#pragma unroll
      for (int sl = 0; sl < kSlots; ++sl) {
        const uint32_t so = (uint32_t)(((sl & 1) ? t1 - t0 : 0) * P + q) * kPcb;
        const i32x4 crs = sl >= 2 ? crb : cra;
        const uint32_t dst = st_lds + kXBytes + sl * kSlotCode;
        dma_b128(crs, (uint32_t)lane * 16u, so, dst);
        if constexpr (BITS == 6) dma_b128(crs, hvo, so, dst + 1024);
        else if constexpr (BITS != 4) dma_b128(crs, (uint32_t)lane * 16u + 1024u, so, dst + 1024);
      }
#pragma unroll
      for (int h = 0; h < kSlots / 2; ++h) {
        if (h >= 1) dma_b32(srb, svo, (uint32_t)q * kPairSbBytes, st_lds + kXBytes + kSlots * kSlotCode + 2 * h * kPairSbBytes);
        else dma_b32(sra, svo, (uint32_t)q * kPairSbBytes, st_lds + kXBytes + kSlots * kSlotCode + 2 * h * kPairSbBytes);
      }
    };

    const int i16 = lane & 15, kc = lane >> 4;
    const int mine = wave < P ? (P - 1 - wave) / NP + 1 : 0;  // pairs of this wave
    if (mine > 0) issue(wave);
    for (int n = 0; n < mine; ++n) {
      const int q = wave + n * NP;
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // pair q's DMA has landed
      // the stage into registers: the activation fragments (row j, 16-byte
      // chunk 2 ks + hl), the lane's code words and scale/bias words. Code
      // words of k steps 0, 2 come from lane L = jj + 16 hl of the block,
      // of steps 1, 3 from lane L + 32: c0 and c1 (4-bit: .xy the nibble words
      // of steps 0, 2 | 1, 3; 8-bit and FP8: the 16 bytes; 6-bit: the two
      // nibble words and the high-pair word)
      u32x4 xa[2][4];
      u32x4 c0[2][kTiles], c1[2][kTiles];
      uint32_t w[2][kTiles];
      const uint8_t* cs = st + kXBytes;
      const uint8_t* sbs = st + kXBytes + kSlots * kSlotCode;
      const int L = jj + 16 * hl;
#pragma unroll
      for (int gh = 0; gh < 2; ++gh) {
        const uint8_t* xb = st + gh * kFlowRows * kXRowBytes;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) xa[gh][ks] = *(const u32x4*)(xb + xs_off(j, 2 * ks + hl));
#pragma unroll
        for (int t = 0; t < kTiles; ++t) {
          const int sl = 2 * t + (j >> 4);
          w[gh][t] = *(const uint32_t*)(sbs + sl * kPairSbBytes + jj * 8 + gh * 4);
          const uint8_t* blk = cs + sl * kSlotCode;
          if constexpr (BITS == 4) {
            const u32x2 a = *(const u32x2*)(blk + L * 16 + gh * 8), b = *(const u32x2*)(blk + L * 16 + gh * 8 + 512);
            c0[gh][t] = u32x4{a[0], a[1], 0u, 0u};
            c1[gh][t] = u32x4{b[0], b[1], 0u, 0u};
          } else if constexpr (BITS == 6) {
            const u32x2 a = *(const u32x2*)(blk + L * 16 + gh * 8), b = *(const u32x2*)(blk + (L + 32) * 16 + gh * 8);
            c0[gh][t] = u32x4{a[0], a[1], *(const uint32_t*)(blk + 1024 + L * 8 + gh * 4), 0u};
            c1[gh][t] = u32x4{b[0], b[1], *(const uint32_t*)(blk + 1024 + (L + 32) * 8 + gh * 4), 0u};
          } else {
            c0[gh][t] = *(const u32x4*)(blk + gh * 1024 + L * 16);
            c1[gh][t] = *(const u32x4*)(blk + gh * 1024 + L * 16 + 512);
          }
        }
      }
      // the reads have completed: the stage takes the next pair
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      if (n + 1 < mine) issue(q + NP);

      f32x16 Pm[2][kTiles];
      f32x4 Sv[2][2];
#pragma unroll
      for (int gh = 0; gh < 2; ++gh) {
#pragma unroll
        for (int t = 0; t < kTiles; ++t) {
          // the exact bf16 codes of k steps 0..3 (as the other window kernels convert them)
          bf16x8 qk[4];
          const u32x4 a = c0[gh][t], b = c1[gh][t];
          if constexpr (BITS == 4) {
            qk[0] = codes_to_bf16(a[0]);
            qk[2] = codes_to_bf16(a[1]);
            qk[1] = codes_to_bf16(b[0]);
            qk[3] = codes_to_bf16(b[1]);
          } else if constexpr (BITS == 6) {
            qk[0] = six_to_bf16<0>(a[0], a[2]);
            qk[2] = six_to_bf16<1>(a[1], a[2]);
            qk[1] = six_to_bf16<0>(b[0], b[2]);
            qk[3] = six_to_bf16<1>(b[1], b[2]);
          } else if constexpr (BITS == kFmtFp8) {
            qk[0] = fp8_to_bf16(a[0], a[1]);
            qk[2] = fp8_to_bf16(a[2], a[3]);
            qk[1] = fp8_to_bf16(b[0], b[1]);
            qk[3] = fp8_to_bf16(b[2], b[3]);
          } else {
            qk[0] = bytes_to_bf16(a[0], a[1]);
            qk[2] = bytes_to_bf16(a[2], a[3]);
            qk[1] = bytes_to_bf16(b[0], b[1]);
            qk[3] = bytes_to_bf16(b[2], b[3]);
          }
          Pm[gh][t] = mfma32(__builtin_bit_cast(bf16x8, xa[gh][0]), qk[0], f32x16{});
          Pm[gh][t] = mfma32(__builtin_bit_cast(bf16x8, xa[gh][1]), qk[1], Pm[gh][t]);
          Pm[gh][t] = mfma32(__builtin_bit_cast(bf16x8, xa[gh][2]), qk[2], Pm[gh][t]);
          Pm[gh][t] = mfma32(__builtin_bit_cast(bf16x8, xa[gh][3]), qk[3], Pm[gh][t]);
        }
        if constexpr (kBias) {
        // the sums' operands: lane i16 + 16 kc of row block v takes chunks
        // kc and kc + 4 of row 16 v + i16. Lane 16 v + i16 + 32 (kc & 1) holds
        // them in xa[kc / 2] and xa[2 + kc / 2]; a swap of lane halves (32)
        // and then of lane quarters (16) between the two registers brings
        // row block 0's operand to one register and row block 1's to the other
        u32x4 X[2], Y[2];
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
#pragma unroll
          for (int d = 0; d < 4; ++d) {
            const auto r = __builtin_amdgcn_permlane32_swap(xa[gh][2 * h2][d], xa[gh][2 * h2 + 1][d], false, false);
            const auto s = __builtin_amdgcn_permlane16_swap(r[0], r[1], false, false);
            X[h2][d] = s[0];
            Y[h2][d] = s[1];
          }
        }
        Sv[gh][0] = mfma16(ones, __builtin_bit_cast(bf16x8, X[0]), f32x4{0.f, 0.f, 0.f, 0.f});
        Sv[gh][0] = mfma16(ones, __builtin_bit_cast(bf16x8, X[1]), Sv[gh][0]);
        Sv[gh][1] = mfma16(ones, __builtin_bit_cast(bf16x8, Y[0]), f32x4{0.f, 0.f, 0.f, 0.f});
        Sv[gh][1] = mfma16(ones, __builtin_bit_cast(bf16x8, Y[1]), Sv[gh][1]);
        }
      }
      // hand the pair to the folder. The folder releases a pair's entries
      // together (the second after the first), so the second slot's flag
      // frees both; one wait for the writes, then both flags.
      const int g0 = 2 * q, gl = 2 * q + 1 < G ? 2 * q + 1 : 2 * q;
      if (gl >= R) {
        for (int it = 0; it < (1 << 20); ++it) {
          if (__hip_atomic_load(&done[gl % R], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) == (uint32_t)(gl - R + 1)) break;
          __builtin_amdgcn_s_sleep(1);  // poll gently: the folder's LDS traffic comes first
        }
        asm volatile("" ::: "memory");
      }
#pragma unroll
      for (int gh = 0; gh < 2; ++gh) {
        const int g = g0 + gh;
        if (g >= G) break;
        const int slot = g % R;
#pragma unroll
        for (int t = 0; t < kTiles; ++t) {
#pragma unroll
          for (int i = 0; i < 4; ++i)
            ringP[slot][t][i][lane] = f32x4{Pm[gh][t][4 * i], Pm[gh][t][4 * i + 1], Pm[gh][t][4 * i + 2], Pm[gh][t][4 * i + 3]};
          ringC[slot][t][lane] = BITS == kFmtFp8 ? __uint_as_float(w[gh][t]) : bf16_lo(w[gh][t]);
        }
        if constexpr (!kBias) continue;
        // this group's share of its chunk's bias operands: position
        // (m, hl, e) = (gg / 4, gg / 2 % 2, gg % 2) of chunk c
        const int c = g / kPgemmChunk, gg = g % kPgemmChunk, m = gg >> 2, hg = (gg >> 1) & 1, e = gg & 1;
        if (kc == 0) {
#pragma unroll
          for (int v = 0; v < 2; ++v) {
            uint32_t h, mm, l;
            split3(Sv[gh][v][0], h, mm, l);
            u32x2* dst = (u32x2*)&biasA[c & 1][m][16 * v + i16 + 32 * hg] + e;
            *dst = u32x2{h | (mm << 16), l};
          }
        }
        if (hl == 0) {
#pragma unroll
          for (int t = 0; t < kTiles; ++t) {
            const uint32_t bb = w[gh][t] >> 16;
            u32x2* dst = (u32x2*)&biasB[c & 1][t][m][j + 32 * hg] + e;
            *dst = u32x2{bb | (bb << 16), bb};
          }
        }
      }
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      __hip_atomic_store(&ready[g0 % R], (uint32_t)(g0 + 1), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
      if (gl != g0) __hip_atomic_store(&ready[gl % R], (uint32_t)(gl + 1), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    }
    return;
  }

  // ---------------- folder ------------------------------------------------
  f32x16 acc[kTiles];
#pragma unroll
  for (int t = 0; t < kTiles; ++t)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[t][r] = 0.f;

  // chunk c's bias term on the matrix cores, added into acc. The producers
  // write every word of a whole chunk's operands; in the last chunk the
  // positions of groups past G may hold words of chunk c - 2 and are zeroed
  // here, in registers (lane j + 32 hl holds groups 4 m + 2 hl and + 1)
  auto bias_chunk = [&](int c) {
    const int valid = G - c * kPgemmChunk;
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      const int gb = 4 * m + 2 * hl;
      const bool k0 = gb < valid, k1 = gb + 1 < valid;
      u32x4 a = biasA[c & 1][m][lane];
      if (!k0) a[0] = a[1] = 0u;
      if (!k1) a[2] = a[3] = 0u;
#pragma unroll
      for (int t = 0; t < kTiles; ++t) {
        u32x4 b = biasB[c & 1][t][m][lane];
        if (!k0) b[0] = b[1] = 0u;
        if (!k1) b[2] = b[3] = 0u;
        acc[t] = mfma32(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), acc[t]);
      }
    }
  };

  struct Entry {
    f32x4 P[kTiles][4];
    float sc[kTiles];
  };
  auto read = [&](Entry& e, int g) {
    const int slot = g % R;
#pragma unroll
    for (int t = 0; t < kTiles; ++t) {
#pragma unroll
      for (int i = 0; i < 4; ++i) e.P[t][i] = ringP[slot][t][i][lane];
      e.sc[t] = ringC[slot][t][lane];
    }
  };
  // the fold of group g; after the fold of a chunk's first group, the
  // previous chunk's bias term
  auto fold = [&](const Entry& e, int g) {
#pragma unroll
    for (int t = 0; t < kTiles; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int u = 0; u < 4; ++u) acc[t][4 * i + u] = __builtin_fmaf(e.sc[t], e.P[t][i][u], acc[t][4 * i + u]);
    if constexpr (kBias)
      if ((g & (kPgemmChunk - 1)) == 0 && g > 0) bias_chunk(g / kPgemmChunk - 1);
  };
  // Pair q's flag (of its second group: a producer publishes a pair's groups
  // in order) and entries, read back to back. The LDS serves one wave's
  // accesses in order, so when the flag shows the pair, the entries read
  // after it are the pair's.
  auto issue_reads = [&](Entry& a, Entry& b, int q) -> uint32_t {
    const int g0 = 2 * q, g1 = g0 + 1 < G ? g0 + 1 : g0;
    const uint32_t f = __hip_atomic_load(&ready[g1 % R], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    asm volatile("" ::: "memory");
    read(a, g0);
    if (g1 != g0) read(b, g1);
    return f;
  };
  auto shows = [&](uint32_t f, int q) {
    const int g1 = 2 * q + 1 < G ? 2 * q + 1 : 2 * q;
    return __builtin_amdgcn_readfirstlane(f) == (uint32_t)(g1 + 1);
  };
  // read pair q until its flag shows it (bounded)
  auto fetch = [&](Entry& a, Entry& b, int q) {
    for (int it = 0; it < (1 << 22); ++it) {
      const uint32_t f = issue_reads(a, b, q);
      if (shows(f, q)) break;
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    }
  };
  // fold pair q (in ca, cb) while pair q + 1's reads are in flight, then
  // release pair q: every value of its entries has been consumed by then
  auto step = [&](Entry& ca, Entry& cb, Entry& na, Entry& nb2, int q) {
    // pair q's reads were issued a step ago: wait for them here, where the
    // compiler sees it, so that its own wait before the folds does not also
    // cover the reads of pair q + 1 issued below
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
    uint32_t f = 0;
    if (q + 1 < P) f = issue_reads(na, nb2, q + 1);
    fold(ca, 2 * q);
    if (2 * q + 1 < G) fold(cb, 2 * q + 1);
    const int g0 = 2 * q, g1 = g0 + 1 < G ? g0 + 1 : g0;
    asm volatile("" ::: "memory");
    __hip_atomic_store(&done[g0 % R], (uint32_t)(g0 + 1), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    if (g1 != g0) __hip_atomic_store(&done[g1 % R], (uint32_t)(g1 + 1), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    if (q + 1 < P && !shows(f, q + 1)) {
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      fetch(na, nb2, q + 1);
    }
  };
  {
    Entry a0, b0, a1, b1;
    fetch(a0, b0, 0);
    for (int q = 0; q < P; q += 2) {
      step(a0, b0, a1, b1, q);
      if (q + 1 < P) step(a1, b1, a0, b0, q + 1);
    }
  }
  // the last chunk's producers published before the folder consumed their
  // groups, so its operands are in place
  if constexpr (kBias) bias_chunk((G - 1) / kPgemmChunk);

  // ---- epilogue: element r is row 8 (r / 4) + 4 hl + r % 4, column jj of the
  // lane's weight tile
  if (wtile >= ntiles) return;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int row = 8 * (r / 4) + 4 * hl + (r % 4);
    if (row >= mt) continue;
    const int64_t at = (int64_t)(m0 + row) * ldy + (int64_t)wtile * kTileN + jj;
    const float z = SWIGLU ? silu_f32(acc[0][r]) * acc[kTiles - 1][r] : acc[0][r];
    if constexpr (OUT_BF16) ((uint16_t*)yv)[at] = f32_to_bf16_rne(z);
    else ((float*)yv)[at] = z;
  }
}

}  // namespace q4
