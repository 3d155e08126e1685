// Prompt GEMM for short windows. Codes of 4, 6 or 8 bits (MLX affine) or
// block FP8.
//
// A window of a few hundred rows gives pgemm_kernel's 128-row x 256-column
// workgroups too few tiles to fill the chip (a 128-row window of w1/w3 is
// 64 workgroups), and every workgroup walks all of K in sequence. Here a
// workgroup of 4 waves owns 128 rows and only 4 weight tiles of 16 columns
// (64 weight columns; SwiGLU: 2 tiles of w1 and the same 2 of w3, 32 output
// columns), and wave w owns rows 32w .. 32w + 31 of all of them: a quarter of
// the work per workgroup, four times the workgroups, each wave converting the
// codes of all 64 columns for its one row tile. 4-bit codes are staged a
// group pair at a time, the wider ones a group at a time (pgemm_kernel's
// stages and fragment reads for each format).
//
// Per output the arithmetic is pgemm_kernel's, step for step: the same four
// chained 32 x 32 x 16 matrix steps per group on the same exact bf16 codes,
// the same fold fma(s_g, P_g, acc), the same activation sums (16 x 16 x 32
// against ones, two per 16 rows) and the same bias term per chunk of 8
// groups. A row's bits are therefore the same whichever kernel computes
// them, and the window cut stays free (TensorFold PR #1696, later revision,
// "What it adds", prompt GEMM item; "Checks": every row alone equals the row
// inside a window).
#pragma once

#include "pgemm.h"

namespace q4 {

constexpr int kNarrowSlots = 4;     // 16-column weight tiles per workgroup
constexpr int kNarrowSbSlot = 256;  // scale/bias stage bytes per slot (128 used, then the DMA's padding)
constexpr int kNarrowSbStage = kNarrowSlots * kNarrowSbSlot;  // 1 KiB
// code bytes per slot and stage: a group pair of 4-bit codes, a group of the wider ones
__host__ __device__ constexpr int narrow_slot_stage_bytes(int bits) { return bits == 4 ? kPairCodeBytes : pgemm_group_code_bytes(bits); }

// Output columns covered by one workgroup.
__host__ __device__ constexpr int pgemm_narrow_cols(bool swiglu) { return swiglu ? 2 * kTileN : kNarrowSlots * kTileN; }

template <bool SWIGLU, bool OUT_BF16, int BITS = 4>
__global__ __launch_bounds__(kPgemmThreads, 2) void pgemm_narrow_kernel(const uint8_t* __restrict__ pa, const uint8_t* __restrict__ pb,
                                                                         int N, int K, const uint16_t* __restrict__ x, int64_t ldx, int M,
                                                                         void* __restrict__ yv, int64_t ldy, int nblk, int mblk) {
  __shared__ __align__(16) uint8_t xs[kXStages * kXStageBytes];
  constexpr int kSlotStage = narrow_slot_stage_bytes(BITS);
  constexpr int kCSt = kNarrowSlots * kSlotStage;  // one code stage (3 or 4 KiB)
  constexpr int kPcb = pair_code_bytes(BITS);
  static_assert(BITS == 4 || BITS == 6 || BITS == 8 || BITS == kFmtFp8, "4-, 6- or 8-bit codes or block FP8");
  __shared__ __align__(16) uint8_t cs[2 * kCSt];
  __shared__ __align__(16) uint8_t sbs[2 * kNarrowSbStage];
  __shared__ __align__(16) float ssum[kSumFloats];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  int mb, nb;
  pgemm_tile(blockIdx.x, nblk, mblk, mb, nb);
  const int m0 = mb * kPgemmRows;
  const int mt = M - m0 < kPgemmRows ? M - m0 : kPgemmRows;  // rows of this tile inside the window
  const int G = K / kGroup;
  const int P = (G + 1) / 2;
  const int ntiles = N / kTileN;
  const int64_t cb = codes_bytes(N, K, BITS);
  const bf16x8 ones = ones_bf16x8();

  // slot (0..3) -> weight tile (unclamped)
  auto slot_tile = [&](int slot) { return SWIGLU ? nb * 2 + (slot & 1) : nb * kNarrowSlots + slot; };
  auto clamp_tile = [&](int t) { return t < ntiles ? t : ntiles - 1; };

  // ---- DMA set-up --------------------------------------------------------
  // activations: as pgemm_kernel, wave w stages rows 32w + 8u + lane / 8
  const i32x4 xr = make_srsrc(x + (int64_t)m0 * ldx, (uint32_t)((int64_t)mt * ldx * 2));
  uint32_t xvo[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int r = 32 * wave + 8 * u + (lane >> 3);
    const int rc = r < mt ? r : mt - 1;
    xvo[u] = (uint32_t)(rc * ldx * 2) + (uint32_t)(xs_slot(r, lane & 7) << 4);
  }
  const uint32_t xs_lds = lds_addr(xs) + wave * 4096;
  // codes and scale/bias words: wave w stages slot w (SwiGLU: waves 0, 1 the
  // two w1 tiles, waves 2, 3 the same two tiles of w3). The scale/bias DMA
  // writes 64 words per wave; lanes 32..63 read out of range and fill the
  // slot's padding with zeros.
  const uint8_t* mat = (SWIGLU && wave >= 2) ? pb : pa;
  const int tw = clamp_tile(slot_tile(wave));
  const i32x4 cr = make_srsrc(mat + (int64_t)tw * P * kPcb, (uint32_t)(P * kPcb));
  const i32x4 sr = make_srsrc(mat + cb + (int64_t)tw * P * kPairSbBytes, (uint32_t)(P * kPairSbBytes));
  const uint32_t cvo = (uint32_t)lane * 16u;
  const uint32_t svo = lane < 32 ? (uint32_t)lane * 4u : kOffBuffer;
  const uint32_t cs_lds = lds_addr(cs) + wave * kSlotStage;
  const uint32_t sb_lds = lds_addr(sbs) + wave * kNarrowSbSlot;

  auto issue_x = [&](int g) {
    const uint32_t dst = xs_lds + (uint32_t)(g % kXStages) * kXStageBytes;
#pragma unroll
    for (int u = 0; u < 4; ++u) dma_b128(xr, xvo[u], (uint32_t)g * kXRowBytes, dst + u * 1024);
  };
  auto issue_sb = [&](int p) { dma_b32(sr, svo, (uint32_t)p * kPairSbBytes, sb_lds + (uint32_t)(p & 1) * kNarrowSbStage); };
  // 4-bit: the codes and scale/bias words of pair p into stage p & 1: two loads
  auto issue_c = [&](int p) {
    dma_b128(cr, cvo, (uint32_t)p * kPairCodeBytes, cs_lds + (uint32_t)(p & 1) * kCSt);
    issue_sb(p);
  };
  // 6- and 8-bit: the codes of group g into stage g & 1 (one or three loads)
  auto issue_cg = [&](int g) {
    const uint32_t dst = cs_lds + (uint32_t)(g & 1) * kCSt;
    const uint32_t blk = (uint32_t)(g >> 1) * kPcb, gh = (uint32_t)(g & 1);
    if constexpr (code_bits(BITS) == 8) {
      dma_b128(cr, cvo, blk + gh * 1024u, dst);
    } else {
      dma_b32(cr, (uint32_t)lane * 16u + gh * 8u, blk, dst);
      dma_b32(cr, (uint32_t)lane * 16u + gh * 8u + 4u, blk, dst + 256);
      dma_b32(cr, 1024u + (uint32_t)lane * 8u + gh * 4u, blk, dst + 512);
    }
  };

  // ---- consumer set-up ---------------------------------------------------
  const int j = lane & 31, hl = lane >> 5, jj = j & 15;
  // column tile s: slot of this lane's column (s = 0: slots 0, 1; s = 1: slots 2, 3)
  int lslot[kPgemmNT];
#pragma unroll
  for (int s = 0; s < kPgemmNT; ++s) lslot[s] = 2 * s + (j >> 4);
  const int rbase = 32 * wave;

  f32x16 acc[kPgemmNT];
#pragma unroll
  for (int s = 0; s < kPgemmNT; ++s)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[s][r] = 0.f;
  uint32_t bsel[kPgemmNT][2][2];
#pragma unroll
  for (int s = 0; s < kPgemmNT; ++s) bsel[s][0][0] = bsel[s][0][1] = bsel[s][1][0] = bsel[s][1][1] = 0u;

  // the bias term of chunk c on the matrix cores, added into acc
  auto bias_chunk = [&](int c) {
    const float* sp = ssum + (c & 1) * kPgemmRows * kPgemmChunk;
    bf16x8 bfr[kPgemmNT][2];
#pragma unroll
    for (int s = 0; s < kPgemmNT; ++s)
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        const uint32_t b0 = bsel[s][m][0] >> 16, b1 = bsel[s][m][1] >> 16;
        bfr[s][m] = __builtin_bit_cast(bf16x8, u32x4{b0 | (b0 << 16), b0, b1 | (b1 << 16), b1});
        bsel[s][m][0] = bsel[s][m][1] = 0u;
      }
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      const int g0 = kPgemmChunk * c + 4 * m + 2 * hl;
      const bool v0 = g0 < G, v1 = g0 + 1 < G;
      const int row = rbase + j;
      const float2 S2 = *(const float2*)(sp + row * kPgemmChunk + 4 * m + 2 * hl);
      const float s0 = v0 ? S2.x : 0.f, s1 = v1 ? S2.y : 0.f;
      uint32_t h0, mm0, l0, h1, mm1, l1;
      split3(s0, h0, mm0, l0);
      split3(s1, h1, mm1, l1);
      const bf16x8 afr = __builtin_bit_cast(bf16x8, u32x4{h0 | (mm0 << 16), l0, h1 | (mm1 << 16), l1});
#pragma unroll
      for (int s = 0; s < kPgemmNT; ++s) acc[s] = mfma32(afr, bfr[s][m], acc[s]);
    }
  };

  // Group g's products are folded at the start of group g + 1 (the last
  // group's after the loop), so acc still takes fold(0), fold(1), ... in
  // ascending order, each chunk's bias term after the fold of the next
  // chunk's first group, exactly as in pgemm_kernel.
  f32x16 Pd[kPgemmNT];
  float scd[kPgemmNT];
  uint32_t wd[kPgemmNT];
#pragma unroll
  for (int s = 0; s < kPgemmNT; ++s) {
#pragma unroll
    for (int r = 0; r < 16; ++r) Pd[s][r] = 0.f;
    scd[s] = 0.f;
    wd[s] = 0u;
  }
  // after the fold of group gp (half ghp of its pair): the previous chunk's
  // bias term when gp opens a chunk (its sums are visible since the barrier
  // of the group that follows gp), then gp's bias word joins its chunk
  auto prev_bias = [&](int gp, auto ghpc) {
    constexpr int ghp = decltype(ghpc)::value;
    const int ggp = gp & (kPgemmChunk - 1);
    if constexpr (ghp == 0) {
      if (ggp == 0 && gp > 0) bias_chunk(gp / kPgemmChunk - 1);
    }
    const bool take = gp >= 0 && ((ggp >> 1) & 1) == hl;
#pragma unroll
    for (int s = 0; s < kPgemmNT; ++s) {
      if (take && ggp < 4) bsel[s][0][ghp] = wd[s];
      if (take && ggp >= 4) bsel[s][1][ghp] = wd[s];
    }
  };

  // one group; gh (compile time) is the group's half of its pair
  auto group = [&](int g, auto ghc) {
    constexpr int gh = decltype(ghc)::value;
    const int p = g >> 1, gg = g & (kPgemmChunk - 1);
    const uint8_t* xb = xs + (g % kXStages) * kXStageBytes;
    const uint8_t* cb0 = cs + (BITS == 4 ? (p & 1) : (g & 1)) * kCSt;
    const uint8_t* sb0 = sbs + (p & 1) * kNarrowSbStage;

    uint32_t w[kPgemmNT];
    float sc[kPgemmNT];
#pragma unroll
    for (int s = 0; s < kPgemmNT; ++s) {
      w[s] = *(const uint32_t*)(sb0 + lslot[s] * kNarrowSbSlot + jj * 8 + gh * 4);
      sc[s] = BITS == kFmtFp8 ? __uint_as_float(w[s]) : bf16_lo(w[s]);
    }

    bf16x8 q[kPgemmNT][4];
#pragma unroll
    for (int s = 0; s < kPgemmNT; ++s) {
      const int L = jj + 16 * hl;
      if constexpr (BITS == 4) {
        const uint8_t* cl = cb0 + lslot[s] * kPairCodeBytes + L * 16 + gh * 8;
        const u32x2 c02 = *(const u32x2*)cl, c13 = *(const u32x2*)(cl + 512);
        q[s][0] = codes_to_bf16(c02[0]);
        q[s][2] = codes_to_bf16(c02[1]);
        q[s][1] = codes_to_bf16(c13[0]);
        q[s][3] = codes_to_bf16(c13[1]);
      } else if constexpr (BITS == 8) {
        const uint8_t* cl = cb0 + lslot[s] * kSlotStage + L * 16;
        const u32x4 c02 = *(const u32x4*)cl, c13 = *(const u32x4*)(cl + 512);
        q[s][0] = bytes_to_bf16(c02[0], c02[1]);
        q[s][2] = bytes_to_bf16(c02[2], c02[3]);
        q[s][1] = bytes_to_bf16(c13[0], c13[1]);
        q[s][3] = bytes_to_bf16(c13[2], c13[3]);
      } else if constexpr (BITS == kFmtFp8) {
        const uint8_t* cl = cb0 + lslot[s] * kSlotStage + L * 16;
        const u32x4 c02 = *(const u32x4*)cl, c13 = *(const u32x4*)(cl + 512);
        q[s][0] = fp8_to_bf16(c02[0], c02[1]);
        q[s][2] = fp8_to_bf16(c02[2], c02[3]);
        q[s][1] = fp8_to_bf16(c13[0], c13[1]);
        q[s][3] = fp8_to_bf16(c13[2], c13[3]);
      } else {
        const uint32_t* cl = (const uint32_t*)(cb0 + lslot[s] * kSlotStage);
        q[s][0] = six_to_bf16<0>(cl[L], cl[128 + L]);
        q[s][2] = six_to_bf16<1>(cl[64 + L], cl[128 + L]);
        q[s][1] = six_to_bf16<0>(cl[L + 32], cl[128 + L + 32]);
        q[s][3] = six_to_bf16<1>(cl[64 + L + 32], cl[128 + L + 32]);
      }
    }
    // keeps the previous group's fold below the DMA issue that precedes
    // this group (the compiler would otherwise hoist it there, ahead of
    // this group's reads, where nothing hides it)
    static_assert(kPgemmNT == 2, "one register per column tile below");
    asm volatile("" : "+v"(scd[0]), "+v"(scd[1]));
    f32x16 Pn[kPgemmNT];
    {
      const int row = rbase + j;
      bf16x8 xa[4];
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) xa[ks] = __builtin_bit_cast(bf16x8, *(const u32x4*)(xb + xs_off(row, 2 * ks + hl)));
#pragma unroll
      for (int s = 0; s < kPgemmNT; ++s) {
        Pn[s] = mfma32(xa[0], q[s][0], f32x16{});
#pragma unroll
        for (int ks = 1; ks < 4; ++ks) Pn[s] = mfma32(xa[ks], q[s][ks], Pn[s]);
      }
    }
    // the previous group's fold: independent of this group's matrix steps,
    // so it can issue while they run (for g = 0: fma(0, 0, +0) = +0 leaves
    // acc as it is)
#pragma unroll
    for (int s = 0; s < kPgemmNT; ++s)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[s][r] = __builtin_fmaf(scd[s], Pd[s][r], acc[s][r]);

    // activation sums of this wave's 32 rows (16 x 16 tiles); block FP8 has
    // no bias term and needs none
    if constexpr (BITS != kFmtFp8) {
      const int i = lane & 15, kc = lane >> 4;
      float* sw = ssum + ((g / kPgemmChunk) & 1) * kPgemmRows * kPgemmChunk + gg;
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int row = rbase + 16 * u + i;
        const bf16x8 xa0 = __builtin_bit_cast(bf16x8, *(const u32x4*)(xb + xs_off(row, kc)));
        const bf16x8 xa1 = __builtin_bit_cast(bf16x8, *(const u32x4*)(xb + xs_off(row, kc + 4)));
        f32x4 S = mfma16(ones, xa0, f32x4{0.f, 0.f, 0.f, 0.f});
        S = mfma16(ones, xa1, S);
        // every row of the ones-product holds the same sums, so all four
        // lanes of a column store the same value (no divergent branch)
        sw[row * kPgemmChunk] = S[0];
      }
    }

    // the previous group's bias step, now that its fold is in acc
    if constexpr (BITS != kFmtFp8) prev_bias(g - 1, std::integral_constant<int, 1 - gh>{});
#pragma unroll
    for (int s = 0; s < kPgemmNT; ++s) {
      Pd[s] = Pn[s];
      scd[s] = sc[s];
      wd[s] = w[s];
    }
    // 8-bit codes: the fold ends with its group (without this the compiler
    // sinks it past the next branch, away from the matrix steps it hides
    // under; measured 7% on 128-row windows, and slower for the other formats)
    if constexpr (BITS == 8) asm volatile("" : "+v"(acc[0]), "+v"(acc[1]));
  };

  // ---- pipeline (as pgemm_kernel's; 4-bit: two code loads per pair and
  // wave, the wider codes: one group of codes in flight) ---------------------
  if constexpr (BITS == 4) {
    issue_x(0);
    issue_c(0);
    for (int p = 0; p < P; ++p) {
      const int g = 2 * p;
      dma_wait_barrier<0>();
      if (g + 1 < G) issue_x(g + 1);
      if (p + 1 < P) issue_c(p + 1);
      group(g, std::integral_constant<int, 0>{});
      if (g + 1 < G) {
        if (p + 1 < P) dma_wait_barrier<2>();
        else dma_wait_barrier<0>();
        if (g + 2 < G) issue_x(g + 2);
        group(g + 1, std::integral_constant<int, 1>{});
      }
    }
  } else {
    issue_x(0);
    issue_cg(0);
    issue_sb(0);
    for (int p = 0; p < P; ++p) {
      const int g = 2 * p;
      dma_wait_barrier<0>();
      if (g + 1 < G) {
        issue_x(g + 1);
        issue_cg(g + 1);
      }
      group(g, std::integral_constant<int, 0>{});
      if (g + 1 < G) {
        dma_wait_barrier<0>();
        if (g + 2 < G) {
          issue_x(g + 2);
          issue_cg(g + 2);
          issue_sb(p + 1);
        }
        group(g + 1, std::integral_constant<int, 1>{});
      }
    }
  }
  dma_wait_barrier<0>();  // the last group's sums
  // the last group's fold and bias step, then its chunk's bias term
#pragma unroll
  for (int s = 0; s < kPgemmNT; ++s)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[s][r] = __builtin_fmaf(scd[s], Pd[s][r], acc[s][r]);
  if constexpr (BITS != kFmtFp8) {
    if ((G - 1) & 1) prev_bias(G - 1, std::integral_constant<int, 1>{});
    else prev_bias(G - 1, std::integral_constant<int, 0>{});
    bias_chunk((G - 1) / kPgemmChunk);
  }

  // ---- epilogue: element r of tile s is row rbase + 8 (r / 4) + 4 hl + r % 4
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int row = rbase + 8 * (r / 4) + 4 * hl + (r % 4);
    if (row >= mt) continue;
    const int64_t yrow = (int64_t)(m0 + row) * ldy;
    if constexpr (SWIGLU) {
      const int t = slot_tile(lslot[0]);
      if (t >= ntiles) continue;
      const float z = silu_f32(acc[0][r]) * acc[1][r];
      const int64_t at = yrow + (int64_t)t * kTileN + jj;
      if constexpr (OUT_BF16) ((uint16_t*)yv)[at] = f32_to_bf16_rne(z);
      else ((float*)yv)[at] = z;
    } else {
#pragma unroll
      for (int s = 0; s < kPgemmNT; ++s) {
        const int t = slot_tile(lslot[s]);
        if (t >= ntiles) continue;
        const int64_t at = yrow + (int64_t)t * kTileN + jj;
        if constexpr (OUT_BF16) ((uint16_t*)yv)[at] = f32_to_bf16_rne(acc[s][r]);
        else ((float*)yv)[at] = acc[s][r];
      }
    }
  }
}

}  // namespace q4
