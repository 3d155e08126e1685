// Prefill window GEMM (pgemm) on the matrix cores.
//
// A workgroup of 4 waves owns 128 window rows and 16 weight column tiles of
// 16 columns (256 output columns; SwiGLU: 128 output columns, 8 tiles of w1
// and the same 8 tiles of w3). Wave w covers all 128 rows and 64 weight
// columns (SwiGLU: 32 columns of w1 and the same 32 of w3), held as 4 x 2
// output tiles of 32 x 32 for v_mfma_f32_32x32x16_bf16. A workgroup uses
// 76 KiB of LDS, so two run on each CU: each SIMD then holds one wave of
// each, and the two drift independently, one issuing matrix work while the
// other waits at its barrier or converts codes.
//
// Operands move from HBM to LDS by buffer-to-LDS DMA, which costs no
// registers while in flight: the 128 x 64 activation tile of a group in two
// stages (one group of lookahead), the codes and scale/bias words of a pair
// of groups in two stages. One barrier per group. Each wave turns the codes
// of its columns into exact bf16 integers once per group and reuses them for
// its four row tiles. The activation sum S_g of a row is formed once per
// workgroup (each wave forms it for 32 of the 128 rows) and shared through
// LDS.
//
// Per output (r, n) the order is, with chunks c of 8 consecutive groups:
//
//   acc = 0
//   for each group g (ascending):
//     P_g = four chained 16-wide k steps on the matrix cores       exact products
//     acc = fma(s_g, P_g, acc)                                    one VALU op per output
//     S_g = sum of x[g, :] on the matrix cores (A = ones)
//     if g = 8 (c + 1) for a chunk c:  acc = B_c(acc)
//   acc = B_c(acc) for the last chunk
//   y = acc
//
// where B_c(acc) = mfma(A = exact bf16 pieces h, m, l of S_g for groups
// 4..7 of chunk c, B = b_g repeated over the pieces, C = mfma(the same for
// groups 0..3, C = acc)) adds the chunk's bias term.
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

constexpr int kPgemmWaves = 4;                  // 4 column quarters
constexpr int kPgemmThreads = kPgemmWaves * 64;
constexpr int kPgemmRT = 4;                     // 32-row tiles per wave
constexpr int kPgemmNT = 2;                     // 32-column tiles per wave (2 weight tiles each)
constexpr int kPgemmRows = 128;                 // window rows per workgroup
constexpr int kPgemmSlots = 16;                 // 16-column weight tiles per workgroup
constexpr int kPgemmChunk = 8;                  // groups per bias chunk
constexpr int kXStages = 2;
constexpr int kXRowBytes = kGroup * 2;          // one staged activation row of a group
constexpr int kXStageBytes = kPgemmRows * kXRowBytes;       // 16 KiB
constexpr int kCStageBytes = kPgemmSlots * kPairCodeBytes;  // 16 KiB
// Wider codes are staged one group at a time (a pair would not fit two
// workgroups per CU): per slot, 8-bit is the group's 1 KiB sub-block as is;
// 6-bit is the group's two nibble words of every lane then its high-pair
// word of every lane, each as a 256-byte row (three dword copies).
__host__ __device__ constexpr int pgemm_group_code_bytes(int bits) { return code_bits(bits) == 8 ? 1024 : 768; }
__host__ __device__ constexpr int pgemm_cstage_bytes(int bits) {
  return bits == 4 ? kCStageBytes : kPgemmSlots * pgemm_group_code_bytes(bits);
}
constexpr int kSbStageBytes = kPgemmSlots * kPairSbBytes;   // 2 KiB
constexpr int kSumFloats = 2 * kPgemmRows * kPgemmChunk;    // activation sums, 2 chunks
static_assert(kPgemmRows == kPgemmRT * 32, "kPgemmRT row tiles of 32");
static_assert(kPgemmSlots == 4 * 2 * kPgemmNT, "four column quarters");

typedef float f32x16 __attribute__((ext_vector_type(16)));
// D = A B + C on 32 x 32 x 16 bf16: A[i][k] in lane i + 32 (k / 8), element
// k % 8; B[k][j] in lane j + 32 (k / 8), element k % 8; D[i][j] in lane
// j + 32 ((i / 4) % 2), element 4 (i / 8) + i % 4.
__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
static_assert(kPgemmRows * kXRowBytes == kPgemmWaves * 4 * 1024, "each wave stages 4 KiB of a group");
static_assert(kPgemmSlots == 4 * kPgemmWaves, "each wave stages 4 weight slots");

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
  static_assert(n == 0 || n == 2 || n == 6, "wait depths used by the pipelines");
  if constexpr (n == 6) asm volatile("s_waitcnt vmcnt(6)\n\ts_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  else if constexpr (n == 2) asm volatile("s_waitcnt vmcnt(2)\n\ts_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
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

template <bool SWIGLU, bool OUT_BF16, int BITS>
__global__ __launch_bounds__(kPgemmThreads, 2) void pgemm_kernel(const uint8_t* __restrict__ pa, const uint8_t* __restrict__ pb,
                                                                  int N, int K, const uint16_t* __restrict__ x, int64_t ldx, int M,
                                                                  void* __restrict__ yv, int64_t ldy, int nblk, int mblk) {
  __shared__ __align__(16) uint8_t xs[kXStages * kXStageBytes];
  constexpr int kCSt = pgemm_cstage_bytes(BITS);
  constexpr int kPcb = pair_code_bytes(BITS);
  __shared__ __align__(16) uint8_t cs[2 * kCSt];
  __shared__ __align__(16) uint8_t sbs[2 * kSbStageBytes];
  __shared__ __align__(16) float ssum[kSumFloats];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int cw = wave;
  int mb, nb;
  pgemm_tile(blockIdx.x, nblk, mblk, mb, nb);
  const int m0 = mb * kPgemmRows;
  const int mt = M - m0 < kPgemmRows ? M - m0 : kPgemmRows;  // rows of this tile inside the window
  const int G = K / kGroup;
  const int P = (G + 1) / 2;
  const int ntiles = N / kTileN;
  const int64_t cb = codes_bytes(N, K, BITS);
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
  // codes and scale/bias words: wave w stages slots 4w .. 4w + 3, all of one
  // matrix and (up to the clamp at N) consecutive tiles
  const uint8_t* mat = (SWIGLU && wave >= 2) ? pb : pa;
  int tsl[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) tsl[u] = clamp_tile(slot_tile(4 * wave + u));
  const int t0 = tsl[0];
  const i32x4 cr = make_srsrc(mat + (int64_t)t0 * P * kPcb, (uint32_t)((tsl[3] - t0 + 1) * P * kPcb));
  const i32x4 sr = make_srsrc(mat + cb + (int64_t)t0 * P * kPairSbBytes, (uint32_t)((tsl[3] - t0 + 1) * P * kPairSbBytes));
  const uint32_t cvo = (uint32_t)lane * 16u;
  uint32_t svo[2];
#pragma unroll
  for (int u = 0; u < 2; ++u)
    svo[u] = (uint32_t)((lane >> 5) * (tsl[2 * u + 1] - tsl[2 * u]) * P * kPairSbBytes) + (uint32_t)(lane & 31) * 4u;
  constexpr int kSlotStage = BITS == 4 ? kPairCodeBytes : pgemm_group_code_bytes(BITS);  // bytes per slot per stage
  const uint32_t cs_lds = lds_addr(cs) + 4 * wave * kSlotStage;
  const uint32_t sb_lds = lds_addr(sbs) + 4 * wave * kPairSbBytes;

  auto issue_x = [&](int g) {
    const uint32_t dst = xs_lds + (uint32_t)(g % kXStages) * kXStageBytes;
#pragma unroll
    for (int u = 0; u < 4; ++u) dma_b128(xr, xvo[u], (uint32_t)g * kXRowBytes, dst + u * 1024);
  };
  auto issue_sb = [&](int p) {
    const uint32_t st = (uint32_t)(p & 1);
#pragma unroll
    for (int u = 0; u < 2; ++u)
      dma_b32(sr, svo[u], (uint32_t)((tsl[2 * u] - t0) * P + p) * kPairSbBytes, sb_lds + st * kSbStageBytes + 2 * u * kPairSbBytes);
  };
  // 4-bit: the codes of pair p (both groups) into stage p & 1
  auto issue_c = [&](int p) {
    const uint32_t st = (uint32_t)(p & 1);
#pragma unroll
    for (int u = 0; u < 4; ++u)
      dma_b128(cr, cvo, (uint32_t)((tsl[u] - t0) * P + p) * kPairCodeBytes, cs_lds + st * kCStageBytes + u * kPairCodeBytes);
    issue_sb(p);
  };
  // 6- and 8-bit: the codes of group g into stage g & 1
  auto issue_cg = [&](int g) {
    const uint32_t dst = cs_lds + (uint32_t)(g & 1) * kCSt;
    const int p = g >> 1, gh = g & 1;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const uint32_t blk = (uint32_t)((tsl[u] - t0) * P + p) * kPcb;
      if constexpr (code_bits(BITS) == 8) {
        dma_b128(cr, cvo, blk + (uint32_t)gh * 1024u, dst + u * kSlotStage);
      } else {
        dma_b32(cr, (uint32_t)lane * 16u + (uint32_t)gh * 8u, blk, dst + u * kSlotStage);
        dma_b32(cr, (uint32_t)lane * 16u + (uint32_t)gh * 8u + 4u, blk, dst + u * kSlotStage + 256);
        dma_b32(cr, 1024u + (uint32_t)lane * 8u + (uint32_t)gh * 4u, blk, dst + u * kSlotStage + 512);
      }
    }
  };

  // ---- consumer set-up ---------------------------------------------------
  // 32 x 32 fragments: lane = j + 32 hl; j is the row (A) or column (B, D)
  // of the tile, hl the 8-wide k half of a 16-wide step
  const int j = lane & 31, hl = lane >> 5, jj = j & 15;
  // column tile s: weight slot of this lane's column (two 16-column slots)
  int lslot[kPgemmNT];
#pragma unroll
  for (int s = 0; s < kPgemmNT; ++s) lslot[s] = (SWIGLU ? (s == 0 ? 2 * cw : 8 + 2 * cw) : 4 * cw + 2 * s) + (j >> 4);
  constexpr int rbase = 0;

  f32x16 acc[kPgemmRT][kPgemmNT];
#pragma unroll
  for (int rt = 0; rt < kPgemmRT; ++rt)
#pragma unroll
    for (int s = 0; s < kPgemmNT; ++s)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[rt][s][r] = 0.f;
  // raw scale/bias words of this lane's column for the groups its bias
  // operand carries: 4 m + 2 hl + e (e = 0, 1) of the current chunk, m = 0, 1
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
#pragma unroll
      for (int rt = 0; rt < kPgemmRT; ++rt) {
        const int row = rbase + rt * 32 + j;
        const float2 S2 = *(const float2*)(sp + row * kPgemmChunk + 4 * m + 2 * hl);
        // groups past K hold no sum in this chunk; their slots must be zero
        const float s0 = v0 ? S2.x : 0.f, s1 = v1 ? S2.y : 0.f;
        uint32_t h0, mm0, l0, h1, mm1, l1;
        split3(s0, h0, mm0, l0);
        split3(s1, h1, mm1, l1);
        const bf16x8 afr = __builtin_bit_cast(bf16x8, u32x4{h0 | (mm0 << 16), l0, h1 | (mm1 << 16), l1});
#pragma unroll
        for (int s = 0; s < kPgemmNT; ++s) acc[rt][s] = mfma32(afr, bfr[s][m], acc[rt][s]);
      }
    }
  };

  // one group; gh (compile time) is the group's half of its pair
  auto group = [&](int g, auto ghc) {
    constexpr int gh = decltype(ghc)::value;
    const int p = g >> 1, gg = g & (kPgemmChunk - 1);
    const uint8_t* xb = xs + (g % kXStages) * kXStageBytes;
    const uint8_t* cb0 = cs + (BITS == 4 ? (p & 1) : (g & 1)) * kCSt;
    const uint8_t* sb0 = sbs + (p & 1) * kSbStageBytes;

    // codes of this lane's column: k steps 0 and 2 are halves 0 and 1 of the
    // group in lane jj + 16 hl of the block, steps 1 and 3 in lane jj + 32 + 16 hl
    uint32_t w[kPgemmNT];
    float sc[kPgemmNT];
#pragma unroll
    for (int s = 0; s < kPgemmNT; ++s) {
      w[s] = *(const uint32_t*)(sb0 + lslot[s] * kPairSbBytes + jj * 8 + gh * 4);
      sc[s] = BITS == kFmtFp8 ? __uint_as_float(w[s]) : bf16_lo(w[s]);
    }

    // activation sums of this wave's 32 of the 128 rows (16 x 16 tiles);
    // block FP8 has no bias term and needs none
    if constexpr (BITS != kFmtFp8) {
      const int i = lane & 15, kc = lane >> 4;
      float* sw = ssum + ((g / kPgemmChunk) & 1) * kPgemmRows * kPgemmChunk + gg;
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int row = rbase + 32 * cw + 16 * u + i;
        const bf16x8 xa0 = __builtin_bit_cast(bf16x8, *(const u32x4*)(xb + xs_off(row, kc)));
        const bf16x8 xa1 = __builtin_bit_cast(bf16x8, *(const u32x4*)(xb + xs_off(row, kc + 4)));
        f32x4 S = mfma16(ones, xa0, f32x4{0.f, 0.f, 0.f, 0.f});
        S = mfma16(ones, xa1, S);
        if (kc == 0) sw[row * kPgemmChunk] = S[0];
      }
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
#pragma unroll
    for (int rt = 0; rt < kPgemmRT; ++rt) {
      const int row = rbase + rt * 32 + j;
      bf16x8 xa[4];
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) xa[ks] = __builtin_bit_cast(bf16x8, *(const u32x4*)(xb + xs_off(row, 2 * ks + hl)));
#pragma unroll
      for (int s = 0; s < kPgemmNT; ++s) {
        f32x16 Pm = mfma32(xa[0], q[s][0], f32x16{});
#pragma unroll
        for (int ks = 1; ks < 4; ++ks) Pm = mfma32(xa[ks], q[s][ks], Pm);
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[rt][s][r] = __builtin_fmaf(sc[s], Pm[r], acc[rt][s][r]);
      }
    }

    // the previous chunk's bias term follows the fold of its next chunk's
    // first group (its sums are visible since this group's barrier); only
    // then does this group's bias word join the new chunk's operand
    if constexpr (BITS == kFmtFp8) {
      // No bias term: an empty statement that takes and returns every
      // accumulator ends the group instead, so that the scheduler does not
      // interleave consecutive groups (their live ranges overflow the
      // register file: 100 to 1800 spilled registers without it).
#pragma unroll
      for (int rt = 0; rt < kPgemmRT; ++rt)
#pragma unroll
        for (int s = 0; s < kPgemmNT; ++s) asm volatile("" : "+v"(acc[rt][s]));
    } else {
      if constexpr (gh == 0) {
        if (gg == 0 && g > 0) bias_chunk(g / kPgemmChunk - 1);
      }
      const bool take = ((gg >> 1) & 1) == hl;
#pragma unroll
      for (int s = 0; s < kPgemmNT; ++s) {
        if (take && gg < 4) bsel[s][0][gh] = w[s];
        if (take && gg >= 4) bsel[s][1][gh] = w[s];
      }
    }
  };

  // ---- pipeline ------------------------------------------------------------
  // During group g the wave issues the activations of group g + 1 (4 loads)
  // and, when g is even, then the weights of the next pair (6 loads). At the
  // top of group g everything but those weights must have landed: vmcnt(6)
  // after an even group that issued them, vmcnt(0) otherwise; the barrier
  // then makes every wave's stage visible and frees the stages the next DMA
  // overwrites (read during group g - 1).
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
        if (p + 1 < P) dma_wait_barrier<6>();
        else dma_wait_barrier<0>();
        if (g + 2 < G) issue_x(g + 2);
        group(g + 1, std::integral_constant<int, 1>{});
      }
    }
  } else {
    // one group of activations and codes in flight; the scale/bias words of
    // a pair are issued with its first group's codes
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
  dma_wait_barrier<0>();  // the last group's sums from every wave
  if constexpr (BITS != kFmtFp8) bias_chunk((G - 1) / kPgemmChunk);

  // ---- epilogue: element r of tile (rt, s) is row rbase + 32 rt + 8 (r / 4)
  // + 4 hl + r % 4, column jj of the lane's weight slot
  if constexpr (SWIGLU && OUT_BF16) {
    // the workgroup's 128 x 128 bf16 block goes through LDS (the activation
    // stages are free once every wave is past its last group) and out as
    // whole 16-byte pieces of rows, when the output allows 16-byte stores
    if ((((uintptr_t)yv) & 15) == 0 && (ldy & 7) == 0) {
      uint16_t* ob = (uint16_t*)xs;  // [128 rows][128 columns]
      __syncthreads();
#pragma unroll
      for (int rt = 0; rt < kPgemmRT; ++rt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = rbase + rt * 32 + 8 * (r / 4) + 4 * hl + (r % 4);
          ob[row * 128 + 32 * cw + j] = f32_to_bf16_rne(silu_f32(acc[rt][0][r]) * acc[rt][1][r]);
        }
      __syncthreads();
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int idx = (int)threadIdx.x + u * kPgemmThreads;
        const int row = idx >> 4, col = (idx & 15) * 8;  // 8 output columns of one 16-column tile
        if (row >= mt || nb * 8 + (col >> 4) >= ntiles) continue;
        *(u32x4*)((uint16_t*)yv + (int64_t)(m0 + row) * ldy + (int64_t)nb * 128 + col) = *(const u32x4*)(ob + row * 128 + col);
      }
      return;
    }
  }
#pragma unroll
  for (int rt = 0; rt < kPgemmRT; ++rt) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = rbase + rt * 32 + 8 * (r / 4) + 4 * hl + (r % 4);
      if (row >= mt) continue;
      const int64_t yrow = (int64_t)(m0 + row) * ldy;
      if constexpr (SWIGLU) {
        const int t = slot_tile(lslot[0]);
        if (t >= ntiles) continue;
        const float z = silu_f32(acc[rt][0][r]) * acc[rt][1][r];
        const int64_t at = yrow + (int64_t)t * kTileN + jj;
        if constexpr (OUT_BF16) ((uint16_t*)yv)[at] = f32_to_bf16_rne(z);
        else ((float*)yv)[at] = z;
      } else {
#pragma unroll
        for (int s = 0; s < kPgemmNT; ++s) {
          const int t = slot_tile(lslot[s]);
          if (t >= ntiles) continue;
          const int64_t at = yrow + (int64_t)t * kTileN + jj;
          if constexpr (OUT_BF16) ((uint16_t*)yv)[at] = f32_to_bf16_rne(acc[rt][s][r]);
          else ((float*)yv)[at] = acc[rt][s][r];
        }
      }
    }
  }
}

}  // namespace q4
