// Prefill window GEMM (pgemm) on the matrix cores.
//
// A workgroup of 4 waves owns 64 window rows and 4 x 64 output columns
// (SwiGLU: 4 x 32 columns, each wave holding the same 32 columns of w1 and of
// w3). Per 64-wide k group it stages the 128 x 64 activation tile in LDS
// (double buffered, one barrier per group); each wave streams the codes of
// its four 16-column tiles with 128-bit loads, turns them into exact bf16
// integers once, and reuses them for its four 16-row tiles.
//
// Per output (r, n) the order is, with chunks of 8 consecutive groups:
//
//   acc = 0, Yb = 0
//   for each chunk (ascending):
//     for each group g of the chunk (ascending):
//       P_g = mfma(x[g, 32..63], q, mfma(x[g, 0..31], q, 0))     exact products
//       acc = fma(s_g, P_g, acc)                                  one VALU op per output
//       S_g = sum of x[g, :] on the matrix cores (A = ones)
//     Yb = mfma(A = exact bf16 pieces h, m, l of S_g for the chunk's groups,
//               B = b_g repeated over the pieces, C = Yb)          the bias term
//   y = acc + Yb
//
// Nothing in it depends on M, on the row's offset in the window or on the
// other rows, so a row's bits are the same for every cut of the prompt
// (TensorFold PR #1696, later revision, "What it adds", prompt GEMM item: a
// chain per 64-wide k block, blocks added in order; "Checks": every row alone
// equals the row inside a window).
#pragma once

#include "common.h"

namespace q4 {

constexpr int kPgemmWaves = 4;
constexpr int kPgemmRT = 4;     // 16-row tiles per wave (all waves share the workgroup's rows)
constexpr int kPgemmNT = 4;     // 16-column tiles per wave
constexpr int kPgemmRows = kPgemmRT * 16;
constexpr int kXsStride = 64;   // bf16 per staged activation row (16-byte chunks XOR-swizzled by row)
constexpr int kPgemmChunk = 8;  // groups per bias chunk

// LDS byte offset of 16-byte chunk c (0..7) of staged row r: chunk slots are
// XOR-swizzled by the row so the 16 rows a fragment read touches spread over
// the banks.
__device__ __forceinline__ int xs_off(int r, int c) { return r * (kXsStride * 2) + ((c ^ (r & 7)) << 4); }

template <bool SWIGLU, bool OUT_BF16>
__global__ __launch_bounds__(kPgemmWaves * 64, 1) void pgemm_kernel(const uint8_t* __restrict__ pa, const uint8_t* __restrict__ pb,
                                                                 int N, int K, const uint16_t* __restrict__ x, int64_t ldx, int M,
                                                                 void* __restrict__ yv, int64_t ldy) {
  constexpr int kColsPerWave = SWIGLU ? 32 : 64;
  __shared__ __align__(16) uint8_t xs[2][kPgemmRows * kXsStride * 2];  // two activation tiles
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int i = lane & 15, kc = lane >> 4;
  const int n0 = (blockIdx.x * kPgemmWaves + wave) * kColsPerWave;
  const bool active = n0 < N;  // inactive waves still stage activations and meet barriers
  const int m0 = blockIdx.y * kPgemmRows;
  const int G = K / kGroup;
  const int P = (G + 1) / 2;
  const int64_t cb = codes_bytes(N, K);
  const bf16x8 ones = ones_bf16x8();

  // weight resources of this wave's four column tiles
  rsrc_t cres[kPgemmNT], sres[kPgemmNT];
#pragma unroll
  for (int s = 0; s < kPgemmNT; ++s) {
    const uint8_t* pk = (SWIGLU && s >= 2) ? pb : pa;
    int tile = SWIGLU ? n0 / kTileN + (s & 1) : n0 / kTileN + s;
    tile = active ? tile : 0;
    cres[s] = make_rsrc(pk + (int64_t)tile * P * kPairCodeBytes, (uint32_t)P * kPairCodeBytes);
    sres[s] = make_rsrc(pk + cb + (int64_t)tile * P * kPairSbBytes, (uint32_t)P * kPairSbBytes);
  }
  // activation tile staging: thread t loads 16-byte chunk t & 7 of rows
  // (t >> 3) + 32 * u, u < kStageRows (rows past M read row M - 1; their
  // results are never stored)
  constexpr int kStageRows = kPgemmRows / (kPgemmWaves * 64 / 8);
  static_assert(kStageRows * kPgemmWaves * 64 / 8 == kPgemmRows, "staging covers the tile exactly");
  const int sc = threadIdx.x & 7, sr = threadIdx.x >> 3;
  const rsrc_t xres = make_rsrc(x + (int64_t)m0 * ldx, (uint32_t)((int64_t)(M - m0 < kPgemmRows ? M - m0 : kPgemmRows) * ldx * 2));
  int srow[kStageRows];
#pragma unroll
  for (int u = 0; u < kStageRows; ++u) {
    const int r = sr + 32 * u;
    srow[u] = m0 + r < M ? r : M - 1 - m0;
  }
  auto stage_load = [&](int g, u32x4 (&v)[kStageRows]) {
#pragma unroll
    for (int u = 0; u < kStageRows; ++u) v[u] = buf_load16(xres, (uint32_t)(srow[u] * ldx * 2 + sc * 16), (uint32_t)g * kGroup * 2);
  };
  auto stage_store = [&](int buf, const u32x4 (&v)[kStageRows]) {
#pragma unroll
    for (int u = 0; u < kStageRows; ++u) *(u32x4*)(xs[buf] + xs_off(sr + 32 * u, sc)) = v[u];
  };

  f32x4 acc[kPgemmRT][kPgemmNT];
  f32x4 yb[kPgemmRT][kPgemmNT];
#pragma unroll
  for (int rt = 0; rt < kPgemmRT; ++rt)
#pragma unroll
    for (int s = 0; s < kPgemmNT; ++s) {
      acc[rt][s] = f32x4{0.f, 0.f, 0.f, 0.f};
      yb[rt][s] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
  // per chunk: S of groups 2*kc, 2*kc+1 (this lane's bias-operand slots) and
  // the raw scale/bias words of those groups for this lane's column
  float ssel[kPgemmRT][2];
  uint32_t bsel[kPgemmNT][2];

  // prologue: stage group 0, load the codes of pair 0
  {
    u32x4 v[kStageRows];
    stage_load(0, v);
    stage_store(0, v);
  }
  u32x4 cw[kPgemmNT];
  u32x2 sbw[kPgemmNT];
#pragma unroll
  for (int s = 0; s < kPgemmNT; ++s) {
    cw[s] = buf_load16(cres[s], (uint32_t)lane * 16u, 0u);
    sbw[s] = buf_load8(sres[s], (uint32_t)i * 8u, 0u);
  }
  __syncthreads();

  for (int g = 0; g < G; ++g) {
    const int buf = g & 1, gh = g & 1, gg = g % kPgemmChunk;
    if (gg == 0) {
#pragma unroll
      for (int rt = 0; rt < kPgemmRT; ++rt) ssel[rt][0] = ssel[rt][1] = 0.f;
#pragma unroll
      for (int s = 0; s < kPgemmNT; ++s) bsel[s][0] = bsel[s][1] = 0u;
    }
    // next activation tile and (at the start of a pair) the next pair's codes
    u32x4 nv[kStageRows];
    const bool more = g + 1 < G;
    if (more) stage_load(g + 1, nv);
    u32x4 cwn[kPgemmNT];
    u32x2 sbn[kPgemmNT];
    if (gh == 1 && more) {
      const int pn = (g + 1) >> 1;
#pragma unroll
      for (int s = 0; s < kPgemmNT; ++s) {
        cwn[s] = buf_load16(cres[s], (uint32_t)lane * 16u, (uint32_t)pn * kPairCodeBytes);
        sbn[s] = buf_load8(sres[s], (uint32_t)i * 8u, (uint32_t)pn * kPairSbBytes);
      }
    }

    // this group's B fragments, scales; capture the bias words this lane's
    // bias operand holds (groups 2*kc, 2*kc+1 of the chunk)
    bf16x8 q[kPgemmNT][2];
    float sc4[kPgemmNT];
#pragma unroll
    for (int s = 0; s < kPgemmNT; ++s) {
      q[s][0] = codes_to_bf16(gh ? cw[s][2] : cw[s][0]);
      q[s][1] = codes_to_bf16(gh ? cw[s][3] : cw[s][1]);
      const uint32_t w = gh ? sbw[s][1] : sbw[s][0];
      sc4[s] = bf16_lo(w);
      if (kc == (gg >> 1)) bsel[s][gh] = w;
    }

    const uint8_t* xb = xs[buf];
#pragma unroll
    for (int rt = 0; rt < kPgemmRT; ++rt) {
      const int r = rt * 16 + i;
      const bf16x8 xa0 = __builtin_bit_cast(bf16x8, *(const u32x4*)(xb + xs_off(r, kc)));
      const bf16x8 xa1 = __builtin_bit_cast(bf16x8, *(const u32x4*)(xb + xs_off(r, kc + 4)));
      // activation sums of rows rt*16 + (lane & 15), in every slot of the lane
      f32x4 S = mfma16(ones, xa0, f32x4{0.f, 0.f, 0.f, 0.f});
      S = mfma16(ones, xa1, S);
      if (kc == (gg >> 1)) ssel[rt][gh] = S[0];
#pragma unroll
      for (int s = 0; s < kPgemmNT; ++s) {
        f32x4 Pm = mfma16(xa0, q[s][0], f32x4{0.f, 0.f, 0.f, 0.f});
        Pm = mfma16(xa1, q[s][1], Pm);
#pragma unroll
        for (int v = 0; v < 4; ++v) acc[rt][s][v] = __builtin_fmaf(sc4[s], Pm[v], acc[rt][s][v]);
      }
    }

    // end of a chunk (or of K): the bias term of its groups on the matrix cores
    if (gg == kPgemmChunk - 1 || g == G - 1) {
      bf16x8 bfr[kPgemmNT];
#pragma unroll
      for (int s = 0; s < kPgemmNT; ++s) {
        const uint32_t b0 = bsel[s][0] >> 16, b1 = bsel[s][1] >> 16;
        bfr[s] = __builtin_bit_cast(bf16x8, u32x4{b0 | (b0 << 16), b0, b1 | (b1 << 16), b1});
      }
#pragma unroll
      for (int rt = 0; rt < kPgemmRT; ++rt) {
        uint32_t h0, m0p, l0, h1, m1p, l1;
        split3(ssel[rt][0], h0, m0p, l0);
        split3(ssel[rt][1], h1, m1p, l1);
        const bf16x8 afr = __builtin_bit_cast(bf16x8, u32x4{h0 | (m0p << 16), l0, h1 | (m1p << 16), l1});
#pragma unroll
        for (int s = 0; s < kPgemmNT; ++s) yb[rt][s] = mfma16(afr, bfr[s], yb[rt][s]);
      }
    }

    if (more) stage_store(buf ^ 1, nv);
    if (gh == 1 && more) {
#pragma unroll
      for (int s = 0; s < kPgemmNT; ++s) {
        cw[s] = cwn[s];
        sbw[s] = sbn[s];
      }
    }
    __syncthreads();
  }

  if (!active) return;
  // epilogue: lane holds rows m0 + rt*16 + 4*kc + v of column i of each tile
#pragma unroll
  for (int rt = 0; rt < kPgemmRT; ++rt) {
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int row = m0 + rt * 16 + 4 * kc + v;
      if (row >= M) continue;
      if constexpr (SWIGLU) {
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          const float a = acc[rt][s][v] + yb[rt][s][v];
          const float c = acc[rt][s + 2][v] + yb[rt][s + 2][v];
          const float z = silu_f32(a) * c;
          const int64_t at = (int64_t)row * ldy + n0 + s * kTileN + i;
          if constexpr (OUT_BF16) ((uint16_t*)yv)[at] = f32_to_bf16_rne(z);
          else ((float*)yv)[at] = z;
        }
      } else {
#pragma unroll
        for (int s = 0; s < kPgemmNT; ++s) {
          const float o = acc[rt][s][v] + yb[rt][s][v];
          const int64_t at = (int64_t)row * ldy + n0 + s * kTileN + i;
          if constexpr (OUT_BF16) ((uint16_t*)yv)[at] = f32_to_bf16_rne(o);
          else ((float*)yv)[at] = o;
        }
      }
    }
  }
}

}  // namespace q4
