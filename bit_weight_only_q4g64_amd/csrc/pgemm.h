// Prefill window GEMM (pgemm) on the matrix cores.
//
// A workgroup of 4 waves owns RT*16 window rows and 4 column slots of 16
// columns per wave (plain: 64 columns of one matrix; SwiGLU: the same 32
// columns of w1 and of w3, paired in one wave so the epilogue can form
// silu(a) * c). Weight codes stream in with 128-bit loads (one per lane per
// column tile and pair of groups), are turned into exact bf16 integers in
// registers once, and are reused for all RT row tiles. Per output the order
// is a single chain over the groups of K:
//
//   acc = 0
//   for g = 0 .. K/64-1:  P = mfma(x[g, 32..63], q, mfma(x[g, 0..31], q, 0))
//                         S = mfma(x[g, 32..63], 1, mfma(x[g, 0..31], 1, 0))
//                         acc = fma(s_g, P, fma(b_g, S, acc))
//
// It depends neither on M, nor on the row's offset in the window, nor on its
// slot, so a row's bits are the same for every cut of the prompt (TensorFold
// PR #1696, later revision, "What it adds", prompt GEMM item).
#pragma once

#include "common.h"

namespace q4 {

constexpr int kPgemmWaves = 4;

template <bool SWIGLU, bool OUT_BF16, int RT>
__global__ __launch_bounds__(256) void pgemm_kernel(const uint8_t* __restrict__ pa, const uint8_t* __restrict__ pb, int N,
                                                  int K, const uint16_t* __restrict__ x, int64_t ldx, int M,
                                                  void* __restrict__ yv, int64_t ldy) {
  constexpr int kColsPerWave = SWIGLU ? 32 : 64;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int i = lane & 15, kc = lane >> 4;
  const int n0 = (blockIdx.x * kPgemmWaves + wave) * kColsPerWave;
  if (n0 >= N) return;
  const int m0 = blockIdx.y * RT * 16;
  const int G = K / kGroup;
  const int64_t P = (G + 1) / 2;
  const int64_t cb = codes_bytes(N, K);
  const bf16x8 ones = ones_bf16x8();

  const uint8_t* spk[4];
  int64_t stile[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    if constexpr (SWIGLU) {
      spk[s] = s < 2 ? pa : pb;
      stile[s] = n0 / kTileN + (s & 1);
    } else {
      spk[s] = pa;
      stile[s] = n0 / kTileN + s;
    }
  }

  f32x4 acc[RT][4];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int s = 0; s < 4; ++s) acc[rt][s] = f32x4{0.f, 0.f, 0.f, 0.f};

  bool row_ok[RT];
  const uint16_t* xrow[RT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int row = m0 + rt * 16 + i;
    row_ok[rt] = row < M;
    xrow[rt] = x + (int64_t)(row_ok[rt] ? row : 0) * ldx + kc * 8;
  }

  u32x4 cw[4];
  u32x2 sbw[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    cw[s] = *(const u32x4*)(spk[s] + (stile[s] * P) * kPairCodeBytes + lane * 16);
    sbw[s] = *(const u32x2*)(spk[s] + cb + (stile[s] * P) * kPairSbBytes + i * 8);
  }

  for (int64_t p = 0; p < P; ++p) {
    // prefetch the next pair's codes and scale/bias while this pair computes
    u32x4 cwn[4];
    u32x2 sbn[4];
    const int64_t pn = p + 1 < P ? p + 1 : p;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      cwn[s] = *(const u32x4*)(spk[s] + (stile[s] * P + pn) * kPairCodeBytes + lane * 16);
      sbn[s] = *(const u32x2*)(spk[s] + cb + (stile[s] * P + pn) * kPairSbBytes + i * 8);
    }
#pragma unroll
    for (int gh = 0; gh < 2; ++gh) {
      const int g = (int)(2 * p + gh);
      if (g >= G) break;
      bf16x8 q[4][2];
      float sc[4], bs[4];
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        q[s][0] = codes_to_bf16(gh ? cw[s][2] : cw[s][0]);
        q[s][1] = codes_to_bf16(gh ? cw[s][3] : cw[s][1]);
        const uint32_t w = gh ? sbw[s][1] : sbw[s][0];
        sc[s] = bf16_lo(w);
        bs[s] = bf16_hi(w);
      }
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        bf16x8 xa0 = zero_bf16x8(), xa1 = zero_bf16x8();
        if (row_ok[rt]) {
          xa0 = __builtin_bit_cast(bf16x8, *(const u32x4*)(xrow[rt] + (int64_t)g * kGroup));
          xa1 = __builtin_bit_cast(bf16x8, *(const u32x4*)(xrow[rt] + (int64_t)g * kGroup + 32));
        }
        f32x4 S = mfma16(xa0, ones, f32x4{0.f, 0.f, 0.f, 0.f});
        S = mfma16(xa1, ones, S);
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          f32x4 Pm = mfma16(xa0, q[s][0], f32x4{0.f, 0.f, 0.f, 0.f});
          Pm = mfma16(xa1, q[s][1], Pm);
#pragma unroll
          for (int v = 0; v < 4; ++v) acc[rt][s][v] = __builtin_fmaf(sc[s], Pm[v], __builtin_fmaf(bs[s], S[v], acc[rt][s][v]));
        }
      }
    }
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      cw[s] = cwn[s];
      sbw[s] = sbn[s];
    }
  }

  // Epilogue: lane holds rows m0 + rt*16 + 4*kc + v of column i of each slot.
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int row = m0 + rt * 16 + 4 * kc + v;
      if (row >= M) continue;
      if constexpr (SWIGLU) {
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          const float z = silu_f32(acc[rt][s][v]) * acc[rt][s + 2][v];
          const int64_t at = (int64_t)row * ldy + n0 + s * kTileN + i;
          if constexpr (OUT_BF16) ((uint16_t*)yv)[at] = f32_to_bf16_rne(z);
          else ((float*)yv)[at] = z;
        }
      } else {
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const int64_t at = (int64_t)row * ldy + n0 + s * kTileN + i;
          if constexpr (OUT_BF16) ((uint16_t*)yv)[at] = f32_to_bf16_rne(acc[rt][s][v]);
          else ((float*)yv)[at] = acc[rt][s][v];
        }
      }
    }
  }
}

}  // namespace q4
