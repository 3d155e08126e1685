// Decode matvecs over 1..16 activation rows (qmv) on the matrix cores.
//
// One workgroup owns one 16-column tile of the weight matrix (or the same
// tile of w1 and w3 for the fused SwiGLU variant) and all of K. Its waves
// split K into segments of kSegGroups groups (a fixed function of K): each
// wave streams its segment's codes with 128-bit loads, turns them into exact
// bf16 integers in registers, and reduces them with v_mfma_f32_16x16x32_bf16
// against the activation rows, which fill the 16 row slots (unused slots are
// zero). Per output the order is:
//
//   for each segment s (ascending):   part_s = 0
//     for each group g in s:           P = mfma(x[g, 32..63], q, mfma(x[g, 0..31], q, 0))
//                                      S = mfma(x[g, 32..63], 1, mfma(x[g, 0..31], 1, 0))
//                                      part_s = fma(s_g, P, fma(b_g, S, part_s))
//   y = ((part_0 + part_1) + part_2) + ...
//
// Nothing in it depends on R, on the slot a row occupies or on the launch
// shape, so every row is bit-equal to its one-row result (TensorFold PR #1696,
// later revision, "What it adds": rows that share a decode step are summed as
// the one-row kernels sum them).
#pragma once

#include "common.h"

namespace q4 {

constexpr int kSegGroups = 4;                 // groups per k segment (256 k)
constexpr int kSegPairs = kSegGroups / 2;
// Waves per workgroup: 16 for bf16 activations; 8 for float32 activations,
// whose three-piece split needs more registers per wave.
template <int XF32>
struct QmvLimits {
  static constexpr int kMaxWaves = XF32 ? 8 : 16;
};

__host__ __device__ inline int qmv_segments(int64_t K) { return (int)((K / kGroup + kSegGroups - 1) / kSegGroups); }

// Activation fragment of row i (lane & 15), k = k0 + 8*(lane >> 4) .. +7 as
// bf16 pieces. bf16 input: one piece. float32 input: three exact pieces.
template <int XF32>
struct XFrag {
  static constexpr int kPieces = XF32 ? 3 : 1;
  bf16x8 p[kPieces];
};

template <int XF32>
__device__ __forceinline__ XFrag<XF32> load_xfrag(const void* __restrict__ xv, int64_t ldx, int row, bool ok, int64_t k0,
                                                   int kc) {
  XFrag<XF32> f;
  if constexpr (!XF32) {
    if (ok) {
      const uint16_t* p = (const uint16_t*)xv + (int64_t)row * ldx + k0 + kc * 8;
      f.p[0] = __builtin_bit_cast(bf16x8, *(const u32x4*)p);
    } else {
      f.p[0] = zero_bf16x8();
    }
  } else {
    if (ok) {
      const float* p = (const float*)xv + (int64_t)row * ldx + k0 + kc * 8;
      const f32x4 a = *(const f32x4*)p;
      const f32x4 b = *(const f32x4*)(p + 4);
      const float v[8] = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
      uint32_t h[8], m[8], l[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) split3(v[e], h[e], m[e], l[e]);
      u32x4 H, Mi, L;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        H[j] = h[2 * j] | (h[2 * j + 1] << 16);
        Mi[j] = m[2 * j] | (m[2 * j + 1] << 16);
        L[j] = l[2 * j] | (l[2 * j + 1] << 16);
      }
      f.p[0] = __builtin_bit_cast(bf16x8, H);
      f.p[1] = __builtin_bit_cast(bf16x8, Mi);
      f.p[2] = __builtin_bit_cast(bf16x8, L);
    } else {
      f.p[0] = f.p[1] = f.p[2] = zero_bf16x8();
    }
  }
  return f;
}

// NMAT = 1: y = W x (float32 out). NMAT = 2: y = silu(W1 x) * (W3 x).
template <int XF32, int NMAT>
__global__ __launch_bounds__(QmvLimits<XF32>::kMaxWaves * 64) void qmv_kernel(const uint8_t* __restrict__ pk0, const uint8_t* __restrict__ pk1,
                                                 int N, int K, const void* __restrict__ xv, int64_t ldx, int R,
                                                 float* __restrict__ y, int64_t ldy) {
  extern __shared__ f32x4 part[];  // [segment][matrix][lane]
  const int64_t t = blockIdx.x;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nwaves = blockDim.x >> 6;
  const int i = lane & 15, kc = lane >> 4;
  const int G = K / kGroup;
  const int64_t P = (G + 1) / 2;
  const int nseg = qmv_segments(K);
  const int64_t cb = codes_bytes(N, K);
  const bf16x8 ones = ones_bf16x8();
  const bool row_ok = i < R;
  const uint8_t* pks[2] = {pk0, pk1};

  for (int seg = wave; seg < nseg; seg += nwaves) {
    const int g0 = seg * kSegGroups;
    // Issue every load of the segment first: codes, scale/bias, activations.
    u32x4 cw[NMAT][kSegPairs];
    u32x2 sbw[NMAT][kSegPairs];
#pragma unroll
    for (int m = 0; m < NMAT; ++m) {
#pragma unroll
      for (int pp = 0; pp < kSegPairs; ++pp) {
        const int64_t p = g0 / 2 + pp;
        if (p < P) {
          cw[m][pp] = __builtin_nontemporal_load((const u32x4*)(pks[m] + (t * P + p) * kPairCodeBytes + lane * 16));
          sbw[m][pp] = *(const u32x2*)(pks[m] + cb + (t * P + p) * kPairSbBytes + i * 8);
        } else {
          cw[m][pp] = u32x4{0u, 0u, 0u, 0u};
          sbw[m][pp] = u32x2{0u, 0u};
        }
      }
    }
    XFrag<XF32> xf[kSegGroups][2];
#pragma unroll
    for (int gg = 0; gg < kSegGroups; ++gg) {
      const int g = g0 + gg;
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) xf[gg][hh] = load_xfrag<XF32>(xv, ldx, i, row_ok && g < G, (int64_t)g * kGroup + hh * 32, kc);
    }

    f32x4 acc[NMAT];
#pragma unroll
    for (int m = 0; m < NMAT; ++m) acc[m] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int gg = 0; gg < kSegGroups; ++gg) {
      const int g = g0 + gg;
      if (g >= G) break;
      const int pp = gg >> 1, gh = gg & 1;
      f32x4 S = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int pc = 0; pc < XFrag<XF32>::kPieces; ++pc) {
        S = mfma16(xf[gg][0].p[pc], ones, S);
        S = mfma16(xf[gg][1].p[pc], ones, S);
      }
#pragma unroll
      for (int m = 0; m < NMAT; ++m) {
        const bf16x8 q0 = codes_to_bf16(gh ? cw[m][pp][2] : cw[m][pp][0]);
        const bf16x8 q1 = codes_to_bf16(gh ? cw[m][pp][3] : cw[m][pp][1]);
        f32x4 Pm = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int pc = 0; pc < XFrag<XF32>::kPieces; ++pc) {
          Pm = mfma16(xf[gg][0].p[pc], q0, Pm);
          Pm = mfma16(xf[gg][1].p[pc], q1, Pm);
        }
        const uint32_t sbword = gh ? sbw[m][pp][1] : sbw[m][pp][0];
        const float s = bf16_lo(sbword), b = bf16_hi(sbword);
#pragma unroll
        for (int v = 0; v < 4; ++v) acc[m][v] = __builtin_fmaf(s, Pm[v], __builtin_fmaf(b, S[v], acc[m][v]));
      }
    }
#pragma unroll
    for (int m = 0; m < NMAT; ++m) part[(seg * NMAT + m) * 64 + lane] = acc[m];
  }
  __syncthreads();
  if (wave != 0) return;
  f32x4 tot[NMAT];
#pragma unroll
  for (int m = 0; m < NMAT; ++m) tot[m] = part[m * 64 + lane];
  for (int seg = 1; seg < nseg; ++seg) {
#pragma unroll
    for (int m = 0; m < NMAT; ++m) {
      const f32x4 ps = part[(seg * NMAT + m) * 64 + lane];
#pragma unroll
      for (int v = 0; v < 4; ++v) tot[m][v] = tot[m][v] + ps[v];
    }
  }
  const int64_t n = t * kTileN + i;
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const int r = 4 * kc + v;
    if (r < R) {
      float out;
      if constexpr (NMAT == 1) {
        out = tot[0][v];
      } else {
        out = silu_f32(tot[0][v]) * tot[1][v];
      }
      y[(int64_t)r * ldy + n] = out;
    }
  }
}

}  // namespace q4
