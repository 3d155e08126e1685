// Decode FFN step in one launch: z = silu(W1 x) * (W3 x), then y = W2 z.
//
// It computes exactly what qmv_w13_swiglu followed by qmv_rows (float32 x)
// compute, with the same per-tile arithmetic (qmv_fold_segment and
// qmv_ordered_sum) and the same exact three-piece split of z, so z and y are
// bit-identical to the two calls (TensorFold PR #1696, "What it adds":
// w1 + w3 + SwiGLU in one pass; PR #1514, "What changes": the fusion keeps
// every rounding boundary). What changes is the schedule:
//
//   * one persistent workgroup per CU (16 waves);
//   * at the start each workgroup issues the loads of its w1/w3 tiles AND of
//     its first w2 work item, so the whole step's weights stream from HBM
//     together instead of w2 waiting for a second launch;
//   * phase 1: w1/w3 tiles two at a time (8 waves each); z is written with
//     device-scope (write-through) stores;
//   * a grid barrier: workgroups arrive at one of 16 counters (each on its
//     own 128-byte line), the last of each counter at a top counter, the last
//     of all bumps a generation word; one release and one acquire per
//     workgroup; the wait polls with relaxed loads and gives up after a
//     bounded time, recording an error, so every wave finishes;
//   * phase 2: z staged in LDS as its three bf16 planes (the staging
//     qmv_rows does), w2 over 8-column half-tiles (two per 16-column tile) so
//     a 2048-row w2 still covers every CU; the lanes of the other half load
//     nothing and store nothing.
#pragma once

#include "common.h"
#include "qmv.h"

namespace q4 {

constexpr int kFfnWaves = 16;
constexpr int kFfnThreads = kFfnWaves * 64;
constexpr int kFfnP1Waves = 8;               // waves per w1/w3 tile in phase 1
constexpr int kFfnGroups = 16;               // first-level barrier counters
constexpr int kFfnLine = 128;                // bytes between barrier words
constexpr uint64_t kFfnSpinTicks = 2000000;  // barrier give-up: 20 ms of the 100 MHz real-time clock

// Workspace: the barrier state only. Byte offsets: counter c at c * 128
// (c < 16), the top counter at 16 * 128, the generation at 17 * 128, the
// error word at 18 * 128.
constexpr size_t kFfnWorkBytes = 4096;
constexpr size_t kFfnTopOff = kFfnGroups * kFfnLine;
constexpr size_t kFfnGenOff = (kFfnGroups + 1) * kFfnLine;
constexpr size_t kFfnErrOff = (kFfnGroups + 2) * kFfnLine;
static_assert(kFfnErrOff + 4 <= kFfnWorkBytes, "barrier words fit the workspace");

__device__ __forceinline__ uint32_t* ffn_word(uint8_t* work, size_t off) { return (uint32_t*)(work + off); }

// Grid barrier over nwg co-resident workgroups. g0 is the generation thread
// 0 read at kernel start: it cannot change before this
// workgroup arrives, because the barrier needs every arrival. Returns false
// if this workgroup gave up waiting (then the error word is set, the
// counters are left mid-count and the results are invalid).
__device__ __forceinline__ bool ffn_grid_barrier(uint8_t* work, int b, int nwg, uint32_t g0, uint32_t* flag) {
  __syncthreads();  // every wave's stores of this workgroup are done
  if (threadIdx.x == 0) {
    uint32_t ok = 1;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    const int c = b % kFfnGroups;
    const uint32_t nc = (uint32_t)((nwg - c + kFfnGroups - 1) / kFfnGroups);  // workgroups on counter c
    const uint32_t ncount = (uint32_t)(nwg < kFfnGroups ? nwg : kFfnGroups);   // counters in use
    uint32_t* cnt = ffn_word(work, (size_t)c * kFfnLine);
    uint32_t* top = ffn_word(work, kFfnTopOff);
    uint32_t* gen = ffn_word(work, kFfnGenOff);
    bool last = false;
    if (__hip_atomic_fetch_add(cnt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == nc - 1) {
      __hip_atomic_store(cnt, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (__hip_atomic_fetch_add(top, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == ncount - 1) {
        __hip_atomic_store(top, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_fetch_add(gen, 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
        last = true;
      }
    }
    if (!last) {
      const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
      while (__hip_atomic_load(gen, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == g0) {
        if (__builtin_amdgcn_s_memrealtime() - t0 > kFfnSpinTicks) {
          ok = 0;
          __hip_atomic_store(ffn_word(work, kFfnErrOff), 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          break;
        }
        __builtin_amdgcn_s_sleep(2);
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    *flag = ok;
  }
  __syncthreads();
  return *flag != 0;
}

// LDS of the fused kernel (bytes): phase 1 stages x and holds the partials of
// two tiles; phase 2 reuses the space for its partials and, when xl2, z's
// three bf16 planes ([3][R][K2 + 8], the layout qmv_rows stages).
__host__ __device__ inline int ffn_rtf(int R) { return (R + 3) / 4 <= 1 ? 1 : ((R + 3) / 4 <= 2 ? 2 : 4); }
__host__ __device__ inline size_t ffn_part2_bytes(int64_t K2, int R) {
  return (size_t)qmv_segments(K2) * ffn_rtf(R) * 64 * sizeof(float);
}
__host__ __device__ inline size_t ffn_lds_bytes(int64_t K1, int64_t K2, int R, bool xl2) {
  const int nv = qmv_nv(R);
  const size_t p1 = 2 * (size_t)qmv_segments(K1) * 2 * nv * 64 * sizeof(float) + (size_t)R * qmv_xs_stride(K1) * 2;
  const size_t p2 = ffn_part2_bytes(K2, R) + (xl2 ? (size_t)3 * R * qmv_xs_stride(K2) * 2 : 0);
  return (p1 > p2 ? p1 : p2) + 16;
}

// NV: row slots per lane group of phase 1 (as qmv_w13_swiglu); RTF: row tiles
// of phase 2 (as qmv_rows with float32 x); SPW1 / SPW2: segments per wave.
// xl2: z fits in LDS as three bf16 planes (else fragments are read from z
// and split in registers, as qmv_rows does when its staging does not fit).
template <int NV, int RTF, int SPW1, int SPW2>
__global__ __launch_bounds__(kFfnThreads) void ffn_kernel(const uint8_t* __restrict__ p1, const uint8_t* __restrict__ p3,
                                                        const uint8_t* __restrict__ p2, int N1, int K1, int N2,
                                                        const uint16_t* __restrict__ x, int64_t ldx, int R,
                                                        float* __restrict__ z, int64_t ldz, float* __restrict__ y, int64_t ldy,
                                                        uint8_t* __restrict__ work, int xl2) {
  extern __shared__ __align__(16) uint8_t smem[];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int i = lane & 15, kc = lane >> 4;
  const int nwg = gridDim.x, b = blockIdx.x;
  const int K2 = N1;
  const int G1 = K1 / kGroup, P1 = (G1 + 1) / 2, nseg1 = qmv_segments(K1);
  const int G2 = K2 / kGroup, P2 = (G2 + 1) / 2, nseg2 = qmv_segments(K2);
  const int64_t cb1 = codes_bytes(N1, K1), cb2 = codes_bytes(N2, K2);
  const int T1 = N1 / kTileN, pairs1 = (T1 + 1) / 2;
  const int items2 = 2 * (N2 / kTileN);
  // the barrier generation of this call (only thread 0 uses it). Relaxed:
  // the previous call's last update precedes this launch, and a relaxed load
  // does not hold back the weight loads issued after it.
  uint32_t g0 = 0;
  if (threadIdx.x == 0) g0 = __hip_atomic_load(ffn_word(work, kFfnGenOff), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);

  // ---- phase 1 set-up: x staged in LDS, the first tile pair's weights -----
  const int grp = wave / kFfnP1Waves, wg = wave % kFfnP1Waves;
  const int xsi = (int)qmv_xs_stride(K1);
  const size_t part1_bytes = (size_t)nseg1 * 2 * NV * 64 * sizeof(float);
  float* part1 = (float*)(smem + grp * part1_bytes);
  uint16_t* xs = (uint16_t*)(smem + 2 * part1_bytes);
  uint32_t* flag = (uint32_t*)(smem + ffn_lds_bytes(K1, K2, R, xl2 != 0) - 16);
  const rsrc_t xres = make_rsrc(x, (uint32_t)(R * ldx * 2));
  const int per_row = K1 / 8;  // 16-byte chunks of one bf16 row
  constexpr int kBatch = 4;
  const int jmax = (per_row + kFfnThreads - 1) / kFfnThreads;
  auto xload = [&](int r, int j) -> u32x4 {
    int c = (int)threadIdx.x + j * kFfnThreads;
    c = c < per_row ? c : per_row - 1;
    return buf_load16(xres, (uint32_t)c * 16u, (uint32_t)(r * ldx * 2));
  };
  auto xput = [&](int r, int j, const u32x4& v) {
    const int c = (int)threadIdx.x + j * kFfnThreads;
    if (c < per_row) *(u32x4*)(xs + r * xsi + c * 8) = v;
  };
  u32x4 xv0[kBatch];
  {
    int r = 0, j = 0;
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      if (r >= R) break;
      xv0[u] = xload(r, j);
      if (++j == jmax) { j = 0; ++r; }
    }
  }
  auto tile_rsrc = [&](const uint8_t* pk, int64_t cb, int t, int P, rsrc_t& cr, rsrc_t& sr) {
    cr = make_rsrc(pk + (int64_t)t * P * kPairCodeBytes, (uint32_t)P * kPairCodeBytes);
    sr = make_rsrc(pk + cb + (int64_t)t * P * kPairSbBytes, (uint32_t)P * kPairSbBytes);
  };
  // w1/w3 tile of this wave's group for tile pair pr (clamped to the last tile)
  auto p1_rsrc = [&](int pr, rsrc_t (&cr)[2], rsrc_t (&sr)[2]) {
    int t = 2 * pr + grp;
    t = t < T1 ? t : T1 - 1;
    tile_rsrc(p1, cb1, t, P1, cr[0], sr[0]);
    tile_rsrc(p3, cb1, t, P1, cr[1], sr[1]);
  };
  // (issued on every path, with a workgroup past the last tile loading
  // nothing, so that staging x below waits for x alone)
  QmvWeights<2, SPW1> w13;
  {
    rsrc_t cr[2], sr[2];
    p1_rsrc(b < pairs1 ? b : pairs1 - 1, cr, sr);
    qmv_issue_weights<2, SPW1>(w13, cr, sr, wg, kFfnP1Waves, P1, lane, b < pairs1);
  }
  // the first w2 item: tile it / 2, columns 8 (it % 2) .. + 7 of that tile
  auto p2_rsrc = [&](int it, rsrc_t (&cr)[1], rsrc_t (&sr)[1]) { tile_rsrc(p2, cb2, it / 2, P2, cr[0], sr[0]); };
  QmvWeights<1, SPW2> w2w;
  {
    rsrc_t cr[1], sr[1];
    p2_rsrc(b < items2 ? b : items2 - 1, cr, sr);
    qmv_issue_weights<1, SPW2>(w2w, cr, sr, wave, kFfnWaves, P2, lane, b < items2 && (i >> 3) == (b & 1));
  }
  {
    int r = 0, j = 0;
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      if (r >= R) break;
      xput(r, j, xv0[u]);
      if (++j == jmax) { j = 0; ++r; }
    }
    while (r < R) {
      const u32x4 v = xload(r, j);
      xput(r, j, v);
      if (++j == jmax) { j = 0; ++r; }
    }
  }
  __syncthreads();

  // ---- phase 1: w1/w3 + SwiGLU, two tiles per pass --------------------------
  const int frow = i < R ? i : R - 1;
  auto xfrag1 = [&](int, int g, int hh) -> bf16x8 {
    return __builtin_bit_cast(bf16x8, *(const u32x4*)(xs + frow * xsi + g * kGroup + hh * 32 + kc * 8));
  };
  const rsrc_t zres = make_rsrc(z, (uint32_t)(R * ldz * 4));
  for (int pr = b; pr < pairs1; pr += nwg) {
    if (pr != b) {
      rsrc_t cr[2], sr[2];
      p1_rsrc(pr, cr, sr);
      qmv_issue_weights<2, SPW1>(w13, cr, sr, wg, kFfnP1Waves, P1, lane, true);
    }
#pragma unroll
    for (int j = 0; j < SPW1; ++j) {
      const int seg = wg + j * kFfnP1Waves;
      if (seg >= nseg1) break;
      float acc[2][1][NV];
      qmv_fold_segment<0, 2, 1, NV>(acc, w13.cw[j], w13.sbw[j], seg * kSegGroups, G1, xfrag1);
#pragma unroll
      for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int v = 0; v < NV; ++v) part1[qmv_part_index<2, 1, NV>(seg, m, 0, v, lane)] = acc[m][0][v];
    }
    __syncthreads();
    const int t = 2 * pr + grp;
    if (wg == 0 && t < T1) {
      float tot[2][1][NV];
      qmv_ordered_sum<2, 1, NV>(tot, part1, nseg1, lane);
      const int n = t * kTileN + i;
#pragma unroll
      for (int v = 0; v < NV; ++v) {
        const int r = 4 * kc + v;
        if (r >= R) continue;
        const float zz = silu_f32(tot[0][0][v]) * tot[1][0][v];
        // device scope (sc1): written through the XCD's L2
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(zz), zres, (int)((r * ldz + n) * 4), 0, 16);
      }
    }
    __syncthreads();  // the partials are reused by the next pass
  }

  // ---- grid barrier: every row of z written and visible --------------------
  if (!ffn_grid_barrier(work, b, nwg, g0, flag)) return;

  // ---- phase 2: w2 on the three bf16 pieces of z, half-tiles ---------------
  float* part2 = (float*)smem;
  const uint32_t zrow = (uint32_t)(ldz * 4);
  // one phase-2 work item with fragment source xf: compute, reduce, store
  auto item = [&](int it, const auto& xf) {
    const bool on = (i >> 3) == (it & 1);
    if (it != b) {
      rsrc_t cr[1], sr[1];
      p2_rsrc(it, cr, sr);
      qmv_issue_weights<1, SPW2>(w2w, cr, sr, wave, kFfnWaves, P2, lane, on);
    }
#pragma unroll
    for (int j = 0; j < SPW2; ++j) {
      const int seg = wave + j * kFfnWaves;
      if (seg >= nseg2) break;
      float acc[1][RTF][1];
      qmv_fold_segment<1, 1, RTF, 1>(acc, w2w.cw[j], w2w.sbw[j], seg * kSegGroups, G2, xf);
#pragma unroll
      for (int rt = 0; rt < RTF; ++rt) part2[qmv_part_index<1, RTF, 1>(seg, 0, rt, 0, lane)] = acc[0][rt][0];
    }
    __syncthreads();
    if (wave == 0) {
      float tot[1][RTF][1];
      qmv_ordered_sum<1, RTF, 1>(tot, part2, nseg2, lane);
      const int n = (it / 2) * kTileN + i;
#pragma unroll
      for (int rt = 0; rt < RTF; ++rt) {
        const int r = rt * 4 + kc;
        if (on && r < R) y[(int64_t)r * ldy + n] = tot[0][rt][0];
      }
    }
    __syncthreads();
  };
  if (xl2) {
    // z into LDS as three exact bf16 planes h, m, l of [R][K2 + 8] (the
    // staging qmv_rows does for a float32 input), loads four deep per thread
    uint16_t* xs2 = (uint16_t*)(smem + ffn_part2_bytes(K2, R));
    const int xsi2 = (int)qmv_xs_stride(K2), plane = R * xsi2;
    const uint32_t per_zrow = (uint32_t)K2 / 4, total = (uint32_t)R * per_zrow;  // 16-byte chunks of z
    for (uint32_t c0 = threadIdx.x; c0 < total; c0 += 4 * kFfnThreads) {
      u32x4 v[4];
#pragma unroll
      for (uint32_t u = 0; u < 4; ++u) {
        uint32_t c = c0 + u * kFfnThreads;
        c = c < total ? c : total - 1;
        v[u] = buf_load16(zres, (c / per_zrow) * zrow + (c % per_zrow) * 16u, 0u);
      }
#pragma unroll
      for (uint32_t u = 0; u < 4; ++u) {
        const uint32_t c = c0 + u * kFfnThreads;
        if (c >= total) continue;
        uint32_t h[4], m[4], l[4];
#pragma unroll
        for (int w = 0; w < 4; ++w) split3(__uint_as_float(v[u][w]), h[w], m[w], l[w]);
        uint16_t* d = xs2 + (c / per_zrow) * xsi2 + (c % per_zrow) * 4;
        *(u32x2*)d = u32x2{h[0] | (h[1] << 16), h[2] | (h[3] << 16)};
        *(u32x2*)(d + plane) = u32x2{m[0] | (m[1] << 16), m[2] | (m[3] << 16)};
        *(u32x2*)(d + 2 * plane) = u32x2{l[0] | (l[1] << 16), l[2] | (l[3] << 16)};
      }
    }
    __syncthreads();
    auto xf = [&](int rt, int g, int hh) -> bf16x8 {
      const int k0 = g * kGroup + hh * 32 + kc * 8;
      int row = rt * 4 + (i >> 2);
      row = row < R ? row : R - 1;
      int piece = i & 3;
      piece = piece < 3 ? piece : 2;
      return __builtin_bit_cast(bf16x8, *(const u32x4*)(xs2 + (piece * R + row) * xsi2 + k0));
    };
    for (int it = b; it < items2; it += nwg) item(it, xf);
  } else {
    // fragments straight from z, split in registers (as qmv_rows does when
    // its input does not fit in LDS)
    auto xf = [&](int rt, int g, int hh) -> bf16x8 {
      const int k0 = g * kGroup + hh * 32 + kc * 8;
      int row = rt * 4 + (i >> 2);
      row = row < R ? row : R - 1;
      int piece = i & 3;
      piece = piece < 3 ? piece : 2;
      const u32x4 a = buf_load16(zres, (uint32_t)row * zrow + (uint32_t)k0 * 4u, 0u);
      const u32x4 c = buf_load16(zres, (uint32_t)row * zrow + (uint32_t)k0 * 4u + 16u, 0u);
      uint32_t o[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        uint32_t h, m, l;
        split3(__uint_as_float(e < 4 ? a[e] : c[e - 4]), h, m, l);
        o[e] = piece == 0 ? h : (piece == 1 ? m : l);
      }
      return __builtin_bit_cast(bf16x8, u32x4{o[0] | (o[1] << 16), o[2] | (o[3] << 16), o[4] | (o[5] << 16), o[6] | (o[7] << 16)});
    };
    for (int it = b; it < items2; it += nwg) item(it, xf);
  }
}

}  // namespace q4
