// Decode FFN step in one launch, with data handed between workgroups as it
// becomes ready (no grid-wide wait): z = silu(W1 x) * (W3 x), then y = W2 z,
// for R <= 4 activation rows.
//
// The arithmetic of every output is that of qmv_w13_swiglu followed by
// qmv_rows on the float32 z (TensorFold PR #1696, "What it adds": w1 + w3 +
// SwiGLU in one pass; PR #1514, "What changes": fusions keep every rounding
// boundary), so z and y are bit-identical to the two calls. The schedule:
//
//   * one workgroup per CU (16 waves), all resident at once;
//   * at the start each workgroup requests x and the weights of its w1/w3
//     tile pair; each wave requests its first w2 item's weights after its
//     first w1/w3 folds, so the bytes that z waits for come first;
//   * phase 1 (w1/w3, SwiGLU): each z value goes to the caller's z and, with
//     a tag, to a workspace copy: one 64-bit store of {z bits, tag}, where
//     the tag is this call's number (the workspace's call counter + 1);
//   * phase 2 (w2): an item is one 16-column tile of w2 over one half of K.
//     Wave w of the item takes one 256-wide segment: it polls the tagged z
//     of that segment until every tag is this call's, splits the floats into
//     their three exact bf16 pieces in LDS (qmv_rows' staging) and folds the
//     segment with the decode kernels' own arithmetic;
//   * the item of the lower half adds its segments' partials in ascending
//     order and hands the running sum to the item of the upper half (a tagged
//     64-bit store per lane), which continues the same ascending sum over its
//     own segments: ((p_0 + p_1) + ...) + p_last, the order qmv_rows uses;
//   * each upper-half item, once it has its hand-over, raises the call
//     counter to this call's number (a non-returning atomic maximum). Every
//     workgroup has read the counter by then: each one produces z, and the
//     item and its lower-half partner have consumed every producer's z.
//
// Every wait polls with agent-scope loads and gives up after a bounded time
// (the error word is set and y is left undefined), so every wave finishes.
#pragma once

#include "common.h"
#include "ffn.h"
#include "qmv.h"

namespace q4 {

// Workspace layout (bytes): the error word at kFfnErrOff, then from byte
// 4096 this step's state.
constexpr size_t kFlowEpochOff = 4096;        // call counter
constexpr size_t kFlowZOff = 4096 + 256;      // tagged z: [R][N1] of {bits, tag}
constexpr int kFlowMaxRows = 4;
__host__ __device__ inline size_t flow_hand_off(int64_t N1, int R) { return kFlowZOff + (size_t)R * N1 * 8; }
__host__ __device__ inline size_t flow_work_bytes(int64_t N1, int64_t N2, int R) { return flow_hand_off(N1, R) + (size_t)(N2 / kTileN) * 64 * 8; }

// LDS: phase 1 stages x and holds the partials of two tiles; phase 2 holds
// per-wave z pieces ([3][R][256 + 8] bf16 per wave) and the item's partials.
constexpr int kFlowZsi = 256 + 8;
__host__ __device__ inline size_t flow_lds_bytes(int64_t K1, int R) {
  const int nv = qmv_nv(R);
  const size_t p1 = 2 * (size_t)qmv_segments(K1) * 2 * nv * 64 * sizeof(float) + (size_t)R * qmv_xs_stride(K1) * 2;
  const size_t p2 = (size_t)kFfnWaves * 3 * R * kFlowZsi * 2 + (size_t)kFfnWaves * 64 * sizeof(float);
  return (p1 > p2 ? p1 : p2) + 16;
}

__device__ __forceinline__ uint64_t flow_ld(const uint64_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void flow_st(uint64_t* p, float v, uint32_t tag) {
  __hip_atomic_store(p, ((uint64_t)tag << 32) | __float_as_uint(v), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <int NV, int SPW1>
__global__ __launch_bounds__(kFfnThreads) void ffn_flow_kernel(const uint8_t* __restrict__ p1, const uint8_t* __restrict__ p3,
                                                             const uint8_t* __restrict__ p2, int N1, int K1, int N2,
                                                             const uint16_t* __restrict__ x, int64_t ldx, int R,
                                                             float* __restrict__ z, int64_t ldz, float* __restrict__ y, int64_t ldy,
                                                             uint8_t* __restrict__ work) {
  extern __shared__ __align__(16) uint8_t smem[];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int i = lane & 15, kc = lane >> 4;
  const int nwg = gridDim.x, b = blockIdx.x;
  const int K2 = N1;
  const int G1 = K1 / kGroup, P1 = (G1 + 1) / 2, nseg1 = qmv_segments(K1);
  const int G2 = K2 / kGroup, P2 = (G2 + 1) / 2, nseg2 = qmv_segments(K2);
  const int64_t cb1 = codes_bytes(N1, K1), cb2 = codes_bytes(N2, K2);
  const int T1 = N1 / kTileN, pairs1 = T1 / 2;
  const int T2 = N2 / kTileN, items2 = 2 * T2;
  const int half2 = (nseg2 + 1) / 2;  // segments of the lower half of K2
  uint32_t* epoch = (uint32_t*)(work + kFlowEpochOff);
  uint32_t* err = (uint32_t*)(work + kFfnErrOff);
  uint64_t* zt = (uint64_t*)(work + kFlowZOff);
  uint64_t* hand = (uint64_t*)(work + flow_hand_off(N1, R));

  // ---- start: x, the first tile pair's w1/w3 weights, the first w2 item's ----
  const int grp = wave / kFfnP1Waves, wg = wave % kFfnP1Waves;
  const int xsi = (int)qmv_xs_stride(K1);
  const size_t part1_bytes = (size_t)nseg1 * 2 * NV * 64 * sizeof(float);
  float* part1 = (float*)(smem + grp * part1_bytes);
  uint16_t* xs = (uint16_t*)(smem + 2 * part1_bytes);
  const rsrc_t xres = make_rsrc(x, (uint32_t)(R * ldx * 2));
  const int per_row = K1 / 8;  // 16-byte chunks of one bf16 row
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
  constexpr int kBatch = 4;
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
  auto p1_rsrc = [&](int pr, rsrc_t (&cr)[2], rsrc_t (&sr)[2]) {
    const int t = 2 * pr + grp;
    tile_rsrc(p1, cb1, t, P1, cr[0], sr[0]);
    tile_rsrc(p3, cb1, t, P1, cr[1], sr[1]);
  };
  QmvWeights<2, SPW1> w13;
  {
    rsrc_t cr[2], sr[2];
    p1_rsrc(b < pairs1 ? b : pairs1 - 1, cr, sr);
    qmv_issue_weights<2, SPW1>(w13, cr, sr, wg, kFfnP1Waves, P1, lane, b < pairs1);
  }
  // a w2 item: tile it % T2 over the half it / T2 of K2; wave w folds segment
  // half * half2 + w of it
  auto item_seg = [&](int it) { return (it / T2) * half2 + wave; };
  auto item_seg_end = [&](int it) { return it / T2 == 0 ? half2 : nseg2; };
  QmvWeights<1, 1> w2w;
  auto issue_w2 = [&](int it, bool on) {
    rsrc_t cr[1], sr[1];
    tile_rsrc(p2, cb2, it % T2, P2, cr[0], sr[0]);
    const int seg = item_seg(it);
    qmv_issue_weights<1, 1>(w2w, cr, sr, seg, 1, P2, lane, on && seg < item_seg_end(it));
  };
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
  // this call's number (the previous call advanced the counter before it
  // ended). Requested after x and the w1/w3 weights, which phase 1 waits for
  // anyway, and before the w2 weights, which it does not.
  const uint32_t tag = __hip_atomic_load(epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) + 1u;
  // the first w2 item's weights are requested once this wave's w1/w3 weights
  // have landed (after its first folds): until then x and the w1/w3 weights,
  // which the whole step waits for, have the memory system to themselves

  // ---- phase 1: w1/w3 + SwiGLU, two tiles per pass -------------------------
  const int frow = i < R ? i : R - 1;
  auto xfrag1 = [&](int, int g, int hh) -> bf16x8 {
    return __builtin_bit_cast(bf16x8, *(const u32x4*)(xs + frow * xsi + g * kGroup + hh * 32 + kc * 8));
  };
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
    if (pr == b) issue_w2(b < items2 ? b : items2 - 1, b < items2);
    __syncthreads();
    if (wg == 0) {
      float tot[2][1][NV];
      qmv_ordered_sum<2, 1, NV>(tot, part1, nseg1, lane);
      const int n = (2 * pr + grp) * kTileN + i;
#pragma unroll
      for (int v = 0; v < NV; ++v) {
        const int r = 4 * kc + v;
        if (r >= R) continue;
        const float zz = silu_f32(tot[0][0][v]) * tot[1][0][v];
        z[(int64_t)r * ldz + n] = zz;
        flow_st(zt + (int64_t)r * N1 + n, zz, tag);
      }
    }
    // the partials are reused by the next pass: wait for LDS only, not for
    // the z stores in flight
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  }

  // ---- phase 2: w2 items ---------------------------------------------------
  // The w2 weights are first touched here: without this the compiler moves
  // work on them into phase 1, whose folds would then wait for their loads.
#pragma unroll
  for (int pp = 0; pp < kSegPairs; ++pp) asm volatile("" : "+v"(w2w.cw[0][0][pp].a), "+v"(w2w.sbw[0][0][pp]));
  uint16_t* zs = (uint16_t*)smem + (size_t)wave * 3 * R * kFlowZsi;  // this wave's pieces
  float* part2 = (float*)(smem + (size_t)kFfnWaves * 3 * R * kFlowZsi * 2);
  bool ok = true;
  for (int it = b; it < items2; it += nwg) {
    if (it != b) issue_w2(it, true);
    const int seg = item_seg(it);
    const bool active = seg < item_seg_end(it);
    if (active) {
      // the codes as exact bf16 fragments, converted before z is waited for
      bf16x8 q2[kSegGroups][2];
#pragma unroll
      for (int gg = 0; gg < kSegGroups; ++gg) {
        const int pp = gg >> 1;
        if (gg & 1) {
          q2[gg][0] = code_frag<4, 1, 0>(w2w.cw[0][0][pp]);
          q2[gg][1] = code_frag<4, 1, 1>(w2w.cw[0][0][pp]);
        } else {
          q2[gg][0] = code_frag<4, 0, 0>(w2w.cw[0][0][pp]);
          q2[gg][1] = code_frag<4, 0, 1>(w2w.cw[0][0][pp]);
        }
        asm volatile("" : "+v"(q2[gg][0]), "+v"(q2[gg][1]));
      }
      // this segment's z: lane L holds columns 4 L .. 4 L + 3 of every row
      const uint64_t* src = zt + (int64_t)seg * 256 + 4 * lane;
      uint64_t v[kFlowMaxRows][4];
      const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
      while (true) {
        bool mine = true;
#pragma unroll
        for (int r = 0; r < kFlowMaxRows; ++r) {
          if (r >= R) break;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            v[r][e] = flow_ld(src + (int64_t)r * N1 + e);
            mine = mine && (uint32_t)(v[r][e] >> 32) == tag;
          }
        }
        if (__builtin_amdgcn_ballot_w64(!mine) == 0) break;
        if (__builtin_amdgcn_s_memrealtime() - t0 > kFfnSpinTicks) {
          ok = false;
          __hip_atomic_store(err, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          break;
        }
        __builtin_amdgcn_s_sleep(1);
      }
      // the three exact bf16 pieces, planes [3][R][256 + 8]
#pragma unroll
      for (int r = 0; r < kFlowMaxRows; ++r) {
        if (r >= R) break;
        uint32_t h[4], m[4], l[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) split3(__uint_as_float((uint32_t)v[r][e]), h[e], m[e], l[e]);
        uint16_t* d = zs + r * kFlowZsi + 4 * lane;
        *(u32x2*)d = u32x2{h[0] | (h[1] << 16), h[2] | (h[3] << 16)};
        *(u32x2*)(d + R * kFlowZsi) = u32x2{m[0] | (m[1] << 16), m[2] | (m[3] << 16)};
        *(u32x2*)(d + 2 * R * kFlowZsi) = u32x2{l[0] | (l[1] << 16), l[2] | (l[3] << 16)};
      }
      // the wave's own pieces are read back below: its LDS writes complete first
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      __builtin_amdgcn_wave_barrier();
      // fragments of the staged pieces: row (i >> 2), piece (i & 3, slot 3 repeats piece 2)
      auto xf = [&](int, int g, int hh) -> bf16x8 {
        const int k0 = (g - seg * kSegGroups) * kGroup + hh * 32 + kc * 8;
        int row = i >> 2;
        row = row < R ? row : R - 1;
        int piece = i & 3;
        piece = piece < 3 ? piece : 2;
        return __builtin_bit_cast(bf16x8, *(const u32x4*)(zs + (piece * R + row) * kFlowZsi + k0));
      };
      float acc[1][1][1];
      auto qf = [&](int, int gg, int h) { return q2[gg][h]; };
      qmv_fold_segment<1, 1, 1, 1>(acc, w2w.cw[0], w2w.sbw[0], seg * kSegGroups, G2, xf, qf);
      part2[wave * 64 + lane] = acc[0][0][0];
    }
    __syncthreads();
    if (wave == 0) {
      const int t = it % T2, h = it / T2;
      const int nloc = item_seg_end(it) - h * half2;  // this item's segments, at most one per wave
      // the item's segment partials, all requested at once: read one by one
      // inside the sum, each would cost an LDS round trip on the step's
      // critical path
      float pv[kFfnWaves];
#pragma unroll
      for (int j = 0; j < kFfnWaves; ++j) pv[j] = part2[(j < nloc ? j : 0) * 64 + lane];
      if (h == 0) {
        float tot = pv[0];
#pragma unroll
        for (int j = 1; j < kFfnWaves; ++j)
          if (j < nloc) tot = tot + pv[j];
        flow_st(hand + (int64_t)t * 64 + lane, tot, tag);
      } else {
        // the lower half's running sum, polled with two loads in flight
        // (each check waits for its own load only), so a value that lands
        // just after one load has passed is seen by the next, not a whole
        // round trip later
        const uint64_t* src = hand + (int64_t)t * 64 + lane;
        const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
        uint64_t ha = flow_ld(src), hb, hv;
        while (true) {
          __builtin_amdgcn_s_sleep(2);
          hb = flow_ld(src);
          if (__builtin_amdgcn_ballot_w64((uint32_t)(ha >> 32) != tag) == 0) {
            hv = ha;
            asm volatile("" ::"v"(hb));  // the load still in flight lands here, not in a register reused below
            break;
          }
          __builtin_amdgcn_s_sleep(2);
          ha = flow_ld(src);
          if (__builtin_amdgcn_ballot_w64((uint32_t)(hb >> 32) != tag) == 0) {
            hv = hb;
            asm volatile("" ::"v"(ha));
            break;
          }
          if (__builtin_amdgcn_s_memrealtime() - t0 > kFfnSpinTicks) {
            ok = false;
            hv = hb;
            asm volatile("" ::"v"(ha));
            __hip_atomic_store(err, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            break;
          }
        }
        float tot = __uint_as_float((uint32_t)hv);
#pragma unroll
        for (int j = 0; j < kFfnWaves; ++j)
          if (j < nloc) tot = tot + pv[j];
        const int r = kc;
        if (r < R) y[(int64_t)r * ldy + (int64_t)t * kTileN + i] = tot;
        // every workgroup has read the call counter by now (each produces z,
        // and this item and its partner have consumed every producer's z):
        // advance it, without waiting for the result
        if (lane == 0) (void)__hip_atomic_fetch_max(epoch, tag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
    // part2 and the staged pieces are reused by the next item (LDS only)
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  }
  (void)ok;
}

}  // namespace q4
