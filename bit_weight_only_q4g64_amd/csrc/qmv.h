// Decode matvecs over 1..16 activation rows (qmv) on the matrix cores.
//
// One workgroup owns one 16-column tile of the weight matrix (or the same
// tile of w1 and w3 for the fused SwiGLU variant) and all of K. K is cut into
// segments of kSegGroups groups (a fixed function of K); each wave owns up to
// SPW segments and issues every weight load of all of them before any
// compute, so a workgroup has its whole column tile in flight at once. Codes
// become exact bf16 integers in registers and are reduced with
// v_mfma_f32_16x16x32_bf16 against the activation rows. Per output the order
// is:
//
//   for each segment s (ascending):   part_s = 0
//     for each group g in s:           P = mfma(x[g, 32..63], q, mfma(x[g, 0..31], q, 0))
//                                      S = mfma(x[g, 32..63], 1, mfma(x[g, 0..31], 1, 0))
//                                      part_s = fma(s_g, P, fma(b_g, S, part_s))
//   y = ((part_0 + part_1) + part_2) + ...
//
// bf16 activations: the 16 row slots of the instruction hold rows 0..15.
// float32 activations: each float is split exactly into three bf16 pieces
// h + m + l; row r of a 4-row tile uses slots 4r (h), 4r+1 (m), 4r+2 (l)
// (slot 4r+3 repeats a piece or holds anything: its result is never used),
// and P = (P_h + P_m) + P_l, S = (S_h + S_m) + S_l are combined in-lane
// before the fold. R > 4 uses 2 or 4 row tiles; with the pieces given in
// fragment order the tiles may be spread over workgroups along y.
//
// Nothing in the order depends on R, on the slot a row occupies or on the
// launch shape, so every row is bit-equal to its one-row result (TensorFold
// PR #1696, later revision, "What it adds": rows that share a decode step are
// summed as the one-row kernels sum them).
#pragma once

#include <cstddef>
#include <type_traits>

#include "common.h"

namespace q4 {

constexpr int kSegGroups = 4;  // groups per k segment (256 k)
constexpr int kSegPairs = kSegGroups / 2;
constexpr int kQmvMaxWaves = 16;
constexpr int kQmvMaxSpw = 4;  // segments per wave the kernels instantiate
constexpr int64_t kQmvMaxK = (int64_t)kQmvMaxWaves * kQmvMaxSpw * kSegGroups * kGroup;  // 16384

__host__ __device__ inline int qmv_segments(int64_t K) { return (int)((K / kGroup + kSegGroups - 1) / kSegGroups); }

// Layout of the dynamic LDS: per-segment partials, then (XLDS) the staged
// activations. bf16 x: [R][K + 8] bf16 (rows padded by 16 bytes against bank
// conflicts). float32 x: three bf16 planes h, m, l of [R][K + 8] each.
__host__ __device__ inline int64_t qmv_xs_stride(int64_t K) { return K + 8; }
__host__ __device__ inline size_t qmv_part_bytes(int64_t K, int xf32, int nmat, int rt, int nv = 4) {
  return (size_t)qmv_segments(K) * nmat * rt * (xf32 ? 1 : nv) * 64 * sizeof(float);
}
// Row slots per lane group the bf16 path keeps for R rows.
__host__ __device__ inline int qmv_nv(int R) { return R <= 1 ? 1 : (R <= 2 ? 2 : 4); }
// Row tiles the float32 path instantiates for R rows (1, 2 or 4 tiles of 4 rows).
__host__ __device__ inline int qmv_row_tiles(int xf32, int R) {
  if (!xf32) return 1;
  const int rtf = (R + 3) / 4;
  return rtf <= 1 ? 1 : (rtf <= 2 ? 2 : 4);
}
// Planes in fragment order: piece p (0..2) of element k of row r sits where
// the matvec's lane reads it, so one 16-byte read per lane covers a whole
// fragment and a wave's read is 1 KiB of consecutive bytes. Layout
// [K/64 groups][tiles][2 halves][64 lanes][8 values]: lane i + 16 kc holds
// matrix row i = 4 (r % 4) + p of tile r / 4, values kc * 8 .. + 7 of the
// half. Slots of piece 3 and of rows >= R are never written and never enter
// a stored result.
__host__ __device__ inline int64_t qmv_x3t_offset(int k, int r, int p, int tiles) {
  const int g = k >> 6, hh = (k >> 5) & 1, kc = (k >> 3) & 3, e = k & 7;
  const int ln = 4 * (r & 3) + p + 16 * kc;
  return ((((int64_t)g * tiles + (r >> 2)) * 2 + hh) * 64 + ln) * 8 + e;
}
__host__ __device__ inline int64_t qmv_x3t_bytes(int64_t K, int R) { return (K / kGroup) * qmv_row_tiles(1, R) * 2048; }
// workgroups up to which float32 rows read from memory split their row tiles
constexpr int64_t kQmvSplitBelow = 256;
// column tiles from which a bf16 matvec of one matrix runs two tiles per
// workgroup (at least 512 column tiles; K up to 8192, as the fused kernel)
constexpr int64_t kQmvPairTilesFrom = 512;
__host__ __device__ inline size_t qmv_xs_bytes(int64_t K, int xf32, int R) {
  return (size_t)(xf32 ? 3 : 1) * R * qmv_xs_stride(K) * sizeof(uint16_t);
}

// Weight registers of one wave's segments of one column tile (codes: one
// 128-bit word per lane per pair; scale/bias: one 64-bit word per pair).
template <int NMAT, int SPW, int BITS = 4>
struct QmvWeights {
  CodeWords<BITS> cw[SPW][NMAT][kSegPairs];
  u32x2 sbw[SPW][NMAT][kSegPairs];
};

// Issue every weight load of segments seg0 + j * step (j < SPW), with the
// streaming cache policy (each weight is read once per launch). Pair indices
// past the matrix are clamped to its last pair (those values are never
// used). Lanes with on == false, and slots at or past seg_end, read past the
// buffer's end, which the hardware answers with zeros and no memory access:
// the loads stay unconditional, so the count of loads in flight is the same
// on every path.
template <int NMAT, int SPW, int BITS = 4>
__device__ __forceinline__ void qmv_issue_weights(QmvWeights<NMAT, SPW, BITS>& w, const rsrc_t (&cres)[NMAT], const rsrc_t (&sres)[NMAT],
                                                  int seg0, int step, int P, int lane, bool on, int seg_end = 0x7fffffff) {
  const int i = lane & 15;
  constexpr uint32_t kPcb = pair_code_bytes(BITS);
#pragma unroll
  for (int j = 0; j < SPW; ++j) {
    const int seg = seg0 + j * step;
    const bool onj = on && seg < seg_end;
    const uint32_t cv = onj ? (uint32_t)lane * 16u : kOffBuffer, sv = onj ? (uint32_t)i * 8u : kOffBuffer;
    const uint32_t cv8 = onj ? (uint32_t)lane * 8u : kOffBuffer;
#pragma unroll
    for (int pp = 0; pp < kSegPairs; ++pp) {
      int p = seg * kSegPairs + pp;
      p = p < P ? p : P - 1;
#pragma unroll
      for (int m = 0; m < NMAT; ++m) {
        w.cw[j][m][pp].a = buf_load16_nt(cres[m], cv, (uint32_t)p * kPcb);
        if constexpr (BITS == 6) w.cw[j][m][pp].b = buf_load8_nt(cres[m], cv8, (uint32_t)p * kPcb + 1024u);
        if constexpr (code_bits(BITS) == 8) w.cw[j][m][pp].b = buf_load16_nt(cres[m], cv, (uint32_t)p * kPcb + 1024u);
        w.sbw[j][m][pp] = buf_load8_nt(sres[m], sv, (uint32_t)p * kPairSbBytes);
      }
    }
  }
}

// Fold the groups of one segment (g0 .. g0 + kSegGroups - 1, those below G)
// into acc, from zero. xfrag(rt, g, hh) returns this lane's activation
// fragment of row tile rt, group g, half hh. This is the decode order:
//   P = mfma(x[g, 32..63], q, mfma(x[g, 0..31], q, 0))
//   S = the same with q replaced by ones
//   acc = fma(s_g, P, fma(b_g, S, acc))
// with float32 rows combining their three pieces in-lane first. Block FP8
// has no bias: acc = fma(s_g, P, acc) with s_g the float32 block scale.
// AHEAD (fragments read from memory rather than LDS): every fragment of a
// group is requested before its first use and the next group's during this
// one, so a wave waits for one memory round trip per segment, not one per
// row tile and group.
// QF: nullptr (codes converted here), or qfrag(m, gg, half) returning codes
// converted earlier.
template <int XF32, int NMAT, int kRT, int kPerLane, bool AHEAD = false, int BITS, typename XF, typename QF = std::nullptr_t>
__device__ __forceinline__ void qmv_fold_segment(float (&acc)[NMAT][kRT][kPerLane], const CodeWords<BITS> (&cw)[NMAT][kSegPairs],
                                                 const u32x2 (&sbw)[NMAT][kSegPairs], int g0, int G, const XF& xfrag,
                                                 const QF& qfrag = nullptr) {
  const bf16x8 ones = ones_bf16x8();
  bf16x8 xn[kRT][2];  // AHEAD: the fragments of the next group
  if constexpr (AHEAD) {
    if (g0 < G) {
#pragma unroll
      for (int rt = 0; rt < kRT; ++rt) {
        xn[rt][0] = xfrag(rt, g0, 0);
        xn[rt][1] = xfrag(rt, g0, 1);
      }
    }
  }
#pragma unroll
  for (int m = 0; m < NMAT; ++m)
#pragma unroll
    for (int rt = 0; rt < kRT; ++rt)
#pragma unroll
      for (int v = 0; v < kPerLane; ++v) acc[m][rt][v] = 0.f;
#pragma unroll
  for (int gg = 0; gg < kSegGroups; ++gg) {
    const int g = g0 + gg;
    if (g >= G) break;
    const int pp = gg >> 1, gh = gg & 1;
    bf16x8 xc[kRT][2];
    if constexpr (AHEAD) {
#pragma unroll
      for (int rt = 0; rt < kRT; ++rt) {
        xc[rt][0] = xn[rt][0];
        xc[rt][1] = xn[rt][1];
      }
      if (gg + 1 < kSegGroups && g + 1 < G) {
#pragma unroll
        for (int rt = 0; rt < kRT; ++rt) {
          xn[rt][0] = xfrag(rt, g + 1, 0);
          xn[rt][1] = xfrag(rt, g + 1, 1);
        }
      }
    }
    bf16x8 q[NMAT][2];
    float sc[NMAT], bs[NMAT];
#pragma unroll
    for (int m = 0; m < NMAT; ++m) {
      if constexpr (std::is_same_v<QF, std::nullptr_t>) {
        q[m][0] = gh ? code_frag<BITS, 1, 0>(cw[m][pp]) : code_frag<BITS, 0, 0>(cw[m][pp]);
        q[m][1] = gh ? code_frag<BITS, 1, 1>(cw[m][pp]) : code_frag<BITS, 0, 1>(cw[m][pp]);
      } else {
        q[m][0] = qfrag(m, gg, 0);
        q[m][1] = qfrag(m, gg, 1);
      }
      const uint32_t w = gh ? sbw[m][pp][1] : sbw[m][pp][0];
      if constexpr (BITS == kFmtFp8) {
        sc[m] = __uint_as_float(w);
        bs[m] = 0.f;
      } else {
        sc[m] = bf16_lo(w);
        bs[m] = bf16_hi(w);
      }
    }
#pragma unroll
    for (int rt = 0; rt < kRT; ++rt) {
      const bf16x8 xa0 = AHEAD ? xc[rt][0] : xfrag(rt, g, 0), xa1 = AHEAD ? xc[rt][1] : xfrag(rt, g, 1);
      f32x4 S = {0.f, 0.f, 0.f, 0.f};
      if constexpr (BITS != kFmtFp8) {
        S = mfma16(xa0, ones, S);
        S = mfma16(xa1, ones, S);
      }
#pragma unroll
      for (int m = 0; m < NMAT; ++m) {
        f32x4 Pm = mfma16(xa0, q[m][0], f32x4{0.f, 0.f, 0.f, 0.f});
        Pm = mfma16(xa1, q[m][1], Pm);
        if constexpr (BITS == kFmtFp8) {
          if constexpr (!XF32) {
#pragma unroll
            for (int v = 0; v < kPerLane; ++v) acc[m][rt][v] = __builtin_fmaf(sc[m], Pm[v], acc[m][rt][v]);
          } else {
            const float Pr = (Pm[0] + Pm[1]) + Pm[2];
            acc[m][rt][0] = __builtin_fmaf(sc[m], Pr, acc[m][rt][0]);
          }
        } else if constexpr (!XF32) {
#pragma unroll
          for (int v = 0; v < kPerLane; ++v) acc[m][rt][v] = __builtin_fmaf(sc[m], Pm[v], __builtin_fmaf(bs[m], S[v], acc[m][rt][v]));
        } else {
          const float Pr = (Pm[0] + Pm[1]) + Pm[2];
          const float Sr = (S[0] + S[1]) + S[2];
          acc[m][rt][0] = __builtin_fmaf(sc[m], Pr, __builtin_fmaf(bs[m], Sr, acc[m][rt][0]));
        }
      }
    }
  }
}

// Segment partials in LDS: [segment][matrix][row tile][per lane][lane].
template <int NMAT, int kRT, int kPerLane>
__device__ __forceinline__ int qmv_part_index(int seg, int m, int rt, int v, int lane) {
  return (((seg * NMAT + m) * kRT + rt) * kPerLane + v) * 64 + lane;
}

// The segments' partials added in ascending order, a batch of reads in flight
// at a time (8 to 32 segments, by register room): every read of a batch is
// issued (indices clamped to the last segment) before its adds, and the adds
// past the last segment are dropped by a select rather than a branch, so the
// compiler cannot sink the reads into the adds (which costs one LDS round
// trip per segment).
template <int NMAT, int kRT, int kPerLane>
__device__ __forceinline__ void qmv_ordered_sum(float (&tot)[NMAT][kRT][kPerLane], const float* part, int nseg, int lane) {
#pragma unroll
  for (int m = 0; m < NMAT; ++m)
#pragma unroll
    for (int rt = 0; rt < kRT; ++rt)
#pragma unroll
      for (int v = 0; v < kPerLane; ++v) tot[m][rt][v] = part[qmv_part_index<NMAT, kRT, kPerLane>(0, m, rt, v, lane)];
  // as many reads in flight as 32 registers hold (at least 8)
  constexpr int kVals = NMAT * kRT * kPerLane;
  constexpr int kSumBatch = kVals >= 4 ? 8 : 32 / kVals;
  for (int seg0 = 1; seg0 < nseg; seg0 += kSumBatch) {
    float pv[kSumBatch][NMAT][kRT][kPerLane];
#pragma unroll
    for (int b = 0; b < kSumBatch; ++b) {
      const int seg = seg0 + b < nseg ? seg0 + b : nseg - 1;
#pragma unroll
      for (int m = 0; m < NMAT; ++m)
#pragma unroll
        for (int rt = 0; rt < kRT; ++rt)
#pragma unroll
          for (int v = 0; v < kPerLane; ++v) pv[b][m][rt][v] = part[qmv_part_index<NMAT, kRT, kPerLane>(seg, m, rt, v, lane)];
    }
#pragma unroll
    for (int b = 0; b < kSumBatch; ++b) {
      const bool in = seg0 + b < nseg;
#pragma unroll
      for (int m = 0; m < NMAT; ++m)
#pragma unroll
        for (int rt = 0; rt < kRT; ++rt)
#pragma unroll
          for (int v = 0; v < kPerLane; ++v) {
            const float t = tot[m][rt][v] + pv[b][m][rt][v];
            tot[m][rt][v] = in ? t : tot[m][rt][v];
          }
    }
  }
}

// XF32 = 0: bf16 x, one row tile of 16 rows.  XF32 = 1: float32 x, RTF row
// tiles of 4 rows x 3 pieces.  XF32 = 2: the same float32 values given as
// their three exact bf16 pieces, planes [3][R][ldx] (x = h + m + l, see
// split3): the arithmetic of XF32 = 1 without splitting in the kernel.
// NMAT = 1: y = W x.  NMAT = 2: y = silu(W1 x) * (W3 x); with Y3 the result
// is written as its three bf16 pieces, planes [3][R][ldy], instead of float32.
// SPW: maximum segments per wave.  XLDS: activations staged in LDS once per
// workgroup (else each wave reads its fragments from global memory). NV:
// row slots per lane group kept by the bf16 path. None of these changes the
// arithmetic of a stored row.
// XF32: 0 bf16 rows, 1 float32 rows, 2 float32 rows as three bf16 planes
// [3][R][ldx], 3 the same planes in fragment order (qmv_x3t_offset; read
// from memory, never staged). Y3: 0 float32 output, 1 three bf16 planes
// [3][R][ldy], 2 the planes in fragment order, 3 no SwiGLU: the two
// "matrices" are column tiles 2t and 2t + 1 of one matrix, each written as
// its own float32 columns (twice the weight loads in flight per wave; every
// column's arithmetic is the one-tile kernel's).
//
// K split (sp.nshare > 1): the sp.nshare workgroups along z of one column
// tile each fold a run of consecutive segments and store their partials in
// the caller's workspace; the last of them to arrive (an agent-scope counter
// per tile, which it resets) reads the others' partials and adds all of the
// tile's segments in the same ascending order, so the results are the
// unsplit kernel's bit for bit.
struct QmvSplit {
  int nshare;     // workgroups per column tile along z (1: no split)
  float* part;    // [tile id][segment][values per segment], tile id = x + gridDim.x * y
  uint32_t* cnt;  // [tile id] arrival counters, zero between calls
  // fused SwiGLU writing fragment-ordered planes (Y3 = 2): when set, the
  // same values also as float32 rows [R][ldz32]
  float* z32 = nullptr;
  int64_t ldz32 = 0;
};

template <int XF32, int NMAT, int SPW, int RTF, bool XLDS, int NV, int BITS, int Y3 = 0>
__global__ __launch_bounds__(kQmvMaxWaves * 64) void qmv_kernel(const uint8_t* __restrict__ pk0, const uint8_t* __restrict__ pk1,
                                                              int N, int K, const void* __restrict__ xv, int64_t ldx, int R,
                                                              float* __restrict__ y, int64_t ldy, QmvSplit sp) {
  static_assert(!Y3 || NMAT == 2, "the three-plane output is the fused SwiGLU's");
  static_assert(XF32 != 3 || !XLDS, "fragment-ordered planes are read from memory");
  constexpr int kRT = XF32 ? RTF : 1;  // row tiles
  // accumulators per lane per row tile: bf16 x keeps row slots 4*kc + v for
  // v < NV (NV = 4 when R > 4, else the smallest of 1, 2, 4 covering R); the
  // slots left out hold rows >= R and are never stored
  constexpr int kPerLane = XF32 ? 1 : NV;
  constexpr int kXElem = XF32 == 1 ? 4 : 2;  // bytes per activation element
  const int XR = XF32 == 2 ? 3 * R : R;        // activation rows in memory (planes: piece-major)
  extern __shared__ __align__(16) uint8_t smem[];
  // The segment partials ([segment][matrix][row tile][kPerLane][lane]) are
  // written only after every wave has finished reading the staged
  // activations, so the two share the same LDS: a workgroup needs the larger
  // of the two, which keeps two workgroups per CU at up to 16 rows.
  float* part = (float*)smem;
  uint16_t* xs = (uint16_t*)smem;
  const int t = blockIdx.x;
  // float32 rows read from memory may split their row tiles over
  // blockIdx.y: this workgroup's first tile of the T = qmv_row_tiles(R)
  // (a row's arithmetic is the same whichever workgroup computes it)
  const int rt0 = XF32 ? (int)blockIdx.y * kRT : 0;
  const int T = XF32 ? qmv_row_tiles(1, R) : kRT;
  const int lane = threadIdx.x & 63, nwaves = blockDim.x >> 6;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform per wave
  const int i = lane & 15, kc = lane >> 4;
  const int G = K / kGroup;
  const int P = (G + 1) / 2;
  const int nseg = qmv_segments(K);
  const int64_t cb = codes_bytes(N, K, BITS);
  // this workgroup's segments [sb, se) and the k range [kb, kb + kl) they read
  const int per = (nseg + sp.nshare - 1) / sp.nshare;
  const int sb = (int)blockIdx.z * per;
  const int se = sb + per < nseg ? sb + per : nseg;
  const int kb = sb * kSegGroups * kGroup;
  const int kl = (se * kSegGroups * kGroup < K ? se * kSegGroups * kGroup : K) - kb;
  const int xsi = (int)qmv_xs_stride(kl);
  const uint32_t xrow = (uint32_t)(ldx * kXElem);  // bytes per activation row

  // buffer resources: this column tile's codes and scale/bias, and x
  rsrc_t cres[NMAT], sres[NMAT];
#pragma unroll
  for (int m = 0; m < NMAT; ++m) {
    const uint8_t* pk = m ? pk1 : pk0;
    const int64_t tm = Y3 == 3 ? 2 * (int64_t)t + m : t;  // this matrix's column tile
    cres[m] = make_rsrc(pk + tm * P * pair_code_bytes(BITS), (uint32_t)P * pair_code_bytes(BITS));
    sres[m] = make_rsrc(pk + cb + tm * P * kPairSbBytes, (uint32_t)P * kPairSbBytes);
  }
  const rsrc_t xres = make_rsrc(xv, XF32 == 3 ? (uint32_t)qmv_x3t_bytes(K, R) : (uint32_t)XR * xrow);

  // 1) activations: the first batch of staging loads is issued before the
  //    weight loads (after them with PRE below), so writing it to LDS waits
  //    for nothing else. The R rows
  //    are cut into 16-byte chunks, numbered row after row; slot u of a
  //    thread holds chunk threadIdx.x + u * blockDim.x, so every thread has
  //    work whatever the row length.
  // eight loads in flight where the weight registers leave room, else four
  constexpr int kBatch = (XF32 || SPW * NMAT * code_bits(BITS) > 8) ? 4 : 8;
  const int nthr = blockDim.x;
  const int per_row = kl * kXElem / 16;  // 16-byte chunks per staged row
  const int total = XR * per_row;
  const int nslots = (total + nthr - 1) / nthr;
  // (row, chunk) of slot 0, and the step from one slot to the next
  const int r0 = (int)threadIdx.x / per_row, c0 = (int)threadIdx.x - r0 * per_row;
  const int step_r = nthr / per_row, step_c = nthr - step_r * per_row;
  auto advance = [&](int& r, int& c) {
    c += step_c;
    r += step_r;
    if (c >= per_row) { c -= per_row; ++r; }
  };
  auto xload = [&](int r, int c) -> u32x4 {
    if (r >= XR) { r = XR - 1; c = per_row - 1; }  // past the last chunk: a valid, unused read
    return buf_load16(xres, (uint32_t)c * 16u + (uint32_t)r * xrow, (uint32_t)kb * kXElem);
  };
  // PRE (one row tile, one slot per lane, codes of at most 64 registers once
  // converted): the weights are requested first and their codes converted
  // while the activations are still in flight; the folds after the staging
  // barrier then run only matrix steps and fmas
  constexpr bool kPre = XLDS && kRT == 1 && kPerLane == 1 && SPW * NMAT * kSegGroups * 2 <= 16;
  QmvWeights<NMAT, SPW, BITS> wts;
  if constexpr (kPre) qmv_issue_weights<NMAT, SPW, BITS>(wts, cres, sres, sb + wave, nwaves, P, lane, true, se);
  u32x4 xv0[kBatch];
  if constexpr (XLDS) {
    int r = r0, c = c0;
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      if (u >= nslots) break;
      xv0[u] = xload(r, c);
      advance(r, c);
    }
  }

  // 2) every weight load of this wave's segments
  if constexpr (!kPre) qmv_issue_weights<NMAT, SPW, BITS>(wts, cres, sres, sb + wave, nwaves, P, lane, true, se);
  bf16x8 qpre[SPW][NMAT][kSegGroups][2];
  if constexpr (kPre) {
#pragma unroll
    for (int j = 0; j < SPW; ++j)
#pragma unroll
      for (int m = 0; m < NMAT; ++m)
#pragma unroll
        for (int gg = 0; gg < kSegGroups; ++gg) {
          const int pp = gg >> 1;
          if (gg & 1) {
            qpre[j][m][gg][0] = code_frag<BITS, 1, 0>(wts.cw[j][m][pp]);
            qpre[j][m][gg][1] = code_frag<BITS, 1, 1>(wts.cw[j][m][pp]);
          } else {
            qpre[j][m][gg][0] = code_frag<BITS, 0, 0>(wts.cw[j][m][pp]);
            qpre[j][m][gg][1] = code_frag<BITS, 0, 1>(wts.cw[j][m][pp]);
          }
          // converted here, before the activations are waited for
          asm volatile("" : "+v"(qpre[j][m][gg][0]), "+v"(qpre[j][m][gg][1]));
        }
  }

  // 3) write the staged activations (float32 rows as three exact bf16 planes)
  if constexpr (XLDS) {
    const int plane = R * xsi;
    auto put = [&](int r, int c, const u32x4& v) {
      if (r >= XR) return;
      if constexpr (XF32 != 1) {  // bf16 rows, or the planes row after row (piece * R + row)
        *(u32x4*)(xs + r * xsi + c * 8) = v;
      } else {
        uint32_t h[4], m[4], l[4];
#pragma unroll
        for (int w = 0; w < 4; ++w) split3(__uint_as_float(v[w]), h[w], m[w], l[w]);
        uint16_t* d = xs + r * xsi + c * 4;
        *(u32x2*)d = u32x2{h[0] | (h[1] << 16), h[2] | (h[3] << 16)};
        *(u32x2*)(d + plane) = u32x2{m[0] | (m[1] << 16), m[2] | (m[3] << 16)};
        *(u32x2*)(d + 2 * plane) = u32x2{l[0] | (l[1] << 16), l[2] | (l[3] << 16)};
      }
    };
    int r = r0, c = c0;
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      if (u >= nslots) break;
      put(r, c, xv0[u]);
      advance(r, c);
    }
    // slots beyond the first batch (large R * K): kBatch loads, then their writes
    for (int u0 = kBatch; u0 < nslots; u0 += kBatch) {
      u32x4 v[kBatch];
      int rl = r, cl = c;
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        if (u0 + u < nslots) v[u] = xload(rl, cl);
        advance(rl, cl);
      }
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        if (u0 + u < nslots) put(r, c, v[u]);
        advance(r, c);
      }
    }
    __syncthreads();
  }

  // Activation fragment of row tile rt, group g, half hh for this lane. Slots
  // of rows >= R (and the unused fourth piece slot) read a valid row: their
  // results are independent of the other slots and never stored.
  const int frow = XF32 ? 0 : (i < R ? i : R - 1);
  auto xfrag = [&](int rt, int g, int hh) -> bf16x8 {
    const int k0 = g * kGroup + hh * 32 + kc * 8;
    if constexpr (!XF32) {
      if constexpr (XLDS) return __builtin_bit_cast(bf16x8, *(const u32x4*)(xs + frow * xsi + (k0 - kb)));
      else return __builtin_bit_cast(bf16x8, buf_load16(xres, (uint32_t)frow * xrow + (uint32_t)k0 * 2u, 0u));
    } else if constexpr (XF32 == 3) {
      return __builtin_bit_cast(bf16x8, buf_load16(xres, (uint32_t)((((g * T + rt0 + rt) * 2 + hh) * 64 + lane) * 16), 0u));
    } else {
      int row = (rt0 + rt) * 4 + (i >> 2);
      row = row < R ? row : R - 1;
      int piece = i & 3;
      piece = piece < 3 ? piece : 2;
      if constexpr (XLDS) return __builtin_bit_cast(bf16x8, *(const u32x4*)(xs + (piece * R + row) * xsi + (k0 - kb)));
      else if constexpr (XF32 == 2) return __builtin_bit_cast(bf16x8, buf_load16(xres, (uint32_t)(piece * R + row) * xrow + (uint32_t)k0 * 2u, 0u));
      else {
        const u32x4 a = buf_load16(xres, (uint32_t)row * xrow + (uint32_t)k0 * 4u, 0u);
        const u32x4 b = buf_load16(xres, (uint32_t)row * xrow + (uint32_t)k0 * 4u + 16u, 0u);
        uint32_t o[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          uint32_t h, m, l;
          split3(__uint_as_float(e < 4 ? a[e] : b[e - 4]), h, m, l);
          o[e] = piece == 0 ? h : (piece == 1 ? m : l);
        }
        return __builtin_bit_cast(bf16x8, u32x4{o[0] | (o[1] << 16), o[2] | (o[3] << 16), o[4] | (o[5] << 16), o[6] | (o[7] << 16)});
      }
    }
  };

  // fragments read from memory are requested a group ahead where the
  // registers allow (the weights of at most 8 code bits x segments x
  // matrices per lane are held; more spills)
  constexpr bool kAhead = !XLDS && SPW * NMAT * code_bits(BITS) <= 8;

  // 4) compute, one segment after another; the partials wait in registers
  //    until every wave is past its last activation read
  float keep[SPW][NMAT][kRT][kPerLane];
#pragma unroll
  for (int j = 0; j < SPW; ++j) {
    const int seg = sb + wave + j * nwaves;
    if (seg >= se) break;
    if constexpr (kPre) {
      auto qfrag = [&](int m, int gg, int h) { return qpre[j][m][gg][h]; };
      qmv_fold_segment<XF32, NMAT, kRT, kPerLane, kAhead>(keep[j], wts.cw[j], wts.sbw[j], seg * kSegGroups, G, xfrag, qfrag);
    } else {
      qmv_fold_segment<XF32, NMAT, kRT, kPerLane, kAhead>(keep[j], wts.cw[j], wts.sbw[j], seg * kSegGroups, G, xfrag);
    }
  }
  if constexpr (XLDS) __syncthreads();
  constexpr int kSegVals = NMAT * kRT * kPerLane * 64;  // partials per segment
  const int64_t tid = (int64_t)t + (int64_t)gridDim.x * blockIdx.y;
  uint32_t* wpart = (uint32_t*)sp.part + tid * nseg * kSegVals;
#pragma unroll
  for (int j = 0; j < SPW; ++j) {
    const int seg = sb + wave + j * nwaves;
    if (seg >= se) break;
#pragma unroll
    for (int m = 0; m < NMAT; ++m)
#pragma unroll
      for (int rt = 0; rt < kRT; ++rt)
#pragma unroll
        for (int v = 0; v < kPerLane; ++v) {
          const int at = qmv_part_index<NMAT, kRT, kPerLane>(seg, m, rt, v, lane);
          part[at] = keep[j][m][rt][v];
          // agent-scope stores: coherent for a workgroup on any XCD
          if (sp.nshare > 1) __hip_atomic_store(wpart + at, __float_as_uint(keep[j][m][rt][v]), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
  }
  if (sp.nshare > 1) {
    // every partial of this wave is stored before the workgroup arrives
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  }
  __syncthreads();
  if (sp.nshare > 1) {
    __shared__ uint32_t s_last;
    if (threadIdx.x == 0) {
      const uint32_t old = __hip_atomic_fetch_add(sp.cnt + tid, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      const uint32_t last = old == (uint32_t)(sp.nshare - 1);
      // every workgroup of this tile has arrived: the counter is free for the next call
      if (last) __hip_atomic_store(sp.cnt + tid, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      s_last = last;
    }
    __syncthreads();
    if (!s_last) return;
    // the last arrival: the other workgroups' segments, from the workspace
    for (int at = (int)threadIdx.x; at < nseg * kSegVals; at += nthr) {
      const int seg = at / kSegVals;
      if (seg >= sb && seg < se) continue;
      part[at] = __uint_as_float(__hip_atomic_load(wpart + at, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
    }
    __syncthreads();
  }
  if (wave != 0) return;

  // 5) add the segments in ascending order; epilogue
  float tot[NMAT][kRT][kPerLane];
  qmv_ordered_sum<NMAT, kRT, kPerLane>(tot, part, nseg, lane);

  const int64_t n = (int64_t)t * kTileN + i;
#pragma unroll
  for (int rt = 0; rt < kRT; ++rt) {
#pragma unroll
    for (int v = 0; v < kPerLane; ++v) {
      const int r = XF32 ? (rt0 + rt) * 4 + kc : 4 * kc + v;
      if (r >= R) continue;
      if constexpr (Y3 == 3) {
        y[(int64_t)r * ldy + 2 * (int64_t)t * kTileN + i] = tot[0][rt][v];
        y[(int64_t)r * ldy + (2 * (int64_t)t + 1) * kTileN + i] = tot[1][rt][v];
        continue;
      }
      float out;
      if constexpr (NMAT == 1) {
        out = tot[0][rt][v];
      } else {
        out = silu_f32(tot[0][rt][v]) * tot[1][rt][v];
      }
      if constexpr (Y3 == 1) {
        uint32_t h, m, l;
        split3(out, h, m, l);
        uint16_t* y3 = (uint16_t*)y;
        const int64_t plane = (int64_t)R * ldy;
        y3[(int64_t)r * ldy + n] = (uint16_t)h;
        y3[plane + (int64_t)r * ldy + n] = (uint16_t)m;
        y3[2 * plane + (int64_t)r * ldy + n] = (uint16_t)l;
      } else if constexpr (Y3 == 2) {
        uint32_t h, m, l;
        split3(out, h, m, l);
        uint16_t* y3 = (uint16_t*)y;
        const int tiles = qmv_row_tiles(1, R);
        y3[qmv_x3t_offset((int)n, r, 0, tiles)] = (uint16_t)h;
        y3[qmv_x3t_offset((int)n, r, 1, tiles)] = (uint16_t)m;
        y3[qmv_x3t_offset((int)n, r, 2, tiles)] = (uint16_t)l;
        if (sp.z32 != nullptr) sp.z32[(int64_t)r * sp.ldz32 + n] = out;
      } else {
        y[(int64_t)r * ldy + n] = out;
      }
    }
  }
}

// Largest dynamic LDS a workgroup may use (queried once per process, on the
// device current at the first call; the initialisation is thread-safe).
inline size_t qmv_max_lds() {
  static const size_t cached = [] {
    int dev = 0, v = 0;
    if (hipGetDevice(&dev) == hipSuccess && hipDeviceGetAttribute(&v, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) == hipSuccess && v > 0)
      return (size_t)v;
    return (size_t)64 * 1024;
  }();
  return cached;
}

// Compute units of the device (queried once per process, like qmv_max_lds;
// used only to choose among kernels that give the same bits).
inline int device_cus() {
  static const int cached = [] {
    int dev = 0, v = 0;
    if (hipGetDevice(&dev) == hipSuccess && hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && v > 0)
      return v;
    return 256;
  }();
  return cached;
}

// Let a kernel use the largest dynamic LDS a workgroup may have beside the
// kernel's own static LDS. A failed query or setting keeps the 64 KiB default
// and clears the error it raised, so that the launch after it reports only
// its own status.
inline bool allow_max_dynamic_lds(const void* kern) {
  hipFuncAttributes fa{};
  size_t stat = 0;
  if (hipFuncGetAttributes(&fa, kern) == hipSuccess) stat = fa.sharedSizeBytes;
  const size_t mx = qmv_max_lds();
  const bool ok = mx > stat && hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)(mx - stat)) == hipSuccess;
  if (!ok) (void)hipGetLastError();
  return ok;
}

// LDS needed without staging (partials only); the launch adds the staged
// activations when they fit.
inline size_t qmv_lds_bytes(int64_t K, int xf32, int nmat, int R) {
  return qmv_part_bytes(K, xf32, nmat, qmv_row_tiles(xf32, R), xf32 ? 1 : qmv_nv(R));
}

// Segments per workgroup of a tile split nshare ways, and the k extent of
// the activations such a workgroup stages.
__host__ __device__ inline int qmv_share_segments(int64_t K, int nshare) { return (qmv_segments(K) + nshare - 1) / nshare; }
__host__ __device__ inline int64_t qmv_share_k(int64_t K, int nshare) {
  const int64_t k = (int64_t)qmv_share_segments(K, nshare) * kSegGroups * kGroup;
  return k < K ? k : K;
}

template <int XF32, int NMAT, int SPW, int RTF, bool XLDS, int NV, int BITS, int Y3>
inline void qmv_launch_t(const uint8_t* pk0, const uint8_t* pk1, int N, int K, const void* x, int64_t ldx, int R, float* y,
                         int64_t ldy, int nwaves, size_t lds, hipStream_t s, const QmvSplit& sp) {
  // float32 rows: the row tiles not covered by RTF go to more workgroups along y
  const unsigned ysplit = XF32 ? (unsigned)(qmv_row_tiles(1, R) / RTF) : 1u;
  auto kern = qmv_kernel<XF32, NMAT, SPW, RTF, XLDS, NV, BITS, Y3>;
  // allow dynamic LDS beyond the 64 KB default, once per instantiation
  static const bool lds_ok = allow_max_dynamic_lds((const void*)kern);
  (void)lds_ok;
  const unsigned gx = (unsigned)(N / kTileN / (Y3 == 3 ? 2 : 1));
  hipLaunchKernelGGL(kern, dim3(gx, ysplit, (unsigned)sp.nshare), dim3(nwaves * 64), lds, s, pk0, pk1, N, K, x, ldx, R, y, ldy, sp);
}

template <int XF32, int NMAT, int RTF, bool XLDS, int NV, int BITS, int Y3>
inline void qmv_launch_spw(const uint8_t* pk0, const uint8_t* pk1, int N, int K, const void* x, int64_t ldx, int R, float* y,
                           int64_t ldy, size_t lds, hipStream_t s, const QmvSplit& sp) {
  const int per = qmv_share_segments(K, sp.nshare);
  const int nwaves = per < kQmvMaxWaves ? per : kQmvMaxWaves;
  const int spw = (per + nwaves - 1) / nwaves;
  if (spw <= 1) {
    qmv_launch_t<XF32, NMAT, 1, RTF, XLDS, NV, BITS, Y3>(pk0, pk1, N, K, x, ldx, R, y, ldy, nwaves, lds, s, sp);
  } else if (spw <= 2) {
    qmv_launch_t<XF32, NMAT, 2, RTF, XLDS, NV, BITS, Y3>(pk0, pk1, N, K, x, ldx, R, y, ldy, nwaves, lds, s, sp);
  } else {
    // the fused two-matrix variant is limited to K <= 8192 (two segments per wave)
    if constexpr (NMAT == 1) qmv_launch_t<XF32, NMAT, 4, RTF, XLDS, NV, BITS, Y3>(pk0, pk1, N, K, x, ldx, R, y, ldy, nwaves, lds, s, sp);
  }
}

template <int XF32, int NMAT, int RTF, int NV, int BITS, int Y3>
inline void qmv_launch_lds(const uint8_t* pk0, const uint8_t* pk1, int N, int K, const void* x, int64_t ldx, int R, float* y,
                           int64_t ldy, hipStream_t s, const QmvSplit& sp) {
  const size_t part = qmv_part_bytes(K, XF32, NMAT, XF32 ? RTF : 1, NV);
  if constexpr (XF32 == 3) {
    qmv_launch_spw<XF32, NMAT, RTF, false, NV, BITS, Y3>(pk0, pk1, N, K, x, ldx, R, y, ldy, part, s, sp);
  } else {
    const size_t xsb = qmv_xs_bytes(qmv_share_k(K, sp.nshare), XF32, R);
    const size_t staged = part > xsb ? part : xsb;  // the partials reuse the staging area
    // staged rows are not split: a workgroup then covers every row tile
    if ((!XF32 || RTF == qmv_row_tiles(1, R)) && staged <= qmv_max_lds())
      qmv_launch_spw<XF32, NMAT, RTF, true, NV, BITS, Y3>(pk0, pk1, N, K, x, ldx, R, y, ldy, staged, s, sp);
    else
      qmv_launch_spw<XF32, NMAT, RTF, false, NV, BITS, Y3>(pk0, pk1, N, K, x, ldx, R, y, ldy, part, s, sp);
  }
}

template <int NMAT, int BITS, int Y3>
inline void qmv_launch_bf16(const uint8_t* pk0, const uint8_t* pk1, int N, int K, const void* x, int64_t ldx, int R, float* y,
                            int64_t ldy, hipStream_t s, const QmvSplit& sp) {
  const int nv = qmv_nv(R);
  if (nv == 1)
    qmv_launch_lds<0, NMAT, 1, 1, BITS, Y3>(pk0, pk1, N, K, x, ldx, R, y, ldy, s, sp);
  else if (nv == 2)
    qmv_launch_lds<0, NMAT, 1, 2, BITS, Y3>(pk0, pk1, N, K, x, ldx, R, y, ldy, s, sp);
  else
    qmv_launch_lds<0, NMAT, 1, 4, BITS, Y3>(pk0, pk1, N, K, x, ldx, R, y, ldy, s, sp);
}

// Row tiles per workgroup of a float32 matvec: rows read from memory
// (fragment-ordered planes, or rows that do not fit in LDS) split their row
// tiles over more workgroups (1, 2 or 4 tiles each) while the column tiles
// and K shares leave CUs idle.
inline int qmv_pieces_rt(int xf32, int N, int K, int R, int nshare) {
  int rt = qmv_row_tiles(1, R);
  bool from_memory = xf32 == 3;
  if (!from_memory) {
    const size_t part = qmv_part_bytes(K, xf32, 1, rt, 1), xsb = qmv_xs_bytes(qmv_share_k(K, nshare), xf32, R);
    from_memory = (part > xsb ? part : xsb) > qmv_max_lds();
  }
  if (from_memory)
    while (rt > 1 && (int64_t)(N / kTileN) * nshare * (qmv_row_tiles(1, R) / rt) * 2 <= kQmvSplitBelow) rt /= 2;
  return rt;
}

template <int XF32, int BITS>
inline void qmv_launch_pieces(const uint8_t* pk0, int N, int K, const void* x, int64_t ldx, int R, float* y, int64_t ldy,
                              hipStream_t s, const QmvSplit& sp) {
  const int rt = qmv_pieces_rt(XF32, N, K, R, sp.nshare);
  if (rt == 1)
    qmv_launch_lds<XF32, 1, 1, 1, BITS, 0>(pk0, pk0, N, K, x, ldx, R, y, ldy, s, sp);
  else if (rt == 2)
    qmv_launch_lds<XF32, 1, 2, 1, BITS, 0>(pk0, pk0, N, K, x, ldx, R, y, ldy, s, sp);
  else
    qmv_launch_lds<XF32, 1, 4, 1, BITS, 0>(pk0, pk0, N, K, x, ldx, R, y, ldy, s, sp);
}

// Whether a bf16 matvec of one matrix runs two column tiles per workgroup.
inline bool qmv_pairs_tiles(int nmat, int xmode, int N, int K, int nshare) {
  return nmat == 1 && xmode == 0 && nshare == 1 && N / kTileN >= kQmvPairTilesFrom && K <= kQmvMaxK / 2;
}

// xmode: 0 bf16 rows, 1 float32 rows, 2 float32 rows as three bf16 planes,
// 3 the planes in fragment order (one matrix only). y3: the fused SwiGLU
// writes three bf16 planes (1) or the planes in fragment order (2).
template <int BITS>
inline void qmv_launch_bits(const uint8_t* pk0, const uint8_t* pk1, int nmat, int N, int K, const void* x, int xmode, int64_t ldx,
                            int R, float* y, int64_t ldy, hipStream_t s, int y3, const QmvSplit& sp) {
  if (xmode == 0) {
    if (qmv_pairs_tiles(nmat, xmode, N, K, sp.nshare))
      qmv_launch_bf16<2, BITS, 3>(pk0, pk0, N, K, x, ldx, R, y, ldy, s, sp);
    else if (nmat == 1)
      qmv_launch_bf16<1, BITS, 0>(pk0, pk1, N, K, x, ldx, R, y, ldy, s, sp);
    else if (y3 == 1)
      qmv_launch_bf16<2, BITS, 1>(pk0, pk1, N, K, x, ldx, R, y, ldy, s, sp);
    else if (y3 == 2)
      qmv_launch_bf16<2, BITS, 2>(pk0, pk1, N, K, x, ldx, R, y, ldy, s, sp);
    else
      qmv_launch_bf16<2, BITS, 0>(pk0, pk1, N, K, x, ldx, R, y, ldy, s, sp);
  } else if (xmode == 1) {
    qmv_launch_pieces<1, BITS>(pk0, N, K, x, ldx, R, y, ldy, s, sp);
  } else if (xmode == 2) {
    qmv_launch_pieces<2, BITS>(pk0, N, K, x, ldx, R, y, ldy, s, sp);
  } else {
    qmv_launch_pieces<3, BITS>(pk0, N, K, x, ldx, R, y, ldy, s, sp);
  }
}

// Workspace of a K split: one arrival counter per tile id (a 256-byte
// aligned block), then the partials [tile id][segment][values per segment].
// Tile ids are column tiles (pairs for the fused two-matrix kernel count
// once) times the row-tile workgroups of float32 rows read from memory.
struct QmvSplitShape {
  int64_t tile_ids;
  int64_t seg_vals;  // floats per segment and tile id
};
inline QmvSplitShape qmv_split_shape(int nmat, int xmode, int N, int K, int R, int nshare) {
  QmvSplitShape sh{};
  const int64_t tiles = N / kTileN;
  if (xmode == 0) {
    sh.tile_ids = tiles;
    sh.seg_vals = (int64_t)nmat * qmv_nv(R) * 64;
  } else {
    const int rt = qmv_pieces_rt(xmode, N, K, R, nshare);
    sh.tile_ids = tiles * (qmv_row_tiles(1, R) / rt);
    sh.seg_vals = (int64_t)rt * 64;
  }
  return sh;
}
inline size_t qmv_split_counter_bytes(const QmvSplitShape& sh) { return (size_t)((sh.tile_ids * 4 + 255) / 256 * 256); }
inline size_t qmv_split_work_bytes(int nmat, int xmode, int N, int K, int R, int nshare) {
  const QmvSplitShape sh = qmv_split_shape(nmat, xmode, N, K, R, nshare);
  return qmv_split_counter_bytes(sh) + (size_t)sh.tile_ids * qmv_segments(K) * sh.seg_vals * sizeof(float);
}

// bits: 4, 6, 8 or kFmtFp8 (checked by the caller). sp: the K split and its
// workspace (nshare = 1: none).
inline void qmv_launch(const uint8_t* pk0, const uint8_t* pk1, int nmat, int N, int K, const void* x, int xmode, int64_t ldx,
                       int R, float* y, int64_t ldy, hipStream_t s, int bits = 4, int y3 = 0, QmvSplit sp = QmvSplit{1, nullptr, nullptr}) {
  if (bits == 6)
    qmv_launch_bits<6>(pk0, pk1, nmat, N, K, x, xmode, ldx, R, y, ldy, s, y3, sp);
  else if (bits == 8)
    qmv_launch_bits<8>(pk0, pk1, nmat, N, K, x, xmode, ldx, R, y, ldy, s, y3, sp);
  else if (bits == kFmtFp8)
    qmv_launch_bits<kFmtFp8>(pk0, pk1, nmat, N, K, x, xmode, ldx, R, y, ldy, s, y3, sp);
  else
    qmv_launch_bits<4>(pk0, pk1, nmat, N, K, x, xmode, ldx, R, y, ldy, s, y3, sp);
}

}  // namespace q4
