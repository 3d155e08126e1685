// Attention-side decode epilogue: QK norm, partial RoPE and the KV store on
// the output of the stacked q/k/v matvec (TensorFold PR #1696, "What it adds":
// kernels for QK norm with partial RoPE and GQA attention over a KV ring;
// decode fuses RoPE with the KV store).
//
// One row of the stacked matvec output is [q heads | k heads | v heads], 64
// values per head. Per head, on one wave (lane d holds dimension d):
//   * q and k, when a gamma is given: x <- (x * r) * gamma[d] with
//     r = 1 / sqrt(sum(x^2) / 64 + eps), the sum over a fixed xor butterfly;
//   * q and k: the first `rot` dims rotate in half-split pairs (i, i + rot/2)
//     by the angle pos * theta^(-2i/rot): the inverse frequencies are formed
//     on the host in double, the angle on the device in double, reduced
//     modulo 2 pi in double and rounded once to float for sincosf:
//       x_i' = fma(x_i, c, -(x_{i+h} s)),  x_{i+h}' = fma(x_{i+h}, c, x_i s);
//   * q goes to q_out[r], k and v to slot pos mod ring of their caches
//     ([ring][kv_heads][64], float32 or bf16 rounded to nearest even; row r's
//     ring starts row_stride * r elements in, 0 = one ring for all rows);
//   * gate heads (gated attention's fourth matvec, after the v heads) go to
//     gate_out[r] unchanged.
// The same function serves the stand-alone epilogue and the fused matvec, so
// the fused results are bit-identical to the composition.
#pragma once

#include "common.h"
#include "qmv.h"

namespace q4 {

constexpr int kHeadDim = 64;

struct RopeKvArgs {
  double inv[32];  // theta^(-2i/rot), i < rot/2
  const int32_t* pos;
  int n_q, n_kv, rot;
  float theta, eps;
  const float* gamma_q;
  const float* gamma_k;
  float* q_out;
  int64_t ldq;
  void* k_cache;
  void* v_cache;
  int cache_bf16;
  int64_t ring;
  int64_t row_stride;  // elements between the rows' rings (0: one shared ring)
  int n_gate;
  float* gate_out;
  int64_t ldg;
};

// Head hd (wave-uniform) of row r; x is this lane's value of dimension d.
__device__ __forceinline__ void rope_kv_head(float x, int d, int hd, int r, const RopeKvArgs& a) {
  const int n_qkv = a.n_q + 2 * a.n_kv;
  if (hd >= n_qkv) {
    a.gate_out[(int64_t)r * a.ldg + (int64_t)(hd - n_qkv) * kHeadDim + d] = x;
    return;
  }
  const bool is_q = hd < a.n_q, is_k = !is_q && hd < a.n_q + a.n_kv;
  const int p = a.pos[r];
  if (is_q || is_k) {
    const float* gamma = is_q ? a.gamma_q : a.gamma_k;
    if (gamma != nullptr) {
      float ss = x * x;
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) ss = ss + __shfl_xor(ss, o, 64);
      const float rn = 1.0f / __builtin_sqrtf(ss * (1.0f / 64.0f) + a.eps);
      x = (x * rn) * gamma[d];
    }
    if (a.rot > 0) {
      const int h = a.rot >> 1;
      const int partner = d < h ? d + h : (d < a.rot ? d - h : d);
      const float xp = __shfl(x, partner, 64);
      if (d < a.rot) {
        const int i = d < h ? d : d - h;
        const double ang = (double)p * a.inv[i];
        const double kk = rint(ang * 0.15915494309189535);  // 1 / (2 pi)
        const float red = (float)__builtin_fma(-kk, 6.283185307179586, ang);
        float s, c;
        sincosf(red, &s, &c);
        x = d < h ? __builtin_fmaf(x, c, -(xp * s)) : __builtin_fmaf(x, c, xp * s);
      }
    }
  }
  if (is_q) {
    a.q_out[(int64_t)r * a.ldq + (int64_t)hd * kHeadDim + d] = x;
    return;
  }
  int64_t slot = a.ring > 0 ? (int64_t)p % a.ring : 0;
  if (slot < 0) slot += a.ring;
  const int kvh = is_k ? hd - a.n_q : hd - a.n_q - a.n_kv;
  const int64_t at = (int64_t)r * a.row_stride + (slot * a.n_kv + kvh) * kHeadDim + d;
  void* cache = is_k ? a.k_cache : a.v_cache;
  if (a.cache_bf16) ((uint16_t*)cache)[at] = f32_to_bf16_rne(x);
  else ((float*)cache)[at] = x;
}

// Stand-alone epilogue: one wave per (head, row) of a float32 q/k/v output.
__global__ __launch_bounds__(64) void rope_kv_kernel(const float* __restrict__ qkv, int64_t ld, RopeKvArgs a) {
  const int hd = blockIdx.x, r = blockIdx.y, d = threadIdx.x;
  rope_kv_head(qkv[(int64_t)r * ld + (int64_t)hd * kHeadDim + d], d, hd, r, a);
}

// Fused: the q/k/v matvec (bf16 x) with the epilogue. One workgroup per head
// (four 16-column tiles); wave w folds segments (w & 3) + 4 j of tile w >> 2
// with the decode kernels' own per-tile arithmetic (qmv_fold_segment, then
// qmv_ordered_sum), so the head's 64 values are bit-identical to qmv_rows
// before the epilogue runs on them.
constexpr int kQkvWaves = 16;
__host__ __device__ inline size_t qkv_rope_lds_bytes(int64_t K, int NV, int R) {
  return 4 * (size_t)qmv_segments(K) * NV * 64 * sizeof(float) + (size_t)R * kHeadDim * sizeof(float) +
         (size_t)R * qmv_xs_stride(K) * 2;
}

template <int SPW, int NV, int BITS>
__global__ __launch_bounds__(kQkvWaves * 64) void qkv_rope_kernel(const uint8_t* __restrict__ pk, int N, int K,
                                                                 const uint16_t* __restrict__ x, int64_t ldx, int R, RopeKvArgs a) {
  extern __shared__ __align__(16) uint8_t smem[];
  const int hd = blockIdx.x;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int tt = wave >> 2, sub = wave & 3;
  const int i = lane & 15, kc = lane >> 4;
  const int G = K / kGroup, P = (G + 1) / 2, nseg = qmv_segments(K);
  const size_t part_tile = (size_t)nseg * NV * 64;  // floats per tile
  float* part = (float*)smem + tt * part_tile;
  float* hb = (float*)smem + 4 * part_tile;  // [R][64] the head's values
  uint16_t* xs = (uint16_t*)(hb + R * kHeadDim);
  const int xsi = (int)qmv_xs_stride(K);
  const int64_t cb = codes_bytes(N, K, BITS);
  const int t = 4 * hd + tt;
  rsrc_t cres[1], sres[1];
  cres[0] = make_rsrc(pk + (int64_t)t * P * pair_code_bytes(BITS), (uint32_t)P * pair_code_bytes(BITS));
  sres[0] = make_rsrc(pk + cb + (int64_t)t * P * kPairSbBytes, (uint32_t)P * kPairSbBytes);
  const rsrc_t xres = make_rsrc(x, (uint32_t)(R * ldx * 2));

  // activations first, then every weight load, then the staging stores
  constexpr int kThreads = kQkvWaves * 64;
  const int per_row = K / 8;
  const int jmax = (per_row + kThreads - 1) / kThreads;
  auto xload = [&](int r, int j) -> u32x4 {
    int c = (int)threadIdx.x + j * kThreads;
    c = c < per_row ? c : per_row - 1;
    return buf_load16(xres, (uint32_t)c * 16u, (uint32_t)(r * ldx * 2));
  };
  auto xput = [&](int r, int j, const u32x4& v) {
    const int c = (int)threadIdx.x + j * kThreads;
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
  QmvWeights<1, SPW, BITS> wts;
  qmv_issue_weights<1, SPW, BITS>(wts, cres, sres, sub, 4, P, lane, true);
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

  const int frow = i < R ? i : R - 1;
  auto xfrag = [&](int, int g, int hh) -> bf16x8 {
    return __builtin_bit_cast(bf16x8, *(const u32x4*)(xs + frow * xsi + g * kGroup + hh * 32 + kc * 8));
  };
#pragma unroll
  for (int j = 0; j < SPW; ++j) {
    const int seg = sub + 4 * j;
    if (seg >= nseg) break;
    float acc[1][1][NV];
    qmv_fold_segment<0, 1, 1, NV>(acc, wts.cw[j], wts.sbw[j], seg * kSegGroups, G, xfrag);
#pragma unroll
    for (int v = 0; v < NV; ++v) part[qmv_part_index<1, 1, NV>(seg, 0, 0, v, lane)] = acc[0][0][v];
  }
  __syncthreads();
  if (sub == 0) {
    float tot[1][1][NV];
    qmv_ordered_sum<1, 1, NV>(tot, part, nseg, lane);
#pragma unroll
    for (int v = 0; v < NV; ++v) {
      const int r = 4 * kc + v;
      if (r < R) hb[r * kHeadDim + tt * kTileN + i] = tot[0][0][v];
    }
  }
  __syncthreads();
  if (wave < R) rope_kv_head(hb[wave * kHeadDim + lane], lane, hd, wave, a);
}

}  // namespace q4
