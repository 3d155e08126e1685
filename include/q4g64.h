/*
 * q4g64 — 4-bit group-64 weight-only quantized matmul for MI355X (gfx950).
 *
 * C ABI. Plain pointers and sizes; no HIP, torch or C++ types in signatures.
 *
 * The operation (TensorFold PR #1696, "What it adds": the LFM3 projections use
 * MLX 4-bit group-64 weights read as stored; later revision, "What it adds":
 * N-row decode matvecs, fused w1 + w3 + SwiGLU and fused attention matvecs,
 * and the prompt GEMM that dequantizes weight tiles as it loads them):
 *
 *     q[n][k] = (wq[n][k/8] >> 4*(k%8)) & 0xF               codes, low nibble first
 *     w[n][k] = scale[n][k/64] * q[n][k] + bias[n][k/64]    affine dequantization
 *     y[r][n] = sum_k w[n][k] * x[r][k]                     float32 result
 *     SwiGLU:  z = silu(w1 x) * (w3 x),  silu(a) = a / (1 + exp(-a))
 *
 * Canonical weight input ("MLX q4g64"):
 *     wq      uint32 [N][K/8]    (row-major, contiguous)
 *     scales  uint16 [N][K/64]   bf16 bit patterns
 *     biases  uint16 [N][K/64]   bf16 bit patterns
 *
 * Device ("packed") layout, produced by pack_q4g64 and read by every kernel.
 * With T = N/16 column tiles, G = K/64 groups and P = ceil(G/2) group pairs:
 *   - codes: T*P blocks of 1024 bytes, block (t, p) at byte (t*P + p)*1024.
 *     Lane L (0..63) of a wave reads the 16 bytes at L*16: four 32-bit words
 *     h = 0..3 holding the 8 codes of column n = 16t + L%16 at
 *     k = 128p + 32h + 8*(L/16) + e, e = 0..7, code e at nibble 2e (e < 4)
 *     or 2(e-4)+1 (e >= 4). Words past K (odd G) are zero.
 *   - scale/bias: T*P blocks of 128 bytes after the codes; block (t, p),
 *     column c = 0..15 at byte c*8: bf16 {scale, bias} of group 2p then of
 *     group 2p+1 (zero past G).
 *   Size: T*P*1152 bytes = 0.5625*N*K bytes for even G.
 *
 * Wider codes (the *_qg64 calls with bits = 6 or 8; PR #1514, "What
 * changes": the MLX 4-, 6- and 8-bit checkpoints are served as stored; the
 * pages give no bit layout, so this reading is the plain generalisation of
 * the 4-bit one):
 *   - canonical wq is uint32 [N][K*bits/32]; the words of a row form one
 *     little-endian bit stream and code k occupies bits bits*k .. bits*k +
 *     bits - 1 (8-bit: the bytes of each word in order; 6-bit: codes
 *     straddle words). Scales, biases and the dequantization are unchanged.
 *   - packed codes: T*P blocks of 256*bits bytes. 8-bit: two 1024-byte
 *     sub-blocks, one per group of the pair; lane L's 16 bytes in sub-block
 *     j hold, for half hh = 0, 1 (k = 128p + 64j + 32hh + 8*(L/16) + e), two
 *     words with codes e = 0..3 and 4..7, one per byte in order. 6-bit: a
 *     1024-byte sub-block of the low four bits laid out exactly as the
 *     4-bit codes above, then a 512-byte sub-block where lane L's two words
 *     j = 0, 1 hold the top two bits of halves h = 2j and 2j+1: byte b
 *     carries, from bit 0, those of codes b and 4+b of half 2j, then of
 *     codes b and 4+b of half 2j+1.
 *   - scale/bias blocks follow the codes as for 4 bits.
 *   The matrix cores take every code as an exact bf16 integer, so the
 *   summation orders below are the same for every width.
 *
 * Summation order. Each 64-wide group is reduced on the matrix cores into
 * P_g = sum q*x and S_g = sum x (exact products, float32 sums). Decode calls
 * (qmv_rows, qmv_w13_swiglu) fold acc = fma(s_g, P_g, fma(b_g, S_g, acc)) in
 * ascending g within each 256-wide k segment, from zero, and add the
 * segments in ascending order. qmm_window folds one chain over all of K:
 * acc = fma(s_g, P_g, acc) in ascending g, and after every 8 groups (and
 * after the last) acc = acc + sum over those groups of b_g * S_g, formed on
 * the matrix cores from the exact bf16 pieces h + m + l = S_g.
 * Each order is a function of K alone: a row's bits never depend on R, on M,
 * on the window cut, on the row's position or on the other rows.
 *
 * Conventions for every call below:
 *   - All array arguments are DEVICE pointers owned by the caller; the
 *     library allocates nothing and keeps no device state between calls
 *     (except the fixed scratch array of qmv_rows_split_noalloc, below).
 *   - Host-side caches, per process: the largest dynamic LDS a workgroup may
 *     use and the number of compute units are queried once, on the device
 *     current at the first call that needs them, and each kernel's LDS limit
 *     is raised once, at its first launch. Every GPU this library runs on must therefore be of the same
 *     kind (all MI355X); results never depend on these values.
 *   - `stream` is a hipStream_t (NULL = the default stream). Kernels are
 *     enqueued asynchronously on it; execution errors surface at the caller's
 *     next synchronization.
 *   - Arguments are validated on the host before anything is enqueued; on any
 *     error nothing is enqueued and a negative status is returned, with a
 *     message available from q4_last_error() on the calling thread.
 *   - N and K must be positive multiples of 64. Packed buffers, x and wq must
 *     be 16-byte aligned; x row strides (ldx, in elements) must keep every row
 *     16-byte aligned. Outputs must not alias inputs.
 *   - Every row stride (ldx, ldy, ldz, ldq, ldg, ldqkv, cache_row_stride) is
 *     at most 2^40 elements (Q4_EINVAL otherwise), so no offset a call forms
 *     overflows 64-bit arithmetic.
 *   - The caller passes the same (N, K) to pack_q4g64 and to every use.
 */
#ifndef Q4G64_H
#define Q4G64_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define Q4_OK 0
#define Q4_EINVAL (-1)       /* bad shape, count, stride or dtype */
#define Q4_EALIGN (-2)       /* null or misaligned pointer / stride */
#define Q4_EDEVICE (-3)      /* a HIP call or kernel launch failed */
#define Q4_EUNSUPPORTED (-4) /* valid request outside what this build implements */

#define Q4_BF16 0   /* bf16 bit patterns stored as uint16 */
#define Q4_F32 1    /* IEEE float32 */
#define Q4_BF16X3 2 /* float32 values as three exact bf16 pieces, planes [3][R][ld] of uint16:
                     * h = the top 16 bits of x, m = the top 16 bits of x - h, l = x - h - m
                     * (each exact in bf16), x = h + m + l; plane p starts R * ld elements
                     * after plane p - 1 */
#define Q4_BF16X3T 3 /* the same pieces in fragment order, q4g64_x3t_bytes(K, R) bytes:
                      * piece p (0..2) of element k of row r is uint16 number
                      * ((((k/64) * T + r/4) * 2 + (k/32)%2) * 64 + 4*(r%4) + p + 16*((k/8)%4)) * 8 + k%8,
                      * T = 1, 2 or 4 row tiles for R <= 4, <= 8, <= 16. Slots of
                      * p = 3 and of rows >= R are not read into any result. One
                      * 16-byte read per lane then fetches a whole matrix fragment
                      * (a wave reads 1 KiB of consecutive bytes) */

/* ABI version of this header (incremented on incompatible changes). */
int q4g64_abi_version(void);

/* Bytes of the packed device layout for an N x K matrix; 0 if (N, K) is invalid. */
size_t q4g64_packed_bytes(int64_t N, int64_t K);

/* Bytes of R rows of K activations as Q4_BF16X3T; 0 if K is not a positive
 * multiple of 64 (at most 16384) or R is outside 1..16. */
size_t q4g64_x3t_bytes(int64_t K, int R);

/* Canonical MLX q4g64 (wq, scales, biases on the device) -> packed layout.
 * An integer permutation of the input bits: bit-exact and invertible.
 * `packed` must hold q4g64_packed_bytes(N, K) bytes. */
int pack_q4g64(const uint32_t* wq, const uint16_t* scales, const uint16_t* biases, int64_t N, int64_t K,
               void* packed, void* stream);

/* Inverse of pack_q4g64: packed layout -> canonical wq [N][K/8], scales and biases [N][K/64]. */
int unpack_q4g64(const void* packed, int64_t N, int64_t K, uint32_t* wq, uint16_t* scales, uint16_t* biases,
                 void* stream);

/* The same three calls for bits = 4, 6 or 8 (Q4_EINVAL otherwise; 0 bytes
 * from qg64_packed_bytes). wq is [N][K*bits/32]; bits = 4 is identical to
 * the q4g64 calls. The caller passes the same bits, N and K to every use. */
size_t qg64_packed_bytes(int bits, int64_t N, int64_t K);
int pack_qg64(int bits, const uint32_t* wq, const uint16_t* scales, const uint16_t* biases, int64_t N, int64_t K,
              void* packed, void* stream);
int unpack_qg64(int bits, const void* packed, int64_t N, int64_t K, uint32_t* wq, uint16_t* scales, uint16_t* biases,
                void* stream);

/* Decode matvec over R = 1..16 rows (PR #1696, later revision, "What it adds":
 * N-row matvecs for streams that share a decode step).
 *   x: R rows of K activations, row stride ldx elements; x_dtype Q4_BF16,
 *      Q4_F32 (float32 rows are split into three exact bf16 pieces), or
 *      Q4_BF16X3 (the same pieces given as planes, as qmv_w13_swiglu_x3
 *      writes them: bit-identical results to Q4_F32 on the same values,
 *      without the split in every workgroup), or Q4_BF16X3T (the pieces in
 *      fragment order, as qmv_w13_swiglu_x3t writes them for the same R;
 *      ldx must equal K; bit-identical results again; from 4 rows on the
 *      fragments come from memory, where this order reads whole cache
 *      lines). The layout depends on R through its row-tile count, so a
 *      buffer written for one R is read with that R.
 *   y: float32 [R][ldy], ldy >= N.
 * Row r of y is bit-identical to the result of the same call with R = 1 on
 * that row alone. Limits: K <= 16384 (bf16 x) / 16384 (float32 x). */
int qmv_rows(const void* packed, int64_t N, int64_t K, const void* x, int x_dtype, int64_t ldx, int R, float* y,
             int64_t ldy, void* stream);

/* qmv_rows for bits = 4, 6 or 8 (`packed` from pack_qg64 with the same bits). */
int qmv_rows_qg64(int bits, const void* packed, int64_t N, int64_t K, const void* x, int x_dtype, int64_t ldx, int R,
                  float* y, int64_t ldy, void* stream);

/* qmv_rows (bits = 4, 6 or 8) with K split over several workgroups per
 * 16-column tile, for matrices with too few column tiles to give every CU
 * one (TensorFold PR #1696, later revision, "What it adds" > Exact speed
 * work: the rows sharing a decode step are summed as the one-row kernels sum
 * them). Each workgroup of a tile folds a run of consecutive 256-wide k
 * segments; the last of them to finish adds all of the tile's segment
 * partials in the same ascending order as qmv_rows, so y is bit-identical to
 * qmv_rows_qg64 on the same arguments, for every value of splits.
 *   splits: workgroups per tile, 1..16 (at most the K/256 segments), or 0
 *           for the smallest power of two that gives each CU a workgroup.
 *   work:   a DEVICE buffer of at least qmv_split_work_bytes(bits, N, K,
 *           x_dtype, R, splits) bytes (work_bytes says how many it holds),
 *           256-byte aligned, zero-filled by the caller before its first
 *           use: it holds one arrival counter per tile, which every
 *           completed call returns to zero, and the segment partials. One
 *           workspace serves any later call of any shape that fits in it;
 *           calls that share a workspace must not run concurrently. When
 *           the split comes out as 1, work may be NULL.
 * Other arguments and limits as qmv_rows. qmv_split_work_bytes returns 0 for
 * invalid arguments. */
size_t qmv_split_work_bytes(int bits, int64_t N, int64_t K, int x_dtype, int R, int splits);
int qmv_rows_split(int bits, const void* packed, int64_t N, int64_t K, const void* x, int x_dtype, int64_t ldx, int R, float* y,
                   int64_t ldy, int splits, void* work, size_t work_bytes, void* stream);

/* qmv_rows_split without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, serving loops that
 * forbid allocation). It allocates nothing: its workspace is a fixed
 * device array inside the library, qmv_split_noalloc_max_bytes() bytes
 * (8 MiB) on each GPU it runs on, held until the process ends. The first
 * call on a device looks the array up and clears its counters with a kernel
 * on `stream`. Shapes whose qmv_split_work_bytes exceeds the array return
 * Q4_EUNSUPPORTED. Every call on one GPU shares that GPU's array: calls that
 * overlap on one GPU (other streams, other threads) race and must not be
 * issued. Results are bit-identical to qmv_rows_split and qmv_rows. */
size_t qmv_split_noalloc_max_bytes(void);
int qmv_rows_split_noalloc(int bits, const void* packed, int64_t N, int64_t K, const void* x, int x_dtype, int64_t ldx, int R,
                           float* y, int64_t ldy, int splits, void* stream);

/* Fused decode FFN gate (PR #1696, "What it adds": w1 + w3 + SwiGLU in one
 * pass): y[r][n] = silu(a) * c with a = (w1 x)[r][n], c = (w3 x)[r][n], each
 * computed in qmv_rows' order; bit-equal to composing two qmv_rows results
 * with the same float32 silu. x bf16 [R][ldx], y float32 [R][ldy], R = 1..16,
 * K <= 8192. */
int qmv_w13_swiglu(const void* packed_w1, const void* packed_w3, int64_t N, int64_t K, const uint16_t* x,
                   int64_t ldx, int R, float* y, int64_t ldy, void* stream);

/* qmv_w13_swiglu for bits = 4, 6 or 8 (both matrices packed with that bits). */
int qmv_w13_swiglu_qg64(int bits, const void* packed_w1, const void* packed_w3, int64_t N, int64_t K, const uint16_t* x,
                        int64_t ldx, int R, float* y, int64_t ldy, void* stream);

/* qmv_w13_swiglu (bits = 4, 6 or 8) writing each float32 result as its three
 * exact bf16 pieces: z3 is Q4_BF16X3 planes [3][R][ldz], ldz >= N, ldz * 2 a
 * multiple of 16 so the planes feed qmv_rows directly (the decode FFN's w2
 * takes the SwiGLU output unrounded). h + m + l equals the float32 result of
 * qmv_w13_swiglu_qg64 bit for bit. */
int qmv_w13_swiglu_x3(int bits, const void* packed_w1, const void* packed_w3, int64_t N, int64_t K, const uint16_t* x,
                      int64_t ldx, int R, uint16_t* z3, int64_t ldz, void* stream);

/* The same with the pieces written as Q4_BF16X3T for N activations per row:
 * z3t holds q4g64_x3t_bytes(N, R) bytes (16-byte aligned), the x of a
 * following qmv_rows over a matrix with K = N. Slots the layout leaves
 * unread are not written. */
int qmv_w13_swiglu_x3t(int bits, const void* packed_w1, const void* packed_w3, int64_t N, int64_t K, const uint16_t* x,
                       int64_t ldx, int R, uint16_t* z3t, void* stream);

/* Prompt-window GEMM (PR #1696, later revision, "What it adds": pgemm).
 *   x: bf16 [M][ldx], any M >= 1.
 *   packed_b == NULL: y = A x.  packed_b != NULL: y = silu(A x) * (B x), the
 *   paired w1/w3 projections with the SwiGLU epilogue (PR #1514, "What
 *   changes": paired FFN projections keep their rounding boundaries).
 *   y: [M][ldy], y_dtype Q4_F32 or Q4_BF16 (round to nearest even).
 * A row's result does not depend on M, on its offset or on the other rows.
 * Limits: M <= 2^24, K <= 2^20, 512 * ldx < 2^31, M * ldx and M * ldy at
 * most 2^48 elements (Q4_EINVAL / Q4_EUNSUPPORTED). */
int qmm_window(const void* packed_a, const void* packed_b, int64_t N, int64_t K, const uint16_t* x, int64_t ldx,
               int64_t M, void* y, int y_dtype, int64_t ldy, void* stream);

/* qmm_window for bits = 4, 6 or 8 (both matrices packed with that bits). */
int qmm_window_qg64(int bits, const void* packed_a, const void* packed_b, int64_t N, int64_t K, const uint16_t* x,
                    int64_t ldx, int64_t M, void* y, int y_dtype, int64_t ldy, void* stream);

/* Window driver: runs qmm_window over consecutive windows of a prompt.
 * window_rows is a HOST array of n_windows positive row counts; window w
 * covers rows [sum of earlier counts, + window_rows[w]) of x and y. The
 * result is bit-identical for every cut (PR #1696, later revision, "Checks":
 * windows of 64, 128, 256 and a ragged cut agree bit for bit). Every count
 * is checked before any window is enqueued, and the total rows obey the
 * 2^48-element span limit of qmm_window. */
int qmm_cut(const void* packed_a, const void* packed_b, int64_t N, int64_t K, const uint16_t* x, int64_t ldx,
            const int64_t* window_rows, int n_windows, void* y, int y_dtype, int64_t ldy, void* stream);

/* qmm_cut for bits = 4, 6 or 8. */
int qmm_cut_qg64(int bits, const void* packed_a, const void* packed_b, int64_t N, int64_t K, const uint16_t* x, int64_t ldx,
                 const int64_t* window_rows, int n_windows, void* y, int y_dtype, int64_t ldy, void* stream);

/* Decode FFN step (PR #1696, "What it adds": w1 + w3 + SwiGLU in one pass;
 * PR #1514, "What changes": the fusion keeps every rounding boundary):
 *   z = silu(W1 x) * (W3 x)   float32 [R][ldz], bit-identical to qmv_w13_swiglu;
 *   y = W2 z                  float32 [R][ldy], bit-identical to qmv_rows on z
 *                             with x_dtype = Q4_F32.
 * W1, W3: N1 x K1 packed; W2: N2 x N1 packed. x bf16 [R][ldx], R = 1..16.
 * work: a DEVICE buffer of q4g64_ffn_work_bytes(N1, N2, R) bytes (0 means
 * the arguments are invalid; the size does not depend on R), 256-byte
 * aligned, zero-filled by the caller before its first use; every completed
 * call leaves it ready for the next, and one workspace serves any later call
 * with the same N1 and N2 and any R (calls on one workspace must not run
 * concurrently). Two schedules:
 *   - R <= 2 with K1 and N1 multiples of 256: one launch, one workgroup per
 *     CU with every workgroup resident at once (the call needs the whole
 *     device). Each z value is also stored in the workspace with this call's
 *     number (a counter in the workspace that every such call advances), and
 *     each w2 k segment starts as soon as its 256 z values carry that number;
 *     the two halves of K of a w2 tile hand over a running sum the same way.
 *     No workgroup waits for the whole grid. A workgroup that waits more than
 *     about 20 ms gives up, sets the 32-bit word at byte 2304 of work to 1 and
 *     leaves y undefined; the workspace must then be zero-filled again.
 *   - otherwise: two launches, w1/w3 + SwiGLU writing z and its three exact
 *     bf16 pieces in fragment order (Q4_BF16X3T) into the workspace, then w2
 *     reading those (qmv_rows gives the same bits for them as for z).
 * Limits: K1 <= 4096, N1 <= 8192 (Q4_EUNSUPPORTED otherwise). */
size_t q4g64_ffn_work_bytes(int64_t N1, int64_t N2, int R);
int qmv_ffn(const void* packed_w1, const void* packed_w3, const void* packed_w2, int64_t N1, int64_t K1, int64_t N2,
            const uint16_t* x, int64_t ldx, int R, float* z, int64_t ldz, float* y, int64_t ldy, void* work, void* stream);

/* Message of the last failed call on this thread ("" if none). */
const char* q4_last_error(void);

/* Block FP8, weight-only (TensorFold PR #1696, first revision, "Stacked on"
 * and "Checks": the CUDA engine it builds on and checks against serves the
 * LFM3 block FP8 export weight-only; the pages give no format, so this
 * reading is the common block-FP8 checkpoint layout):
 *     w8      uint8 [N][K]   OCP FP8 E4M3 bytes (bias 7, 3 mantissa bits,
 *                            exponent field 0 subnormal, 0x7F/0xFF NaN)
 *     scales  float32 [ceil(N/128)][ceil(K/128)], one per 128 x 128 block
 *     w[n][k] = e4m3(w8[n][k]) * scales[n/128][k/128]
 * Packed layout: the 8-bit code layout above holding the E4M3 bytes, then
 * the scale/bias blocks with both 32-bit words of pair p of column n set to
 * the float32 scale of block (n/128, p) (fp8b_packed_bytes = the 8-bit size).
 * The calls mirror their q4g64 counterparts (same arguments, limits and
 * row/cut bit rules). Every finite E4M3 value is a bf16 value, so the codes
 * enter the matrix cores exactly; there is no bias, so each group folds as
 * acc = fma(s_g, P_g, acc) in the decode order and the window order. */
size_t fp8b_packed_bytes(int64_t N, int64_t K);
int pack_fp8b(const uint8_t* w8, const float* scales, int64_t N, int64_t K, void* packed, void* stream);
int unpack_fp8b(const void* packed, int64_t N, int64_t K, uint8_t* w8, float* scales, void* stream);
int qmv_rows_fp8b(const void* packed, int64_t N, int64_t K, const void* x, int x_dtype, int64_t ldx, int R, float* y,
                  int64_t ldy, void* stream);
int qmv_w13_swiglu_fp8b(const void* packed_w1, const void* packed_w3, int64_t N, int64_t K, const uint16_t* x, int64_t ldx,
                        int R, float* y, int64_t ldy, void* stream);
int qmv_w13_swiglu_x3_fp8b(const void* packed_w1, const void* packed_w3, int64_t N, int64_t K, const uint16_t* x, int64_t ldx,
                           int R, uint16_t* z3, int64_t ldz, void* stream);
int qmv_w13_swiglu_x3t_fp8b(const void* packed_w1, const void* packed_w3, int64_t N, int64_t K, const uint16_t* x, int64_t ldx,
                            int R, uint16_t* z3t, void* stream);
int qmm_window_fp8b(const void* packed_a, const void* packed_b, int64_t N, int64_t K, const uint16_t* x, int64_t ldx,
                    int64_t M, void* y, int y_dtype, int64_t ldy, void* stream);
int qmm_cut_fp8b(const void* packed_a, const void* packed_b, int64_t N, int64_t K, const uint16_t* x, int64_t ldx,
                 const int64_t* window_rows, int n_windows, void* y, int y_dtype, int64_t ldy, void* stream);

/* Attention-side decode epilogue (PR #1696, "What it adds": the LFM3 kernels
 * include QK norm with partial RoPE and GQA attention over a KV ring; decode
 * fuses RoPE with the KV store). The pages give no formulas; readings:
 *   - a row of the stacked q/k/v matvec output is [q heads | k heads | v
 *     heads], 64 values per head, N = (n_q_heads + 2 n_kv_heads) * 64;
 *   - QK norm (when gamma_q / gamma_k is not NULL): per q (k) head,
 *     x <- (x * r) * gamma[d], r = 1 / sqrt(sum(x^2) / 64 + eps);
 *   - partial RoPE on q and k: the first rot_dims dims of a head rotate in
 *     half-split pairs (i, i + rot_dims/2) by pos * theta^(-2i/rot_dims)
 *     (cos and sin of the angle formed in double, rounded once to float);
 *   - q goes to q_out; k and v go to slot pos mod ring_len of k_cache and
 *     v_cache, each [ring_len][n_kv_heads][64] of cache_dtype (Q4_F32, or
 *     Q4_BF16 rounded to nearest even). Other slots are not touched;
 *   - rows of separate streams keep separate rings: row r writes the ring
 *     that starts cache_row_stride * r elements after k_cache (v_cache).
 *     cache_row_stride = 0 makes every row write one shared ring; rows whose
 *     slots coincide then write the same words and which row's values
 *     remain is undefined (the positions are device data, so the host
 *     cannot check). A nonzero stride must be at least ring_len *
 *     n_kv_heads * 64, so the rows' rings do not overlap;
 *   - gated attention's fourth matvec: n_gate_heads further heads may follow
 *     the v heads in the stacked output (PR #1696, "What it adds": gated GQA
 *     attention; decode fuses the four attention matvecs). Their values go
 *     to gate_out unchanged (no norm, no rotation): the gate acts inside
 *     attention, which these calls do not compute.
 * All pointers in the struct are DEVICE pointers except the struct itself,
 * which is read on the host when the call is made. */
typedef struct q4_rope_kv {
  const int32_t* pos;     /* [R] position of each row (slot = pos mod ring_len) */
  int32_t n_q_heads;      /* >= 1 */
  int32_t n_kv_heads;     /* >= 1 */
  int32_t rot_dims;       /* even, 0..64 */
  float theta;            /* rotary base, > 0 */
  const float* gamma_q;   /* [64] or NULL: no norm on q */
  const float* gamma_k;   /* [64] or NULL: no norm on k */
  float eps;              /* >= 0 */
  float* q_out;           /* float32 [R][ldq], ldq >= n_q_heads * 64 */
  int64_t ldq;
  void* k_cache;          /* [ring_len][n_kv_heads][64] */
  void* v_cache;
  int32_t cache_dtype;    /* Q4_F32 or Q4_BF16 */
  int64_t ring_len;       /* 1..2^31 (positions are int32) */
  int32_t n_gate_heads;   /* >= 0 gate heads after the v heads */
  float* gate_out;        /* float32 [R][ldg], ldg >= n_gate_heads * 64; may be NULL when n_gate_heads = 0 */
  int64_t ldg;
  int64_t cache_row_stride; /* elements between row r's ring and row r+1's; 0 = one shared ring (ABI 3) */
} q4_rope_kv;

/* The epilogue alone, on a float32 q/k/v(/gate) output qkv [R][ldqkv], ldqkv
 * >= (n_q_heads + 2 n_kv_heads + n_gate_heads) * 64 (for example qmv_rows
 * over the stacked [Wq; Wk; Wv; Wg]); R >= 1. */
int rope_kv_store(const float* qkv, int64_t ldqkv, int R, const q4_rope_kv* args, void* stream);

/* The stacked q/k/v matvec (bits = 4, 6 or 8, bf16 x [R][ldx], R = 1..16,
 * K <= 4096, N = (n_q_heads + 2 n_kv_heads + n_gate_heads) * 64) with the
 * epilogue in the same launch, one workgroup per head. q_out, gate_out and
 * the cache contents are bit-identical to qmv_rows_qg64 followed by
 * rope_kv_store, and a row's results do not depend on R or on the other
 * rows. */
int qmv_qkv_rope(int bits, const void* packed_qkv, int64_t K, const uint16_t* x, int64_t ldx, int R, const q4_rope_kv* args,
                 void* stream);

/* Window-cost table (TensorFold PR #1696, later revision, "What it adds" >
 * Exact speed work: the cost of a window is measured once, when the model
 * loads, at five row counts from 1 to 16, and costs in between are
 * interpolated; a planner uses them to choose how many streams' rows share
 * a decode step).
 *
 * qmv_window_costs times qmv_rows_qg64 on `packed` at R = 1, 2, 4, 8, 16
 * (bits = 4, 6 or 8; x and y must hold 16 rows), each as the average of `reps` (1..10000)
 * back-to-back launches between two HIP events on `stream`, and writes the
 * five averages in microseconds to the HOST array us_out[5]. It blocks until
 * the timing is done (a load-time call) and creates and destroys its two
 * events; it allocates no device memory. Arguments are validated as for
 * qmv_rows_qg64 at R = 16; timing failures return Q4_EDEVICE.
 *
 * qmv_window_cost returns the cost of R rows (1..16) read off the table by
 * linear interpolation between the two timed row counts around R (exact at
 * 1, 2, 4, 8, 16); NaN for R outside 1..16 or a NULL table. Host only. */
int qmv_window_costs(int bits, const void* packed, int64_t N, int64_t K, const void* x, int x_dtype, int64_t ldx, float* y,
                     int64_t ldy, int reps, float* us_out, void* stream);
float qmv_window_cost(const float* us, int R);

#ifdef __cplusplus
}
#endif

#endif /* Q4G64_H */
