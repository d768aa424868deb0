/*
 * fa.h -- C ABI of libfa.so: exact tiled softmax attention on AMD MI355X
 * (gfx950).
 *
 * What is computed.  For every batch b and head h, with S = scale * Q K^T
 * (N x N) and, when causal, S[i][j] = -inf for key j > query i (top-left
 * alignment, equal query and key lengths):
 *
 *     O   = softmax_rows(S) V
 *     LSE = m + ln(sum_j exp(S[i][j] - m)),   m = max_j S[i][j]   (natural log)
 *
 * This is exact attention ("FlashAttention: Fast and Memory-Efficient Exact
 * Attention with IO-Awareness", abstract): the kernels stream key/value tiles
 * through on-chip memory with an online softmax (running row maximum and
 * normaliser, rescaled output accumulator; FlashAttention-4 related-papers
 * page, online-softmax snippet) so the N x N matrix never reaches HBM, but
 * the result is the definition above up to floating-point rounding.
 *
 * Layout.  Q, K, V, O, dO, dK, dV and the fp8 tensors are contiguous
 * row-major [B][H][N][d] (d fastest).  LSE, the backward's D = rowsum(dO o O)
 * and the fp8 block scales are contiguous [B][H][N] / [B][H][ceil(N/128)].
 * Base pointers must be 16-byte aligned.  Offsets are 64-bit inside the
 * library, so any tensor that fits in device memory is addressable.
 *
 * Ownership.  Every pointer is device memory owned by the caller.  The
 * library allocates nothing, frees nothing and never synchronises; work is
 * enqueued on the caller's stream (a hipStream_t passed as void*, NULL = the
 * null stream) and completes asynchronously.  Inputs are read only; outputs
 * are fully overwritten.  No global mutable state: calls are reentrant and may
 * run concurrently on different streams as long as their output buffers do
 * not overlap.
 *
 * Errors.  Argument problems are reported synchronously, before anything is
 * enqueued: FA_ERR_INVALID for null pointers, non-positive sizes, unknown
 * dtype, misaligned pointers or a non-finite or non-positive scale;
 * FA_ERR_UNSUPPORTED for a head dimension other than 64, 128 or 256 (and,
 * for fa_bwd and fa_bwd_workspace_size, for d = 256: the backward is built
 * for d = 64 and 128 only).
 * FA_ERR_LAUNCH means the HIP runtime refused a kernel launch.  Faults inside
 * a kernel surface at the caller's next synchronisation.
 */
#ifndef FA_H_
#define FA_H_

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. */
#define FA_OK 0
#define FA_ERR_INVALID (-1)
#define FA_ERR_UNSUPPORTED (-2)
#define FA_ERR_LAUNCH (-3)
#define FA_ERR_TOO_LARGE (-4) /* above the fixed scratch of fa_bwd_noalloc */

/* Element types of the 16-bit inputs. */
#define FA_BF16 0
#define FA_FP16 1

/* Rows per fp8 quantisation block (per (b, h), all d columns). */
#define FA_FP8_BLOCK 128

/* Scale modes of fa_quant_fp8. */
#define FA_FP8_BLOCK_SCALES 0
#define FA_FP8_TENSOR_SCALE 1
#define FA_FP8_BLOCK_POW2 2

/*
 * fa_fwd -- attention forward.
 *   q, k, v : [B][H][N][d] of `dtype` (FA_BF16 or FA_FP16), read only.
 *   o       : [B][H][N][d] of `dtype`, written (rounded to nearest even).
 *   lse     : [B][H][N] float, written; natural-log log-sum-exp of each
 *             query row's scaled scores (scale included).  May be NULL when
 *             the caller does not need it.
 *   B, H, N : >= 1.  d : 64, 128 or 256.
 *   scale   : softmax scale (1/sqrt(d) is the usual choice), finite, > 0.
 *   causal  : 0 = full attention, 1 = key j visible to query i iff j <= i.
 *   stream  : hipStream_t.
 * The scores, probabilities and accumulators are fp32 inside the kernel;
 * both products run on bf16/fp16 matrix-core instructions.
 */
int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
           int B, int H, int N, int d, int dtype, float scale, int causal,
           void* stream);

/*
 * fa_quant_fp8 -- e4m3 quantisation for the fp8 forward
 * ("FlashAttention-3: Fast and Accurate Attention with Asynchrony and
 * Low-precision", abstract: block quantisation and incoherent processing).
 *   x         : [B][H][N][d] of `dtype`, read only.
 *   x8        : [B][H][N][d] uint8 e4m3 codes (OCP E4M3FN: bias 7, max 448,
 *               no infinities), written.
 *   scales    : [B][H][ceil(N/128)] float, written.  Dequantised element =
 *               code value * scales[b][h][row/128].
 *   signs     : device array of d floats, each +1 or -1, or NULL.  Non-NULL
 *               applies the incoherent-processing rotation x' = H_d (s o x)
 *               with H_d the unnormalised Sylvester Hadamard matrix,
 *               computed in fp32 by the fast Walsh-Hadamard transform
 *               (half-widths 1, 2, ..., d/2 in that order).  NULL = x' = x.
 *   scale_mul : multiplies every stored scale (1/d for a rotated Q, so that
 *               dequantised Q.K equals the unrotated product; else 1).
 *   mode      : FA_FP8_BLOCK_SCALES (0): one scale per 128-row block of
 *               each (b, h); FA_FP8_TENSOR_SCALE (1): one scale for the whole
 *               tensor, written to every slot; FA_FP8_BLOCK_POW2 (2): block
 *               scales rounded up to the nearest power of two (for V: the
 *               fp8 forward then applies them as exact exponents of its
 *               matrix instructions).  Other values: FA_ERR_INVALID.
 *   Scale = amax(|x'|) / 448 in fp32 (1 if the amax is 0), in mode 2 rounded
 *   up to a power of two, times scale_mul; code = round-to-nearest-even of
 *   x' / scale (that scale, before scale_mul) in fp32, saturated to +-448.
 *   Mode 1 enqueues three kernels (block amax, reduction into every slot of
 *   `scales`, quantisation); modes 0 and 2 enqueue one.
 */
int fa_quant_fp8(const void* x, int dtype, void* x8, float* scales,
                 const float* signs, float scale_mul, int mode,
                 int B, int H, int N, int d, void* stream);

/*
 * fa_fwd_fp8 -- attention forward on e4m3 operands: the FP8 variant of the
 * same exact attention, with one scale per block of rows instead of per
 * tensor and incoherent processing of Q and K ("FlashAttention-3: Fast and
 * Accurate Attention with Asynchrony and Low-precision", abstract and core
 * claim: block quantization and incoherent processing on hardware FP8
 * support).  The block scales and the rotation come from fa_quant_fp8.
 *   q8, k8, v8        : [B][H][N][d] e4m3 codes from fa_quant_fp8 (Q and K
 *                       rotated with the same signs, Q with scale_mul 1/d).
 *   q_scale, k_scale,
 *   v_scale           : [B][H][ceil(N/128)] float block scales.
 *   o                 : [B][H][N][d] bf16, written.
 *   lse               : [B][H][N] float or NULL, as in fa_fwd.
 *   scale, causal     : as in fa_fwd (the ordinary softmax scale).
 *   Errors            : as in fa_fwd (no dtype argument: the codes are
 *                       e4m3, the output bf16).
 * S = Q8 K8^T runs on fp8 matrix-core instructions with fp32 accumulation
 * (each instruction aligns the products of 8 consecutive head-dim slots to
 * the largest of them with 14 bits below its leading bit, so a dominant
 * product costs the others of its group up to 2^-13 of it); block scales
 * are folded into the fp32 scores.  Value block scales that differ by
 * powers of two (FA_FP8_BLOCK_POW2, or one scale per tensor) are applied as
 * exact exponents of the P V instructions; any other value scales re-express
 * the output accumulator at each new block (slower, most at d = 256).  The
 * probabilities are rounded to e4m3 for the second product while the row
 * normaliser is summed from the fp32 values.  The result is exact attention
 * on the dequantised operands up to that rounding of the probabilities (at
 * most 2^-4 relative per probability), the score accumulation and fp32
 * rounding.
 */
int fa_fwd_fp8(const void* q8, const void* k8, const void* v8,
               const float* q_scale, const float* k_scale,
               const float* v_scale, void* o, float* lse, int B, int H, int N,
               int d, float scale, int causal, void* stream);

/*
 * fa_bwd -- attention backward by recomputation.  FlashAttention trains
 * Transformers ("FlashAttention: Fast and Memory-Efficient Exact Attention
 * with IO-Awareness", abstract), so the exact attention above needs its
 * gradient; the abstract does not spell the backward out.  This computes the gradient of <dO, O> for O of fa_fwd, rebuilding
 * the probabilities tile by tile from Q, K and the saved LSE so that the
 * N x N matrix again never reaches HBM.
 *   q, k, v, o, dout : [B][H][N][d] of `dtype`, read only; o is the forward
 *                      output and lse the forward's log-sum-exp [B][H][N].
 *   dq               : [B][H][N][d] float, written (fp32 accumulation).
 *   dk, dv           : [B][H][N][d] of `dtype`, written.
 *   workspace        : device memory of at least
 *                      fa_bwd_workspace_size(B, H, N, d) bytes, 16-byte
 *                      aligned; its contents on entry are ignored and on
 *                      exit unspecified.
 *   d                : 64 or 128 (d = 256 returns FA_ERR_UNSUPPORTED, and
 *                      fa_bwd_workspace_size returns 0 for it).
 *   Other arguments and errors as in fa_fwd.
 * With P the probabilities rebuilt from Q, K and LSE, D = rowsum(dO o O),
 * dS = P o (dO V^T - D), the outputs are dV = P^T dO, dK = scale dS^T Q and
 * dQ = scale dS K.  dQ, dK and dV are deterministic: every element is
 * written once, by one workgroup, with no atomics.
 */
size_t fa_bwd_workspace_size(int B, int H, int N, int d);
int fa_bwd(const void* q, const void* k, const void* v, const void* o,
           const void* dout, const float* lse, float* dq, void* dk, void* dv,
           void* workspace, int B, int H, int N, int d, int dtype, float scale,
           int causal, void* stream);

/*
 * fa_bwd_noalloc -- fa_bwd for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same computation and outputs (bit for bit), with the
 * workspace taken from a fixed scratch array in the library's device code
 * instead of a caller buffer.  It calls no hipMalloc, hipFree or other
 * allocating routine; on its first call on a device it looks up that
 * device's copy of the array (hipGetSymbolAddress) and keeps the address.
 *   Arguments : as in fa_bwd, without `workspace`.
 *   Limit     : B * H * N <= FA_BWD_NOALLOC_MAX_ROWS (the scratch is
 *               FA_BWD_NOALLOC_MAX_ROWS * 8 bytes = 16 MiB per device, held
 *               until the process ends); larger problems return
 *               FA_ERR_TOO_LARGE before anything is enqueued.
 *   Errors    : as in fa_bwd; FA_ERR_LAUNCH also if the scratch cannot be
 *               looked up on the current device.
 * Every call on one device shares that device's scratch: calls that
 * overlap in time on one device (different streams, or host threads) race
 * and must be serialised by the caller.  Nothing in the scratch needs to
 * start at zero (each call overwrites what it reads).
 */
#define FA_BWD_NOALLOC_MAX_ROWS 2097152
int fa_bwd_noalloc(const void* q, const void* k, const void* v, const void* o,
                   const void* dout, const float* lse, float* dq, void* dk,
                   void* dv, int B, int H, int N, int d, int dtype,
                   float scale, int causal, void* stream);

/*
 * Split-KV attention: partial results over parts of the keys, and their
 * log-sum-exp merge.  For a key set split into parts p, the attention of a
 * query row over all keys is
 *     L = ln sum_p exp(L_p),    O = sum_p exp(L_p - L) O_p,
 * where O_p is the row's attention output over part p alone (normalised
 * over that part) and L_p its log-sum-exp (-inf when no key of the part is
 * visible; O_p is then 0).  This is the online softmax's rescaling (a
 * running maximum and normaliser; FlashAttention-4 related-papers page,
 * online-softmax snippet) applied across parts; Ring Attention and Lean
 * Attention, in the reference list of "FlashAttention-3: Fast and Accurate
 * Attention with Asynchrony and Low-precision", combine per-device and
 * per-split partials this way.
 *
 * Positions.  With causal = 1, query row i of q sits at global position
 * q_pos0 + i, key row j of k at k_pos0 + j, and the key is visible iff its
 * position <= the query's.  (q_pos0 = k_pos0 = 0 with equal lengths is
 * fa_fwd's top-left mask.)
 */

/*
 * fa_fwd_partial -- attention of q over one key/value part.
 *   q        : [B][H][Nq][d] of `dtype`;  k, v : [B][H][Nk][d] of `dtype`.
 *   o        : [B][H][Nq][d] float, written: O_p (fp32, normalised over
 *              the part; 0 for rows that see no key of the part).
 *   lse      : [B][H][Nq] float, written: L_p (natural log; -inf for rows
 *              that see no key).  Required (it is the merge's input).
 *   Nq, Nk   : >= 1, <= 2^29.  q_pos0, k_pos0 : >= 0, <= 2^29.
 *   Other arguments as in fa_fwd.
 */
int fa_fwd_partial(const void* q, const void* k, const void* v, float* o,
                   float* lse, int B, int H, int Nq, int Nk, int d, int dtype,
                   float scale, int causal, int q_pos0, int k_pos0,
                   void* stream);

/*
 * fa_merge -- combine n_parts partial results into the attention output.
 *   o_parts   : [n_parts][B][H][N][d] float (part p's O_p), read only.
 *   lse_parts : [n_parts][B][H][N] float (part p's L_p), read only.
 *   o         : [B][H][N][d] of `dtype`, written (rounded to nearest even).
 *   lse       : [B][H][N] float, written (L), or NULL.
 *   n_parts   : >= 1.  Parts whose L_p is -inf contribute nothing (their
 *               O_p is not used).  A row with every L_p = -inf gets O = 0
 *               and L = -inf.
 */
int fa_merge(const float* o_parts, const float* lse_parts, int n_parts,
             void* o, float* lse, int B, int H, int N, int d, int dtype,
             void* stream);

/*
 * fa_fwd_splitkv -- attention of Nq queries over Nk keys, the keys split
 * into up to n_splits parts that run as independent workgroups (more
 * parallelism when Nq is small, as in decoding), then merged.
 *   q : [B][H][Nq][d];  k, v : [B][H][Nk][d];  o : [B][H][Nq][d] (`dtype`).
 *   lse       : [B][H][Nq] float or NULL.
 *   workspace : device memory of at least
 *               fa_splitkv_workspace_size(B, H, Nq, d, n_splits) bytes,
 *               16-byte aligned; contents on entry ignored, on exit
 *               unspecified.
 *   n_splits  : >= 1.  Parts are ceil(Nk / n_splits) keys rounded up to a
 *               multiple of 64, so fewer parts may be used.
 *   causal    : 1 aligns the queries with the last Nq keys (query i at
 *               position Nk - Nq + i, key j at j): the decoding convention,
 *               and fa_fwd's mask when Nq = Nk.
 */
size_t fa_splitkv_workspace_size(int B, int H, int Nq, int d, int n_splits);
int fa_fwd_splitkv(const void* q, const void* k, const void* v, void* o,
                   float* lse, void* workspace, int B, int H, int Nq, int Nk,
                   int d, int dtype, float scale, int causal, int n_splits,
                   void* stream);

/*
 * fa_fwd_blocksparse -- block-sparse attention: exact attention restricted
 * by a block mask ("FlashAttention: Fast and Memory-Efficient Exact
 * Attention with IO-Awareness", abstract: the extension to block-sparse
 * attention).  The N x N score matrix is cut into blocks of 128 query rows
 * by 128 keys; query row i may attend to key j only when
 * block_mask[i / 128][j / 128] is nonzero (and, when causal, j <= i).  Key
 * tiles of blocks no query row of a workgroup attends to are skipped; the
 * others are computed with the mask applied, so the result is the
 * definition above up to rounding.  Rows that see no key get O = 0 and
 * LSE = -inf.
 *   block_mask     : uint8, nb = ceil(N / 128): [H][nb][nb] shared by the
 *                    batch (mask_per_batch = 0) or [B][H][nb][nb] (1).
 *   workspace      : at least fa_blocksparse_workspace_size(B, H, N, d,
 *                    mask_per_batch) bytes, 4-byte aligned; holds the
 *                    per-tile lists of live key tiles built from the mask
 *                    on the stream; contents on entry ignored.
 *   Other arguments as in fa_fwd.
 */
size_t fa_blocksparse_workspace_size(int B, int H, int N, int d,
                                     int mask_per_batch);
int fa_fwd_blocksparse(const void* q, const void* k, const void* v, void* o,
                       float* lse, const void* block_mask, int mask_per_batch,
                       void* workspace, int B, int H, int N, int d, int dtype,
                       float scale, int causal, void* stream);

/* Static, NUL-terminated description of a status code. */
const char* fa_status_str(int status);

#ifdef __cplusplus
}
#endif

#endif /* FA_H_ */
