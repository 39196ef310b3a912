/*
 * slim.h — C ABI of the SLiM compressed linear layer on AMD Instinct MI355X
 * (gfx950).
 *
 * The layer (Compression Trinity thesis, Fig. 7.1 caption and the Ch. 4
 * introduction on parallel sparse and low-rank paths):
 *
 *     Y[M,N] = X[M,K] . deq(W_c)^T + (X . L[K,r]) . R[r,N]
 *
 * where W_c is W [N,K] quantised to symmetric int4 with one fp16 scale per
 * 128 consecutive k (thesis §1.2.2 per-group quantisation; group size 128 in
 * the developinglight.com summary) and then pruned to 2:4 along k, the
 * reduction dimension (thesis §2.2.3 "Sparse Tensor Core Acceleration").
 * Y = X W^T is the linear layer of thesis §2.1.
 *
 * Conventions for every call:
 *  - All tensor pointers are DEVICE pointers owned by the caller, dense and
 *    row-major, 16-byte aligned.  Half-precision tensors are passed as
 *    uint16_t (IEEE binary16 bit patterns).
 *  - Calls only enqueue work on `stream` (0 = the null stream) and return;
 *    they never allocate, free or synchronise (the one exception is the
 *    query slim_linear_giveups).  Outputs must not alias inputs.
 *  - Every argument is checked before anything is launched: a call that
 *    returns an error has enqueued nothing.  No call aborts or throws.
 *  - Not checked (undefined results): W holding non-finite values or
 *    |W| >= 7 * 65504; device pointers that do not cover the stated sizes.
 *
 * Packed weight format (per row n of W; the pages fix only "packed kept
 * values + small position indices"), per block of 16 consecutive k:
 *    values: one little-endian uint32: bits [4j,4j+4) = the kept value with the
 *            lower index in group j (k = 16b+4j .. 16b+4j+3), bits
 *            [16+4j,16+4j+4) = the kept value with the higher index, both
 *            4-bit two's complement in [-7, 7];
 *    meta:   one little-endian uint16: bits [4j,4j+2) = lower kept index,
 *            bits [4j+2,4j+4) = higher kept index (0..3, lower < higher).
 *    scales: one fp16 per 128 consecutive k; dequantised weight = q * scale.
 * Arrangement in memory: rows in blocks of 16 (the last block holds N mod 16
 * rows if that is not 0); inside a block the 128-k groups in order; inside a
 * group the rows in order, each with its 8 values words (32 B), 8 metadata
 * half-words (16 B) and 1 scale.  For a block of R rows starting at row 16b:
 *    values byte offset of (group g, row i): 16b*K/4 + (g*R + i)*32
 *    meta   byte offset of (group g, row i): 16b*K/8 + (g*R + i)*16
 *    scales element of     (group g, row i): 16b*K/128 + g*R + i
 * so one block's data of one group is contiguous (wide loads, no 16-row
 * strided fragments); the array sizes are N*K/4, N*K/8 and N*K/128*2 bytes.
 */
#ifndef SLIM_H
#define SLIM_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    SLIM_OK = 0,
    SLIM_EINVAL = 1,        /* bad argument: null pointer, bad size, misaligned, workspace too small */
    SLIM_EUNSUPPORTED = 2,  /* group != 128, or the current device is not gfx950 */
    SLIM_EHIP = 3           /* a HIP runtime call failed; detail in slim_last_error() */
} slim_status;

/* Static description of a status code; never NULL. */
const char* slim_status_string(int status);

/* Detail of the last failed call on this thread ("" if none); valid until the
 * next call on this thread. */
const char* slim_last_error(void);

/* ABI version, currently 1. */
int slim_version(void);

/* Byte sizes of the packed triple for a weight W [N,K]; 0 if K % 128 != 0,
 * N or K <= 0, or N or K > 2^24 (no call accepts such a weight).
 * values = N*K/4, meta = N*K/8, scales = N*(K/group)*2.
 * Every call and size query accepts dimensions up to 2^24 (r up to 4096 and
 * N*K up to 2^40 for one weight); the size queries return 0 for any shape
 * their call would reject, and never wrap around. */
size_t slim_values_bytes(int64_t N, int64_t K);
size_t slim_meta_bytes(int64_t N, int64_t K);
size_t slim_scales_bytes(int64_t N, int64_t K, int64_t group);

/*
 * slim_pack — one-shot quantise -> 2:4 prune -> pack (thesis Fig. 7.1 steps
 * 1-2: the quantised weights are the ones that get sparsified).
 *   W       fp32 [N][K], device.
 *   group   must be 128.
 *   values  uint8 [N*K/4], meta uint8 [N*K/8], scales fp16 [N*K/128]: outputs,
 *           in the arrangement above.
 * Per row n and group j: s = fp16_rne(absmax / 7); q = clamp(rint(w / s), -7, 7)
 * (fp32 division, half-to-even), q = 0 if s == 0; in every 4 consecutive k the
 * two largest |q| are kept (ties to the lower index), the others dropped.
 * The result is bit-exact and deterministic.
 * Errors: SLIM_EINVAL if a pointer is NULL or misaligned, N <= 0, K <= 0 or
 * K % 128 != 0; SLIM_EUNSUPPORTED if group != 128.
 */
slim_status slim_pack(const float* W, int64_t N, int64_t K, int64_t group,
                      uint8_t* values, uint8_t* meta, uint16_t* scales,
                      hipStream_t stream);

/*
 * Workspace needed by slim_linear for this shape, in bytes (a multiple of 256).
 * The workspace is caller-owned device scratch for intermediate results (the
 * adapter's T = X L) and, in its first 16384 bytes, the hand-off state of the
 * one-launch decode path (workgroups that wait for each other's rows of T):
 * a 64-bit epoch, a 64-bit give-up count (slim_linear_giveups) and tagged
 * rows of T.  Zero the whole workspace (or at least those first 16384 bytes)
 * before its first use; every call leaves that state valid for the next call,
 * of any shape, and the rest of the workspace undefined.  Calls that share one
 * workspace must be ordered on one stream.  If a call's workgroups cannot all
 * be resident at once (the GPU shared with other work), a workgroup of that
 * path gives up after a bounded wait (slim_set_wait_limit), writes NaN to its
 * rows of Y and adds one to the workspace's give-up count; the state stays
 * valid, so the next call on the workspace computes a correct result.  One
 * workspace serves up to 2^48 - 1 one-launch calls (the tags are 48 bits).
 */
size_t slim_linear_workspace_bytes(int64_t M, int64_t N, int64_t K, int64_t r);  /* 0: shape rejected */

/*
 * slim_linear_giveups — the number of workgroups of the one-launch decode
 * path that gave up their bounded wait on this workspace (their rows of Y
 * read NaN) since it was zeroed or last reset.  Unlike every other call this
 * one synchronises `stream` (it reads device memory after the calls enqueued
 * before it) and must not be captured in a graph; reset != 0 also sets the
 * count back to 0.  workspace: the caller's workspace of slim_linear or
 * slim_linear_qa (the first problem's, for the batched call); count: host.
 * Errors: SLIM_EINVAL (NULL or misaligned pointer); SLIM_EHIP (copy failed).
 */
slim_status slim_linear_giveups(const void* workspace, int reset, uint64_t* count, hipStream_t stream);

/*
 * slim_set_wait_limit — poll passes of the one-launch decode path's bounded
 * wait before a workgroup gives up, for calls made after it returns
 * (process-wide; default 262144, a fraction of a second).  0 makes every such
 * wait give up at once, which forces the give-up path from the host (tests);
 * a negative value restores the default; values above 2^30 are clamped.
 * Returns the previous limit.
 */
int64_t slim_set_wait_limit(int64_t limit);

/*
 * slim_linear — Y = X . deq(W_c)^T + (X . L) . R, fp16 in and out, fp32
 * accumulation (thesis §2.1 linear layer; Ch. 4 introduction: the sparse
 * weight and the dense adapter are separate paths).
 *   X       fp16 [M][K]            M >= 0 (M == 0: nothing to do, SLIM_OK)
 *   values, meta, scales           the packed W [N][K] from slim_pack
 *   group   must be 128
 *   Lt      fp16 [r][K] = L^T, Rt fp16 [N][r] = R^T: the rank-r adapter
 *           (L [K][r], R [r][N]) stored output-major like a linear layer's
 *           weight, i.e. like W itself and like LoRA-style adapter factors;
 *           these are the thesis' own factors of W ~ L R (§1.2.3: a
 *           [d_out x r] and an [r x d_in] matrix).  Every product of the
 *           layer then contracts along contiguous memory.
 *           r % 32 == 0; r == 0 means no adapter (Lt and Rt may then be NULL)
 *   Y       fp16 [M][N], output
 *   workspace / workspace_bytes    see slim_linear_workspace_bytes
 * Constraints: N % 16 == 0, K % 128 == 0.
 * Errors: SLIM_EINVAL (NULL or misaligned pointer, N, K <= 0, M < 0, shape
 * constraint broken, r < 0 or r % 32 != 0, workspace too small);
 * SLIM_EUNSUPPORTED (group != 128); SLIM_EHIP (launch failure).
 */
slim_status slim_linear(const uint16_t* X, int64_t M, int64_t N, int64_t K,
                        const uint8_t* values, const uint8_t* meta,
                        const uint16_t* scales, int64_t group,
                        const uint16_t* Lt, const uint16_t* Rt, int64_t r,
                        uint16_t* Y, void* workspace, size_t workspace_bytes,
                        hipStream_t stream);

/*
 * slim_linear_noalloc — slim_linear without a workspace argument, for callers
 * that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid allocation).  Its scratch is one
 * library-owned array per GPU of 64 MiB (67108864 bytes), held until the
 * process ends; the call allocates and frees nothing.  Shapes whose
 * slim_linear_workspace_bytes(M, N, K, r) exceeds 64 MiB are rejected with
 * SLIM_EINVAL.  Every call on one GPU shares that GPU's array and leaves its
 * contents for the next: calls that overlap on one GPU (other streams, other
 * threads) race and must be ordered by the caller.  A workgroup that gives
 * up its bounded wait writes NaN to its rows of Y as in slim_linear; the
 * count of such give-ups lives in the library's array and is not reported.
 * Arguments, results and other errors as slim_linear.
 */
slim_status slim_linear_noalloc(const uint16_t* X, int64_t M, int64_t N, int64_t K,
                                const uint8_t* values, const uint8_t* meta,
                                const uint16_t* scales, int64_t group,
                                const uint16_t* Lt, const uint16_t* Rt, int64_t r,
                                uint16_t* Y, hipStream_t stream);

/*
 * slim_linear_batched — `batch` independent problems of one shape (M,N,K,r),
 * e.g. the q/k/v or gate/up projections of one decoder block.  Problem b reads
 * X + b*stride_X, values + b*stride_values, ... and writes Y + b*stride_Y.
 * Strides are in elements of each array's type; stride_X == 0 shares one X
 * among all problems.  Output strides must keep the Y blocks disjoint.  With
 * batch > 1 every stride must keep each problem 16-byte aligned and be at
 * most 2^40 elements; batch <= 65535.
 * The workspace needs batch * slim_linear_workspace_bytes(M, N, K, r) bytes.
 * Other rules as slim_linear.  batch == 0 is a no-op.
 */
slim_status slim_linear_batched(int64_t batch, int64_t M, int64_t N, int64_t K,
                                int64_t r, int64_t group,
                                const uint16_t* X, int64_t stride_X,
                                const uint8_t* values, int64_t stride_values,
                                const uint8_t* meta, int64_t stride_meta,
                                const uint16_t* scales, int64_t stride_scales,
                                const uint16_t* Lt, int64_t stride_Lt,
                                const uint16_t* Rt, int64_t stride_Rt,
                                uint16_t* Y, int64_t stride_Y,
                                void* workspace, size_t workspace_bytes,
                                hipStream_t stream);

/*
 * Quantised adapters ("Quantized SLiM": the thesis' Tables E.13 and E.14
 * quantise the low-rank adapters as well; the pages give no adapter
 * quantiser, so W's is used without pruning).  A factor is given
 * output-major, rows x cols with cols its reduction dimension: Lt = L^T
 * [r][K] with group 128 along K, Rt = R^T [N][r] with group 32 along r.
 * Per row and group: s = fp16_rne(absmax / 7); q = clamp(rint(a / s), -7, 7)
 * (fp32 division, half to even), q = 0 if s == 0.
 *   codes   uint8 [rows][cols/2]: per row, per 8 consecutive elements one
 *           little-endian uint32 in which element e occupies nibble
 *           (0,4,1,5,2,6,3,7)[e] (4-bit two's complement)
 *   scales  fp16 [rows][cols/group], row-major
 * slim_adapter_codes_bytes / slim_adapter_scales_bytes give the sizes (0 for
 * an invalid shape).  slim_pack_adapter is bit-exact and deterministic.
 * Errors: SLIM_EINVAL (NULL or misaligned pointer, rows <= 0, cols not a
 * positive multiple of group); SLIM_EUNSUPPORTED (group not 32 or 128).
 */
size_t slim_adapter_codes_bytes(int64_t rows, int64_t cols);
size_t slim_adapter_scales_bytes(int64_t rows, int64_t cols, int64_t group);
slim_status slim_pack_adapter(const float* A, int64_t rows, int64_t cols, int64_t group,
                              uint8_t* codes, uint16_t* scales, hipStream_t stream);

/*
 * slim_linear_qa — slim_linear with quantised adapters:
 *   Y = X . deq(W_c)^T + (X . deq(L)) . deq(R)
 *   Lq, Ls  codes and scales of Lt [r][K] (group 128) from slim_pack_adapter
 *   Rq, Rs  codes and scales of Rt [N][r] (group 32) from slim_pack_adapter
 *   r > 0, r % 32 == 0; other arguments as slim_linear.
 * The workspace needs slim_linear_qa_workspace_bytes(M, N, K, r) bytes with
 * the rules of slim_linear_workspace_bytes (zero it before its first use).
 * One or two tokens on the one-launch decode path read the int4 factors
 * directly; other shapes dequantise them (q * s in fp16) into the workspace.
 * Errors: as slim_linear; SLIM_EINVAL also for r == 0 or a NULL factor.
 */
size_t slim_linear_qa_workspace_bytes(int64_t M, int64_t N, int64_t K, int64_t r);
slim_status slim_linear_qa(const uint16_t* X, int64_t M, int64_t N, int64_t K,
                           const uint8_t* values, const uint8_t* meta,
                           const uint16_t* scales, int64_t group,
                           const uint8_t* Lq, const uint16_t* Ls,
                           const uint8_t* Rq, const uint16_t* Rs, int64_t r,
                           uint16_t* Y, void* workspace, size_t workspace_bytes,
                           hipStream_t stream);

/*
 * 4-bit weights with an 8-bit input (thesis Appendix E.2 "Input
 * Quantization"; captions of Tables E.2 and E.5: 4-bit weights and 8-bit
 * input).  The pages give no input quantiser; per token (row of X):
 *   s = fp16_rne(absmax / 127),  q = clamp(rint(x / s), -127, 127)
 * (fp32 division, half to even), q = 0 if s == 0.  The layer then computes
 *   Y = deq(X) . deq(W_c)^T + (deq(X) . L) . R,   deq(X) = q * s.
 *
 * slim_quantize_input — X fp16 [M][K] -> q int8 [M][K], s fp16 [M]
 *   (device).  K % 8 == 0.  Bit-exact and deterministic.
 *   Errors: SLIM_EINVAL (NULL or misaligned pointer, M < 0, K not a positive
 *   multiple of 8); SLIM_EHIP (launch failure).  M == 0 is a no-op.
 *
 * slim_linear_a8 — the layer on q [M][K] int8 and s [M] fp16 (device, from
 *   slim_quantize_input), other arguments as slim_linear.  Without an
 *   adapter (r == 0), at prefill shapes (the 256 x 128 output tiles number
 *   at least 128) the main term runs on the int8 sparse matrix core: one
 *   v_smfmac_i32_16x16x128_i8 per 128-k scale group, its exact int32 sums
 *   scaled by the group scale in fp32, the token scale applied to the
 *   finished sums.  Other calls dequantise the input (q * s rounded once to
 *   fp16) into the workspace and run the fp16 kernels (decode is bound by
 *   the weight and adapter bytes, not the input; with an adapter the fp16
 *   one-pass prefill is the faster one).
 *   The workspace needs slim_linear_a8_workspace_bytes(M, N, K, r) bytes,
 *   with the rules of slim_linear_workspace_bytes.
 *   Errors: as slim_linear; SLIM_EINVAL also for a NULL or misaligned s.
 */
slim_status slim_quantize_input(const uint16_t* X, int64_t M, int64_t K, int8_t* q, uint16_t* s,
                                hipStream_t stream);
size_t slim_linear_a8_workspace_bytes(int64_t M, int64_t N, int64_t K, int64_t r);
slim_status slim_linear_a8(const int8_t* qx, const uint16_t* sx, int64_t M, int64_t N, int64_t K,
                           const uint8_t* values, const uint8_t* meta,
                           const uint16_t* scales, int64_t group,
                           const uint16_t* Lt, const uint16_t* Rt, int64_t r,
                           uint16_t* Y, void* workspace, size_t workspace_bytes,
                           hipStream_t stream);

/*
 * Hybrid dense / 2:4 tiles (PATCH, thesis Ch. 6 and the Ch. 1 list of
 * contributions: weight tiles are either dense or 2:4 sparse, an effective
 * sparsity between 0% and 50%, composable with SLiM's quantisation and
 * adapter; Fig. 6.1 caption: a per-tile mask).  The pages learn the mask and
 * fix neither the tile size nor a format; here a tile is 16 rows x one 128-k
 * scale group, and the mask is an input:
 *   dense   int32 [ceil(N/16)][K/128], nonzero = the tile stays dense.
 * slim_pack_hybrid quantises every tile as slim_pack does (same scales),
 * prunes the 2:4 tiles as slim_pack does, and keeps every code of a dense
 * tile: its codes at positions 0 and 1 of each group of 4 go to values /
 * meta (metadata 0, 1) in slim_pack's format, those at positions 2 and 3 to
 *   dvalues  uint8 [N*K/4], the arrangement of values (zero in 2:4 tiles).
 * Bit-exact and deterministic.  Errors as slim_pack; SLIM_EINVAL also for a
 * NULL or misaligned dense or dvalues.
 *
 * slim_linear_hybrid — Y = X . deq(W_h)^T + (X . L) . R on the hybrid weight;
 * arguments as slim_linear plus dvalues and dense (one problem).  At 1-16
 * tokens (two launches: adapter-down, then the main kernel) and at prefill
 * shapes the kernels read a dense tile's second pair and issue a second
 * sparse matrix instruction for it; 2:4 tiles cost what they cost in
 * slim_linear.  The workspace is slim_linear_workspace_bytes(M, N, K, r).
 */
slim_status slim_pack_hybrid(const float* W, int64_t N, int64_t K, int64_t group, const int32_t* dense,
                             uint8_t* values, uint8_t* meta, uint16_t* scales, uint8_t* dvalues,
                             hipStream_t stream);
slim_status slim_linear_hybrid(const uint16_t* X, int64_t M, int64_t N, int64_t K,
                               const uint8_t* values, const uint8_t* meta, const uint16_t* scales,
                               const uint8_t* dvalues, const int32_t* dense, int64_t group,
                               const uint16_t* Lt, const uint16_t* Rt, int64_t r,
                               uint16_t* Y, void* workspace, size_t workspace_bytes,
                               hipStream_t stream);

/*
 * slim_pack_transposed — the double-pruned transpose of a packed weight
 * (SLoPe, thesis Ch. 4 list of contributions: the forward N:M-pruned weight
 * is transposed and pruned N:M again, so that the backward product
 * dX = dY . W, whose reduction runs over n, is 2:4 sparse too).  The pages
 * give no procedure for the quantised weight; this call:
 *   D[k][n] = fp16_rne(q[n][k] * scale)    (deq(W_c)^T, exact product, one
 *                                           rounding, as the forward kernels)
 *   in every 4 consecutive n of a row k the 2 largest |D| are kept, ties to
 *   the lower index.
 *   values, meta, scales   the packed W [N][K] from slim_pack (inputs)
 *   tvalues  fp16 [K][N/2]: per row k, per 16 consecutive n (4 groups j of
 *            4), 8 values: group j's kept value with the lower index, then
 *            the one with the higher index
 *   tmeta    uint16 [K][N/16]: per 16 n one half-word, bits [4j,4j+2) =
 *            lower kept index of group j, bits [4j+2,4j+4) = higher one
 *            (the metadata bit order of the forward format).
 * slim_transposed_values_bytes = N*K, slim_transposed_meta_bytes = N*K/8
 * (0 for an invalid shape).  Bit-exact and deterministic; scales must be
 * finite (slim_pack's are).
 * Errors: SLIM_EINVAL (NULL or misaligned pointer, N not a positive multiple
 * of 16, K not a positive multiple of 128, N*K/16 > 2^40); SLIM_EUNSUPPORTED
 * (group != 128); SLIM_EHIP (launch failure).
 */
size_t slim_transposed_values_bytes(int64_t N, int64_t K);
size_t slim_transposed_meta_bytes(int64_t N, int64_t K);
slim_status slim_pack_transposed(const uint8_t* values, const uint8_t* meta,
                                 const uint16_t* scales, int64_t N, int64_t K,
                                 int64_t group, uint16_t* tvalues, uint16_t* tmeta,
                                 hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* SLIM_H */
