/*
 * qpn.h -- C ABI of the QPN weight-streaming skinny GEMM for MI355X (gfx950).
 *
 * The operation.  Decode steps of single-request speculative decoding
 * multiply each projection's weights by a block of 1..8 FP16 activation rows
 * (the target token plus up to 7 draft candidates checked in the same verify
 * round).  The weights stay in their published compressed formats while they
 * stream from HBM and are expanded to FP16 in registers, in small pieces,
 * right before the matrix unit consumes them; there is no dequantise-first
 * pass.  NVFP4 regions and FP8 regions each get their own path, activations
 * are FP16, accumulation is FP32, outputs are FP16.  Sources:
 *   taozi.news, "四张 2017 年 V100 跑通 Qwen 3 NVFP4 推理，性能追平 RTX 5090":
 *     section "自研 QPN 内核：让 Volta 跑 NVFP4" (the kernel idea, the NVFP4
 *     M=1 / M=8 and FP8 M=1..4 paths, the 4-bit lm_head, the 8-row verify
 *     tile) and section "v1.1 的关键改进：保留官方混合精度分配" (FP4 regions
 *     -> NVFP4 path, FP8 regions -> FP8 path, activations FP16);
 *   aiwitness.kr, "VOLTA에서 NVFP4 구동! ...": section "내가 실제로 만든 것"
 *     (weights stay compressed and are translated in registers) and the v1.1
 *     section (the published FP4/FP8 assignment is preserved);
 *   lcz.me, "前情提要 整台洋垃圾V100 16G雙卡": table
 *     "NVFP4 （V100 sm_70 + E5-2686 v4）的支援狀況" (NVFP4 = E2M1 codes with
 *     UE4M3 scales, decodable in software).
 * The pages fix no bit layout, block size or rounding.  This library uses:
 *   NVFP4: E2M1 codes, one UE4M3 scale per 16 consecutive K elements of a
 *          row, one FP32 tensor scale g = amax / (6 * 448);
 *   FP8:   E4M3 (OCP "FN": bias 7, max 448) codes, one FP32 scale per output
 *          row s = row amax / 448;
 *   both:  round to nearest, ties to the even code, saturating.
 *
 * Conventions for every call.
 *   - W is [n, k] row-major FP32 (row = output channel).  X is [m, k]
 *     row-major FP16, Y is [m, n] row-major FP16: Y = X * What^T.
 *   - FP16 data is passed as uint16_t bit patterns.
 *   - Pointers named w, packed, x, y, logits, argmax, workspace are DEVICE
 *     pointers on the current HIP device.  `stream` is a hipStream_t (NULL =
 *     the default stream).  All work is enqueued on that stream; no call
 *     allocates, frees, copies to the host or synchronises.
 *   - The caller owns every buffer.  A packed blob is opaque and versioned;
 *     it records its own n, k and scales, so GEMM calls need no host reads.
 *     A GEMM reads at most qpn_*_packed_bytes(n, k) bytes of `packed` for
 *     its own format; passing a smaller buffer is undefined behaviour.
 *   - Workspace (split-K exchange slots, prefill partial sums and arrival
 *     counters, lm_head argmax keys) must be zero-filled before its first use; every call leaves it
 *     zero-filled again, so a workspace is zeroed once and then reused.
 *     Calls that share a workspace must not overlap.
 *   - Argument checks run on the host before anything is enqueued; on any
 *     error nothing is launched.  Device faults surface, as usual for HIP,
 *     at the caller's next synchronisation.  Nothing is printed and no C++
 *     exception crosses the ABI.
 *   - Shapes: 0 <= m <= 8, n >= 0, k >= 0; n <= 2^24, k <= 2^20.  NVFP4
 *     needs k % 16 == 0, FP8 needs k % 8 == 0.  m == 0 or n == 0 is a valid
 *     empty call (QPN_OK, nothing launched); k == 0 gives Y = 0.
 *   - Alignment: packed 256 B, x 16 B, w 16 B, workspace 8 B, y and
 *     logits 2 B, argmax 4 B.
 *   - Inputs to pack must be finite; this is a precondition, not checked.
 */
#ifndef QPN_H
#define QPN_H

#include <stddef.h>
#include <stdint.h>

#if defined(__GNUC__)
#define QPN_API __attribute__((visibility("default")))
#else
#define QPN_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes returned by every call. */
#define QPN_OK 0
#define QPN_ERR_NULL 1   /* a required pointer is NULL                      */
#define QPN_ERR_SHAPE 2  /* m, n or k outside the documented range         */
#define QPN_ERR_ALIGN 3  /* a pointer is not aligned as documented         */
#define QPN_ERR_BUFFER 4 /* packed or workspace buffer smaller than needed */
#define QPN_ERR_DEVICE 5 /* current device is not gfx950 or not usable     */
#define QPN_ERR_LAUNCH 6 /* the HIP runtime rejected a kernel launch       */
#define QPN_ERR_SCRATCH 7 /* needs more than the static scratch (noalloc)  */

/* Formats, for qpn_workspace_bytes. */
#define QPN_OP_GEMM_NVFP4 1
#define QPN_OP_GEMM_FP8 2
#define QPN_OP_LMHEAD_NVFP4 3
#define QPN_OP_PREFILL_NVFP4 4
#define QPN_OP_PREFILL_FP8 5

/* Human-readable name of a status code (static string, never NULL). */
QPN_API const char *qpn_status_string(int status);

/* Version of the packed-blob layout this library reads and writes. */
QPN_API int qpn_layout_version(void);

/* Bytes a packed NVFP4 blob of an [n, k] weight occupies (header, codes and
 * block scales, padded to whole tiles); 0 when (n, k) is not a valid NVFP4
 * shape.  Pure host computation. */
QPN_API size_t qpn_nvfp4_packed_bytes(int64_t n, int64_t k);

/* Bytes a packed FP8 blob of an [n, k] weight occupies (header, row scales
 * and codes, padded to whole tiles); 0 when (n, k) is not a valid FP8 shape.
 * Pure host computation. */
QPN_API size_t qpn_fp8_packed_bytes(int64_t n, int64_t k);

/* Workspace bytes a call of kind `op` (QPN_OP_*) with these sizes uses for
 * its preferred launch plan: 0 when that plan does not split K (the GEMMs
 * then accept a NULL workspace), else room for the slots in which the K
 * splits' partial sums meet (1 KiB per 16-row panel per node of the
 * pairwise tree over the splits); the lm_head needs at least 8 * m * 256
 * bytes for its argmax keys plus any split-K room.  A call
 * given less workspace than this still runs, with fewer K splits, as long as
 * the fewest splits whose activation slice (m * K / splits FP16 values) fits
 * in LDS still fit the workspace; otherwise it returns QPN_ERR_BUFFER (only
 * for large m * k, e.g. m > 4 with k = 17408).  The prefill ops take
 * 0 <= m <= 256; above 16 rows, when output tiles are cut between
 * workgroups, they need one arrival counter per tile and room for two FP32
 * partial tiles per workgroup, and on any smaller workspace every workgroup
 * takes whole tiles.  Returns (size_t)-1 for an unknown op or invalid shape.  Pure
 * host. */
QPN_API size_t qpn_workspace_bytes(int op, int m, int64_t n, int64_t k);

/* Launch plan a call of kind `op` (QPN_OP_*) uses for (m, n, k) when given
 * the workspace qpn_workspace_bytes asks for: the number of workgroups; the
 * wavefronts per 16-row panel (they interleave the panel's k-steps); the
 * panels per workgroup; the k-steps each wavefront keeps in flight; the
 * number of K ranges ("splits", > 1 when partial sums are combined across
 * workgroups); the activation rows staged in LDS (1, 2, 4 or 8 >= m); and
 * split_workgroups, the workgroups that work on K ranges (split_workgroups
 * / splits panel groups of the last panels, dispatched first).  The other
 * workgroups - 0 unless the plan balances whole panels per CU - each take
 * panels_per_workgroup whole panels.  For the prefill ops on the tiled
 * kernel (above 16 rows, and at 9-16 rows of large calls: see
 * qpn_gemm_prefill_nvfp4) a workgroup covers either 8 panels
 * (waves_per_panel 2: a wavefront per half of the activation rows) or 16
 * panels (waves_per_panel 1; above 128 rows; at 65-128 rows when there
 * are more than 128 tiles of 128 channels and the 256-channel launch has
 * 192 workgroups or more; and for NVFP4 up to 64 rows when that launch
 * still has 128 workgroups or more) by activation_rows = 32, 64 or 128 rows (the fewest that hold m, at
 * most 128; more rows are further row blocks, as separate workgroups).  The
 * workgroups cut the (tile, k-step) pairs into contiguous ranges: equal
 * ones, or, where the partial tiles are summed in shares (128 rows or 16
 * panels), a whole piece of one tile each, the workgroup count a multiple
 * of the tile count.  splits is the most workgroups that one output tile
 * is cut between (1: whole tiles), and split_workgroups equals
 * workgroups.  A pure function of its
 * arguments, independent of any declared maximum.  Any output pointer may
 * be NULL.  Returns QPN_OK or QPN_ERR_SHAPE.  Pure host. */
QPN_API int qpn_gemm_plan(int op, int m, int64_t n, int64_t k, int64_t *workgroups,
                          int *waves_per_panel, int *panels_per_workgroup,
                          int *prefetch_depth, int *splits, int *activation_rows,
                          int64_t *split_workgroups);

/* NVFP4 pack ("pure round" quantisation, lcz.me quantisation-option table,
 * NVFP4-NVIDIA row; format per the lcz.me NVFP4 support table).
 * w: device FP32 [n, k].  packed: device buffer of packed_bytes >=
 * qpn_nvfp4_packed_bytes(n, k).  Computes, in FP32 with IEEE division:
 *   amax = max|w|;  g = amax / 2688;
 *   per 16-block of a row: sc = E4M3(nearest-even, saturating) of
 *     (blockmax / 6) / g  (sc = 0 when g == 0);  S = value of sc;
 *   codes = 0 when S == 0, else E2M1(nearest-even, saturating) of w / (S*g).
 * Writes the whole blob (header, codes, scales, zeroed padding).  Three
 * kernels on `stream`, no host synchronisation. */
QPN_API int qpn_pack_nvfp4(const float *w, int64_t n, int64_t k, void *packed,
                   size_t packed_bytes, void *stream);

/* FP8 pack (taozi.news section "v1.1 的关键改进", FP8 regions kept as FP8).
 * w: device FP32 [n, k].  Per row: s = max|w_row| / 448 (stored FP32);
 * codes = 0 when s == 0, else E4M3(nearest-even, saturating) of w / s.
 * Writes the whole blob.  One kernel plus a header kernel on `stream`. */
QPN_API int qpn_pack_fp8(const float *w, int64_t n, int64_t k, void *packed,
                 size_t packed_bytes, void *stream);

/* FP8 -> NVFP4 conversion of a packed weight: the derived-checkpoint variant
 * (taozi.news section "v1.1 的关键改进" and aiwitness.kr section
 * "내가 실제로 만든 것": before FP8 regions had an execution path of their
 * own, they were converted to NVFP4).  Every weight is decoded to its FP8
 * value E4M3(code) * s_n (the exact product rounded once to FP32) and that
 * FP32 tensor is packed exactly as qpn_pack_nvfp4 packs its input.
 * fp8_packed: a blob from qpn_pack_fp8 for this (n, k), fp8_bytes >=
 * qpn_fp8_packed_bytes(n, k); nvfp4_packed: output, nvfp4_bytes >=
 * qpn_nvfp4_packed_bytes(n, k).  Both device, 256-byte aligned, not
 * overlapping (QPN_ERR_BUFFER otherwise).  k % 16 == 0.  If the source
 * header does not describe an FP8 [n, k] weight the output is marked
 * invalid and GEMMs on it write NaN.  Three kernels on `stream`. */
QPN_API int qpn_requant_fp8_to_nvfp4(const void *fp8_packed, size_t fp8_bytes, int64_t n,
                                     int64_t k, void *nvfp4_packed, size_t nvfp4_bytes,
                                     void *stream);

/* QPN NVFP4 skinny GEMM (taozi.news section "自研 QPN 内核", the NVFP4 path
 * at M=1 and M=8; aiwitness.kr section "내가 실제로 만든 것").
 * Y[m, n] = FP16_RNE( sum_k X[m, k] * What[n, k] ), What = E2M1 * UE4M3 * g,
 * with FP32 accumulation.  packed: blob from qpn_pack_nvfp4 for this (n, k).
 * x: [m, k] FP16, y: [m, n] FP16.  workspace: zero-filled device memory of
 * workspace_bytes bytes (see qpn_workspace_bytes; NULL with 0 bytes is
 * valid and only limits the launch plan).  If the blob header does not
 * describe an NVFP4 [n, k] weight the kernel writes FP16 NaN to every
 * output. */
QPN_API int qpn_gemm_nvfp4(const void *packed, const uint16_t *x, uint16_t *y, int m,
                   int64_t n, int64_t k, void *workspace,
                   size_t workspace_bytes, void *stream);

/* qpn_gemm_nvfp4 for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * Same product, arguments (minus the workspace), kernels and failure
 * behaviour as qpn_gemm_nvfp4.  The split-K partials and counters live in
 * the library's own static device array (4 MiB per GPU, allocated when the
 * library's code is loaded on that GPU and held until the process ends);
 * this call allocates nothing, and nothing else is needed from the caller.
 * The launch plan is the one qpn_gemm_nvfp4 uses when given 4 MiB of
 * workspace: fewer K splits where more would not fit.  Returns
 * QPN_ERR_SCRATCH when even the fewest K splits the activation slice needs
 * exceed 4 MiB (only for very large n * k at m > 4); QPN_ERR_DEVICE when the
 * scratch could not be located on the current device.  Every call on one
 * GPU shares that GPU's scratch and leaves it zero-filled: calls that
 * overlap on one GPU (concurrent streams, or host threads on one device)
 * race and must be serialised by the caller. */
QPN_API int qpn_gemm_nvfp4_noalloc(const void *packed, const uint16_t *x, uint16_t *y, int m,
                                   int64_t n, int64_t k, void *stream);

/* QPN FP8 skinny GEMM (taozi.news section "自研 QPN 内核", the FP8 M=1..4
 * path; section "v1.1 的关键改进" for FP8 regions).
 * Y[m, n] = FP16_RNE( s_n * sum_k X[m, k] * E4M3(code[n, k]) ), FP32
 * accumulation.  Arguments and failure behaviour as qpn_gemm_nvfp4. */
QPN_API int qpn_gemm_fp8(const void *packed, const uint16_t *x, uint16_t *y, int m,
                 int64_t n, int64_t k, void *workspace, size_t workspace_bytes,
                 void *stream);

/* Prefill-sized activation blocks against the same packed weights (lcz.me
 * page, "strata" section: prompt processing on FP16 tensor-core tiles, with
 * activations in FP16; aiwitness.kr page, questions section: prefill is the
 * phase that the old card loses).  The same product as qpn_gemm_nvfp4 /
 * qpn_gemm_fp8 for 0 <= m <= 256 activation rows: Y[m, n] = FP16_RNE(scale *
 * sum_k X[m, k] * W[n, k]), FP32 accumulation, weights decoded in registers,
 * no dequantised copy.  Up to 16 rows it runs the skinny kernel of
 * qpn_gemm_nvfp4 / qpn_gemm_fp8 with a 16-row activation tile (the weights
 * stream once); from 17 rows, at 9-16 rows of large calls (NVFP4: 1536 or
 * more 16-row panels, or 1024 or more with k > 8064; FP8: k > 8128, or
 * 3072 or more panels), or when the workspace given cannot hold the K
 * splits the skinny kernel needs, a tiled MFMA kernel.  Both reach the same
 * parity bar.  x: [m, k] FP16, 16-byte aligned; y: [m, n] FP16.
 * workspace: zero-filled device memory, 16-byte aligned, of
 * qpn_workspace_bytes(QPN_OP_PREFILL_*, m, n, k) bytes for the preferred
 * plan (NULL with 0 bytes is valid and runs whole tiles per workgroup);
 * every call leaves it zero-filled.  Output tiles cut between workgroups are
 * summed in an order fixed by the launch (a pairwise tree over the pieces,
 * or each output in piece order), so results are deterministic.  m > 256 gives QPN_ERR_SHAPE.  A blob whose
 * header does not match gives FP16 NaN outputs.  One kernel on `stream`. */
QPN_API int qpn_gemm_prefill_nvfp4(const void *packed, const uint16_t *x, uint16_t *y,
                                   int m, int64_t n, int64_t k, void *workspace,
                                   size_t workspace_bytes, void *stream);
QPN_API int qpn_gemm_prefill_fp8(const void *packed, const uint16_t *x, uint16_t *y, int m,
                                 int64_t n, int64_t k, void *workspace,
                                 size_t workspace_bytes, void *stream);

/* NVFP4 lm_head with fused greedy argmax (taozi.news section "自研 QPN 内核",
 * the native 4-bit lm_head; section "一些工程细节与长上下文发现", drafts
 * proposed by greedy / local argmax).  Computes logits exactly as
 * qpn_gemm_nvfp4 and, per row m, argmax[m] = the lowest index n whose FP16
 * logit equals the row maximum (values compared as numbers: -0 == +0).
 * n >= 1 is required.  workspace: zero-filled device memory of at least
 * 8 * m * 256 bytes (qpn_workspace_bytes(QPN_OP_LMHEAD_NVFP4, m, n, k) for
 * the preferred plan).  Two kernels on `stream`. */
QPN_API int qpn_lmhead_nvfp4(const void *packed, const uint16_t *x, uint16_t *logits,
                     int32_t *argmax, int m, int64_t n, int64_t k,
                     void *workspace, size_t workspace_bytes, void *stream);

/* NVFP4 lm_head, fused argmax and greedy verification of one speculative
 * round (taozi.news section "自研 QPN 内核": M=8 is the verify step of a
 * round with k=7 drafts; section "一些工程细节与长上下文发现": drafts come
 * from greedy / local argmax and the round is checked without host
 * synchronisation).  Row i of x is the input at position i of the round,
 * so argmax[i] is the target's token after it; draft[i] (i < m - 1) is the
 * drafter's token at that position.  The greedy acceptance read here:
 * result[0] = L, the length of the longest prefix with draft[i] ==
 * argmax[i], and result[1] = argmax[L], the target's token that follows
 * the accepted drafts (the correction, or the bonus token when all m - 1
 * are accepted).  logits and argmax as qpn_lmhead_nvfp4; everything stays
 * on the device, in stream order.  draft: m - 1 int32 device values (may
 * be NULL when m == 1); result: 2 int32 device values, 4-byte aligned.
 * Same workspace and failure behaviour as qpn_lmhead_nvfp4; m == 0 writes
 * nothing.  Two kernels on `stream`. */
QPN_API int qpn_lmhead_verify_nvfp4(const void *packed, const uint16_t *x,
                                    uint16_t *logits, int32_t *argmax,
                                    const int32_t *draft, int32_t *result, int m,
                                    int64_t n, int64_t k, void *workspace,
                                    size_t workspace_bytes, void *stream);

/* --- test exports: the device-side layout and decode, for parity checks --- */

/* Canonical export of an NVFP4 blob: codes [n, k/2] (element 2j in the low
 * nibble of byte j), scales [n, k/16], tensor scale g (1 float).  All three
 * are device pointers.  Reads the blob with the same layout map the GEMM
 * uses. */
QPN_API int qpn_debug_unpack_nvfp4(const void *packed, int64_t n, int64_t k,
                           uint8_t *codes, uint8_t *scales, float *g,
                           void *stream);

/* Canonical export of an FP8 blob: codes [n, k], row scales [n] FP32. */
QPN_API int qpn_debug_unpack_fp8(const void *packed, int64_t n, int64_t k,
                         uint8_t *codes, float *row_scale, void *stream);

/* Runs the GEMM's own NVFP4 register decode on `count` fragments: fragment
 * i is 16 code bytes codes16[16 i ..] (32 E2M1 codes, low nibble first) and
 * 2 UE4M3 bytes scales2[2 i ..] (first for codes 0..15, second for 16..31).
 * out[32 i + e] is the FP16 operand the matrix unit receives for code e,
 * which equals E2M1(code) * UE4M3(scale) exactly.  Scale bytes must be
 * <= 0x7E.  Device pointers; out must be 16-byte aligned. */
QPN_API int qpn_debug_decode_nvfp4(const uint8_t *codes16, const uint8_t *scales2,
                           int64_t count, uint16_t *out, void *stream);

/* Runs the GEMM's own FP8 register decode: fragment i is 16 E4M3 bytes;
 * out[16 i + e] is the FP16 operand for byte e, which equals E4M3(byte)
 * exactly for every byte except the NaN codes 0x7F and 0xFF.  out must be
 * 16-byte aligned. */
QPN_API int qpn_debug_decode_fp8(const uint8_t *codes16, int64_t count,
                         uint16_t *out, void *stream);

/* Diagnostic: the launch plan compiled plan `plan` gives a call of kind
 * `op` (QPN_OP_GEMM_NVFP4, QPN_OP_GEMM_FP8 or QPN_OP_LMHEAD_NVFP4) with
 * (m, n, k), given all the workspace it asks for.  Plan ids 1..13 select a
 * fixed (wavefronts per panel, panels per workgroup, prefetch depth,
 * contraction) configuration; 11 and 12 repeat 2 and 1 with VALU dot
 * products in place of the MFMA (valu_dot = 1), 13 is the eight-panel plan
 * of large-N calls; 0 is the automatic choice (the same answer as
 * qpn_gemm_plan).  The outputs are those of qpn_gemm_plan plus valu_dot and
 * workspace_bytes, the workspace the call uses with that plan (as
 * qpn_workspace_bytes does for the automatic one).  Any output pointer may
 * be NULL.  QPN_ERR_SHAPE for an unknown op or plan id or an invalid shape.
 * A pure function of its arguments; pure host. */
QPN_API int qpn_debug_plan(int op, int plan, int m, int64_t n, int64_t k,
                           int64_t *workgroups, int *waves_per_panel,
                           int *panels_per_workgroup, int *prefetch_depth, int *splits,
                           int *activation_rows, int64_t *split_workgroups, int *valu_dot,
                           size_t *workspace_bytes);

/* Diagnostic: qpn_gemm_nvfp4 (op QPN_OP_GEMM_NVFP4), qpn_gemm_fp8
 * (QPN_OP_GEMM_FP8) or qpn_lmhead_nvfp4 (QPN_OP_LMHEAD_NVFP4, `y` being the
 * logits and `argmax` its argmax output) run with compiled launch plan
 * `plan` instead of the automatic choice (0 = automatic), for A/B timing and
 * parity tests of every configuration on identical inputs.  `argmax` is
 * ignored by the GEMM ops.  Arguments, workspace rules and failure
 * behaviour as the entry point it runs; QPN_ERR_SHAPE for an unknown op or
 * plan id.  Touches no state outside its arguments. */
QPN_API int qpn_debug_run_plan(int op, int plan, const void *packed, const uint16_t *x,
                               uint16_t *y, int32_t *argmax, int m, int64_t n, int64_t k,
                               void *workspace, size_t workspace_bytes, void *stream);

/* Diagnostic: qpn_gemm_prefill_nvfp4 (op QPN_OP_PREFILL_NVFP4) or
 * qpn_gemm_prefill_fp8 (QPN_OP_PREFILL_FP8) with no waiting: where a tile
 * is cut between workgroups that sum it in shares, none waits for the
 * others, so the last one to arrive sums every share (the path taken when a
 * wait runs out).  The results are bit-identical to the entry point's.
 * Arguments, workspace rules and failure behaviour as that entry point;
 * QPN_ERR_SHAPE for another op.  Touches no state outside its arguments. */
QPN_API int qpn_debug_prefill_no_wait(int op, const void *packed, const uint16_t *x, uint16_t *y,
                                      int m, int64_t n, int64_t k, void *workspace,
                                      size_t workspace_bytes, void *stream);

/* Diagnostic: reads `bytes` (a multiple of 16, at most 2^40) of device
 * memory at `buf` once with the same nontemporal 16-byte loads the GEMM
 * kernels use; *sink is written only if a fold of the data equals a fixed
 * constant (so the loads cannot be elided).  Timing it gives the measured
 * HBM read ceiling that bandwidth is also reported against, as the
 * taozi.news and aiwitness.kr pages report theirs against a measured
 * read-only limit. */
QPN_API int qpn_debug_read_ceiling(const void *buf, size_t bytes, uint32_t *sink,
                                   void *stream);

#ifdef __cplusplus
}
#endif

#endif /* QPN_H */
