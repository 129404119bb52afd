/*
 * mxattn.h -- C ABI of the MXFP4 block quantizer and MXFP4 attention for
 * AMD Instinct MI355X (gfx950).
 *
 * What is computed (sources cited by page title and section):
 *  - MXFP4 blocks: 32 consecutive elements share one power-of-two E8M0 scale
 *    2^(X-127); each element is an E2M1 code (magnitudes 0, 0.5, 1, 1.5, 2,
 *    3, 4, 6 plus a sign bit).  Rounding onto those magnitudes is the only
 *    error; the scale applies exactly ("Quantization Error", section "Where
 *    the error comes from"; OCP Microscaling Formats v1.0).
 *  - Scale rules: OCP (the baseline) chooses the smallest exponent e with
 *    amax < 8 * 2^e; Universal Optimal Scaling (UOS) chooses the smallest e
 *    with amax <= 7.25 * 2^e ("MXAttention: Data-Free Optimal Scaling and
 *    Pre-Normalization Quantization for MXFP4 Attention", abstract:
 *    boundary Qmax = 7.25).  e is clamped to >= -127; an all-zero block gets
 *    X = 0.  Elements round to the nearest magnitude, ties to the even code,
 *    saturating at 6.
 *  - Attention: QK^T and P~V as block-scaled FP4 contractions inside a
 *    FlashAttention-style online softmax whose row-max update, history
 *    rescaling, fp32 accumulation and final normalization are unchanged
 *    ("EFQ-Softmax", abstract).  In UOS+PNQ mode the unnormalized
 *    exponentials exp(s - m) are quantized in blocks of 32 keys before the
 *    row sum, and the same P~ feeds both the numerator P~V and the
 *    denominator P~1 (MXAttention abstract, Pre-Normalization
 *    Quantization).  In the OCP and UOS modes P is quantized with the same
 *    rule for P~V but the denominator sums the unquantized P.
 *
 * Layout conventions.
 *  - Packed codes: element 2j in the low nibble of byte j, element 2j+1 in
 *    the high nibble; bit 3 of a code is the sign.  Scales: one byte per 32
 *    elements.
 *  - Attention tensors are contiguous [B, H, S, D] (row-major, D fastest).
 *    Query head h reads KV head h / (Hq / Hkv).  Softmax scale 1/sqrt(D).
 *    Causal masking keeps keys j <= i and requires Sq == Skv.
 *
 * Ownership and errors.
 *  - Every pointer argument is a DEVICE pointer owned by the caller, except
 *    where marked host.  The library never allocates, frees or synchronizes;
 *    all work is enqueued on `stream` (a hipStream_t passed as void*; NULL is
 *    the default stream) and returns before it completes.
 *  - Arguments are validated before any HIP call.  Functions return MX_OK or
 *    a negative mx_status; a failed launch returns MX_ERR_HIP.  Device
 *    pointers must be 16-byte aligned unless stated otherwise
 *    (MX_ERR_ALIGN).
 */
#ifndef MXATTN_H
#define MXATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum mx_status {
    MX_OK = 0,
    MX_ERR_ARG = -1,         /* null pointer, bad enum, bad size */
    /* valid but not implemented: e.g. D not 64/128, or a size whose element
       count or launch passes the library's limits (Q or K/V of more than
       2^40 elements; any launch of 2^32 or more work items in one grid
       dimension, e.g. mxq_quantize with n >= 2^36, mxq_dequantize with
       n >= 2^35, K/V tile images of 2^35 or more padded elements) */
    MX_ERR_UNSUPPORTED = -2,
    MX_ERR_WORKSPACE = -3,   /* workspace missing or too small */
    MX_ERR_HIP = -4,         /* a HIP launch or runtime call failed */
    MX_ERR_ALIGN = -5        /* a device pointer is not 16-byte aligned */
};

enum mx_dtype { MX_F32 = 0, MX_BF16 = 1 };
enum mxq_mode { MXQ_OCP = 0, MXQ_UOS = 1 };
enum mxattn_mode {
  MXATTN_FP16 = 0,
  MXATTN_OCP = 1,
  MXATTN_UOS = 2,
  MXATTN_UOS_PNQ = 3,
  /* UOS operands; P~ by the exp-free EFQ rule (see mxattn_fwd); PNQ denominator */
  MXATTN_UOS_EFQ = 4
};

/* Human-readable text of a status code (static storage). */
const char *mx_strerror(int status);

/*
 * Block-quantize a flat tensor along its contiguous axis.
 *  x      [n] elements of `dtype` (MX_F32 or MX_BF16)
 *  n      element count, n % 32 == 0, n >= 0 (n == 0 is a no-op)
 *  mode   MXQ_OCP or MXQ_UOS (scale rule)
 *  codes  [n/2] bytes out;  scales [n/32] bytes out (E8M0)
 * Inputs must be finite (NaN/Inf give unspecified codes).
 */
int mxq_quantize(const void *x, int64_t n, int dtype, int mode,
                 uint8_t *codes, uint8_t *scales, void *stream);

/*
 * Block-quantize `batch` row-major matrices [rows][cols] along their ROWS
 * (blocks of 32 consecutive rows in one column) and store them transposed:
 *  codes_t  [batch][cols][rows_pad/2],  scales_t [batch][cols][rows_pad/32]
 * rows_pad: output row length in elements; 0 means ceil(rows/32)*32;
 * otherwise a multiple of 32 that is >= rows.  Rows beyond `rows` are
 * quantized as zeros (codes 0, scale byte 0 for all-padding blocks).
 * This is the layout of V~ (blocks along keys) in MXFP4 attention.
 */
int mxq_quantize_t(const void *x, int64_t batch, int64_t rows, int64_t cols,
                   int dtype, int mode, int64_t rows_pad, uint8_t *codes_t,
                   uint8_t *scales_t, void *stream);

/*
 * Dequantize n elements (n % 32 == 0) to `out_dtype` (MX_F32 or MX_BF16):
 * y = sign * magnitude(code) * 2^(X-127).  Exact unless the value lies
 * outside the output type's range (then +-inf) or X == 255 (NaN).
 */
int mxq_dequantize(const uint8_t *codes, const uint8_t *scales, int64_t n,
                   int out_dtype, void *y, void *stream);

/*
 * Workspace needed by mxattn_fwd (and mxattn_prepare, mxattn_fwd_prepared,
 * mxattn_fwd_varlen without a dump) for these sizes and mode (bytes; 0 for
 * invalid arguments).  The workspace holds the quantized K/V operands (MX
 * modes: the KV tile images, followed by one 32-bit arrival counter per
 * (b, KV head) that the short-query calls use (mxattn_prepare and
 * mxattn_prepare_varlen set them to 0) and the prefill kernel's 8-word work
 * queue (cleared by every attention call before its kernel)) or the 16-bit
 * operands (FP16 mode).
 * mxattn_dump_workspace_bytes: the larger workspace of the dump entry points
 * (mxattn_fwd_dump, mxattn_fwd_varlen with a dump), which also receives the
 * kernel's Q~; 0 for the FP16 mode, which has no dump.
 */
size_t mxattn_workspace_bytes(int B, int Hq, int Hkv, int Sq, int Skv, int D,
                              int dtype, int mode);
size_t mxattn_dump_workspace_bytes(int B, int Hq, int Hkv, int Sq, int Skv,
                                   int D, int dtype, int mode);

/*
 * Where the quantized operands of an MX mode lie inside the workspace (host
 * array `off` of 6 entries):
 *   off[2] KV tile images [B][Hkv][skv_ld/128][off[3]], at offset 0
 *   off[0] Q~ codes [B][Hq][Sq][D/2]      off[1] Q~ scales [B][Hq][Sq][D/32]
 *          after the images, the arrival counters (B*Hkv 32-bit words
 *          rounded to 256 bytes) and the work queue (256 bytes), inside the
 *          dump workspace only (written only
 *          by the dump entry points: the attention kernels quantize Q
 *          themselves, and the dump variants store that Q~ here; the
 *          short-query workspace always holds these regions)
 *   off[3] bytes per image (17408 for D = 128, 9216 for D = 64)
 *   off[4] = off[5] = 0
 * and *skv_ld (host) = Skv rounded up to a multiple of the 128-key tile.
 * Image of KV tile T (keys 128T .. 128T+127), all offsets in bytes, in the
 * operand order of the 32 x 32 x 64 block-scaled FP4 matrix instruction
 * (lane l of an operand: row l%32, 32 elements of K-block l/32):
 *   [0, 64D)        K~ codes, [subtile t < 4][d-half i < D/64][lane l < 64]
 *                   [16]: lane l of (t, i) holds key 128T + 64*(t/2) +
 *                   32*((R/4)%2) + 16*(t%2) + 4*(R/8) + R%4 with R = l%32,
 *                   elements 32*(2i + l/32) .. +31 (one 32-element block
 *                   along D)
 *   [64D, 128D)     V~ codes, [channel tile c < D/32][key step s < 2][lane l]
 *                   [16]: lane l of (c, s) holds channel 32c + l%32, keys
 *                   128T + 64s + 32*(l/32) .. +31 (one 32-key block along
 *                   keys)
 *   [128D, 132D)    K~ scales [lane l][t*(D/64) + i], E8M0
 *   [132D, 136D)    V~ scales [lane l][2c + s], E8M0
 *   then zero padding to a multiple of 1 KiB.
 * Codes pack two E2M1 elements per byte, the lower-indexed one in the low
 * nibble.  Keys at or past Skv are quantized as zeros (codes 0, scale 0).
 * Returns MX_ERR_ARG for the FP16 mode.
 */
int mxattn_workspace_layout(int B, int Hq, int Hkv, int Sq, int Skv, int D,
                            int dtype, int mode, size_t *off, int64_t *skv_ld);

/*
 * Keys per KV tile (Bc) of the attention kernel for this head size and mode
 * (128 in the MX modes, 64 in the FP16 mode).  The running max -- and hence
 * the scale of every P~ block -- is updated once per tile, in ascending key
 * order, so a reference must use the same Bc to reproduce P~ (the FP16 mode
 * has no P~; there Bc only changes rounding).  Returns a negative status for
 * unsupported D.
 */
int mxattn_kv_tile(int D, int mode);

/*
 * Attention forward.
 *  q [B][Hq][Sq][D], k and v [B][Hkv][Skv][D], contiguous, dtype MX_F32 or
 *  MX_BF16.  D in {64, 128}; Hq % Hkv == 0; Sq, Skv >= 1; causal (0/1)
 *  requires Sq == Skv.
 *  o [B][Hq][Sq][D] fp32 out.
 *  workspace: >= mxattn_workspace_bytes(...) bytes, 256-byte aligned,
 *  overwritten.  Modes: MXATTN_FP16 (16-bit operands, no quantization),
 *  MXATTN_OCP, MXATTN_UOS, MXATTN_UOS_PNQ, MXATTN_UOS_EFQ.  MXATTN_UOS_EFQ
 *  ("EFQ-Softmax", abstract; constants are a reading, not the page's):
 *  UOS operands and PNQ denominator, with each P~ block generated without
 *  exp: z = log2 of the unnormalized probability, block exponent e = the
 *  smallest e >= -127 with z_max - e < (7.5 - beta)/2 - 2^-10, code =
 *  clamp(round-half-even(2 (z - e) + beta), 0, 7), beta = 1.8678023 (the
 *  least-squares fit of this rule to the E2M1 rounding boundaries of
 *  codes 2..7).
 * In the MX modes the call first quantizes K (blocks along D) and V (blocks
 * along keys) into the workspace as KV tile images in matrix-core operand
 * order, then runs the fused attention kernel, which reads Q itself and
 * quantizes each 32-element block of it (blocks along D, the mode's scale
 * rule) as it loads it; the codes equal mxq_quantize's.  In FP16 mode, V
 * (and, for fp32 inputs, Q and K) is first converted to fp16 in the
 * workspace.
 */
int mxattn_fwd(const void *q, const void *k, const void *v, int dtype,
               int B, int Hq, int Hkv, int Sq, int Skv, int D, int causal,
               int mode, float *o, void *workspace, size_t ws_bytes,
               void *stream);

/*
 * The two halves of mxattn_fwd, for callers that reuse prepared operands or
 * time the attention kernel alone.
 * mxattn_prepare: fills the workspace -- MX modes: K~ / V~ (blocks along D /
 * along keys) as KV tile images (see mxattn_workspace_layout; q is checked
 * but not read);
 * FP16 mode: K and V^T as 16-bit tile images of 64 keys (K bf16 for bf16
 * inputs, else fp16; V fp16), and fp16 Q for fp32 inputs.
 * mxattn_fwd_prepared: the fused attention kernel alone, reading the
 * operands a previous mxattn_prepare with the same sizes, dtype and mode
 * left in the workspace (in the MX modes it also writes the workspace's
 * small work-queue region, which schedules the kernel's query tiles over
 * the XCDs: calls that overlap on one workspace race), and q (quantized in the kernel in the MX modes,
 * read directly in FP16 mode with bf16 inputs; only FP16 mode with fp32
 * inputs does not read it, and then it may be NULL).  k is not read and may
 * be NULL.  Arguments as for mxattn_fwd.  mxattn_fwd == mxattn_prepare followed by mxattn_fwd_prepared.
 */
int mxattn_prepare(const void *q, const void *k, const void *v, int dtype,
                   int B, int Hq, int Hkv, int Sq, int Skv, int D, int mode,
                   void *workspace, size_t ws_bytes, void *stream);
int mxattn_fwd_prepared(const void *q, const void *k, int dtype, int B,
                        int Hq, int Hkv, int Sq, int Skv, int D, int causal,
                        int mode, float *o, void *workspace,
                        size_t ws_bytes, void *stream);

/*
 * mxattn_fwd plus a dump of the quantized probabilities P~ of selected rows
 * (MX modes only; slower).  row_slot [B*Hq*Sq] int32: for query row
 * (b*Hq + h)*Sq + i, the dump slot (>= 0) or -1.  p_codes
 * [nslots][skv_ld/2] and p_scales [nslots][skv_ld/32] receive, for every
 * key block a slot's row visits, its packed codes and E8M0 byte; blocks the
 * row never visits (beyond the causal diagonal tile) are left untouched.
 * The kernel's Q~ (every row) is stored at off[0] / off[1] of the workspace,
 * which must hold mxattn_dump_workspace_bytes(...) bytes (MX_ERR_WORKSPACE).
 */
int mxattn_fwd_dump(const void *q, const void *k, const void *v, int dtype,
                    int B, int Hq, int Hkv, int Sq, int Skv, int D, int causal,
                    int mode, float *o, void *workspace, size_t ws_bytes,
                    const int32_t *row_slot, uint8_t *p_codes,
                    uint8_t *p_scales, void *stream);

/*
 * Short-query attention over key splits (decode): the same attention as
 * mxattn_fwd for few queries against many keys, with the keys cut into
 * splits of mxattn_decode_split(B, Hkv, Skv) keys (a multiple of the
 * 128-key tile, counted from key 0).  Each split runs the tiled online
 * softmax on its own, from m = -inf ("EFQ-Softmax", abstract: running-max
 * update, history rescaling, final normalization), so the P~ blocks of a
 * split are scaled by that split's running max; the splits are then merged
 * in ascending order by rescaling to the largest max.  One wave handles the
 * (Hq/Hkv) x Sq queries of one GQA group on one split, reading the group's
 * K~/V~ once.
 *
 * Arguments as for mxattn_fwd, except: causal queries are aligned to the
 * end of the keys (query i sees keys j <= i + Skv - Sq; Sq <= Skv);
 * (Hq/Hkv) * Sq <= 32 and an MX mode (MXATTN_OCP .. MXATTN_UOS_EFQ), else
 * MX_ERR_UNSUPPORTED (FP16 mode and longer query blocks: mxattn_fwd); the
 * workspace holds mxattn_decode_workspace_bytes(...) bytes (the
 * mxattn_prepare layout followed by the per-split partial states).
 * Q is quantized inside the split kernel (as in mxattn_fwd).
 * One kernel: each wave leaves its split's (m, l, unnormalized O) in the
 * workspace and counts itself in its group's arrival counter; the wave that
 * completes the count merges the group's splits into o and returns the
 * counter to 0, so the next call on the workspace finds it cleared (no
 * memset: the calls can be captured into a graph and replayed).  Calls that
 * overlap on one workspace race.
 * mxattn_decode_prepared runs that kernel on a workspace that
 * mxattn_prepare filled (which also cleared the counters), for the queries
 * q (k, v are not taken: a quantized KV cache is reused across calls; q
 * must not be NULL).
 * mxattn_decode_dump also writes the P~ codes and E8M0 bytes of selected
 * rows, and the kernel's Q~, as mxattn_fwd_dump.
 * mxattn_decode_split returns MX_ERR_ARG, and the workspace size 0, for bad
 * arguments.
 */
int mxattn_decode_split(int B, int Hkv, int Skv);
size_t mxattn_decode_workspace_bytes(int B, int Hq, int Hkv, int Sq, int Skv,
                                     int D, int dtype, int mode);
int mxattn_decode(const void *q, const void *k, const void *v, int dtype,
                  int B, int Hq, int Hkv, int Sq, int Skv, int D, int causal,
                  int mode, float *o, void *workspace, size_t ws_bytes,
                  void *stream);
int mxattn_decode_prepared(const void *q, int dtype, int B, int Hq, int Hkv,
                           int Sq, int Skv, int D, int causal, int mode,
                           float *o, void *workspace, size_t ws_bytes,
                           void *stream);
int mxattn_decode_dump(const void *q, const void *k, const void *v, int dtype,
                       int B, int Hq, int Hkv, int Sq, int Skv, int D,
                       int causal, int mode, float *o, void *workspace,
                       size_t ws_bytes, const int32_t *row_slot,
                       uint8_t *p_codes, uint8_t *p_scales, void *stream);

/*
 * Sequences of different lengths in one padded batch: per entry, exactly the
 * attention of mxattn_fwd / mxattn_decode on that entry's own rows and keys
 * (the pages time their kernels over sequence lengths of 16K to 128K,
 * "EFQ-Softmax", abstract, and fix no batching).  q [B][Hq][Sq][D] and
 * k, v [B][Hkv][Skv][D] as for mxattn_fwd / mxattn_decode, Sq and Skv being
 * the padded extents; seqlens_q and seqlens_k are DEVICE int32 arrays of B
 * entries: batch entry b holds seqlens_q[b] query rows and seqlens_k[b]
 * keys (values are clamped to [0, Sq] and [0, Skv]; the host does not read
 * them).  Keys at or past seqlens_k[b] take no part in entry b: K~ and V~
 * are quantized as if they were zero (so V~'s 32-key blocks end as at Skv),
 * and they are masked.  Query rows at or past seqlens_q[b] are not written
 * (their o rows keep their contents).  Causal queries are aligned to the
 * end of the entry's keys (row i sees keys j <= i + seqlens_k[b] -
 * seqlens_q[b]); an entry with no key, or a causal entry with more query
 * rows than keys, writes no row.
 *
 * mxattn_fwd_varlen: the prefill form (per-entry query and key lengths); MX
 * modes only (MXATTN_FP16 gives MX_ERR_UNSUPPORTED); Sq and Skv may differ
 * also when causal.  Workspace as for mxattn_fwd (mxattn_fwd_dump's size
 * with a dump).
 * mxattn_decode_varlen: the short-query form (every entry has Sq query
 * rows, seqlens_k[b] keys: a padded KV cache), split as mxattn_decode with
 * the split size of the padded Skv; workspace as for mxattn_decode.
 * Both: row_slot, p_codes, p_scales are all NULL (no dump) or all set (the
 * P~ and Q~ dump of mxattn_fwd_dump, rows past an entry's length never
 * dumped, nor the Q~ rows of an entry that writes no row); a mix gives
 * MX_ERR_ARG, as does a NULL seqlens pointer.
 * mxattn_prepare_varlen / mxattn_decode_varlen_prepared: the two halves of
 * mxattn_decode_varlen, for a KV cache quantized once and read by many
 * calls (as mxattn_prepare / mxattn_decode_prepared): the first writes the
 * KV tile images with keys past seqlens_k[b] quantized as zero (MX modes;
 * q is checked, not read; the arrival counters cleared); the second runs
 * the short-query kernel for the queries q with the same seqlens_k (k and v
 * are not taken).
 */
int mxattn_fwd_varlen(const void *q, const void *k, const void *v, int dtype,
                      int B, int Hq, int Hkv, int Sq, int Skv, int D,
                      const int32_t *seqlens_q, const int32_t *seqlens_k,
                      int causal, int mode, float *o, void *workspace,
                      size_t ws_bytes, const int32_t *row_slot,
                      uint8_t *p_codes, uint8_t *p_scales, void *stream);
int mxattn_prepare_varlen(const void *q, const void *k, const void *v,
                          int dtype, int B, int Hq, int Hkv, int Sq, int Skv,
                          int D, const int32_t *seqlens_k, int mode,
                          void *workspace, size_t ws_bytes, void *stream);
int mxattn_decode_varlen_prepared(const void *q, int dtype, int B, int Hq,
                                  int Hkv, int Sq, int Skv, int D,
                                  const int32_t *seqlens_k, int causal,
                                  int mode, float *o, void *workspace,
                                  size_t ws_bytes, void *stream);
int mxattn_decode_varlen(const void *q, const void *k, const void *v,
                         int dtype, int B, int Hq, int Hkv, int Sq, int Skv,
                         int D, const int32_t *seqlens_k, int causal,
                         int mode, float *o, void *workspace, size_t ws_bytes,
                         const int32_t *row_slot, uint8_t *p_codes,
                         uint8_t *p_scales, void *stream);

/*
 * W4A4 product of two MXFP4 operands ("MXCode: Vector Quantization for
 * MX-Native Inference at Scale", abstract: MX-native W4A4 operands; the
 * 32-element blocks and E8M0 scales of the OCP MX format):
 *
 *   y[m][n] = sum_k deq(a)[m][k] * deq(b)[n][k],   accumulated in fp32.
 *
 *   a_codes  [M][K/2], a_scales [M][K/32]: a [M][K] exactly as mxq_quantize
 *            writes a row-major tensor (blocks of 32 along K, element 2j in
 *            the low nibble of byte j, one E8M0 byte per block).  For a
 *            linear layer: the activations, one row per token.
 *   b_codes  [N][K/2], b_scales [N][K/32]: likewise b [N][K] (the weight,
 *            one row per output feature).
 *   y        [M][N] row-major: fp32 (out_dtype MX_F32) or bf16 (MX_BF16,
 *            rounded to nearest even).
 *
 *   workspace: at least mxgemm_workspace_bytes(M, N, K) bytes of device
 *            memory, 256-byte aligned, that the call overwrites (the
 *            operands' E8M0 bytes re-laid out for the kernel); calls that
 *            run concurrently need separate workspaces.
 *
 * M, N >= 1; K >= 128 and K % 128 == 0, else MX_ERR_UNSUPPORTED (the
 * matrix instruction consumes 128 K-elements, four blocks, at a time).
 * M, N < 2^31.  All pointers are device memory owned by the caller; codes
 * and y must be 16-byte aligned (MX_ERR_ALIGN); a NULL pointer or bad
 * out_dtype gives MX_ERR_ARG; a missing or short workspace
 * MX_ERR_WORKSPACE.  Asynchronous on stream; allocates nothing; y must not
 * overlap the operands.  mxgemm_workspace_bytes returns 0 for bad sizes.
 */
size_t mxgemm_workspace_bytes(int64_t M, int64_t N, int64_t K);
int mxgemm(const uint8_t *a_codes, const uint8_t *a_scales,
           const uint8_t *b_codes, const uint8_t *b_scales, int64_t M,
           int64_t N, int64_t K, int out_dtype, void *y, void *workspace,
           size_t ws_bytes, void *stream);

/*
 * mxgemm without a workspace argument, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  Same arguments, result and errors as
 * mxgemm minus workspace/ws_bytes; the same kernels run.  The staging that
 * mxgemm keeps in the caller's workspace lives instead in a scratch array of
 * the library: 32 MiB of device memory per GPU, reserved when the library
 * is loaded on that GPU and held until the process ends.  Shapes whose
 * staging, mxgemm_workspace_bytes(M, N, K), exceeds 32 MiB give
 * MX_ERR_UNSUPPORTED (e.g. M = 32760, N = 13824 fits up to K = 23040).  The
 * call allocates and frees nothing; the first call on a GPU looks up that
 * GPU's address of the array (MX_ERR_HIP if the lookup fails).  Every call
 * on one GPU uses that GPU's one array, so calls that can run at the same
 * time on one GPU (different streams, or host threads) race and give wrong
 * results: serialize them, or use mxgemm with separate workspaces.
 */
int mxgemm_noalloc(const uint8_t *a_codes, const uint8_t *a_scales,
                   const uint8_t *b_codes, const uint8_t *b_scales, int64_t M,
                   int64_t N, int64_t K, int out_dtype, void *y, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* MXATTN_H */
