/*
 * sharq.h -- C ABI of the SharQ linear-layer hot path on AMD Instinct MI355X
 * (gfx950).
 *
 * SharQ ("SharQ: Bridging Activation Sparsity and FP4 Quantization for LLM
 * Inference") approximates a linear layer Y = X W, X in R^{T x K},
 * W in R^{K x D} (xllm-io paper review, §3.1), by an online sparse-dense
 * decomposition of the activations:
 *
 *   y      = RMSNorm(x)                       (fused preparation, review §3.5)
 *   X_sp   = M(y) ⊙ y, M = 4:8 in-pairs mask  (review §3.2; kasblo explainer,
 *                                              4:8 in-pairs section)
 *   X~_sp  = D_sp(Q_sp(X_sp))                 (review §3.3)
 *   R      = y - X~_sp                        (review §3.3)
 *   Y^     = GEMM_sp(Q_sp(X_sp), Q_w,sp(W)) + GEMM_dn(Q_dn(R), Q_w,dn(W))
 *                                             (review §3.4)
 *
 * with one shared FP4 weight payload seen through a sparse and a dense scale
 * view, and the dense path accumulating into the sparse path's output tile
 * (review §3.5).  Three calls implement it: sharq_pack_weight (offline),
 * sharq_prepare and sharq_linear (per forward).
 *
 * Conventions for every entry point:
 *  - Pointers marked (device) are device pointers on the current HIP device;
 *    (host) pointers are read or written synchronously before the call
 *    returns.  The caller allocates and owns every buffer; the library never
 *    allocates device memory, never synchronizes and keeps no state between
 *    calls (entry points are reentrant).
 *  - `stream` is a hipStream_t (NULL = the default stream).  All device work
 *    is enqueued on it; outputs are valid once that stream has reached the
 *    call's work.
 *  - Arguments are validated on the host before anything is enqueued; a call
 *    that returns an error has enqueued nothing.  SHARQ_ERR_HIP reports a
 *    failed kernel launch; faults inside kernels surface at the caller's next
 *    synchronization.  sharq_last_error() gives a message for the last error
 *    of the calling thread.
 *  - Device buffers must be 16-byte aligned.  Row strides are in elements.
 *  - K must be a multiple of 32 (the scale block); the GEMM also needs
 *    K % 128 == 0.  T, D >= 1.
 *
 * Number formats (exact bits; written from the pages plus the readings stated
 * with each):
 *  - E2M1 (FP4): codes 0..7 have magnitudes {0,0.5,1,1.5,2,3,4,6}, bit 3 is
 *    the sign.  Rounding is to nearest, ties to the even code, saturating at
 *    6; the sign is copied from the input.  Two codes per byte, the even K
 *    index in the low nibble.
 *  - MXFP4 block scale (E8M0 byte e+127): e is the smallest integer with
 *    amax <= 6 * 2^e over the 32-value block, clamped to [-127, 127]
 *    (review §3.1 scale max|x| / alpha rounded up to a power of two, review
 *    §5.3 power-of-two MXFP4 scale).
 *  - NVFP4 (emulated): fp32 tensor scale s_T = amax / 2688 (1 for an
 *    all-zero tensor), E4M3 (OCP FP8, saturating at 448) block scale of
 *    (amax_b / 6) / s_T, element codes E2M1(x / (dec * s_T)) in fp32 (review
 *    §3.1 two-level NVFP4 scaling; kasblo explainer: 16 E2M1 + one E4M3).
 */
#ifndef SHARQ_H
#define SHARQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  SHARQ_OK = 0,
  SHARQ_ERR_INVALID_ARGUMENT = 1,   /* null pointer, bad enum, misaligned, bad stride */
  SHARQ_ERR_UNSUPPORTED_SHAPE = 2,  /* K % 32 (GEMM: K % 128), T/D < 1, sizes too large */
  SHARQ_ERR_FORMAT_MISMATCH = 3,    /* activation and weight formats or K differ */
  SHARQ_ERR_WORKSPACE_TOO_SMALL = 4,
  SHARQ_ERR_HIP = 5                 /* a HIP runtime call or kernel launch failed */
} sharq_status;

/* SHARQ_MXFP4_24: MXFP4 activations whose backbone uses the 2:4 element-wise
 * mask (review §3.2 general N:M mask; the pattern the pages pair with MXFP4)
 * instead of 4:8 in pairs: per group of 4 K-values the 2 largest |y| are
 * kept (ties to the lower index); bb_codes holds one byte per group of 4 (the
 * kept codes, lower index in the low nibble), bb_meta one nibble per group
 * of 4 (i0 | i1 << 2, even group in the low nibble: T x K/8 bytes).  An
 * activation format only: it multiplies SHARQ_MXFP4 weights. */
typedef enum { SHARQ_MXFP4 = 0, SHARQ_NVFP4_EMU = 1, SHARQ_MXFP4_24 = 2 } sharq_format;
typedef enum { SHARQ_F32 = 0, SHARQ_BF16 = 1 } sharq_dtype;

/* Packed weight: n_groups stacked matrices (n_groups experts; 1 for a plain
 * linear), each K x D before packing.  Row d of a group's payload holds
 * column d of W (K contiguous).  Review §3.5: one shared FP4 payload, sparse
 * view with one scale per 32 K-values, dense view with one scale per 16
 * K-values holding each per-32 scale twice. */
typedef struct {
  int32_t fmt;           /* sharq_format */
  int32_t K, D;          /* per group */
  int32_t n_groups;      /* >= 1 */
  uint8_t *payload;      /* (device) n_groups x D x K/2 E2M1 codes                          */
  uint8_t *scale_sp;     /* (device) n_groups x D x K/32 (MXFP4 E8M0 | NVFP4 E4M3)          */
  uint8_t *scale_dn;     /* (device) MXFP4: n_groups x D x K/32, identical to scale_sp (may
                                     alias it); NVFP4: n_groups x D x K/16, each sp scale twice */
  float *tensor_scale;   /* (device) NVFP4: n_groups fp32 tensor scales; MXFP4: unused (NULL) */
} sharq_weight;

/* Prepared activations of T rows (review §3.5 fused preparation output).
 *  bb_codes: per group of 8 K-values, the two bytes (pairs) of the backbone
 *            the 4:8 in-pairs mask kept, ascending pair order (2 of 4 bytes);
 *  bb_meta:  per group the nibble i0 | i1 << 2 of the kept pairs (i0 < i1),
 *            even group in the low nibble;
 *  bb_scale: backbone scale per 32 K-positions (16 kept values);
 *  res_codes/res_scale: the dense FP4 residual R = y - X~_sp. */
typedef struct {
  int32_t fmt;           /* sharq_format */
  int32_t T, K;
  uint8_t *bb_codes;     /* (device) T x K/4                                   */
  uint8_t *bb_meta;      /* (device) T x K/16 (2:4: T x K/8)                    */
  uint8_t *bb_scale;     /* (device) T x K/32                                  */
  uint8_t *res_codes;    /* (device) T x K/2                                   */
  uint8_t *res_scale;    /* (device) T x K/32 (MXFP4) | T x K/16 (NVFP4)       */
  float *tensor_scales;  /* (device) NVFP4: 2 fp32 {backbone, residual}; MXFP4: NULL */
} sharq_act;

/* Buffer sizes in bytes of a packed weight: bytes_out[0..4] = payload,
 * scale_sp, scale_dn, tensor_scale, workspace of sharq_pack_weight.
 * (host) bytes_out.  Errors: INVALID_ARGUMENT, UNSUPPORTED_SHAPE. */
sharq_status sharq_weight_sizes(int32_t fmt, int32_t K, int32_t D, int32_t n_groups,
                                size_t bytes_out[5]);

/* Buffer sizes in bytes of prepared activations: bytes_out[0..6] = bb_codes,
 * bb_meta, bb_scale, res_codes, res_scale, tensor_scales, workspace of
 * sharq_prepare.  (host) bytes_out. */
sharq_status sharq_act_sizes(int32_t fmt, int32_t T, int32_t K, size_t bytes_out[7]);

/* Offline weight packer (review §3.5 shared payload with two scale views).
 * W: (device) n_groups matrices K x D of `dtype` (sharq_dtype), element (k, d)
 * of group g at W[g * group_stride + k * ldw + d]; ldw >= D.
 * out: (host) struct whose fields describe the destination buffers (device),
 * sized by sharq_weight_sizes; out->K/D/n_groups/fmt must match.
 * workspace: (device) scratch of sharq_weight_sizes()[4] bytes (NVFP4: the
 * tensor amax reduction; MXFP4: may be NULL when 0 bytes are needed).
 * Errors: INVALID_ARGUMENT, UNSUPPORTED_SHAPE, WORKSPACE_TOO_SMALL, HIP. */
sharq_status sharq_pack_weight(const void *W, int32_t dtype, int32_t K, int32_t D, int32_t n_groups,
                               int64_t ldw, int64_t group_stride, const sharq_weight *out,
                               void *workspace, size_t workspace_bytes, void *stream);

/* Fused activation preparation (review §3.2-§3.5): RMSNorm (fp32, sum of
 * squares as a pairwise tree in K order, no fused multiply-add), 4:8 in-pairs
 * mask (pair score = max |y| of the pair, keep the 2 highest of 4 pairs,
 * ties to the lower pair), backbone quantization and compaction, residual
 * R = y - X~_sp (exact in fp32) and its quantization.
 * X: (device) T x K of `dtype`, row t at X + t * ldx (ldx >= K).
 * gamma: (device) K fp32 RMSNorm weights, or NULL for no normalization (y = x).
 * Input domain of the RMSNorm: every x_k * x_k and the row's sum of squares
 * must be finite in fp32 (a single |x| above about 1.8e19 already overflows).
 * Outside it the sum is +inf, 1/rms is 0 and the row is prepared as signed
 * zeros (deterministic, identical to the fp32 order above; not a supported
 * use).  Non-finite inputs give unspecified codes.
 * out: (host) struct describing (device) outputs sized by sharq_act_sizes.
 * workspace: (device) sharq_act_sizes()[6] bytes (NVFP4 tensor amax
 * partials; MXFP4 needs 0 and may pass NULL).
 * Bit-exact: identical inputs give identical bytes on every call.
 * Errors: INVALID_ARGUMENT, UNSUPPORTED_SHAPE, WORKSPACE_TOO_SMALL, HIP. */
sharq_status sharq_prepare(const void *X, int32_t dtype, int32_t T, int32_t K, int64_t ldx,
                           const float *gamma, float eps, const sharq_act *out,
                           void *workspace, size_t workspace_bytes, void *stream);

/* Allocation-free sharq_prepare, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc): the same outputs as sharq_prepare, bit for bit, with
 * the NVFP4 preparation's scratch taken from a static device array of the
 * library (1 MiB per GPU, held until the process ends) instead of a caller
 * workspace.  MXFP4 formats need no scratch.  Calls that overlap on one GPU
 * share that array and race: order them (one stream, or events).  Nothing
 * is allocated; the array's device address is looked up once per device.
 * Arguments as sharq_prepare.  Errors: as sharq_prepare, and
 * UNSUPPORTED_SHAPE when the NVFP4 scratch (4 T + 8 ceil(T / rows per
 * workgroup) + 256 bytes, sharq_act_sizes()[6]) exceeds 1 MiB. */
sharq_status sharq_prepare_no_alloc(const void *X, int32_t dtype, int32_t T, int32_t K, int64_t ldx,
                                    const float *gamma, float eps, const sharq_act *out, void *stream);

/* Dual-path FP4 GEMM (review §3.4-§3.5): Y^ = X~_sp W~ + R~ W~ with one
 * accumulator per output tile (the dense path accumulates into the sparse
 * path's tile); the backbone runs zero-filled through dense scaled MFMA
 * (gfx950 has no sparse MFMA taking FP4 operands).
 * a: (host) prepared activations; w: (host) packed weight, a->fmt == w->fmt
 * and a->K == w->K.
 * Plain linear (w->n_groups == 1): group_offsets NULL; output row r reads
 * activation row row_index[r] if row_index != NULL (device int32
 * [total_rows], each < a->T), else row r (total_rows == a->T).
 * Grouped (w->n_groups = E > 1): group_offsets (device int32 [E+1],
 * nondecreasing, [0] = 0, [E] = total_rows): rows group_offsets[e] ..
 * group_offsets[e+1]-1 use expert e's weights; row_index as above.
 * Y: (device) fp32 total_rows x D, row r at Y + r * ldy (ldy >= D).
 * Size limit: a->T * K / 2 and D * K / 2 (one group's payload) must each
 * stay under 2 GiB - 256 bytes (buffer offsets below bit 31), else
 * UNSUPPORTED_SHAPE.
 * Errors: INVALID_ARGUMENT, UNSUPPORTED_SHAPE, FORMAT_MISMATCH, HIP. */
sharq_status sharq_linear(const sharq_act *a, const sharq_weight *w, const int32_t *group_offsets,
                          const int32_t *row_index, int32_t total_rows, float *Y, int64_t ldy,
                          void *stream);

/* Single-launch decode (review §3.5: preparation fused ahead of the dual-
 * path GEMM, here in the same kernel launch): sharq_prepare of the T rows
 * of X into act, then sharq_linear(act, w) into Y (plain linear: row t of Y
 * from activation row t, total_rows = T).  For T <= 8 and K <= 16384, and
 * for 9 <= T <= 16 and K <= 7168, one kernel does both: its first T workgroups prepare one row each and signal
 * through counters in `workspace`; the GEMM workgroups stream their weights
 * meanwhile and wait (bounded polling) before reading the activations.
 * Larger shapes run sharq_prepare's and sharq_linear's kernels one after the
 * other.  Either way act holds exactly sharq_prepare's bytes and Y exactly
 * sharq_linear's values.
 * X, dtype, T, K, ldx, gamma, eps: as sharq_prepare; act: (host) MXFP4
 * activation buffers for T rows; w: (host) MXFP4 weight, n_groups == 1;
 * Y, ldy: as sharq_linear.
 * workspace: (device) >= 16 bytes, 16-byte aligned, all zero before the
 * first call; the library keeps four uint32 words there across calls (a
 * running count of prepared rows, a per-call base, a count of GEMM
 * workgroups past their wait, a sticky error word).  Calls that share a
 * workspace must not overlap: run them on one stream (or order them), and
 * give each stream that calls concurrently its own workspace.
 * Failure mode: a GEMM workgroup that waits for the prepared rows longer
 * than a bound (about a second; a correct call waits microseconds) gives
 * up, sets the sticky error word and writes NaN into its columns of Y; every
 * later call on that workspace also writes NaN into Y until the caller
 * clears the workspace.  The kernel always terminates.
 * sharq_prepare_linear_status reports the word.
 * Errors: INVALID_ARGUMENT (also for NVFP4 or n_groups > 1),
 * UNSUPPORTED_SHAPE, FORMAT_MISMATCH, WORKSPACE_TOO_SMALL, HIP. */
sharq_status sharq_prepare_linear(const void *X, int32_t dtype, int32_t T, int32_t K, int64_t ldx,
                                  const float *gamma, float eps, const sharq_act *act,
                                  const sharq_weight *w, float *Y, int64_t ldy, void *workspace,
                                  size_t workspace_bytes, void *stream);

/* Status of a sharq_prepare_linear workspace: SHARQ_OK, or SHARQ_ERR_HIP when
 * a single-launch decode on it gave up waiting (its Y holds NaN; see the
 * failure mode above).  Unlike the other calls this one synchronizes: it
 * copies the workspace's words to the host on `stream` and waits for them.
 * workspace: (device) the workspace, >= 16 bytes, 16-byte aligned.
 * Errors: WORKSPACE_TOO_SMALL, INVALID_ARGUMENT, HIP. */
sharq_status sharq_prepare_linear_status(const void *workspace, size_t workspace_bytes, void *stream);

/* ---- Plain baseline (the unfused pipeline the fused preparation replaces,
 * xllm-io paper review §5 kernel latency breakdown): RMSNorm, plain MXFP4
 * quantization and a dense one-operand MXFP4 GEMM as three launches, for
 * timing and error comparisons against the SharQ path. ---- */

/* RMSNorm of T rows into fp32 y, with the fused preparation's pinned order
 * (so y is bit-identical to the y that sharq_prepare quantizes).
 * X: (device) T x K of `dtype`, row t at X + t * ldx; gamma: (device) K fp32
 * or NULL (y = x); Y: (device) fp32 T x K, row t at Y + t * ldy (ldy >= K,
 * rows 16-byte aligned).  K % 32 == 0, K <= the sharq_prepare maximum.
 * Errors: INVALID_ARGUMENT, UNSUPPORTED_SHAPE, HIP. */
sharq_status sharq_rmsnorm(const void *X, int32_t dtype, int32_t T, int32_t K, int64_t ldx,
                           const float *gamma, float eps, float *Y, int64_t ldy, void *stream);

/* Plain MXFP4 quantization of fp32 rows (review §3.1 block scale rounded up
 * to a power of two, §5.3): per 32-block e = the smallest integer with
 * amax <= 6 * 2^e (E8M0 code e + 127), codes = E2M1 RNE of y / 2^e.
 * Y: (device) fp32 T x K, row t at Y + t * ldy (rows 16-byte aligned);
 * codes: (device) T x K/2 (two codes per byte, even K index in the low
 * nibble); scales: (device) T x K/32.  K % 32 == 0.
 * Errors: INVALID_ARGUMENT, UNSUPPORTED_SHAPE, HIP. */
sharq_status sharq_quantize_mx(const float *Y, int32_t T, int32_t K, int64_t ldy, uint8_t *codes,
                               uint8_t *scales, void *stream);

/* Dense one-operand MXFP4 GEMM Y = X~ W~ (fp32 accumulation) on the prefill
 * tile kernel: the plain FP4 linear the dual-path GEMM is compared with.
 * codes, scales: (device) plain MXFP4 activations as sharq_quantize_mx
 * writes them (T rows); w: (host) MXFP4 weight, n_groups == 1, its dense
 * scale view is used; Y: (device) fp32 T x D, row t at Y + t * ldy.
 * w->K % 512 == 0; the size limits of sharq_linear apply (T * K / 2 and
 * D * K / 2 under 2 GiB - 256 bytes).
 * Errors: INVALID_ARGUMENT, UNSUPPORTED_SHAPE, FORMAT_MISMATCH, HIP. */
sharq_status sharq_linear_dense(const uint8_t *codes, const uint8_t *scales, int32_t T,
                                const sharq_weight *w, float *Y, int64_t ldy, void *stream);

/* ---- Tile timeline (tracing).  The library built with SHARQ_TIMELINE
 * defined (`python -m sparsity_sharq_prepare_amd.build --timeline` writes
 * libsharq_timeline.so beside libsharq.so) has the tile GEMM of
 * sharq_linear (MXFP4, more than 64 rows) record, from wave 0 of each tile,
 * s_memrealtime stamps (a 100 MHz clock): word 0 the tile's start, word 1
 * after its first step's wait and barrier, word 2 after its last step,
 * word 3 after its epilogue stores are issued; word 4 holds the XCC id (high
 * half) and the hardware id register (low half), word 5 the workgroup
 * index, words 6 and 7 are zero.  The persistent 128-row tile (grouped
 * linears, at most 256 experts) writes record t for tile t of its tile
 * order; the 256-row tile writes record b for workgroup b.  Each launch
 * overwrites the records it writes, so read after the launch of interest.
 * The normal build exports the same entry points: its record count is 0
 * and clear / read return INVALID_ARGUMENT.
 * sharq_timeline_records: (host) out, the number of 8-word records.
 * sharq_timeline_clear: zeroes every record (synchronous, device-wide).
 * sharq_timeline_read: copies the first `words` words to `host` (host
 * memory, synchronous); words <= 8 * records.
 * Errors: INVALID_ARGUMENT, HIP. */
sharq_status sharq_timeline_records(size_t *records);
sharq_status sharq_timeline_clear(void);
sharq_status sharq_timeline_read(uint64_t *host, size_t words);

/* Static string naming a status code. */
const char *sharq_status_string(sharq_status s);

/* Message describing the last error returned on the calling thread ("" if none). */
const char *sharq_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* SHARQ_H */
