/*
 * varlen_attn.h -- C ABI of the MI355X (gfx950) ragged THD attention library.
 *
 * Scaled-dot-product attention over ragged, THD-packed batches: a forward pass
 * that also emits the softmax statistics (log-sum-exp, LSE), and a backward
 * pass producing dQ, dK and dV.  Every entry point only validates host-visible
 * arguments and enqueues HIP kernels on the caller's stream; it allocates
 * nothing, keeps no state between calls, copies nothing between host and
 * device and never synchronises, so it can be captured in a HIP graph.
 *
 * Addressing (cudnn-frontend issue on padded THD, sections "Concrete failure"
 * and "Proposal: consume the bound offsets on device"): row i of sequence b of
 * tensor X, head h, element d lives at
 *
 *     X.data[X.ragged[b] + i * X.stride_t + h * X.stride_h + d]
 *
 * with X.ragged a caller-bound device array of element offsets, one array per
 * tensor, so Q/O padding may differ from K/V padding.  Offsets are never
 * re-derived from the sequence lengths.  Lengths come from the cumulative
 * valid-length arrays: Lq(b) = cu_seqlens_q[b+1] - cu_seqlens_q[b], likewise
 * Lk(b) from cu_seqlens_kv; they bound the mask and decide dead rows.
 *
 * Mask (per sequence; TransformerEngine PR #3274, "Description" and the
 * reviewer's policy mapping; Megatron-LM PR #14 commit message for the
 * diagonals): key j is visible to row i iff j < Lk(b) and either the policy is
 * VARLEN_ATTN_PADDING or j <= i + delta(b), where delta(b) is
 *   0                    for VARLEN_ATTN_CAUSAL_TOP_LEFT,
 *   Lk(b) - Lq(b)        for VARLEN_ATTN_CAUSAL_BOTTOM_RIGHT,
 *   q_causal_offset[b]   for either causal policy when that array is given
 *                        (the absolute key index of the segment's q[0]).
 * Sliding window (TransformerEngine PR #3274, "Description": a window size
 * per mask type beside the per-sequence policy): policy p may carry a window
 * (left_p, right_p), -1 meaning unbounded on that side.  With the anchor
 * a(b) = q_causal_offset[b] when given, else 0 for top-left and Lk(b) - Lq(b)
 * for bottom-right and padding, key j is further restricted to
 * i + a(b) - left_p <= j <= i + a(b) + right_p on the bounded sides.
 * A row with no visible key is dead: O = 0, LSE = -inf, dQ = 0.
 *
 * LSE is the natural-log log-sum-exp of the scaled, masked scores, fp32, in
 * any strided layout: token-major [t, h] (stride_t = H_q, stride_h = 1) or
 * head-major [h, t] (stride_t = 1, stride_h >= rows), each with its own ragged
 * offsets in its own element units (cudnn-frontend PR #462, "What").
 *
 * Buffers the kernels never write: pad rows between or around sequences,
 * gap columns of strided views, rows of invalid sequences.  Those elements of
 * O, LSE, dQ, dK and dV keep their previous contents bit for bit.
 *
 * Data types: Q, K, V, O, dO, dQ, dK, dV share one 16-bit element type, bf16
 * or IEEE fp16 (TransformerEngine PR #3274, "Description": the per-sequence
 * policy path supports FP16 and BF16 THD attention), stored as 16-bit
 * patterns and rounded to nearest even on output; products accumulate in
 * fp32.  LSE and the scale are fp32.
 */
#ifndef VARLEN_ATTN_H
#define VARLEN_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---------------------------------------------------------------- codes */

/* Host return codes.  A nonzero code means nothing was enqueued. */
enum {
  VARLEN_ATTN_OK = 0,
  VARLEN_ATTN_ERR_NULL = 1,        /* a required pointer is NULL */
  VARLEN_ATTN_ERR_BATCH = 2,       /* batch < 0 */
  VARLEN_ATTN_ERR_HEAD_DIM = 3,    /* head_dim not 64 or 128 */
  VARLEN_ATTN_ERR_HEADS = 4,       /* h_q or h_kv < 1, or h_q % h_kv != 0 */
  VARLEN_ATTN_ERR_ALIGN = 5,       /* 16-bit data not 16-byte aligned, LSE not
                                      4-byte aligned, workspace not 256-byte
                                      aligned */
  VARLEN_ATTN_ERR_STRIDE = 6,      /* 16-bit strides not multiples of 8, or a
                                      stride smaller than one row/head, or
                                      larger than the span, or 127 * stride_t
                                      + head_dim elements (a 128-row tile)
                                      reaching 2^31 bytes: tiles are
                                      addressed with 32-bit byte offsets */
  VARLEN_ATTN_ERR_SPAN = 7,        /* span_elems smaller than one row */
  VARLEN_ATTN_ERR_WORKSPACE = 8,   /* workspace NULL or too small */
  VARLEN_ATTN_ERR_POLICY = 9,      /* default_policy not 0, 1 or 2 */
  VARLEN_ATTN_ERR_SCALE = 10,      /* scale not finite */
  VARLEN_ATTN_ERR_HIP = 11,        /* a HIP launch failed */
  VARLEN_ATTN_ERR_OFFSETS = 12,    /* a tensor gives both `ragged` and
                                      `ragged_scaled`, or ragged_multiplier is
                                      outside [1, 2^31) */
  VARLEN_ATTN_ERR_WINDOW = 13,     /* a window_size entry below -1 */
  VARLEN_ATTN_ERR_DTYPE = 14,      /* dtype not VARLEN_ATTN_BF16 or _F16 */
  VARLEN_ATTN_ERR_SCRATCH = 15     /* varlen_attn_fwd_noalloc: the forward
                                      workspace this problem needs exceeds
                                      VARLEN_ATTN_NOALLOC_SCRATCH_BYTES */
};

/* Size of the static per-GPU workspace of varlen_attn_fwd_noalloc. */
#define VARLEN_ATTN_NOALLOC_SCRATCH_BYTES (4u << 20)

/* Element types of the 16-bit tensors. */
enum {
  VARLEN_ATTN_BF16 = 0,
  VARLEN_ATTN_F16 = 1
};

/* Mask policies (TransformerEngine names: padding, padding_causal,
 * padding_causal_bottom_right). */
enum {
  VARLEN_ATTN_PADDING = 0,
  VARLEN_ATTN_CAUSAL_TOP_LEFT = 1,
  VARLEN_ATTN_CAUSAL_BOTTOM_RIGHT = 2
};

/* Device status bits.  Device-resident arguments (lengths, offsets,
 * policies) cannot be checked on the host without the device-to-host read
 * the pages rule out (cudnn-frontend issue on padded THD, "Proposal").  The
 * setup kernel checks them instead: an offending sequence is skipped (its
 * outputs stay untouched) and its bits are ORed into *dev_status. */
enum {
  VARLEN_ATTN_ST_NEG_LENGTH = 1,     /* Lq < 0 or Lk < 0 */
  VARLEN_ATTN_ST_BAD_OFFSET = 2,     /* ragged[b] < 0, or a 16-bit tensor's
                                        ragged[b] not a multiple of 8 */
  VARLEN_ATTN_ST_OUT_OF_SPAN = 4,    /* a row of the sequence would reach past
                                        span_elems */
  VARLEN_ATTN_ST_BAD_POLICY = 8,     /* mask_policy[b] not 0, 1 or 2 */
  VARLEN_ATTN_ST_LIST_OVERFLOW = 16, /* more tiles than the output buffers'
                                        rows can hold (sequences overlap):
                                        nothing is computed */
  VARLEN_ATTN_ST_KV_OVERLAP = 32     /* backward only: the sequence's dK or dV
                                        rows intersect those of a sequence
                                        outside its kv group (see
                                        varlen_attn_bwd); every sequence of
                                        both groups is skipped */
};

/* ---------------------------------------------------------------- types */

/* One ragged tensor as the caller binds it.  All pointers are device
 * pointers owned by the caller.  Element strides; the innermost (head_dim)
 * stride is 1.  `span_elems` is the number of elements addressable from
 * `data` (the allocation's or view's element span, not the count of valid
 * tokens: cudnn-frontend PR #462, review of the sizing helper and "Not
 * addressed here").
 *
 * The offset of sequence b's row 0 (in elements from `data`) is given in
 * exactly one of two forms; entry `batch` (past-the-end) is not used for
 * addressing:
 *   ragged         int64 [batch + 1] element offsets, or
 *   ragged_scaled  int32 [batch + 1] values in units of ragged_multiplier
 *                  elements: offset = ragged_scaled[b] * ragged_multiplier,
 *                  formed on the device (cuDNN's ragged-offset multiplier,
 *                  cudnn-frontend issue on padded THD, "What needs
 *                  checking").  One row-offset array such as a padded
 *                  cu_seqlens then serves every tensor, each with its own
 *                  multiplier (its stride_t).
 * The unused pointer is NULL; ragged_multiplier is ignored with `ragged`. */
typedef struct varlen_attn_tensor {
  void* data;
  int64_t span_elems;
  int64_t stride_t;
  int64_t stride_h;
  const int64_t* ragged;
  const int32_t* ragged_scaled;
  int64_t ragged_multiplier;
} varlen_attn_tensor;

/* The problem.  cu_seqlens_q/kv: device int32 [batch+1] cumulative valid
 * lengths.  mask_policy: device int8 [batch] or NULL (then default_policy
 * applies to every sequence).  q_causal_offset: device int32 [batch] or NULL
 * (then each causal policy uses its own alignment).  window_size: HOST int32
 * [6] = {left, right} for padding, top-left, bottom-right, each >= -1 (else
 * VARLEN_ATTN_ERR_WINDOW), read during the call only; NULL means no window
 * for any policy.  dtype: VARLEN_ATTN_BF16 (0) or VARLEN_ATTN_F16 (1), the
 * element type of Q, K, V, O, dO, dQ, dK and dV.  GQA: query head h reads
 * key/value head h / (h_q / h_kv). */
typedef struct varlen_attn_problem {
  int32_t batch;
  int32_t h_q;
  int32_t h_kv;
  int32_t head_dim;
  float scale;
  const int32_t* cu_seqlens_q;
  const int32_t* cu_seqlens_kv;
  const int8_t* mask_policy;
  int32_t default_policy;
  const int32_t* q_causal_offset;
  const int32_t* window_size;
  int32_t dtype;
} varlen_attn_problem;

/* Byte offsets of the workspace regions (each 256-byte aligned) and the tile
 * sizes the kernels use.  Regions are separate so that no buffer can run into
 * another's counters (cudnn-frontend PR #462, "Root cause": an overrun of one
 * intermediate clobbered the next region's tile counter).
 *   counters  int32[64]  tile-claim counters, zeroed by the setup kernel
 *   header    int32[16]  [0] forward tiles, [1] backward tiles, [2] status
 *   seq       int32 lq[B], lk[B], policy[B], hi[B], lo[B], flags[B] (flags:
 *             bit 0 valid, status bits << 8; key j visible to row i iff
 *             i + lo <= j <= i + hi and j < Lk, hi and lo clamped to
 *             [-Lq, Lk], both 0 for invalid sequences), then at
 *             seq + seq_i64_offset int64 base[9][B] in the order Q, K, V, O,
 *             LSE, dO, dQ, dK, dV
 *   fwd_tiles int32[2 * capacity]: (b, t) for the t-th tile of fwd_block_m
 *             query rows of sequence b
 *   bwd_tiles int32[4 * capacity]: (m, members, u, max Lk) for the u-th tile
 *             of bwd_block_n key rows of a kv group (the sequences that bind
 *             the same K, V, dK and dV offsets), whose members are
 *             member_list[m .. m + members)
 *   members   int32[B] member_list: each kv group's sequences in ascending
 *             index, groups in the order of bwd_tiles
 *   scratch   setup kernel scratch
 *   delta     fp32 -rowsum(dO * O), same element offsets as LSE (backward
 *             only)
 *   lse_term  fp32 -LSE * log2(e) / max(|scale * log2(e)|, 1e-30), same
 *             element offsets as LSE (backward only): the row term that
 *             the backward kernels start their score accumulators from */
typedef struct varlen_attn_layout {
  int64_t total_bytes;
  int64_t counters_offset;
  int64_t header_offset;
  int64_t seq_offset;
  int64_t seq_i64_offset;
  int64_t fwd_tiles_offset;
  int64_t fwd_tiles_capacity;
  int64_t bwd_tiles_offset;
  int64_t bwd_tiles_capacity;
  int64_t members_offset;
  int64_t scratch_offset;
  int64_t delta_offset;
  int64_t delta_elems;
  int64_t lse_term_offset;
  int32_t fwd_block_m;
  int32_t fwd_block_n;
  int32_t bwd_block_m;
  int32_t bwd_block_n;
} varlen_attn_layout;

/* ---------------------------------------------------------------- sizing */

/* Workspace layout of a forward call.  Host only (reads no device memory).
 * The tile capacity comes from o's physical row capacity,
 * floor((span - 1 - (h_q-1)*stride_h - (D-1)) / stride_t) + 1, plus batch:
 * never from the number of valid tokens. */
int varlen_attn_fwd_workspace_layout(const varlen_attn_problem* p, const varlen_attn_tensor* o,
                                     varlen_attn_layout* out);

/* Workspace layout of a backward call.  delta and lse_term mirror lse
 * element for element, so it is sized from the caller's span of lse, which counts every
 * axis (cudnn-frontend PR #462, "The fix (commit 1)": size from every stride
 * axis; a head-major [h, t] LSE needs h*t elements, not t).  Host only. */
int varlen_attn_bwd_workspace_layout(const varlen_attn_problem* p, const varlen_attn_tensor* lse,
                                     const varlen_attn_tensor* dq, const varlen_attn_tensor* dk,
                                     varlen_attn_layout* out);

/* total_bytes of the layouts above. */
int varlen_attn_fwd_workspace_size(const varlen_attn_problem* p, const varlen_attn_tensor* o,
                                   size_t* bytes);
int varlen_attn_bwd_workspace_size(const varlen_attn_problem* p, const varlen_attn_tensor* lse,
                                   const varlen_attn_tensor* dq, const varlen_attn_tensor* dk,
                                   size_t* bytes);

/* ---------------------------------------------------------------- compute */

/* Forward.  For every valid sequence b, query head h and row i < Lq(b):
 *   S = scale * Q_b,h K_b,g(h)^T over the keys visible to the row (the mask
 *   above), LSE_i = log sum_j exp(S_ij) and O_i = sum_j exp(S_ij - LSE_i) V_j,
 * i.e. scaled-dot-product attention per sequence, addressed through the bound
 * per-tensor offsets (cudnn-frontend issue on padded THD, "Concrete failure"
 * and "Proposal: consume the bound offsets on device"; per-sequence policy in
 * one launch: TransformerEngine PR #3274, "Description"; LSE as the stats
 * output with its own offsets and layout: cudnn-frontend PR #462, "What").
 * Dead rows get O = 0 and LSE = -inf.
 *   q, k, v    16-bit inputs; read only at valid rows of valid sequences
 *   o          16-bit output [rows, h_q, D] (any strides)
 *   lse        fp32 output [rows, h_q] (any strides, e.g. token- or
 *              head-major)
 *   workspace  device, 256-byte aligned, at least
 *              varlen_attn_fwd_workspace_size bytes; overwritten
 *   dev_status device int32 or NULL: device status bits are ORed in
 *              (atomic); the caller clears it
 *   stream     hipStream_t (NULL: the default stream)
 * Only valid rows of valid sequences are written.  batch == 0 returns
 * VARLEN_ATTN_OK with nothing enqueued.  Returns a host code; on nonzero
 * nothing was enqueued.  The caller owns every buffer; the call allocates
 * nothing and does not synchronise. */
int varlen_attn_fwd(const varlen_attn_problem* p, const varlen_attn_tensor* q,
                    const varlen_attn_tensor* k, const varlen_attn_tensor* v,
                    const varlen_attn_tensor* o, const varlen_attn_tensor* lse, void* workspace,
                    size_t workspace_bytes, int32_t* dev_status, void* stream);

/* Forward without a workspace argument, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation).  Same arguments (minus the workspace), results and
 * host codes as varlen_attn_fwd, whose kernels it runs.  Its workspace is a
 * static array of VARLEN_ATTN_NOALLOC_SCRATCH_BYTES (4 MiB) that the library
 * holds on each GPU it runs on until the process ends; a problem whose
 * varlen_attn_fwd_workspace_size exceeds it returns VARLEN_ATTN_ERR_SCRATCH
 * with nothing enqueued (the size grows with the batch and the output rows:
 * about 204 bytes per sequence plus 8 bytes per 128 rows of o).  Nothing is
 * allocated: the array's device address is looked up once per device, at the
 * first call with that device current.  All calls on one GPU share the
 * array, so calls that overlap in time on one GPU (other streams, other host
 * threads) race and must not be issued; calls in order on one stream are
 * fine. */
int varlen_attn_fwd_noalloc(const varlen_attn_problem* p, const varlen_attn_tensor* q,
                            const varlen_attn_tensor* k, const varlen_attn_tensor* v,
                            const varlen_attn_tensor* o, const varlen_attn_tensor* lse,
                            int32_t* dev_status, void* stream);

/* Backward.  The gradients of sum(dO * O) for the forward above, given dout
 * (dO) and the forward's o and lse:
 *   delta_i = sum_d dO_id O_id,  P = exp(S - LSE),  dV = P^T dO,
 *   dS = P o (dO V^T - delta),   dQ = scale dS K,   dK = scale dS^T Q,
 * with the stats row-sum intermediate laid out on LSE's own strides and the
 * workspace sized from every stride axis (cudnn-frontend PR #462, "Root
 * cause" and "The fix (commit 1)").  Writes dq, dk, dv (16-bit) for valid
 * rows only.
 *   kv groups: sequences whose K, V, dK and dV offsets are all identical
 *   share those key rows (context-parallel query chunks of one document,
 *   Megatron-LM PR #14, commit message), wherever they sit in the batch;
 *   their dK and dV are the sums over the group.  A group owns rows
 *   [0, max Lk) of dK and dV, the element ranges [offset, offset +
 *   max Lk * stride_t).  When two groups' ranges intersect in dK or in dV,
 *   every sequence of both groups is skipped (dQ, dK and dV untouched) and
 *   VARLEN_ATTN_ST_KV_OVERLAP is set: one group's gradients would otherwise
 *   overwrite the other's without an error (cudnn-frontend issue on padded
 *   THD, "Concrete failure").  Distinct buffers for dq, dk and dv, and
 *   disjoint rows between query-side outputs of different sequences, are
 *   the caller's contract (not checked).
 * Workspace, status and stream as for the forward; the workspace size comes
 * from varlen_attn_bwd_workspace_size. */
int varlen_attn_bwd(const varlen_attn_problem* p, const varlen_attn_tensor* q,
                    const varlen_attn_tensor* k, const varlen_attn_tensor* v,
                    const varlen_attn_tensor* o, const varlen_attn_tensor* dout,
                    const varlen_attn_tensor* lse, const varlen_attn_tensor* dq,
                    const varlen_attn_tensor* dk, const varlen_attn_tensor* dv, void* workspace,
                    size_t workspace_bytes, int32_t* dev_status, void* stream);

/* The setup kernel alone, as the forward (varlen_attn_fwd_setup) or the
 * backward (varlen_attn_bwd_setup) runs it first.  It reads the caller's
 * device offsets, lengths and policies on the device (cudnn-frontend issue on
 * padded THD, "Proposal: consume the bound offsets on device": one base per
 * tensor, no device-to-host read) and writes per-sequence metadata, validity,
 * kv groups and tile lists into the workspace regions described by
 * varlen_attn_layout.  Same arguments and codes as the full calls. */
int varlen_attn_fwd_setup(const varlen_attn_problem* p, const varlen_attn_tensor* q,
                          const varlen_attn_tensor* k, const varlen_attn_tensor* v,
                          const varlen_attn_tensor* o, const varlen_attn_tensor* lse,
                          void* workspace, size_t workspace_bytes, int32_t* dev_status,
                          void* stream);
int varlen_attn_bwd_setup(const varlen_attn_problem* p, const varlen_attn_tensor* q,
                          const varlen_attn_tensor* k, const varlen_attn_tensor* v,
                          const varlen_attn_tensor* o, const varlen_attn_tensor* dout,
                          const varlen_attn_tensor* lse, const varlen_attn_tensor* dq,
                          const varlen_attn_tensor* dk, const varlen_attn_tensor* dv,
                          void* workspace, size_t workspace_bytes, int32_t* dev_status,
                          void* stream);

/* One stage at a time, for callers that schedule or time the stages
 * themselves.  Each takes the same arguments as the full call, enqueues one
 * kernel, and reads what the matching *_setup call (same arguments, earlier
 * on the same stream, same workspace) wrote there.  The full calls are
 * exactly: varlen_attn_fwd = fwd_setup, fwd_attention;
 * varlen_attn_bwd = bwd_setup, bwd_dq, bwd_dkdv.
 *   fwd_attention    O and LSE of every listed tile (the forward's
 *                    definition above)
 *   bwd_dq           dQ (16-bit), query-major: Q/dO resident, K/V tiles
 *                    streamed; also writes the row terms -delta =
 *                    -rowsum(dO * O) and lse_term (fp32, in the workspace,
 *                    on LSE's element offsets: cudnn-frontend PR #462,
 *                    "Root cause")
 *   bwd_dkdv         dK and dV (16-bit), key-major: K/V resident, query tiles
 *                    of every member of the kv group streamed (Megatron-LM
 *                    PR #14, commit message); reads the row terms, so it
 *                    follows bwd_dq */
int varlen_attn_fwd_attention(const varlen_attn_problem* p, const varlen_attn_tensor* q,
                              const varlen_attn_tensor* k, const varlen_attn_tensor* v,
                              const varlen_attn_tensor* o, const varlen_attn_tensor* lse,
                              void* workspace, size_t workspace_bytes, int32_t* dev_status,
                              void* stream);
int varlen_attn_bwd_dkdv(const varlen_attn_problem* p, const varlen_attn_tensor* q,
                         const varlen_attn_tensor* k, const varlen_attn_tensor* v,
                         const varlen_attn_tensor* o, const varlen_attn_tensor* dout,
                         const varlen_attn_tensor* lse, const varlen_attn_tensor* dq,
                         const varlen_attn_tensor* dk, const varlen_attn_tensor* dv,
                         void* workspace, size_t workspace_bytes, int32_t* dev_status,
                         void* stream);
int varlen_attn_bwd_dq(const varlen_attn_problem* p, const varlen_attn_tensor* q,
                       const varlen_attn_tensor* k, const varlen_attn_tensor* v,
                       const varlen_attn_tensor* o, const varlen_attn_tensor* dout,
                       const varlen_attn_tensor* lse, const varlen_attn_tensor* dq,
                       const varlen_attn_tensor* dk, const varlen_attn_tensor* dv,
                       void* workspace, size_t workspace_bytes, int32_t* dev_status,
                       void* stream);

/* Static text for a host return code. */
const char* varlen_attn_status_string(int code);

#ifdef __cplusplus
}
#endif

#endif /* VARLEN_ATTN_H */
